// mla_api.cpp - the C ABI (include/mla_decode.h): argument checks, the work
// plan, and the launches. The caller-facing steps follow the FlashMLA
// overview page (flash_api.cpp walk-through): compute the split metadata once
// per decode step, then run the attention call once per layer; the bridge
// checks its inputs and orchestrates the kernels.
#include "../../include/mla_decode.h"
#include "../../include/mla_decode_fp8.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <mutex>
#include <vector>

#include "mla_common.h"
#include "mla_internal.h"
#include "mla_sched.h"

namespace mla {

namespace {

constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];
std::once_flag g_cu_once[kMaxDevices];

// Compute units of the current device (0 if none).
int current_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 0;
    }
    std::call_once(g_cu_once[dev], [dev]() {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
            (void)hipGetLastError();
            n = 0;
        }
        g_cu_count[dev] = n;
    });
    return g_cu_count[dev];
}

// Process-wide overrides of the kernel choice and of where split sequences
// are merged (mla_set_plan_override); -1 keeps the plan's own choice.
std::atomic<int> g_kernel_override{-1};
std::atomic<int> g_merge_override{-1};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Benchmark timing: three events per recorded call (before decode, between
// decode and combine, after combine), pooled and reused. They are created
// without the system-scope fence a default event performs when it completes
// (an L2 writeback and invalidate): they only time work, and that fence
// would add microseconds to every kernel they bracket.
struct CallEvents {
    hipEvent_t ev[3];
};
struct Timing {
    std::mutex mu;
    bool on = false;
    std::vector<CallEvents> pool;
    size_t used = 0;
};
Timing g_timing;
constexpr size_t kMaxTimedCalls = 4096;

// Events for the next call, or nullptr when timing is off or full.
CallEvents* timing_slot() {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (!g_timing.on || g_timing.used >= kMaxTimedCalls) return nullptr;
    if (g_timing.used == g_timing.pool.size()) {
        CallEvents ce{};
        for (int i = 0; i < 3; ++i) {
            if (hipEventCreateWithFlags(&ce.ev[i], hipEventDisableSystemFence) != hipSuccess) {
                (void)hipGetLastError();
                for (int j = 0; j < i; ++j) (void)hipEventDestroy(ce.ev[j]);
                return nullptr;
            }
        }
        g_timing.pool.push_back(ce);
    }
    return &g_timing.pool[g_timing.used++];
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

bool make_plan(int batch, int h_q, int s_q, int num_partitions, int num_cus, Plan* plan, bool fp8) {
    if (batch < 1 || h_q < 1 || s_q < 1) return false;
    const long long m = (long long)h_q * s_q;
    if (m > MLA_MAX_ROWS) return false;
    if (num_partitions > 65536) return false;
    Plan pl{};
    pl.batch = batch;
    pl.h_q = h_q;
    pl.s_q = s_q;
    pl.M = (int)m;
    // Kernel choice (mla_set_plan_override can force one): 16-row blocks
    // below 64 rows, 64-row blocks from 64 rows on (at exactly 64 the 16-row
    // kernel would stream every page four times, once per row block, and
    // its per-CU load rate then bounds it: on the long-context workload the
    // 64-row kernel is 15% faster despite its larger partials). 128-row
    // blocks whose four waves each score and accumulate 32 rows (override 2)
    // stream each page once per 128 rows, but one wave per SIMD keeps too few
    // LDS reads in flight: at 128 heads they are 13-15% slower than two
    // 64-row blocks. Over the FP8 cache the score/value organisation reads
    // the E4M3 cache as it is and is the default at every size (16 rows, 64
    // sequences of 3-5K tokens: decode 41.8 us, against 45.2 us for 16-row
    // blocks whose waves each convert their key stripe into BF16 first).
    const int ov = g_kernel_override.load(std::memory_order_relaxed);
    DecodeKernel k;
    if (fp8) {
        k = DecodeKernel::WaveSplitFp8;
        if (ov == 0) {
            if (pl.M > 64) return false;   // the 16-row FP8 kernel stops at four row blocks
            k = DecodeKernel::Rows16Fp8;
        }
        if (ov == 1) k = DecodeKernel::WaveSplitFp8;
    } else {
        k = pl.M < 64 ? DecodeKernel::Rows16 : DecodeKernel::WaveSplit;
        if (ov == 0) k = DecodeKernel::Rows16;
        if (ov == 1) k = DecodeKernel::WaveSplit;
        if (ov == 2) k = DecodeKernel::FusedWave;
    }
    // the score/value-wave kernel's block: the smallest of 16, 32 and 64
    // rows that holds the sequence's rows, 64 beyond
    const bool rows16 = k == DecodeKernel::Rows16 || k == DecodeKernel::Rows16Fp8;
    const bool ws = k == DecodeKernel::WaveSplit || k == DecodeKernel::WaveSplitFp8;
    const int tm = rows16                        ? 16
                   : k == DecodeKernel::FusedWave ? 128
                   : pl.M <= 16                   ? 16
                   : pl.M <= 32                   ? 32
                                                  : 64;
    pl.kernel = k;
    pl.tm = tm;
    pl.R = (pl.M + tm - 1) / tm;
    int p = num_partitions;
    if (p <= 0) {
        const int cus = num_cus > 0 ? num_cus : 256;
        p = cus / pl.R;
        // A single 64-row block per partition: three partitions per four
        // CUs. The stream still fills HBM (each workgroup could take a third
        // more than its share), and a quarter fewer 128 KB FP32 partials
        // shortens the combine (4 sequences of 1K-64K tokens at 64 heads:
        // call 53.4 vs 55.5 us, decode kernel unchanged).
        if (ws && tm == 64 && pl.R == 1) p = cus * 3 / 4;
        if (p < 1) p = 1;
    }
    pl.P = (p + 7) / 8 * 8;  // whole groups of 8 for the XCD-aware block mapping
    // fixed cost of a segment in page units: the pipeline fill of its first
    // page plus query load and output or partial traffic (~5 KB per row)
    pl.cseg = 1 + tm / 16;
    pl.slots = 2 * pl.P;
    // With no more partitions than sequences most sequences sit in one
    // partition and the few split ones have about two partials: up to 128
    // rows the merge then runs in the decode kernel and the call is one
    // kernel (128 heads, 128 sequences of 4096 tokens, none split: step
    // 212 vs 217 us). With more partitions per sequence the merging
    // workgroups' extra reads land on the critical path, and beyond 128 rows
    // the partials are large enough that writing them through to the
    // coherent level costs more than a second kernel (two tokens at 128
    // heads over 132 sequences of 1-8192 tokens, 60 of them split: step 410
    // vs 407 us); a combine kernel merges them instead (mla_set_plan_override
    // can force either).
    pl.fused_combine = pl.P <= pl.batch && pl.M <= 128;
    const int mo = g_merge_override.load(std::memory_order_relaxed);
    if (mo >= 0) pl.fused_combine = mo == 1;
    // the 128-row kernel leaves every merge to the combine kernel
    if (k == DecodeKernel::FusedWave) pl.fused_combine = false;
    *plan = pl;
    return true;
}

size_t metadata_bytes(const Plan& plan) { return (size_t)meta_ints(plan.batch, plan.P, plan.R) * 4; }

WorkspaceLayout workspace_layout(const Plan& plan, bool with_metadata) {
    WorkspaceLayout w{};
    w.meta_off = 0;
    w.meta_bytes = with_metadata ? align_up(metadata_bytes(plan), 256) : 0;
    w.lse_off = w.meta_off + w.meta_bytes;
    w.lse_bytes = align_up((size_t)plan.slots * plan.M * sizeof(float), 256);
    w.o_off = w.lse_off + w.lse_bytes;
    w.o_bytes = (size_t)plan.slots * plan.M * MLA_HEAD_DIM_V * sizeof(float);
    w.total = w.o_off + w.o_bytes;
    return w;
}

}  // namespace mla

using namespace mla;

extern "C" {

const char* mla_status_string(int status) {
    switch (status) {
        case MLA_OK: return "MLA_OK";
        case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: invalid argument";
        case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: unsupported shape";
        case MLA_ERR_MISALIGNED: return "MLA_ERR_MISALIGNED: pointer alignment";
        case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL: buffer too small";
        case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime or launch failure";
        case MLA_ERR_SCRATCH_LIMIT:
            return "MLA_ERR_SCRATCH_LIMIT: the call needs more scratch than the allocation-free entry point "
                   "holds (MLA_NOALLOC_SCRATCH_BYTES); use mla_decode_fwd with a workspace";
        default: return "MLA_ERR_UNKNOWN";
    }
}

int mla_abi_version(void) { return (1 << 16) | 0; }

int mla_default_num_partitions(int h_q, int s_q) {
    const int cus = current_cu_count();
    if (cus <= 0) return 0;
    Plan pl;
    if (!make_plan(1, h_q, s_q, 0, cus, &pl)) return 0;
    return pl.P;
}

// Sizes cover both the BF16 plan and, where one exists, the FP8 plan of the
// same shape, so one buffer serves either decode call.
size_t mla_metadata_bytes(int batch, int h_q, int s_q, int num_partitions) {
    const int cus = num_partitions > 0 ? 0 : current_cu_count();
    Plan pl, pf;
    if (!make_plan(batch, h_q, s_q, num_partitions, cus, &pl)) return 0;
    size_t n = metadata_bytes(pl);
    if (make_plan(batch, h_q, s_q, num_partitions, cus, &pf, true)) n = std::max(n, metadata_bytes(pf));
    return n;
}

size_t mla_workspace_bytes(int batch, int h_q, int s_q, int num_partitions) {
    const int cus = num_partitions > 0 ? 0 : current_cu_count();
    Plan pl, pf;
    if (!make_plan(batch, h_q, s_q, num_partitions, cus, &pl)) return 0;
    size_t n = workspace_layout(pl, true).total;
    if (make_plan(batch, h_q, s_q, num_partitions, cus, &pf, true)) n = std::max(n, workspace_layout(pf, true).total);
    return n;
}

static mla_status check_meta_args(const int32_t* seqlens, int batch, int h_q, int s_q,
                                  int num_partitions, const int32_t* metadata) {
    if (!seqlens || !metadata) return MLA_ERR_INVALID_ARG;
    if (batch < 1 || h_q < 1 || s_q < 1 || num_partitions > 65536) return MLA_ERR_INVALID_ARG;
    if ((long long)h_q * s_q > MLA_MAX_ROWS) return MLA_ERR_UNSUPPORTED;
    if (!aligned(seqlens, 4) || !aligned(metadata, 4)) return MLA_ERR_MISALIGNED;
    return MLA_OK;
}

static mla_status get_split_metadata(const int32_t* seqlens, int batch, int h_q, int s_q, int num_partitions,
                                     int32_t* metadata, size_t metadata_bytes_, void* stream, bool fp8) {
    mla_status st = check_meta_args(seqlens, batch, h_q, s_q, num_partitions, metadata);
    if (st != MLA_OK) return st;
    Plan pl;
    if (!make_plan(batch, h_q, s_q, num_partitions,
                   num_partitions > 0 ? 0 : current_cu_count(), &pl, fp8))
        return MLA_ERR_UNSUPPORTED;
    if (metadata_bytes_ < metadata_bytes(pl)) return MLA_ERR_WORKSPACE_TOO_SMALL;
    if (launch_split_metadata(seqlens, batch, pl.P, pl.cseg, pl.R, metadata,
                              reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
        return MLA_ERR_HIP;
    return MLA_OK;
}

mla_status mla_get_split_metadata(const int32_t* seqlens, int batch, int h_q, int s_q,
                                  int num_partitions, int32_t* metadata, size_t metadata_bytes_,
                                  void* stream) {
    return get_split_metadata(seqlens, batch, h_q, s_q, num_partitions, metadata, metadata_bytes_, stream, false);
}

mla_status mla_get_split_metadata_fp8(const int32_t* seqlens, int batch, int h_q, int s_q,
                                      int num_partitions, int32_t* metadata, size_t metadata_bytes_,
                                      void* stream) {
    return get_split_metadata(seqlens, batch, h_q, s_q, num_partitions, metadata, metadata_bytes_, stream, true);
}

mla_status mla_check_metadata_host(const int32_t* metadata, size_t metadata_bytes_, int batch, int h_q,
                                   int s_q, int num_partitions, int fp8) {
    if (!metadata || !aligned(metadata, 4) || (fp8 != 0 && fp8 != 1)) return MLA_ERR_INVALID_ARG;
    if (batch < 1 || h_q < 1 || s_q < 1 || num_partitions > 65536) return MLA_ERR_INVALID_ARG;
    if (metadata_bytes_ < (size_t)kMetaHeader * 4) return MLA_ERR_WORKSPACE_TOO_SMALL;
    Plan pl;
    if (!make_plan(batch, h_q, s_q, num_partitions, num_partitions > 0 ? 0 : current_cu_count(), &pl, fp8 != 0))
        return MLA_ERR_UNSUPPORTED;
    return plan_header_matches(metadata[0], metadata[1], metadata[2], metadata[3], metadata[8], pl.batch, pl.P,
                               pl.cseg, pl.R)
               ? MLA_OK
               : MLA_ERR_INVALID_ARG;
}

mla_status mla_get_split_metadata_host(const int32_t* seqlens, int batch, int h_q, int s_q,
                                       int num_partitions, int32_t* metadata,
                                       size_t metadata_bytes_) {
    mla_status st = check_meta_args(seqlens, batch, h_q, s_q, num_partitions, metadata);
    if (st != MLA_OK) return st;
    for (int b = 0; b < batch; ++b)
        if (seqlens[b] < 0) return MLA_ERR_INVALID_ARG;
    Plan pl;
    if (!make_plan(batch, h_q, s_q, num_partitions,
                   num_partitions > 0 ? 0 : current_cu_count(), &pl))
        return MLA_ERR_UNSUPPORTED;
    if (metadata_bytes_ < metadata_bytes(pl)) return MLA_ERR_WORKSPACE_TOO_SMALL;
    split_metadata_host(seqlens, batch, pl.P, pl.cseg, pl.R, metadata);
    return MLA_OK;
}

}  // extern "C"

namespace {

// Scratch of the allocation-free decode call (mla_decode_fwd_noalloc): its
// split partials and, when the caller passes no plan, the plan. One copy per
// GPU, held from the first such call on that GPU until the process ends; the
// calls on one GPU share it. In host code `scratch` is only a handle for the
// symbol lookup below: the device address is what scratch_address returns.
static __device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

void* g_scratch_ptr[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of the current device's scratch, looked up once per device
// with that device current; nullptr if the lookup failed.
void* scratch_address() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::call_once(g_scratch_once[dev], [dev]() {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            ptr = nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    });
    return g_scratch_ptr[dev];
}

// Both decode entry points: the BF16 cache, or FP8 pages (16-row kernel
// only). `noalloc`: workspace and its size are ignored and the call runs in
// this device's scratch instead (never timed).
mla_status decode_fwd_impl(const void* q, const void* kv_cache, const int32_t* block_table,
                           int max_blocks_per_seq, const int32_t* seqlens, int batch, int s_q,
                           int h_q, int num_pages, float softmax_scale, int causal,
                           int32_t* metadata, int num_partitions, void* workspace,
                           size_t workspace_bytes_, void* out, float* lse, void* stream, bool fp8,
                           bool noalloc = false) {
    if (!q || !kv_cache || !block_table || !seqlens || (!workspace && !noalloc) || !out || !lse)
        return MLA_ERR_INVALID_ARG;
    if (batch < 1 || s_q < 1 || h_q < 1 || max_blocks_per_seq < 1 || num_pages < 1)
        return MLA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return MLA_ERR_INVALID_ARG;
    // the kernels take the row maximum of raw scores and scale it, which is
    // the maximum of the scaled scores only for a positive scale; -0.0 and
    // NaN fail this test too
    if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return MLA_ERR_INVALID_ARG;
    if (num_partitions > 65536) return MLA_ERR_INVALID_ARG;
    if ((long long)h_q * s_q > MLA_MAX_ROWS) return MLA_ERR_UNSUPPORTED;
    if ((long long)max_blocks_per_seq * batch > (1LL << 31) - 1) return MLA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(out, 16) || (!noalloc && !aligned(workspace, 16)))
        return MLA_ERR_MISALIGNED;
    if (!aligned(block_table, 4) || !aligned(seqlens, 4) || !aligned(lse, 4) ||
        (metadata && !aligned(metadata, 4)))
        return MLA_ERR_MISALIGNED;

    Plan pl;
    if (!make_plan(batch, h_q, s_q, num_partitions,
                   num_partitions > 0 ? 0 : current_cu_count(), &pl, fp8))
        return MLA_ERR_UNSUPPORTED;
    if (fp8 != (pl.kernel == DecodeKernel::Rows16Fp8 || pl.kernel == DecodeKernel::WaveSplitFp8))
        return MLA_ERR_UNSUPPORTED;
    const WorkspaceLayout wl = workspace_layout(pl, metadata == nullptr);
    if (noalloc) {
        if (wl.total > (size_t)MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_SCRATCH_LIMIT;
        workspace = scratch_address();
        if (!workspace) return MLA_ERR_HIP;
        workspace_bytes_ = MLA_NOALLOC_SCRATCH_BYTES;
    }
    if (workspace_bytes_ < wl.total) return MLA_ERR_WORKSPACE_TOO_SMALL;

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    int32_t* meta = metadata;
    if (!meta) {
        int32_t* m = reinterpret_cast<int32_t*>(ws + wl.meta_off);
        if (launch_split_metadata(seqlens, batch, pl.P, pl.cseg, pl.R, m, st) != hipSuccess)
            return MLA_ERR_HIP;
        meta = m;
    }

    DecodeArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.kv = static_cast<const uint16_t*>(kv_cache);
    a.block_table = block_table;
    a.seqlens = seqlens;
    a.meta = meta;
    a.counters = pl.fused_combine ? meta + meta_counters(batch, pl.P) : nullptr;
    a.part_lse = reinterpret_cast<float*>(ws + wl.lse_off);
    a.lse_stride = pl.slots;
    a.part_o = reinterpret_cast<float*>(ws + wl.o_off);
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.max_blocks = max_blocks_per_seq;
    a.batch = batch;
    a.s_q = s_q;
    a.h_q = h_q;
    a.M = pl.M;
    a.R = pl.R;
    a.P = pl.P;
    a.cseg = pl.cseg;
    a.scale_log2 = softmax_scale * kLog2e;
    a.causal = causal;
    CallEvents* te = noalloc ? nullptr : timing_slot();
    if (te && hipEventRecord(te->ev[0], st) != hipSuccess) return MLA_ERR_HIP;
    if (launch_decode(pl, a, st) != hipSuccess) return MLA_ERR_HIP;
    if (te && hipEventRecord(te->ev[1], st) != hipSuccess) return MLA_ERR_HIP;
    if (!pl.fused_combine && launch_combine(pl, a, st) != hipSuccess) return MLA_ERR_HIP;
    if (te && hipEventRecord(te->ev[2], st) != hipSuccess) return MLA_ERR_HIP;
    return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_decode_fwd(const void* q, const void* kv_cache, const int32_t* block_table,
                          int max_blocks_per_seq, const int32_t* seqlens, int batch, int s_q,
                          int h_q, int num_pages, float softmax_scale, int causal,
                          int32_t* metadata, int num_partitions, void* workspace,
                          size_t workspace_bytes_, void* out, float* lse, void* stream) {
    return decode_fwd_impl(q, kv_cache, block_table, max_blocks_per_seq, seqlens, batch, s_q, h_q, num_pages,
                           softmax_scale, causal, metadata, num_partitions, workspace, workspace_bytes_, out,
                           lse, stream, false);
}

mla_status mla_decode_fwd_noalloc(const void* q, const void* kv_cache, const int32_t* block_table,
                                  int max_blocks_per_seq, const int32_t* seqlens, int batch, int s_q, int h_q,
                                  int num_pages, float softmax_scale, int causal, int32_t* metadata,
                                  int num_partitions, void* out, float* lse, void* stream) {
    return decode_fwd_impl(q, kv_cache, block_table, max_blocks_per_seq, seqlens, batch, s_q, h_q, num_pages,
                           softmax_scale, causal, metadata, num_partitions, nullptr, 0, out, lse, stream, false,
                           true);
}

mla_status mla_decode_fwd_fp8(const void* q, const void* kv_cache, const int32_t* block_table,
                              int max_blocks_per_seq, const int32_t* seqlens, int batch, int s_q, int h_q,
                              int num_pages, float softmax_scale, int causal, int32_t* metadata,
                              int num_partitions, void* workspace, size_t workspace_bytes_, void* out,
                              float* lse, void* stream) {
    return decode_fwd_impl(q, kv_cache, block_table, max_blocks_per_seq, seqlens, batch, s_q, h_q, num_pages,
                           softmax_scale, causal, metadata, num_partitions, workspace, workspace_bytes_, out,
                           lse, stream, true);
}

mla_status mla_set_plan_override(int kernel, int merge) {
    if (kernel < -1 || kernel > 2 || merge < -1 || merge > 1) return MLA_ERR_INVALID_ARG;
    g_kernel_override.store(kernel, std::memory_order_relaxed);
    g_merge_override.store(merge, std::memory_order_relaxed);
    return MLA_OK;
}

mla_status mla_timing_enable(int enable) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    g_timing.on = enable != 0;
    g_timing.used = 0;
    return MLA_OK;
}

mla_status mla_timing_collect(double* decode_ms, double* combine_ms, int* calls) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    double d = 0.0, c = 0.0;
    for (size_t i = 0; i < g_timing.used; ++i) {
        float t0 = 0.f, t1 = 0.f;
        const CallEvents& ce = g_timing.pool[i];
        if (hipEventElapsedTime(&t0, ce.ev[0], ce.ev[1]) != hipSuccess ||
            hipEventElapsedTime(&t1, ce.ev[1], ce.ev[2]) != hipSuccess) {
            (void)hipGetLastError();
            return MLA_ERR_HIP;
        }
        d += t0;
        c += t1;
    }
    if (decode_ms) *decode_ms = d;
    if (combine_ms) *combine_ms = c;
    if (calls) *calls = (int)g_timing.used;
    g_timing.used = 0;
    return MLA_OK;
}

}  // extern "C"
