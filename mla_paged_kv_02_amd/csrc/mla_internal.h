// mla_internal.h - host-side plan and kernel launchers (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// How one decode call is cut into workgroups: R row blocks of tm rows cover
// the M = h_q*s_q rows of a sequence, P partitions cut the page list, and
// the grid is P*R workgroups.
//   Rows16:    tm = 16, four waves each owning a key stripe of every page;
//   WaveSplit: tm = 16, 32 or 64, score waves and four value waves;
//   FusedWave: tm = 128, four waves each scoring and accumulating 32 rows;
//   Rows16Fp8: the Rows16 organisation over the FP8 page format;
//   WaveSplitFp8: the WaveSplit organisation (tm = 64) over the FP8 pages.
enum class DecodeKernel { Rows16, WaveSplit, Rows16Fp8, FusedWave, WaveSplitFp8 };

struct Plan {
    int batch, h_q, s_q, M;
    DecodeKernel kernel;
    int tm;
    int R, P;
    int cseg;
    int slots;  // capacity of the split-partial buffers (sequence splits)
    // the last workgroup of a split sequence merges its partials (few
    // partials per sequence); otherwise a combine kernel runs after decode
    bool fused_combine;
};

// Returns false for unsupported shapes. num_partitions <= 0 selects the default.
// fp8: the plan of the FP8-cache decode (16-row kernel, at most 64 rows).
bool make_plan(int batch, int h_q, int s_q, int num_partitions, int num_cus, Plan* plan, bool fp8 = false);

// Byte layout of the workspace: [metadata (optional)] [partial lse] [partial O].
struct WorkspaceLayout {
    size_t meta_off, meta_bytes;
    size_t lse_off, lse_bytes;
    size_t o_off, o_bytes;
    size_t total;
};
WorkspaceLayout workspace_layout(const Plan& plan, bool with_metadata);
size_t metadata_bytes(const Plan& plan);

struct DecodeArgs {
    const uint16_t* q;
    const uint16_t* kv;
    const int32_t* block_table;
    const int32_t* seqlens;
    const int32_t* meta;
    int32_t* counters;   // partial counters in the metadata; null when a combine kernel runs
    float* part_o;
    float* part_lse;   // row r, slot j at r * lse_stride + j: a row's partials are contiguous
    uint16_t* out;
    float* lse;
    int max_blocks;
    int batch, s_q, h_q, M;
    int R, P;
    int cseg;          // the plan's per-segment cost (checked against its header)
    int lse_stride;    // split-partial slots of the plan
    float scale_log2;  // softmax_scale * log2(e)
    int causal;
};

hipError_t launch_split_metadata(const int32_t* seqlens, int batch, int num_partitions, int cseg,
                                 int row_blocks, int32_t* meta, hipStream_t stream);
hipError_t launch_decode(const Plan& plan, const DecodeArgs& args, hipStream_t stream);
hipError_t launch_decode_rows16(const Plan& plan, const DecodeArgs& args, hipStream_t stream);
hipError_t launch_decode_ws(const Plan& plan, const DecodeArgs& args, hipStream_t stream);
hipError_t launch_decode_fw(const Plan& plan, const DecodeArgs& args, hipStream_t stream);
hipError_t launch_decode_ws_fp8(const Plan& plan, const DecodeArgs& args, hipStream_t stream);
hipError_t launch_decode_rows16_fp8(const Plan& plan, const DecodeArgs& args, hipStream_t stream);
hipError_t launch_combine(const Plan& plan, const DecodeArgs& args, hipStream_t stream);

// Host build of the same plan (tests and host callers).
void split_metadata_host(const int32_t* seqlens, int batch, int num_partitions, int cseg,
                         int row_blocks, int32_t* meta);

}  // namespace mla
