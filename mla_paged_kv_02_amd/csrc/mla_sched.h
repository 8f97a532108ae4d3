// mla_sched.h - split-KV work plan for paged MLA decode (host and device).
//
// The decode work of one step is the list of (sequence b, page n) pairs, in
// sequence order. Each sequence is laid on a "cost line": a fixed per-segment
// cost `cseg` (query load, output or partial write, and the pipeline fill of
// a fresh segment), then one unit per page. Empty sequences take no room.
// Partition p owns the cost interval [p*W, (p+1)*W), W = ceil(total / P),
// and therefore a contiguous run of pages that may start or end inside a
// sequence. Each boundary is found independently (the last sequence whose
// prefix sum is at most the boundary's position), so the device builds the
// plan in parallel and the host builds the identical plan sequentially from
// the same functions; the device kernel runs that search as radix-4 lifting
// over a copy of the prefix sums in LDS, which finds the same sequence.
//
// Why: decode has one new token per sequence, so parallelising over batch
// alone leaves most compute units idle when batch is small and contexts are
// long (long-text inference page, "Unlocking GPU Potential ...", on decode
// with batch below the SM count). Cutting sequences into page ranges and
// recombining them by log-sum-exp fixes that.
//
// Metadata layout (int32):
//   [0]  magic   [1] batch   [2] P   [3] cseg   [4] ceil(T/P)   [5] total split slots
//   [6]  total cost   [7] active partitions min(P, T)   [8] row blocks R   [9..15] zero
//   [16 + 8p + {0..7}]              partition p: b_begin, n_begin, b_end, n_end
//                                    (end exclusive, (b_end, 0) touches nothing of
//                                    b_end), the length of sequence b_begin (0 past
//                                    the batch), three zeros
//   [16 + 8P + 4b + {0,1,2,3}]      sequence b: slot_base (-1 when not split),
//                                    first partition holding its pages (-1 if none),
//                                    number of partitions holding its pages,
//                                    start of the sequence on the cost line
//   [16 + 8P + 4B + R b + rb]       partial counter of (sequence b, row block rb):
//                                    zero as written; the decode call counts the
//                                    partials written into it and leaves it zero
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MLA_HD __host__ __device__ __forceinline__
#else
#define MLA_HD inline
#endif

namespace mla {

constexpr int32_t kMetaMagic = 0x314C4D41;  // "AML1"
constexpr int kMetaHeader = 16;
constexpr int kPartInts = 8;   // ints per partition record
constexpr int kPageSize = 64;

MLA_HD int meta_ints(int batch, int num_partitions, int row_blocks) {
    return kMetaHeader + kPartInts * num_partitions + 4 * batch + row_blocks * batch;
}

// Offset of the partial counters.
MLA_HD int meta_counters(int batch, int num_partitions) {
    return kMetaHeader + kPartInts * num_partitions + 4 * batch;
}

// Whether a plan's header ([0] magic, [1] batch, [2] P, [3] cseg, [8] R)
// is the one a decode call with these arguments would build. The decode and
// combine kernels test it before reading anything else of the plan, and the
// host check of a host copy uses the same test.
MLA_HD bool plan_header_matches(int32_t magic, int32_t batch_m, int32_t p_m, int32_t cseg_m, int32_t r_m,
                                int batch, int num_partitions, int cseg, int row_blocks) {
    return magic == kMetaMagic && batch_m == batch && p_m == num_partitions && cseg_m == cseg &&
           r_m == row_blocks;
}

MLA_HD int32_t pages_of(int32_t seqlen) { return (seqlen + kPageSize - 1) / kPageSize; }

// Length of sequence b on the cost line.
MLA_HD int64_t cost_len(int32_t seqlen, int32_t cseg) {
    int32_t n = pages_of(seqlen);
    return n > 0 ? (int64_t)n + cseg : 0;
}

// Partitions that get work: min(P, total). Each of them then covers at least
// one unit of the cost line, so the partitions holding pages of one sequence
// are consecutive (none of them can be empty). The rest get nothing.
MLA_HD int32_t active_partitions(int64_t total, int32_t num_partitions) {
    return (int32_t)(total < num_partitions ? total : num_partitions);
}

// Start of partition p (< active partitions) on the cost line.
MLA_HD int64_t partition_start(int64_t p, int64_t total, int32_t num_partitions) {
    return p * total / num_partitions;
}

// Partition owning cost-line position x (0 <= x < total): the largest p with
// partition_start(p) <= x.
MLA_HD int32_t partition_of(int64_t x, int64_t total, int32_t num_partitions) {
    return (int32_t)(((x + 1) * num_partitions - 1) / total);
}

// Maps a cost-line position x to the page where a partition boundary falls.
// `start` is the exclusive prefix sum of cost_len (start[b*stride] = position
// of sequence b), `total` its sum. Positions inside a sequence's fixed cost map
// to its page 0; positions at or past `total` map to (batch, 0).
MLA_HD void boundary_at(int64_t x, const int32_t* start, int start_stride, int batch, int64_t total,
                        int32_t cseg, int32_t* b_out, int32_t* n_out) {
    if (x >= total) {
        *b_out = batch;
        *n_out = 0;
        return;
    }
    // Largest b with start[b] <= x. An empty sequence has the same start as
    // the one after it, so for x < total this b is never an empty sequence.
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (start[(int64_t)mid * start_stride] <= x) lo = mid; else hi = mid - 1;
    }
    int b = lo;
    int64_t off = x - start[(int64_t)b * start_stride] - cseg;
    int32_t n = off < 0 ? 0 : (int32_t)off;
    *b_out = b;
    *n_out = n;
}

// Partitions that hold at least one page of a sequence starting at `start_b`
// with `n_pages` pages: [first, first + count).
MLA_HD void seq_partitions(int64_t start_b, int32_t n_pages, int32_t cseg, int64_t total,
                           int32_t num_partitions, int32_t* first, int32_t* count) {
    if (n_pages <= 0) {
        *first = -1;
        *count = 0;
        return;
    }
    const int32_t a = partition_of(start_b + cseg, total, num_partitions);
    const int32_t z = partition_of(start_b + cseg + n_pages - 1, total, num_partitions);
    *first = a;
    *count = z - a + 1;
}

}  // namespace mla
