// Token-to-expert alignment with block-wise or max padding on gfx950.
//
// Serving-tax notes, "Padding model (Section 5.1)": block-wise padding rounds
// each expert's token count N_i up on its own to a multiple of the block B, so
// the grouped GEMM computes P = sum_i ceil(N_i/B)*B rows; max padding gives
// every expert the slot of the busiest one, P = E * ceil(max_i N_i/B)*B.  The kernel produces the
// grouping that the grouped GEMM reads: per-expert counts and padded offsets,
// the pair index of every row (buckets in ascending pair order, sentinel T*K
// in padding rows), the expert of every B-row block and the inverse map.
//
// One workgroup of 1024 threads does it all; T*K is at most a few tens of
// thousands of pairs, so the pass is a few microseconds.  Wavefront w owns the
// w-th of up to 16 contiguous chunks of the pairs (a multiple of 64 each, at
// least 256), whose ids it loads 4 steps of 64 at a time:
//  1. per-wavefront histograms of the expert ids in LDS (atomics only on
//     counts, so the result does not depend on their order);
//  2. one wavefront sums them per expert and scans the padded counts (E <=
//     256, four per lane; for max padding after a max-reduction of the
//     counts), and each expert's count is turned into per-wavefront starting rows (the rows of the expert's
//     pairs in earlier chunks come first);
//  3. every block gets its expert (binary search over the LDS offsets) and
//     each expert's padding rows, and the rows past the padded total, the
//     sentinel;
//  4. a stable scatter, each wavefront walking its own chunk 64 pairs at a
//     time with no workgroup barrier: lanes holding the same expert are found
//     with 8 ballots (one per bit of the id), a lane's rank is the popcount of
//     the matching lower lanes, and the group's first lane advances the
//     wavefront's starting row for that expert.  The result is the
//     ascending-p order, independent of scheduling.
#include "common.h"
#include "kernels.h"
#include "route_align.h"

namespace moe {

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int64_t TK, int E, int B, int64_t cap, int max_pad,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ inv_pos) {
  __shared__ AlignSmem sm;
  align_body(ids, TK, E, B, cap, max_pad, counts, offsets, sorted_ids, block_expert, inv_pos, sm);
}

hipError_t launch_align(const int32_t* ids, int64_t T, int K, int E, int B, int64_t cap,
                        int max_pad, int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* inv_pos, hipStream_t s) {
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kAlignThreads), 0, s, ids, T * K, E, B, cap,
                     max_pad, counts, offsets, sorted_ids, block_expert, inv_pos);
  return hipGetLastError();
}

}  // namespace moe
