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
// thousands of pairs, so the pass is a few microseconds:
//  1. histogram of the expert ids in LDS (atomics only on counts, so the
//     result does not depend on their order);
//  2. one wavefront scans the padded counts (E <= 256, four per lane; for max
//     padding after a max-reduction of the counts);
//  3. padding rows get the sentinel and every block its expert, each row
//     finding its bucket by binary search over the LDS offsets;
//  4. a stable scatter in rounds of 1024 consecutive pairs: inside a
//     wavefront, lanes holding the same expert are found with 8 ballots (one
//     per bit of the id), a lane's rank is the popcount of the matching lower
//     lanes, and the per-wavefront counts in LDS order the wavefronts; a
//     running fill per expert carries the order across rounds.  The result is
//     the ascending-p order, independent of scheduling.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;
constexpr int kMaxExperts = 256;

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int64_t TK, int E, int B, int64_t cap, int max_pad,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ inv_pos) {
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_fill[kMaxExperts];
  __shared__ int s_wcnt[kAlignWaves][kMaxExperts];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  for (int e = tid; e < kMaxExperts; e += kAlignThreads) {
    s_cnt[e] = 0;
    s_fill[e] = 0;
  }
  for (int i = tid; i < kAlignWaves * kMaxExperts; i += kAlignThreads) (&s_wcnt[0][0])[i] = 0;
  __syncthreads();

  // 1. histogram
  for (int64_t p = tid; p < TK; p += kAlignThreads) {
    const int e = ids[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();

  // 2. exclusive prefix sum of the padded counts, one wavefront
  if (wave == 0) {
    int slot = 0;   // max padding: every expert's padded size
    if (max_pad) {
      int mx = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = lane * 4 + j;
        mx = max(mx, e < E ? s_cnt[e] : 0);
      }
#pragma unroll
      for (int d = kWave / 2; d >= 1; d >>= 1) mx = max(mx, __shfl_xor(mx, d));
      slot = (mx + B - 1) / B * B;
    }
    int loc[4];
    int run = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      const int n = e < E ? s_cnt[e] : 0;
      loc[j] = run;
      run += e < E ? (max_pad ? slot : (n + B - 1) / B * B) : 0;
    }
    int incl = run;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    const int excl = incl - run;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      if (e < E) s_off[e] = excl + loc[j];
    }
    if (lane == kWave - 1) s_off[E] = incl;
  }
  __syncthreads();
  const int num_padded = s_off[E];

  for (int e = tid; e <= E; e += kAlignThreads) {
    offsets[e] = s_off[e];
    if (e < E) counts[e] = s_cnt[e];
  }

  // bucket of row r: the largest e with s_off[e] <= r (so that empty buckets,
  // whose offset equals the next one's, are skipped); r < num_padded
  auto bucket_of = [&](int r) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
  };

  // 3. block map and sentinel rows
  const int64_t nblocks = cap / B;
  for (int64_t b = tid; b < nblocks; b += kAlignThreads) {
    const int64_t r = b * B;
    block_expert[b] = r < num_padded ? bucket_of((int)r) : -1;
  }
  const int sentinel = (int)TK;
  for (int64_t r = tid; r < cap; r += kAlignThreads) {
    if (r >= num_padded) {
      sorted_ids[r] = sentinel;
    } else {
      const int e = bucket_of((int)r);
      if (r - s_off[e] >= s_cnt[e]) sorted_ids[r] = sentinel;
    }
  }

  // 4. stable scatter
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int64_t base = 0; base < TK; base += kAlignThreads) {
    const int64_t p = base + tid;
    int e = p < TK ? ids[p] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    if (!valid && p < TK) inv_pos[p] = -1;   // an unused slot (per-token budget)
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool b = (e >> bit) & 1;
      const uint64_t bal = __ballot(b);
      same &= b ? bal : ~bal;
    }
    const int rank = __popcll(same & lower);
    if (valid && rank == 0) s_wcnt[wave][e] = __popcll(same);
    __syncthreads();
    if (valid) {
      int pos = s_off[e] + s_fill[e] + rank;
      for (int w = 0; w < wave; ++w) pos += s_wcnt[w][e];
      sorted_ids[pos] = (int)p;
      inv_pos[p] = pos;
    }
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&s_fill[e], s_wcnt[wave][e]);
      s_wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

hipError_t launch_align(const int32_t* ids, int64_t T, int K, int E, int B, int64_t cap,
                        int max_pad, int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* inv_pos, hipStream_t s) {
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kAlignThreads), 0, s, ids, T * K, E, B, cap,
                     max_pad, counts, offsets, sorted_ids, block_expert, inv_pos);
  return hipGetLastError();
}

}  // namespace moe
