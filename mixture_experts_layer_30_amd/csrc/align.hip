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

namespace moe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;
constexpr int kMaxExperts = 256;
constexpr int kBatch = 4;   // 64-pair steps whose ids a wavefront loads at once
constexpr int kMinChunk = 256;

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int64_t TK, int E, int B, int64_t cap, int max_pad,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ inv_pos) {
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_wrow[kAlignWaves][kMaxExperts];   // per-wavefront counts, then starting rows

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  for (int i = tid; i < kAlignWaves * kMaxExperts; i += kAlignThreads) (&s_wrow[0][0])[i] = 0;
  __syncthreads();

  // this wavefront's chunk [c0, c1) of the pairs: at least kMinChunk, so
  // that small batches use few wavefronts (nw) and the loops over them stay short
  // (T*K < 2^31, so 32-bit unsigned arithmetic holds these)
  const uint32_t tk = (uint32_t)TK;
  const uint32_t chunk = max((uint32_t)kMinChunk, ((tk + kAlignWaves - 1) / kAlignWaves + kWave - 1) / kWave * kWave);
  const int nw = (int)((tk + chunk - 1) / chunk);
  const int64_t c0 = min(TK, (int64_t)wave * chunk);
  const int64_t c1 = min(TK, c0 + (int64_t)chunk);

  // 1. histograms (up to kBatch loads in flight per lane; the steps past the
  // chunk's end, a wavefront-uniform condition, are skipped)
  for (int64_t b0 = c0; b0 < c1; b0 += kBatch * kWave) {
    int ev[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t p = b0 + j * kWave + lane;
      ev[j] = (b0 + j * kWave < c1 && p < c1) ? ids[p] : -1;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (b0 + j * kWave >= c1) break;
      if ((unsigned)ev[j] < (unsigned)E) atomicAdd(&s_wrow[wave][ev[j]], 1);
    }
  }
  __syncthreads();

  // 2. exclusive prefix sum of the padded counts, one wavefront, which first
  // adds up each of its lane's four experts' per-wavefront counts
  if (wave == 0) {
    int cnt[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      int n = 0;
      if (e < E)
        for (int w = 0; w < nw; ++w) n += s_wrow[w][e];
      cnt[j] = n;
      if (e < E) s_cnt[e] = n;
    }
    int slot = 0;   // max padding: every expert's padded size
    if (max_pad) {
      int mx = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = max(mx, cnt[j]);
#pragma unroll
      for (int d = kWave / 2; d >= 1; d >>= 1) mx = max(mx, __shfl_xor(mx, d));
      slot = (mx + B - 1) / B * B;
    }
    int loc[4];
    int run = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      const int n = cnt[j];
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
    if (e < E) {
      counts[e] = s_cnt[e];
      int row = s_off[e];
      for (int w = 0; w < nw; ++w) {
        const int n = s_wrow[w][e];
        s_wrow[w][e] = row;
        row += n;
      }
    }
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
  // sentinel rows: each expert's padding, then everything past num_padded
  const int sentinel = (int)TK;
  for (int e = wave; e < E; e += kAlignWaves) {   // one wavefront per expert
    const int r1 = s_off[e + 1];
    for (int r = s_off[e] + s_cnt[e] + lane; r < r1; r += kWave) sorted_ids[r] = sentinel;
  }
  for (int64_t r = num_padded + tid; r < cap; r += kAlignThreads) sorted_ids[r] = sentinel;

  __syncthreads();   // every wavefront's starting rows are in LDS

  // 4. stable scatter of this wavefront's chunk
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int64_t b0 = c0; b0 < c1; b0 += kBatch * kWave) {
    int ev[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t p = b0 + j * kWave + lane;
      ev[j] = (b0 + j * kWave < c1 && p < c1) ? ids[p] : -1;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (b0 + j * kWave >= c1) break;
      const int64_t p = b0 + j * kWave + lane;
      const int e = ev[j];
      const bool valid = (unsigned)e < (unsigned)E;
      if (!valid && p < c1) inv_pos[p] = -1;   // an unused slot (per-token budget)
      uint64_t same = __ballot(valid);
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        const bool b = (e >> bit) & 1;
        const uint64_t bal = __ballot(b);
        same &= b ? bal : ~bal;
      }
      const int rank = __popcll(same & lower);
      if (valid) {
        // every lane reads the row before the group's first lane advances it
        // (one wavefront's LDS accesses complete in program order)
        const int pos = s_wrow[wave][e] + rank;
        sorted_ids[pos] = (int)p;
        inv_pos[p] = pos;
      }
      if (valid && rank == 0) s_wrow[wave][e] += __popcll(same);
    }
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
