// Device pieces shared by the routing, alignment and fused routing+alignment
// kernels (route.hip, align.hip, route_align.hip), and the fused launch.
#pragma once

#include "common.h"

namespace moe {

// DPP controls (gfx9 encoding): quad permutations and row mirrors
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  const int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false);
  return fmaxf(v, __int_as_float(o));
}

// Maximum of v over the aligned group of G lanes, in every lane of the group.
template <int G>
__device__ __forceinline__ float group_max(float v) {
  v = dpp_max<kQuadXor1>(v);
  v = dpp_max<kQuadXor2>(v);
  v = dpp_max<kRowHalfMirror>(v);   // the two quads of each 8 lanes
  if constexpr (G >= 16) v = dpp_max<kRowMirror>(v);   // the two 8s of each row
  if constexpr (G == 32) {
    // lane i and lane i ^ 16 inside each 32 (ds_swizzle, bit mode: xor mask 16)
    const int o = __builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F);
    v = fmaxf(v, __int_as_float(o));
  }
  if constexpr (G == 64) {
    // the four row maxima, read as scalars (the whole wavefront is one group)
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    v = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
  }
  return v;
}

// Routing of token t by the aligned group of G lanes holding it (every lane of
// the wavefront calls this, t >= T being inactive): writes its K ids and
// weights to ids / w and, when lds_ids is given, its ids to lds_ids as well.
template <int G, int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int64_t t, int64_t T,
                                            int E, int K, const int32_t* __restrict__ k_tok,
                                            int32_t* __restrict__ ids, float* __restrict__ w,
                                            int32_t* lds_ids) {
  static_assert(G == 8 || G == 16 || G == 32 || G == 64, "group size");
  const int lane = threadIdx.x & (kWave - 1);
  const int gl = lane % G;
  const int gbase = lane - gl;   // first lane of this token's group
  const uint64_t gmask = (G == 64 ? ~0ull : ((1ull << G) - 1)) << gbase;
  const bool active = t < T;

  float v[VPL];
  bool live[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = gl + G * j;
    live[j] = active && e < E;
    v[j] = live[j] ? logits[t * E + e] : 0.0f;
  }

  // the token's budget, clamped to [0, K] (uniform over the group)
  int kt = K;
  if (k_tok && active) {
    const int b = k_tok[t];
    kt = b < 0 ? 0 : (b > K ? K : b);
  }
  // round kk's expert and exp(l - l_0) are kept by lane kk % G of the group in
  // slot kk / G (K <= E <= G * VPL), so the results leave in coalesced stores
  // at the end and the renormalisation reads nothing back from memory
  float first = 0.0f, sum = 0.0f;
  float exk[VPL];
  int idk[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    exk[j] = 0.0f;
    idk[j] = -1;
  }
  for (int kk = 0; kk < K; ++kk) {
    float bv = -INFINITY;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (live[j] && v[j] > bv) bv = v[j];
    const float gm = group_max<G>(bv);
    // the lowest id holding the maximum: slot j's experts are gl + G*j, so the
    // first slot with a match holds the lowest; within it, the lowest lane
    int be = -1;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const uint64_t hit = __ballot(live[j] && v[j] == gm) & gmask;
      if (be < 0 && hit != 0) be = (__ffsll((unsigned long long)hit) - 1 - gbase) + G * j;
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (gl + G * j == be) live[j] = false;
    if (kk == 0) first = gm;
    if (kk < kt) {
      const float ex = expf(gm - first);   // the same value in every lane of the group
      sum += ex;
#pragma unroll
      for (int j = 0; j < VPL; ++j)
        if (gl + G * j == kk) {
          exk[j] = ex;
          idk[j] = be;
        }
    }
  }
  if (active) {
    const float inv = kt > 0 ? 1.0f / sum : 0.0f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int kk = gl + G * j;
      if (kk < K) {
        ids[t * K + kk] = kk < kt ? idk[j] : -1;
        w[t * K + kk] = kk < kt ? exk[j] * inv : 0.0f;
        if (lds_ids) lds_ids[t * K + kk] = kk < kt ? idk[j] : -1;
      }
    }
  }
}

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;
constexpr int kMaxExperts = 256;
constexpr int kBatch = 4;   // 64-pair steps whose ids a wavefront loads at once
constexpr int kMinChunk = 256;

// Shared memory of the alignment: counts, padded offsets, per-wavefront counts
// (then starting rows) of each expert.
struct AlignSmem {
  int cnt[kMaxExperts];
  int off[kMaxExperts + 1];
  int wrow[kAlignWaves][kMaxExperts];
};

// The alignment of the TK pairs whose expert ids ids[p] are in global memory
// or in LDS, by one workgroup of kAlignThreads threads (see align.hip).
__device__ __forceinline__ void align_body(const int32_t* ids, int64_t TK, int E, int B,
                                           int64_t cap, int max_pad, int32_t* __restrict__ counts,
                                           int32_t* __restrict__ offsets,
                                           int32_t* __restrict__ sorted_ids,
                                           int32_t* __restrict__ block_expert,
                                           int32_t* __restrict__ inv_pos, AlignSmem& sm) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  for (int i = tid; i < kAlignWaves * kMaxExperts; i += kAlignThreads) (&sm.wrow[0][0])[i] = 0;
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
      if ((unsigned)ev[j] < (unsigned)E) atomicAdd(&sm.wrow[wave][ev[j]], 1);
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
        for (int w = 0; w < nw; ++w) n += sm.wrow[w][e];
      cnt[j] = n;
      if (e < E) sm.cnt[e] = n;
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
      if (e < E) sm.off[e] = excl + loc[j];
    }
    if (lane == kWave - 1) sm.off[E] = incl;
  }
  __syncthreads();
  const int num_padded = sm.off[E];

  for (int e = tid; e <= E; e += kAlignThreads) {
    offsets[e] = sm.off[e];
    if (e < E) {
      counts[e] = sm.cnt[e];
      int row = sm.off[e];
      for (int w = 0; w < nw; ++w) {
        const int n = sm.wrow[w][e];
        sm.wrow[w][e] = row;
        row += n;
      }
    }
  }

  // bucket of row r: the largest e with sm.off[e] <= r (so that empty buckets,
  // whose offset equals the next one's, are skipped); r < num_padded
  auto bucket_of = [&](int r) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sm.off[mid] <= r) lo = mid; else hi = mid - 1;
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
    const int r1 = sm.off[e + 1];
    for (int r = sm.off[e] + sm.cnt[e] + lane; r < r1; r += kWave) sorted_ids[r] = sentinel;
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
        const int pos = sm.wrow[wave][e] + rank;
        sorted_ids[pos] = (int)p;
        inv_pos[p] = pos;
      }
      if (valid && rank == 0) sm.wrow[wave][e] += __popcll(same);
    }
  }
}

// Routing and alignment in one launch (one workgroup) while the batch has at
// most kFusePairs pairs and one workgroup routes it in one pass (16 * 64 / G
// tokens, G = 8..64 lanes a token by E), else the two launches; the same
// results either way.
constexpr int kFusePairs = 4096;
hipError_t launch_route_align(const float* logits, int64_t T, int E, int K, const int32_t* k_tok,
                              int32_t* ids, float* w, int B, int64_t cap, int max_pad,
                              int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                              int32_t* block_expert, int32_t* inv_pos, hipStream_t s);

}  // namespace moe
