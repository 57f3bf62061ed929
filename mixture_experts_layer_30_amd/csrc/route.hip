// Softmax top-K routing on gfx950.
//
// Routing and top-K selection are the first auxiliary kernels of the MoE
// block in the Serving-tax notes (Table 1, auxiliary-kernel row; finding 5).
// The gating function is softmax over the E logits, the K largest, with the
// K weights renormalised to sum to one.
//
// One group of G lanes of a wavefront owns one token (G = 8..64 by E); each
// lane holds up to 4 of the token's logits in registers, logit j of lane l
// being expert l + G*j.  Each of the K selection rounds takes the group's
// largest remaining logit -- a lane-local max, then a max across the group
// with DPP row permutations (pairs at distance 1 and 2 inside quads, the
// mirrored halves of each 8 and of each 16 lanes), a lane swizzle across
// 16-lane rows and a scalar read across the two halves of the wavefront --
// and then the lowest expert id holding that value, from one ballot per
// register slot (slot j's ids all lie below slot j+1's): the lower id wins
// ties, and the comparison is IEEE equality, so -0 equals +0.  Because the
// first selected logit is the maximum, the renormalised weights are
// exp(l_j - l_0) / sum_i exp(l_i - l_0), the same numbers as renormalising the
// full softmax.
//
// With a per-token budget (the routing top-k as a per-request knob, MoE-Prism
// page) token t keeps only its first k_t selections, renormalised over them;
// its other slots get id -1 and weight 0.
#include "common.h"
#include "kernels.h"

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

template <int G, int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t T,
                                                    int E, int K, const int32_t* __restrict__ k_tok,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  static_assert(G == 8 || G == 16 || G == 32 || G == 64, "group size");
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int gl = lane % G;
  const int gbase = lane - gl;   // first lane of this token's group
  const uint64_t gmask = (G == 64 ? ~0ull : ((1ull << G) - 1)) << gbase;
  const int64_t t =
      ((int64_t)blockIdx.x * (blockDim.x / kWave) + wave) * (kWave / G) + lane / G;
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
      }
    }
  }
}

hipError_t launch_route(const float* logits, int64_t T, int E, int K, const int32_t* k_tok,
                        int32_t* ids, float* w, hipStream_t s) {
  const int threads = 256;
  auto blocks_for = [&](int G) { return (unsigned)((T + (threads / G) - 1) / (threads / G)); };
  if (E <= 8)
    hipLaunchKernelGGL((route_kernel<8, 1>), dim3(blocks_for(8)), dim3(threads), 0, s, logits, T,
                       E, K, k_tok, ids, w);
  else if (E <= 16)
    hipLaunchKernelGGL((route_kernel<16, 1>), dim3(blocks_for(16)), dim3(threads), 0, s, logits,
                       T, E, K, k_tok, ids, w);
  else if (E <= 32)
    hipLaunchKernelGGL((route_kernel<32, 1>), dim3(blocks_for(32)), dim3(threads), 0, s, logits,
                       T, E, K, k_tok, ids, w);
  else if (E <= 64)
    hipLaunchKernelGGL((route_kernel<64, 1>), dim3(blocks_for(64)), dim3(threads), 0, s, logits,
                       T, E, K, k_tok, ids, w);
  else
    hipLaunchKernelGGL((route_kernel<64, 4>), dim3(blocks_for(64)), dim3(threads), 0, s, logits,
                       T, E, K, k_tok, ids, w);
  return hipGetLastError();
}

}  // namespace moe
