// Softmax top-K routing on gfx950.
//
// Routing and top-K selection are the first auxiliary kernels of the MoE
// block in the Serving-tax notes (Table 1, auxiliary-kernel row; finding 5).
// The gating function is softmax over the E logits, the K largest, with the
// K weights renormalised to sum to one.
//
// One group of G lanes of a wavefront owns one token (G = 8..64 by E); each
// lane holds up to 4 of the token's logits in registers.  Each of the K
// selection rounds is a lane-local argmax followed by a butterfly of
// cross-lane swaps (ds_bpermute) inside the group, on the key (logit
// descending, expert id ascending): the lower id wins ties, -0 equals +0.
// Because the first selected logit is the maximum, the renormalised weights
// are exp(l_j - l_0) / sum_i exp(l_i - l_0), the same numbers as renormalising
// the full softmax.
//
// With a per-token budget (the routing top-k as a per-request knob, MoE-Prism
// page) token t keeps only its first k_t selections, renormalised over them;
// its other slots get id -1 and weight 0.
#include "common.h"
#include "kernels.h"

namespace moe {

template <int G, int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t T,
                                                    int E, int K, const int32_t* __restrict__ k_tok,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  constexpr int kNone = 0x7fffffff;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int gl = lane % G;
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
  float first = 0.0f, sum = 0.0f;
  for (int kk = 0; kk < K; ++kk) {
    // lane-local best among the live entries; e grows with j, so strict '>'
    // keeps the lower id among equal logits
    float bv = 0.0f;
    int be = kNone;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (live[j] && (be == kNone || v[j] > bv)) {
        bv = v[j];
        be = gl + G * j;
      }
    // butterfly over the group
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, G);
      const int oe = __shfl_xor(be, off, G);
      if (oe != kNone && (be == kNone || ov > bv || (ov == bv && oe < be))) {
        bv = ov;
        be = oe;
      }
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (gl + G * j == be) live[j] = false;
    if (active && gl == 0) {
      if (kk == 0) first = bv;
      if (kk < kt) {
        const float ex = expf(bv - first);
        sum += ex;
        ids[t * K + kk] = be;
        w[t * K + kk] = ex;
      } else {
        ids[t * K + kk] = -1;
        w[t * K + kk] = 0.0f;
      }
    }
  }
  if (active && gl == 0 && kt > 0) {
    const float inv = 1.0f / sum;
    for (int kk = 0; kk < kt; ++kk) w[t * K + kk] = w[t * K + kk] * inv;
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
