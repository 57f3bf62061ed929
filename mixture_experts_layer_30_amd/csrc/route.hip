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
#include "route_align.h"

namespace moe {

template <int G, int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t T,
                                                    int E, int K, const int32_t* __restrict__ k_tok,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t t =
      ((int64_t)blockIdx.x * (blockDim.x / kWave) + wave) * (kWave / G) + lane / G;
  route_token<G, VPL>(logits, t, T, E, K, k_tok, ids, w, nullptr);
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
