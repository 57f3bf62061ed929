// Routing and alignment in one launch for small batches on gfx950.
//
// At decode a layer pass is a handful of launches, and the first two -- the
// softmax top-K routing and the alignment (Serving-tax notes, Table 1,
// auxiliary-kernel row; finding 5) -- each carry a launch of their own for a
// few microseconds of work.  With at most kFusePairs pairs and few enough
// tokens for one routing pass, one workgroup of 1024 threads does both: its 16 wavefronts route the tokens (route_token, a
// group of G lanes per token, as route.hip does), writing the ids and weights
// to global memory and the ids also to LDS, and after a workgroup barrier the
// same workgroup aligns the pairs from LDS (align_body, as align.hip does).
// The results are those of the two launches, bit for bit.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "route_align.h"

namespace moe {

template <int G, int VPL>
__global__ __launch_bounds__(kAlignThreads) void route_align_kernel(
    const float* __restrict__ logits, int64_t T, int E, int K, const int32_t* __restrict__ k_tok,
    int32_t* __restrict__ ids, float* __restrict__ w, int B, int64_t cap, int max_pad,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ inv_pos) {
  __shared__ int32_t s_ids[kFusePairs];
  __shared__ AlignSmem sm;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  constexpr int kTokPerPass = kAlignWaves * (kWave / G);
  // tokens t = base + wave * (64 / G) + lane / G; the loop bound is the same for
  // every wavefront, so each one's group operations see all of its lanes
  for (int64_t base = 0; base < T; base += kTokPerPass) {
    const int64_t t = base + (int64_t)wave * (kWave / G) + lane / G;
    route_token<G, VPL>(logits, t, T, E, K, k_tok, ids, w, s_ids);
  }
  __syncthreads();
  align_body(s_ids, T * K, E, B, cap, max_pad, counts, offsets, sorted_ids, block_expert, inv_pos,
             sm);
}

hipError_t launch_route_align(const float* logits, int64_t T, int E, int K, const int32_t* k_tok,
                              int32_t* ids, float* w, int B, int64_t cap, int max_pad,
                              int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                              int32_t* block_expert, int32_t* inv_pos, hipStream_t s) {
  // one workgroup routes 16 * 64 / G tokens at a time (G lanes a token); past one
  // such pass the routing launch, spread over many CUs, is the faster (measured on
  // MI355X, DeepSeek-V3-shaped layer at 128 tokens, 8 passes: pass 1089 -> 1135 us
  // fused; one pass: Mixtral-shaped T = 1 143 -> 136 us, T = 8 455 -> 447)
  const int G = E <= 8 ? 8 : E <= 16 ? 16 : E <= 32 ? 32 : 64;
  if (T * K > kFusePairs || T > (int64_t)kAlignWaves * (kWave / G)) {
    hipError_t e = launch_route(logits, T, E, K, k_tok, ids, w, s);
    if (e != hipSuccess) return e;
    return launch_align(ids, T, K, E, B, cap, max_pad, counts, offsets, sorted_ids, block_expert,
                        inv_pos, s);
  }
  auto go = [&](auto g, auto vpl) {
    constexpr int Gc = decltype(g)::value, V = decltype(vpl)::value;
    hipLaunchKernelGGL((route_align_kernel<Gc, V>), dim3(1), dim3(kAlignThreads), 0, s, logits, T,
                       E, K, k_tok, ids, w, B, cap, max_pad, counts, offsets, sorted_ids,
                       block_expert, inv_pos);
  };
  using I1 = std::integral_constant<int, 1>;
  if (E <= 8) go(std::integral_constant<int, 8>{}, I1{});
  else if (E <= 16) go(std::integral_constant<int, 16>{}, I1{});
  else if (E <= 32) go(std::integral_constant<int, 32>{}, I1{});
  else if (E <= 64) go(std::integral_constant<int, 64>{}, I1{});
  else go(std::integral_constant<int, 64>{}, std::integral_constant<int, 4>{});
  return hipGetLastError();
}

}  // namespace moe
