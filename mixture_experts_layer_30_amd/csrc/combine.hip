// Weighted combine ("local sum", finding 5 of the Serving-tax notes) on gfx950.
//
//   out[t][h] = sum_{k in slot order} w[t][k] * y[t*K + k][h]  (+ shared[t][h])
//
// Slots of weight 0 are skipped without reading their rows (the unused slots
// of per-token budgets have no row).
//
// The expert rows are already in pair order (row t*K + k), so each token
// gathers its own K rows: no atomics, no scatter, bit-identical results on
// every run.  One thread owns 8 consecutive h of one token (16-byte loads for
// bf16); the weights of the token are read once per thread from L1/L2.
// HBM-bound: reads T*K*H + T*H elements, writes T*H.
#include "common.h"
#include "kernels.h"

namespace moe {

template <class S>
__device__ __forceinline__ void load8f(const typename S::T* p, float* v);
template <>
__device__ __forceinline__ void load8f<BF16>(const uint16_t* p, float* v) {
  const u32x4 r = *reinterpret_cast<const u32x4*>(p);
  const uint32_t q[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(q[j] << 16);
    v[2 * j + 1] = __uint_as_float(q[j] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8f<F32>(const float* p, float* v) {
  const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
  const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <class S>
__device__ __forceinline__ void store8f(typename S::T* p, const float* v);
template <>
__device__ __forceinline__ void store8f<BF16>(uint16_t* p, const float* v) {
  u32x4 r;
  r.x = pack_bf16x2(v[0], v[1]);
  r.y = pack_bf16x2(v[2], v[3]);
  r.z = pack_bf16x2(v[4], v[5]);
  r.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<u32x4*>(p) = r;
}
template <>
__device__ __forceinline__ void store8f<F32>(float* p, const float* v) {
  reinterpret_cast<f32x4*>(p)[0] = f32x4{v[0], v[1], v[2], v[3]};
  reinterpret_cast<f32x4*>(p)[1] = f32x4{v[4], v[5], v[6], v[7]};
}

template <class SY, class SS, class SO>
__global__ __launch_bounds__(256) void combine_kernel(const typename SY::T* __restrict__ y,
                                                      const float* __restrict__ w,
                                                      const typename SS::T* __restrict__ shared,
                                                      int64_t T, int K, int H,
                                                      typename SO::T* __restrict__ out) {
  const int hv = H / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t = idx / hv;
  if (t >= T) return;
  const int h0 = (int)(idx % hv) * 8;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  for (int k = 0; k < K; ++k) {
    const float wk = w[t * K + k];
    if (wk == 0.0f) continue;   // an unused slot of a per-token budget: its row is never written
    float v[8];
    load8f<SY>(y + (t * K + k) * H + h0, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = fmaf(wk, v[j], acc[j]);
  }
  if (shared) {
    float v[8];
    load8f<SS>(shared + t * H + h0, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += v[j];
  }
  store8f<SO>(out + t * H + h0, acc);
}

template <class SY, class SS, class SO>
static hipError_t launch_combine_t(const void* y, const float* w, const void* shared, int64_t T,
                                   int K, int H, void* out, hipStream_t s) {
  const int64_t n = T * (H / 8);
  const int threads = 256;
  hipLaunchKernelGGL((combine_kernel<SY, SS, SO>), dim3((unsigned)((n + threads - 1) / threads)),
                     dim3(threads), 0, s, static_cast<const typename SY::T*>(y), w,
                     static_cast<const typename SS::T*>(shared), T, K, H,
                     static_cast<typename SO::T*>(out));
  return hipGetLastError();
}

template <class SY, class SS>
static hipError_t dispatch_out(const void* y, const float* w, const void* shared, int64_t T,
                               int K, int H, void* out, int odt, hipStream_t s) {
  return odt == kDtF32 ? launch_combine_t<SY, SS, F32>(y, w, shared, T, K, H, out, s)
                       : launch_combine_t<SY, SS, BF16>(y, w, shared, T, K, H, out, s);
}

template <class SY>
static hipError_t dispatch_shared(const void* y, const float* w, const void* shared, int sdt,
                                  int64_t T, int K, int H, void* out, int odt, hipStream_t s) {
  return sdt == kDtF32 ? dispatch_out<SY, F32>(y, w, shared, T, K, H, out, odt, s)
                       : dispatch_out<SY, BF16>(y, w, shared, T, K, H, out, odt, s);
}

hipError_t launch_combine(const void* y, int ydt, const float* w, const void* shared, int sdt,
                          int64_t T, int K, int H, void* out, int odt, hipStream_t s) {
  return ydt == kDtF32 ? dispatch_shared<F32>(y, w, shared, sdt, T, K, H, out, odt, s)
                       : dispatch_shared<BF16>(y, w, shared, sdt, T, K, H, out, odt, s);
}

}  // namespace moe
