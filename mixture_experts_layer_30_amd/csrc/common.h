// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Storage element types of x and the weights.
struct F32 { typedef float T; static constexpr int kBytes = 4; };
struct BF16 { typedef uint16_t T; static constexpr int kBytes = 2; };
// OCP FP8 E4M3 weight codes (with a per-row fp32 scale held separately)
struct FP8 { typedef uint8_t T; static constexpr int kBytes = 1; };

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// 8 consecutive elements starting at p, as 8 bf16 in 16 bytes (rounding fp32
// storage).  Streaming (read-once) data uses non-temporal loads, which keep it
// from displacing reused data in the caches.
template <class S, bool kStream = false>
__device__ __forceinline__ u32x4 load8(const typename S::T* p);

template <>
__device__ __forceinline__ u32x4 load8<BF16, false>(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
template <>
__device__ __forceinline__ u32x4 load8<BF16, true>(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <>
__device__ __forceinline__ u32x4 load8<F32, false>(const float* p) {
  const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
  const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
  u32x4 r;
  r.x = pack_bf16x2(a.x, a.y);
  r.y = pack_bf16x2(a.z, a.w);
  r.z = pack_bf16x2(b.x, b.y);
  r.w = pack_bf16x2(b.z, b.w);
  return r;
}
template <>
__device__ __forceinline__ u32x4 load8<F32, true>(const float* p) {
  const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
  u32x4 r;
  r.x = pack_bf16x2(a.x, a.y);
  r.y = pack_bf16x2(a.z, a.w);
  r.z = pack_bf16x2(b.x, b.y);
  r.w = pack_bf16x2(b.z, b.w);
  return r;
}

// D += A * B for one 16x16x32 bf16 MFMA.  Lane l supplies row (l % 16) of A
// and column (l % 16) of B, each as 8 consecutive k of the k-group (l / 16);
// it receives rows 4*(l/16) .. 4*(l/16)+3 of column (l % 16) of D.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// 8 FP8 E4M3 codes (two dwords, code j in byte j) as 8 bf16, exactly: every
// E4M3 value is a bf16 value (v_cvt_scalef32_pk_bf16_fp8 with scale 1; checked
// against the format's definition for all 256 codes)
__device__ __forceinline__ u32x4 fp8x8_to_bf16(uint2 v) {
  u32x4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true));
  return r;
}

// Four consecutive outputs with one store instruction (p 8-byte aligned for
// bf16, 16-byte aligned for fp32).  Stores count in vmcnt like loads, so an
// epilogue of single-element stores makes the next wait for a stage in flight
// also wait for them.
template <class S>
__device__ __forceinline__ void store_out4(typename S::T* p, f32x4 v);
template <>
__device__ __forceinline__ void store_out4<F32>(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
template <>
__device__ __forceinline__ void store_out4<BF16>(uint16_t* p, f32x4 v) {
  uint2 q;
  q.x = pack_bf16x2(v.x, v.y);
  q.y = pack_bf16x2(v.z, v.w);
  *reinterpret_cast<uint2*>(p) = q;
}

template <class S>
__device__ __forceinline__ void store_out(typename S::T* p, float v);
template <>
__device__ __forceinline__ void store_out<F32>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<BF16>(uint16_t* p, float v) { *p = f32_to_bf16(v); }

}  // namespace moe
