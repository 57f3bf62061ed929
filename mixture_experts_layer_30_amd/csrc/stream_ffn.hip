// Weight-streaming grouped SwiGLU FFN on gfx950 (the HBM-bound, decode-shape
// schedule).
//
// At decode batch sizes each active expert sees a handful of tokens, so the
// layer's time is the time to read every active expert's weights from HBM
// once (the "weight amplification" of the Serving-tax notes, decode-phase
// section and finding 1).  This schedule reads each weight byte exactly once
// per pass of up to 16*TB tokens and keeps the tokens on the narrow side of
// the MFMA ("swap-AB"): weight rows are the M dimension (16-row tiles) and the
// expert's tokens the N dimension (16-token blocks).
//
// Workgroup = 4 wavefronts = one slab of 64 weight rows of one expert:
//   gate/up half: 32 gate rows and the 32 matching up rows (32 intermediate
//                 columns), so the SwiGLU is applied in the epilogue;
//   down half:    64 rows of W2 (64 output features).
// The wavefronts split the contraction dimension (H, resp. I) four ways; each
// streams its quarter of the 64 rows straight from HBM into MFMA operand
// registers (16-byte loads, the 4 lanes of a row covering 64 contiguous bytes
// per instruction), with D chunks of 64 k in flight, so the loop has no LDS
// traffic and no barrier.  Token rows come the same way (they are small and
// stay in L2).  At the end the four partial sums meet in LDS, where the
// SwiGLU (gate/up half) or the scatter to pair order (down half) happens.
//
// Grid: (slabs, experts).  Workgroups of experts with no tokens return at
// once, so an unused expert's weights are never read.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kStreamThreads = 256;
constexpr int kStreamWaves = kStreamThreads / kWave;
constexpr int kTiles = 4;    // 16-row weight tiles per workgroup
constexpr int kChunk = 64;   // k per pipeline stage: two 16x16x32 MFMA steps

// Tuning knobs: waves per SIMD the register budget must allow, and chunks in
// flight per wavefront for a pass of NB token blocks.
#ifndef MOE_STREAM_WAVES_PER_SIMD
#define MOE_STREAM_WAVES_PER_SIMD 2
#endif
#ifndef MOE_STREAM_DEPTH_1
#define MOE_STREAM_DEPTH_1 4
#endif
#ifndef MOE_STREAM_DEPTH_2
#define MOE_STREAM_DEPTH_2 3
#endif
#ifndef MOE_STREAM_DEPTH_4
#define MOE_STREAM_DEPTH_4 2
#endif

template <class SW, int NB>
constexpr int stream_depth() {
  return sizeof(typename SW::T) == 4 ? 1
         : NB == 1 ? MOE_STREAM_DEPTH_1
         : NB == 2 ? MOE_STREAM_DEPTH_2
                   : MOE_STREAM_DEPTH_4;
}

// acc[q][tb] += W(tile q) * X(token block tb)^T for tb < NB, over chunks
// [c_begin, c_end).  Lane l = 16*g + m supplies row m of every tile and of
// every token block, with k offsets 8g and 32 + 8g inside each chunk (the
// same for both operands, which is all the contraction needs).
//
// NB is the exact number of token blocks of the pass (the caller dispatches
// on it), so every load of the loop is unconditional and the in-order vector
// memory counter lets D chunks stay in flight.  Prefetches past the wave's
// last chunk re-read that chunk (an L1/L2 hit) instead of branching.
template <class SW, class SX, int NB, int TB>
__device__ __forceinline__ void stream_mainloop(const typename SW::T* const (&wrow)[kTiles],
                                                const typename SX::T* const (&xrow)[TB],
                                                int c_begin, int c_end, int g,
                                                f32x4 (&acc)[kTiles][TB]) {
  constexpr int D = stream_depth<SW, NB>();
  if (c_begin >= c_end) return;
  u32x4 wr[D][kTiles][2];
  u32x4 xr[D][NB][2];
  const int kofs = g * 8;
  const int c_last = c_end - 1;

  auto issue = [&](int d, int c) {
    const int k = min(c, c_last) * kChunk + kofs;
#pragma unroll
    for (int q = 0; q < kTiles; ++q) {
      wr[d][q][0] = load8<SW>(wrow[q] + k);
      wr[d][q][1] = load8<SW>(wrow[q] + k + 32);
    }
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      xr[d][tb][0] = load8<SX>(xrow[tb] + k);
      xr[d][tb][1] = load8<SX>(xrow[tb] + k + 32);
    }
  };
  auto compute = [&](int d) {
#pragma unroll
    for (int tb = 0; tb < NB; ++tb)
#pragma unroll
      for (int q = 0; q < kTiles; ++q) {
        acc[q][tb] = mfma16x16x32(wr[d][q][0], xr[d][tb][0], acc[q][tb]);
        acc[q][tb] = mfma16x16x32(wr[d][q][1], xr[d][tb][1], acc[q][tb]);
      }
  };

#pragma unroll
  for (int d = 0; d < D; ++d) issue(d, c_begin + d);
  for (int c = c_begin; c < c_end; c += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (c + d < c_end) compute(d);
      issue(d, c + d + D);
    }
  }
}

// Runs the main loop specialised for the pass's ntb token blocks (1..TB).
template <class SW, class SX, int TB>
__device__ __forceinline__ void stream_pass(const typename SW::T* const (&wrow)[kTiles],
                                            const typename SX::T* const (&xrow)[TB], int ntb,
                                            int c_begin, int c_end, int g,
                                            f32x4 (&acc)[kTiles][TB]) {
  if (TB >= 4 && ntb > 2)
    stream_mainloop<SW, SX, (TB >= 4 ? 4 : TB), TB>(wrow, xrow, c_begin, c_end, g, acc);
  else if (TB >= 2 && ntb == 2)
    stream_mainloop<SW, SX, (TB >= 2 ? 2 : TB), TB>(wrow, xrow, c_begin, c_end, g, acc);
  else
    stream_mainloop<SW, SX, 1, TB>(wrow, xrow, c_begin, c_end, g, acc);
}

struct Bucket {
  int n;     // tokens (rows) of this expert
  int row0;  // first row of the expert in the alignment (0 for dense)
};

template <bool kDense>
__device__ __forceinline__ Bucket bucket_of(const RowMap& rm, int e) {
  if (kDense) return Bucket{(int)rm.dense_rows, 0};
  return Bucket{rm.counts[e], rm.offsets[e]};
}

// Partial sums of the 4 wavefronts: [wave][row of the 64-row slab][token of a 16-block].
// The +1 keeps both the fragment writes and the epilogue reads free of bank conflicts.
struct StreamSmem {
  float part[kStreamWaves][kTiles * 16][17];
  int tok[128];   // token (gate/up) or act row (down) of each row of the pass
  int dst[128];   // down: output row of each row of the pass
};

// Chunks [c_begin, c_end) of wavefront `wave`: the workgroup's slice z =
// blockIdx.z of the gridDim.z-way split of the contraction, cut four ways.
__device__ __forceinline__ void split_range(int nch, int wave, int& c_begin, int& c_end) {
  const int z = blockIdx.z, nz = gridDim.z;
  const int z0 = z * nch / nz, z1 = (z + 1) * nch / nz;
  c_begin = z0 + wave * (z1 - z0) / kStreamWaves;
  c_end = z0 + (wave + 1) * (z1 - z0) / kStreamWaves;
}

// Gate/up half: act[row][i] = silu(W1_e x_t)_i * (W3_e x_t)_i, bf16.
// Tiles of the slab: 0 = gate i0..i0+15, 1 = up i0..i0+15, 2 = gate i0+16..i0+31,
// 3 = up i0+16..i0+31.
template <class S, int TB, bool kDense>
__global__ __launch_bounds__(kStreamThreads, MOE_STREAM_WAVES_PER_SIMD) void stream_gate_up_kernel(
    const typename S::T* __restrict__ x, const typename S::T* __restrict__ w13, RowMap rm, int H,
    int I, uint16_t* __restrict__ act, float* __restrict__ part) {
  __shared__ StreamSmem sm;
  const int e = blockIdx.y;
  const Bucket bk = bucket_of<kDense>(rm, e);
  if (bk.n == 0 || (!kDense && bk.n < rm.min_rows)) return;
  constexpr bool dense = kDense;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int m = lane & 15, g = lane >> 4;
  const int i0 = blockIdx.x * 32;

  const typename S::T* wexp = w13 + (size_t)e * 2 * I * H;
  const typename S::T* const wrow[kTiles] = {
      wexp + (size_t)(i0 + m) * H, wexp + (size_t)(I + i0 + m) * H,
      wexp + (size_t)(i0 + 16 + m) * H, wexp + (size_t)(I + i0 + 16 + m) * H};
  int c_begin, c_end;
  split_range(H / kChunk, wave, c_begin, c_end);

  for (int base = 0; base < bk.n; base += 16 * TB) {
    const int n_pass = min(16 * TB, bk.n - base);
    const int ntb = (n_pass + 15) / 16;
    __syncthreads();
    for (int j = threadIdx.x; j < 16 * TB; j += kStreamThreads) {
      const int jj = j < n_pass ? j : 0;  // rows past the bucket reuse its first token
      sm.tok[j] = dense ? base + jj : rm.sorted_ids[bk.row0 + base + jj] / rm.K;
    }
    __syncthreads();
    const typename S::T* xrow[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) xrow[tb] = x + (size_t)sm.tok[tb * 16 + m] * H;

    f32x4 acc[kTiles][TB];
#pragma unroll
    for (int q = 0; q < kTiles; ++q)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) acc[q][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_pass<S, S, TB>(wrow, xrow, ntb, c_begin, c_end, g, acc);

#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      if (tb >= ntb) break;
#pragma unroll
      for (int q = 0; q < kTiles; ++q) {
        sm.part[wave][q * 16 + 4 * g + 0][m] = acc[q][tb].x;
        sm.part[wave][q * 16 + 4 * g + 1][m] = acc[q][tb].y;
        sm.part[wave][q * 16 + 4 * g + 2][m] = acc[q][tb].z;
        sm.part[wave][q * 16 + 4 * g + 3][m] = acc[q][tb].w;
      }
      __syncthreads();
      const int il = threadIdx.x & 31;
      const int gate_r = (il >> 4) * 32 + (il & 15);
      const int up_r = gate_r + 16;
      for (int tk = threadIdx.x >> 5; tk < 16; tk += kStreamThreads / 32) {
        const int j = tb * 16 + tk;
        if (j < n_pass) {
          float gs = 0.f, us = 0.f;
#pragma unroll
          for (int w = 0; w < kStreamWaves; ++w) {
            gs += sm.part[w][gate_r][tk];
            us += sm.part[w][up_r][tk];
          }
          const size_t row = (size_t)(bk.row0 + base + j);
          if (part) {  // split-K: raw sums, the finish kernel applies the SwiGLU
            float* pr = part + ((size_t)blockIdx.z * rm.dense_rows + row) * (2 * (size_t)I);
            pr[i0 + il] = gs;
            pr[I + i0 + il] = us;
          } else {
            act[row * I + i0 + il] = f32_to_bf16(silu(gs) * us);
          }
        }
      }
      __syncthreads();
    }
  }
}

// Down half: y[p][h] = sum_i W2_e[h][i] act[row][i] for the valid rows of expert e,
// written to the pair's row p = sorted_ids[row] (dense: row = token = output row).
template <class SW, class SY, int TB, bool kDense>
__global__ __launch_bounds__(kStreamThreads, MOE_STREAM_WAVES_PER_SIMD) void stream_down_kernel(
    const typename SW::T* __restrict__ w2, const uint16_t* __restrict__ act, RowMap rm, int H,
    int I, typename SY::T* __restrict__ y, float* __restrict__ part) {
  __shared__ StreamSmem sm;
  const int e = blockIdx.y;
  const Bucket bk = bucket_of<kDense>(rm, e);
  if (bk.n == 0 || (!kDense && bk.n < rm.min_rows)) return;
  constexpr bool dense = kDense;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int m = lane & 15, g = lane >> 4;
  const int h0 = blockIdx.x * 64;

  const typename SW::T* wexp = w2 + (size_t)e * H * I;
  const typename SW::T* const wrow[kTiles] = {
      wexp + (size_t)(h0 + m) * I, wexp + (size_t)(h0 + 16 + m) * I,
      wexp + (size_t)(h0 + 32 + m) * I, wexp + (size_t)(h0 + 48 + m) * I};
  int c_begin, c_end;
  split_range(I / kChunk, wave, c_begin, c_end);

  for (int base = 0; base < bk.n; base += 16 * TB) {
    const int n_pass = min(16 * TB, bk.n - base);
    const int ntb = (n_pass + 15) / 16;
    __syncthreads();
    for (int j = threadIdx.x; j < 16 * TB; j += kStreamThreads) {
      const int jj = j < n_pass ? j : 0;
      const int row = bk.row0 + base + jj;
      sm.tok[j] = row;
      sm.dst[j] = dense ? row : rm.sorted_ids[row];
    }
    __syncthreads();
    const uint16_t* xrow[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) xrow[tb] = act + (size_t)sm.tok[tb * 16 + m] * I;

    f32x4 acc[kTiles][TB];
#pragma unroll
    for (int q = 0; q < kTiles; ++q)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) acc[q][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_pass<SW, BF16, TB>(wrow, xrow, ntb, c_begin, c_end, g, acc);

#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      if (tb >= ntb) break;
#pragma unroll
      for (int q = 0; q < kTiles; ++q) {
        sm.part[wave][q * 16 + 4 * g + 0][m] = acc[q][tb].x;
        sm.part[wave][q * 16 + 4 * g + 1][m] = acc[q][tb].y;
        sm.part[wave][q * 16 + 4 * g + 2][m] = acc[q][tb].z;
        sm.part[wave][q * 16 + 4 * g + 3][m] = acc[q][tb].w;
      }
      __syncthreads();
      const int hl = threadIdx.x & 63;
      for (int tk = threadIdx.x >> 6; tk < 16; tk += kStreamThreads / 64) {
        const int j = tb * 16 + tk;
        if (j < n_pass) {
          float s = 0.f;
#pragma unroll
          for (int w = 0; w < kStreamWaves; ++w) s += sm.part[w][hl][tk];
          if (part)  // split-K: raw sums, the finish kernel adds the slices
            part[((size_t)blockIdx.z * rm.dense_rows + sm.dst[j]) * H + h0 + hl] = s;
          else
            store_out<SY>(y + (size_t)sm.dst[j] * H + h0 + hl, s);
        }
      }
      __syncthreads();
    }
  }
}

// Split-K finish: sums the slices in slice order, V consecutive elements a
// thread (4 where the row length allows: 16-byte loads of the partial sums).
// (gate/up: the partial sums cover columns col0.. of I, W = I - col0 of each)
template <int V>
__global__ __launch_bounds__(256) void finish_gate_up_kernel(const float* __restrict__ part,
                                                             int splits, int64_t rows, int I,
                                                             int col0,
                                                             uint16_t* __restrict__ act,
                                                             const int32_t* __restrict__ out_row) {
  const int W = I - col0;
  const int64_t idx = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * V;
  if (idx >= rows * W) return;
  const int64_t r = idx / W;
  const int i = (int)(idx % W);
  const int64_t o = out_row ? out_row[r] : r;
  if (o < 0) return;
  if constexpr (V == 4) {
    f32x4 g = f32x4{0.f, 0.f, 0.f, 0.f}, u = g;
    for (int z = 0; z < splits; ++z) {
      const float* pr = part + ((size_t)z * rows + r) * (2 * (size_t)W);
      g += *reinterpret_cast<const f32x4*>(pr + i);
      u += *reinterpret_cast<const f32x4*>(pr + W + i);
    }
    uint2 v;
    v.x = pack_bf16x2(silu(g.x) * u.x, silu(g.y) * u.y);
    v.y = pack_bf16x2(silu(g.z) * u.z, silu(g.w) * u.w);
    *reinterpret_cast<uint2*>(act + o * I + col0 + i) = v;
  } else {
    float g = 0.f, u = 0.f;
    for (int z = 0; z < splits; ++z) {
      const float* pr = part + ((size_t)z * rows + r) * (2 * (size_t)W);
      g += pr[i];
      u += pr[W + i];
    }
    act[o * I + col0 + i] = f32_to_bf16(silu(g) * u);
  }
}

template <class SY, int V>
__global__ __launch_bounds__(256) void finish_down_kernel(const float* __restrict__ part,
                                                          int splits, int64_t rows, int H,
                                                          typename SY::T* __restrict__ y,
                                                          const int32_t* __restrict__ skip) {
  const int64_t idx = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * V;
  if (idx >= rows * H) return;
  if (skip && skip[idx / H] < 0) return;
  if constexpr (V == 4) {
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < splits; ++z)
      s += *reinterpret_cast<const f32x4*>(part + (size_t)z * rows * H + idx);
    store_out4<SY>(y + idx, s);
  } else {
    float s = 0.f;
    for (int z = 0; z < splits; ++z) s += part[(size_t)z * rows * H + idx];
    store_out<SY>(y + idx, s);
  }
}

template <class S, int TB>
static void launch_gu(const void* x, const void* w13, const RowMap& rm, int E, int H, int I,
                      int splits, uint16_t* act, float* part, hipStream_t s) {
  if (rm.counts == nullptr)
    hipLaunchKernelGGL((stream_gate_up_kernel<S, TB, true>), dim3(I / 32, E, splits),
                       dim3(kStreamThreads), 0, s, static_cast<const typename S::T*>(x),
                       static_cast<const typename S::T*>(w13), rm, H, I, act, part);
  else
    hipLaunchKernelGGL((stream_gate_up_kernel<S, TB, false>), dim3(I / 32, E, splits),
                       dim3(kStreamThreads), 0, s, static_cast<const typename S::T*>(x),
                       static_cast<const typename S::T*>(w13), rm, H, I, act, part);
}

template <class SW, class SY, int TB>
static void launch_dn(const void* w2, const uint16_t* act, const RowMap& rm, int E, int H, int I,
                      int splits, void* y, float* part, hipStream_t s) {
  if (rm.counts == nullptr)
    hipLaunchKernelGGL((stream_down_kernel<SW, SY, TB, true>), dim3(H / 64, E, splits),
                       dim3(kStreamThreads), 0, s, static_cast<const typename SW::T*>(w2), act, rm,
                       H, I, static_cast<typename SY::T*>(y), part);
  else
    hipLaunchKernelGGL((stream_down_kernel<SW, SY, TB, false>), dim3(H / 64, E, splits),
                       dim3(kStreamThreads), 0, s, static_cast<const typename SW::T*>(w2), act, rm,
                       H, I, static_cast<typename SY::T*>(y), part);
}

template <class S>
static void gu_tb(const void* x, const void* w13, const RowMap& rm, int E, int H, int I, int tb,
                  int splits, uint16_t* act, float* part, hipStream_t s) {
  if (tb <= 1) launch_gu<S, 1>(x, w13, rm, E, H, I, splits, act, part, s);
  else if (tb == 2) launch_gu<S, 2>(x, w13, rm, E, H, I, splits, act, part, s);
  else launch_gu<S, 4>(x, w13, rm, E, H, I, splits, act, part, s);
}

template <class SW, class SY>
static void dn_tb(const void* w2, const uint16_t* act, const RowMap& rm, int E, int H, int I,
                  int tb, int splits, void* y, float* part, hipStream_t s) {
  if (tb <= 1) launch_dn<SW, SY, 1>(w2, act, rm, E, H, I, splits, y, part, s);
  else if (tb == 2) launch_dn<SW, SY, 2>(w2, act, rm, E, H, I, splits, y, part, s);
  else launch_dn<SW, SY, 4>(w2, act, rm, E, H, I, splits, y, part, s);
}

hipError_t launch_stream_gate_up(const void* x, int xdt, const void* w13, const RowMap& rm, int E,
                                 int H, int I, int tok_blocks, int splits, uint16_t* act,
                                 float* part, hipStream_t s) {
  float* p = splits > 1 ? part : nullptr;
  if (xdt == kDtF32) gu_tb<F32>(x, w13, rm, E, H, I, tok_blocks, splits, act, p, s);
  else gu_tb<BF16>(x, w13, rm, E, H, I, tok_blocks, splits, act, p, s);
  if (splits > 1) return launch_finish_gate_up(part, splits, rm.dense_rows, I, act, s);
  return hipGetLastError();
}

hipError_t launch_stream_down(const void* w2, int wdt, const uint16_t* act, const RowMap& rm,
                              int E, int H, int I, int tok_blocks, int splits, void* y, int ydt,
                              float* part, hipStream_t s) {
  float* p = splits > 1 ? part : nullptr;
  if (wdt == kDtF32) {
    if (ydt == kDtF32) dn_tb<F32, F32>(w2, act, rm, E, H, I, tok_blocks, splits, y, p, s);
    else dn_tb<F32, BF16>(w2, act, rm, E, H, I, tok_blocks, splits, y, p, s);
  } else {
    if (ydt == kDtF32) dn_tb<BF16, F32>(w2, act, rm, E, H, I, tok_blocks, splits, y, p, s);
    else dn_tb<BF16, BF16>(w2, act, rm, E, H, I, tok_blocks, splits, y, p, s);
  }
  if (splits > 1) return launch_finish_down(part, splits, rm.dense_rows, H, y, ydt, s);
  return hipGetLastError();
}

hipError_t launch_finish_gate_up(const float* part, int splits, int64_t rows, int I,
                                 uint16_t* act, hipStream_t s, const int32_t* out_row, int col0) {
  const int64_t n = rows * (I - col0);
  if (n == 0) return hipSuccess;
  if ((I - col0) % 4 == 0 && I % 4 == 0 && col0 % 4 == 0)
    hipLaunchKernelGGL(finish_gate_up_kernel<4>, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256),
                       0, s, part, splits, rows, I, col0, act, out_row);
  else
    hipLaunchKernelGGL(finish_gate_up_kernel<1>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       s, part, splits, rows, I, col0, act, out_row);
  return hipGetLastError();
}

hipError_t launch_finish_down(const float* part, int splits, int64_t rows, int H, void* y,
                              int ydt, hipStream_t s, const int32_t* skip) {
  const int64_t n = rows * H;
  if (n == 0) return hipSuccess;
  auto go = [&](auto v) {
    constexpr int V = decltype(v)::value;
    const unsigned blocks = (unsigned)((n / V + 255) / 256);
    if (ydt == kDtF32)
      hipLaunchKernelGGL((finish_down_kernel<F32, V>), dim3(blocks), dim3(256), 0, s, part,
                         splits, rows, H, static_cast<float*>(y), skip);
    else
      hipLaunchKernelGGL((finish_down_kernel<BF16, V>), dim3(blocks), dim3(256), 0, s, part,
                         splits, rows, H, static_cast<uint16_t*>(y), skip);
  };
  if (H % 4 == 0) go(std::integral_constant<int, 4>{});
  else go(std::integral_constant<int, 1>{});
  return hipGetLastError();
}

}  // namespace moe
