// Weight-streaming grouped SwiGLU FFN, LDS-ring variant for bf16 storage (the
// decode-shape schedule when weights and tokens are bf16 and the shapes tile).
//
// Decode time is the time to read every active expert's weights from HBM once
// (weight amplification, Serving-tax notes, decode-phase section).  Register
// loads shaped for the MFMA operands touch half a 128-byte line per row per
// instruction and read HBM at about 5.8 TB/s on gfx950.  This variant streams
// the weights with non-temporal direct global->LDS loads
// (global_load_lds_dwordx4), whose 64 lanes fetch 4 rows x 256 contiguous
// bytes, through a ring of stages in LDS, and reads the MFMA fragments back
// from LDS (a small fraction of LDS bandwidth at HBM rates): 6.3-6.6 TB/s.
//
// Workgroup = 8 wavefronts, one per CU (the ring takes 144-160 KB of LDS),
// persistent.  A work unit is one pass of up to 16*NB of an expert's tokens
// over one contraction slice of one 128-row weight slab; the U units are
// numbered expert-major and workgroup b takes the contiguous run
// [U*b/G, U*(b+1)/G), so every workgroup gets the same number of units
// whatever the experts' loads.  One stage holds, for 128 k, the slab's 128
// weight rows and the pass's token rows; the load side runs ST-1 stages ahead
// of the multiply side across unit boundaries, so the ring never drains
// between units.  Wavefront w owns weight rows 16w..16w+15 of the slab and
// multiplies them by every token block over the whole slice, so no
// cross-wavefront reduction is needed.
//
//   gate/up: a slab is 64 intermediate columns; wavefront w's 16 rows are
//            gate and up rows of 8 columns ordered so that each lane's 4
//            accumulator rows are (gate c, gate c+1, up c, up c+1): the
//            SwiGLU is applied in registers.
//   down:    a slab is 128 consecutive output features.
//
// The token rows share the stage with the weights, so more token blocks per
// pass leave fewer stages in flight; the library runs this kernel with one or
// two blocks and, for bf16, hands experts with more tokens than a pass to the
// register-streaming kernel (RowMap min_rows / max_rows); FP8 experts take as
// many passes as they need (measured faster than a second launch with four
// blocks, whose 64 token rows every wavefront reads from LDS per stage).
//
// Rows of the alignment (token ids, output rows) and the experts' counts are
// read with scalar loads, which complete on a different counter than the
// vector loads: waiting for them does not wait for the stages in flight (a
// vector load of them would, since vector loads complete in order).
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kRWaves = 8;
constexpr int kRThreads = kRWaves * kWave;
constexpr int kRRows = 128;      // weight rows per slab
constexpr int kRK = 128;         // contraction elements per stage of bf16 weights
constexpr int kRLds = 160 * 1024;

// SW: weight storage (BF16, or FP8 codes with row scales).  KS: contraction
// elements per stage: 128 for bf16; 256 for FP8 with at most two token blocks
// where the contraction allows (the weight rows of a stage are then 256 contiguous bytes, as for bf16: HBM
// serves 128-byte pieces of rows 4 KB apart at less than half the rate), else
// 128.  NB: token blocks of 16 per pass.  A slot holds the slab's 128 weight
// rows and the pass's 16*NB bf16 token rows; as many stages as fit (3 to 8).
// Every wavefront issues the same number of loads per stage, so one vmcnt
// bound serves all.
template <class SW, int KS>
constexpr int ring_wrow_bytes() { return KS * SW::kBytes; }
template <class SW, int KS, int NB>
constexpr int ring_slot_bytes() { return kRRows * ring_wrow_bytes<SW, KS>() + 16 * NB * 2 * KS; }
template <class SW, int KS, int NB>
constexpr int ring_stages() {
  return kRLds / ring_slot_bytes<SW, KS, NB>() > 8 ? 8 : kRLds / ring_slot_bytes<SW, KS, NB>();
}
// direct loads per wavefront per stage: its 16 weight rows, its 2*NB token rows
template <class SW, int KS>
constexpr int ring_wloads() { return 16 * ring_wrow_bytes<SW, KS>() / 1024; }
template <int KS, int NB>
constexpr int ring_tok_loads() { return (2 * NB * 2 * KS + 1023) / 1024; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 64 lanes x 16 bytes from global memory (lane's own address) into LDS at
// lds + 16 * lane, without passing through registers.  kStream marks the data
// as read once (non-temporal), which on gfx950 raises the HBM read rate of
// these strided row segments by about 15 % (measured) and keeps them from
// displacing the token rows in the caches.
template <bool kStream>
__device__ __forceinline__ void load_lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 16, 0, kStream ? 2 : 0);
}

// Byte offset of 16-byte segment s of row r in a region of RB-byte rows (RB a
// multiple of 256): segments are permuted by the row's low 4 bits, so the 16
// rows a fragment read touches hit 16 different 16-byte bank groups.
template <int RB>
__device__ __forceinline__ int roff(int r, int s) { return r * RB + ((s ^ (r & 15)) << 4); }

// The same for 128-byte rows (FP8 weights at 128 k per stage): segments
// permuted by bits 1..3 of the row, so the 16 rows of a fragment read (two rows
// per 256 bytes) cover all 64 banks.
__device__ __forceinline__ int roff8(int r, int s) { return r * 128 + ((s ^ ((r >> 1) & 7)) << 4); }

__device__ __forceinline__ void barrier_nf() { asm volatile("s_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

struct RingWork {
  int nslabs;     // 128-row slabs per expert
  int nexp;       // experts (1 for dense rows)
  int ksplit;     // contraction slices
  int nks;        // stages over the whole contraction (Kdim / KS)
  int64_t prows;  // rows of one slice of partial sums: dense rows, or T*K pairs
};

// Position in the workgroup's run of work units.  A unit is one pass of up to
// 16*NB of an expert's tokens over one contraction slice of one 128-row slab;
// units are numbered expert-major, then slab, slice, pass, and workgroup b
// takes the contiguous run [U*b/G, U*(b+1)/G) of the U units, so workgroups
// get equal numbers of units whatever the experts' loads.
struct RingIt {
  int left;                // units still to visit, counting the current one
  int e, slab, z, pass;    // current unit
  int n, row0, npass;      // tokens of expert e, its first alignment row, its passes
  int ks, ks0, ks1;        // stage, and the stages of slice z
};

template <int NB, bool kDense>
__device__ __forceinline__ void ring_expert(RingIt& it, const RowMap& rm,
                                            const int32_t* __restrict__ counts,
                                            const int32_t* __restrict__ offsets) {
  it.n = kDense ? (int)rm.dense_rows : counts[it.e];
  it.row0 = kDense ? 0 : offsets[it.e];
  it.npass = (it.n + 16 * NB - 1) / (16 * NB);
}

__device__ __forceinline__ void ring_slice(RingIt& it, const RingWork& wk) {
  it.ks0 = it.z * wk.nks / wk.ksplit;
  it.ks1 = (it.z + 1) * wk.nks / wk.ksplit;
  it.ks = it.ks0;
}

// Advances one stage; at the end of a unit, to the next unit (skipping experts
// without tokens).  it.left == 0 once the run is done.
template <int NB, bool kDense>
__device__ __forceinline__ void ring_next(RingIt& it, const RowMap& rm, const RingWork& wk,
                                          const int32_t* __restrict__ counts,
                                          const int32_t* __restrict__ offsets) {
  if (++it.ks < it.ks1) return;
  if (--it.left == 0) return;
  it.ks = it.ks0;
  if (++it.pass < it.npass) return;
  it.pass = 0;
  if (++it.z < wk.ksplit) {
    ring_slice(it, wk);
    return;
  }
  it.z = 0;
  ring_slice(it, wk);
  if (++it.slab < wk.nslabs) return;
  it.slab = 0;
  // next expert with units: tokens, min_rows to max_rows of them
  int n;
  do {
    ++it.e;
    n = kDense ? (int)rm.dense_rows : counts[it.e];
  } while (it.e < wk.nexp - 1 && (n == 0 || (!kDense && (n > rm.max_rows || n < rm.min_rows))));
  ring_expert<NB, kDense>(it, rm, counts, offsets);
}

// kGateUp: w = w13 [E][2I][H], xs = x [T][H], writes act [rows][I] (or fp32 gate/up
// sums to part [ksplit][prows][2I]).  Down: w = w2 [E][H][I], xs = act, writes
// y [pairs][H] at the pair of each row (or fp32 sums to part [ksplit][prows][H]).
// Partial sums of grouped rows are indexed by pair, so that a finish kernel
// can add them without the alignment.
// ids / counts / offsets are the plan's sorted_ids, expert_counts and
// expert_offsets (unused for dense rows); passed as restrict-qualified
// arguments, their wave-uniform reads compile to scalar loads.
template <class SW, class SY, int KS, int NB, bool kGateUp, bool kDense>
__global__ __launch_bounds__(kRThreads, 1) void ring_ffn_kernel(
    const typename SW::T* __restrict__ w, const float* __restrict__ wscale,
    const uint16_t* __restrict__ xs, RowMap rm, int H, int I, RingWork wk,
    uint16_t* __restrict__ act, typename SY::T* __restrict__ y, float* __restrict__ part,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets) {
  constexpr bool kFP8 = SW::kBytes == 1;
  constexpr int WB = ring_wrow_bytes<SW, KS>();  // bytes of a weight row per stage
  constexpr int WL = ring_wloads<SW, KS>();      // direct loads per wavefront for its 16 rows
  constexpr int WRPI = 1024 / WB;                // weight rows per direct load
  constexpr int WSEG = WB / 16;                  // 16-byte segments per weight row
  constexpr int TOK0 = kRRows * WB;              // byte offset of the token rows in a slot
  constexpr int TB = 2 * KS;                     // bytes of a token row per stage
  constexpr int TSEG = TB / 16;                  // lanes per token row in a direct load
  constexpr int TRPL = 64 / TSEG;                // token rows per direct load
  constexpr int TRW = 2 * NB;                    // token rows each wavefront loads
  constexpr int ST = ring_stages<SW, KS, NB>();
  constexpr int SB = ring_slot_bytes<SW, KS, NB>();
  constexpr int TL = ring_tok_loads<KS, NB>();
  constexpr int L = WL + TL;  // vector loads per wavefront per stage
  static_assert(WB == 128 || WB == 256, "weight row bytes");
  static_assert(TL * TRPL >= TRW && (TL - 1) * TRPL < TRW, "token loads");
  static_assert(ST >= 3 && (ST - 2) * L < 64, "stages");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[ST * SB];

  RingIt is;
  const int lane = threadIdx.x & (kWave - 1);
  // wave-uniform, so that indices derived from it stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int m = lane & 15, g = lane >> 4;
  const int G = (int)gridDim.x;
  const int Kdim = kGateUp ? H : I;      // contraction length (a multiple of KS)
  const int64_t wrows = kGateUp ? 2 * (int64_t)I : H;  // weight rows per expert

  // Weight row of row t (0..15) of wavefront `wave`'s tile in slab `slab`.
  auto wrow = [&](int slab, int t) -> int64_t {
    if (kGateUp) {
      const int col = slab * 64 + 8 * wave + 2 * (t >> 2) + (t & 1);
      return ((t >> 1) & 1) * (int64_t)I + col;
    }
    return (int64_t)slab * kRRows + 16 * wave + t;
  };
  // Row of the token operand for row r (< 16*NB) of the current pass: rows past
  // the expert's tokens repeat the pass's first row (their products are never
  // stored).  Gate/up: the token's row of x; down: the row of act.
  auto tok_row = [&](const RingIt& it, int r) -> int64_t {
    const int base = it.pass * 16 * NB;
    const int rr = base + r < it.n ? base + r : base;
    if (kDense) return rr;
    if (kGateUp) return ids[it.row0 + rr] / rm.K;
    return it.row0 + rr;
  };

  // ---- load side ----
  // Lane's weight rows for its WL direct loads (WRPI rows x WB bytes each) and
  // token rows for its TL loads, refreshed at the first stage of every pass.
  const uint8_t* wsrc[WL];
  const uint16_t* tsrc[TL];
  auto refresh = [&](const RingIt& it) {
    const uint8_t* wexp =
        reinterpret_cast<const uint8_t*>(w) + (size_t)it.e * wrows * Kdim * SW::kBytes;
#pragma unroll
    for (int j = 0; j < WL; ++j) {
      const int t = WRPI * j + lane / WSEG;  // row within the wavefront's 16
      const int slot = lane % WSEG;
      // logical segment this lane fetches (the row's permuted slot `slot`)
      const int seg = WB == 128 ? (slot ^ ((t >> 1) & 7)) : (slot ^ t);
      wsrc[j] = wexp + (size_t)wrow(it.slab, t) * Kdim * SW::kBytes + seg * 16;
    }
    // token rows TRW*w .. TRW*w + TRW - 1, TRPL of them per load (TSEG lanes
    // each; lanes past the last row idle)
#pragma unroll
    for (int q = 0; q < TL; ++q) {
      const int rbase = TRW * wave + TRPL * q;
      const int i = lane / TSEG;  // row of this load
      int64_t tr = 0;
#pragma unroll
      for (int ii = 0; ii < TRPL; ++ii) {
        if (TRPL * q + ii < TRW) {
          const int64_t ri = tok_row(it, rbase + ii);
          tr = i == ii ? ri : tr;
        }
      }
      const int r = rbase + i;   // token row in the slot
      const int seg = (lane % TSEG) ^ (r & 15);
      tsrc[q] = xs + (size_t)tr * Kdim + seg * 8;
    }
  };
  auto issue = [&](const RingIt& it, int slot) {
    uint8_t* sl = ring + slot * SB;
    const size_t k = (size_t)it.ks * KS;
#pragma unroll
    for (int j = 0; j < WL; ++j)
      load_lds16<true>(wsrc[j] + k * SW::kBytes, sl + (16 * wave + WRPI * j) * WB);
#pragma unroll
    for (int q = 0; q < TL; ++q) {
      const int rbase = TRW * wave + TRPL * q;
      if (TL * TRPL == TRW || TRPL * q + lane / TSEG < TRW)
        load_lds16<false>(tsrc[q] + k, sl + TOK0 + rbase * TB);
    }
  };

  // ---- this workgroup's run of units ----
  {
    // units per expert, scanned across the workgroup (E <= 256 < kRThreads),
    // in LDS that the ring only uses after the barrier below
    int* sc = reinterpret_cast<int*>(ring);
    const int t = threadIdx.x;
    int u = 0;
    if (t < wk.nexp) {
      const int n = kDense ? (int)rm.dense_rows : counts[t];
      if (kDense || (n >= rm.min_rows && n <= rm.max_rows))
        u = (n + 16 * NB - 1) / (16 * NB) * wk.nslabs * wk.ksplit;
    }
    int incl = u;  // inclusive scan within the wavefront
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int v = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += v;
    }
    if (lane == kWave - 1) sc[kRThreads + wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int v = 0; v < kRWaves; ++v) {
      const int sv = sc[kRThreads + v];
      before += v < wave ? sv : 0;
      total += sv;
    }
    incl += before;
    const int b = (int)blockIdx.x;
    const int u0 = (int)((int64_t)total * b / G), u1 = (int)((int64_t)total * (b + 1) / G);
    if (u > 0 && incl - u <= u0 && u0 < incl) {  // the expert holding unit u0
      sc[kRThreads + kRWaves] = t;
      sc[kRThreads + kRWaves + 1] = u0 - (incl - u);
    }
    __syncthreads();
    is.left = u1 - u0;
    if (is.left > 0) {
      is.e = sc[kRThreads + kRWaves];
      const int r = sc[kRThreads + kRWaves + 1];
      ring_expert<NB, kDense>(is, rm, counts, offsets);
      is.pass = r % is.npass;
      const int q = r / is.npass;
      is.z = q % wk.ksplit;
      is.slab = q / wk.ksplit;
      ring_slice(is, wk);
    }
    __syncthreads();  // the scan's LDS is the ring's first slot
  }
  if (is.left == 0) return;
  RingIt ic = is;

  int issued = 0;
#pragma unroll
  for (int d = 0; d < ST - 1; ++d) {
    if (is.left > 0) {
      if (is.ks == is.ks0) refresh(is);
      issue(is, d);
      ++issued;
      ring_next<NB, kDense>(is, rm, wk, counts, offsets);
    }
  }

  f32x4 acc[NB];
#pragma unroll
  for (int tb = 0; tb < NB; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  int computed = 0, slot_c = 0, slot_i = ST - 1;

  while (ic.left > 0) {
    // stage `computed` has landed for this wavefront; the barrier makes every
    // wavefront's loads of it visible and retires every read of the slot
    // about to be refilled (last used by stage computed - 1)
    if (issued - computed - 1 >= ST - 2) wait_vm<(ST - 2) * L>();
    else wait_vm<0>();
    barrier_nf();
    if (is.left > 0) {
      if (is.ks == is.ks0) refresh(is);
      issue(is, slot_i);
      ++issued;
      slot_i = slot_i + 1 == ST ? 0 : slot_i + 1;
      ring_next<NB, kDense>(is, rm, wk, counts, offsets);
    }

    const int ntb = min(NB, (ic.n - ic.pass * 16 * NB + 15) / 16);
    const uint8_t* sl = ring + slot_c * SB;
    if (kFP8) {
      // 64 k per step: lane reads 16 codes of row m at k = 64kk + 16g .. +15 and
      // feeds the first 8 to one MFMA, the last 8 to a second one, with the
      // token values of the same k (the MFMA's k order is immaterial as long as
      // both operands follow it)
#pragma unroll
      for (int kk = 0; kk < KS / 64; ++kk) {
        const int r = 16 * wave + m;
        const u32x4 q = *reinterpret_cast<const u32x4*>(
            sl + (WB == 128 ? roff8(r, 4 * kk + g) : roff<WB>(r, 4 * kk + g)));
        const u32x4 a0 = fp8x8_to_bf16(uint2{q.x, q.y});
        const u32x4 a1 = fp8x8_to_bf16(uint2{q.z, q.w});
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
          if (tb < ntb) {
            const uint8_t* tr = sl + TOK0;
            const u32x4 b0 = *reinterpret_cast<const u32x4*>(tr + roff<TB>(16 * tb + m, 8 * kk + 2 * g));
            const u32x4 b1 =
                *reinterpret_cast<const u32x4*>(tr + roff<TB>(16 * tb + m, 8 * kk + 2 * g + 1));
            acc[tb] = mfma16x16x32(a0, b0, acc[tb]);
            acc[tb] = mfma16x16x32(a1, b1, acc[tb]);
          }
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KS / 32; ++kk) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(sl + roff<WB>(16 * wave + m, 4 * kk + g));
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
          if (tb < ntb) {
            const u32x4 b =
                *reinterpret_cast<const u32x4*>(sl + TOK0 + roff<TB>(16 * tb + m, 4 * kk + g));
            acc[tb] = mfma16x16x32(a, b, acc[tb]);
          }
        }
      }
    }
    ++computed;
    slot_c = slot_c + 1 == ST ? 0 : slot_c + 1;

    if (ic.ks + 1 == ic.ks1) {
      // epilogue of the pass: lane holds rows 4g..4g+3 of its tile for token m of each block
      const int base = ic.pass * 16 * NB;
      const int64_t prows = wk.prows;
      // FP8: the row scales of the lane's 4 rows (scalar loads of the wavefront's
      // 16, then a per-lane pick), applied before the SwiGLU / the store
      f32x4 rs = f32x4{1.f, 1.f, 1.f, 1.f};
      if (kFP8) {
        const float* se = wscale + (size_t)ic.e * wrows;
        float sv[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) sv[t] = se[wrow(ic.slab, t)];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v = sv[q];
#pragma unroll
          for (int gg = 1; gg < 4; ++gg) v = g == gg ? sv[4 * gg + q] : v;
          rs[q] = v;
        }
      }
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) {
        if (tb < ntb) {
          const int j = base + 16 * tb + m;  // row of the pass within the expert
          const f32x4 v = acc[tb] * rs;
          // pair of each token column (grouped down, and grouped partial sums):
          // scalar loads of the block's 16 alignment rows, then a per-lane pick
          int64_t pair = j;
          if (!kDense && (!kGateUp || part)) {
            const int jb = base + 16 * tb;
            const int last = ic.n - 1 - jb;  // last valid column of this block
            int d = 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int di = ids[ic.row0 + jb + (i < last ? i : last)];
              d = m == i ? di : d;
            }
            pair = d;
          }
          if (kGateUp) {
            if (j < ic.n) {
              const int64_t row = (int64_t)ic.row0 + j;
              const int c = ic.slab * 64 + 8 * wave + 2 * g;
              if (part) {
                float* pr = part + ((size_t)ic.z * prows + pair) * (2 * (size_t)I);
                *reinterpret_cast<float2*>(pr + c) = float2{v.x, v.y};   // c is even
                *reinterpret_cast<float2*>(pr + I + c) = float2{v.z, v.w};
              } else {
                *reinterpret_cast<uint32_t*>(act + row * I + c) =
                    pack_bf16x2(silu(v.x) * v.z, silu(v.y) * v.w);
              }
            }
          } else {
            const int64_t dst = pair;  // output row: the token (dense) or the pair
            if (j < ic.n) {
              const int h = ic.slab * kRRows + 16 * wave + 4 * g;
              if (part) {
                *reinterpret_cast<f32x4*>(part + ((size_t)ic.z * prows + dst) * H + h) = v;
              } else {
                typename SY::T* o = y + (size_t)dst * H + h;
                store_out4<SY>(o, v);
              }
            }
          }
        }
        acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    ring_next<NB, kDense>(ic, rm, wk, counts, offsets);
  }
}

namespace {

// compute units of the device current at the first call (a static initialised
// once, so concurrent first calls from several host threads do not race)
int num_cus() {
  static const int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    return cus;
  }();
  return n;
}

// Contraction slices for dense rows: the count minimising the stages on the
// critical path (rounds of G slab slices x stages per slice) plus the fp32 partial
// sums' round trip, in units of one stage of all G workgroups (256-byte weight
// rows per stage).  The round trip is weighted 3x its bytes: scattered fp32
// stores and a separate finish launch move them far slower than the weight
// stream (measured on MI355X at 32 dense rows: Mixtral's DenseFA, 448 gate/up
// slabs, ran 150 us split in 4 and 136 us unsplit, as the weighted model picks;
// DeepSeek-V3's, 288 slabs, stays split in 4: 179 us against 196 unsplit).
int ring_splits(int nslabs, int nks, int64_t rows, int outdim, int G) {
  int best = 1;
  double best_t = 1e30;
  const double stage_bytes = (double)kRRows * 256 * G;
  for (int ks = 1; ks <= 16 && ks * 4 <= nks; ++ks) {
    const int64_t items = (int64_t)nslabs * ks;
    double t = (double)((items + G - 1) / G) * ((nks + ks - 1) / ks);
    if (ks > 1) t += 3.0 * 2.0 * ks * rows * outdim * 4 / stage_bytes;
    if (t < best_t - 1e-9) {
      best_t = t;
      best = ks;
    }
  }
  return best;
}

template <class SW, class SY, int KS, int NB, bool kGateUp, bool kDense>
void ring_go(const void* w, const float* wscale, const void* xs, const RowMap& rm, int E, int H,
             int I, int ksplit, int64_t rows_bound, uint16_t* act, void* y, float* part,
             hipStream_t s) {
  RingWork wk;
  wk.nslabs = kGateUp ? I / 64 : H / kRRows;
  wk.nexp = kDense ? 1 : E;
  wk.ksplit = ksplit;
  wk.nks = (kGateUp ? H : I) / KS;
  wk.prows = kDense ? rm.dense_rows : rows_bound * rm.K;
  // units: at most every expert x slab x slice x pass of T tokens
  const int64_t most = (int64_t)wk.nexp * wk.nslabs * ksplit * ((rows_bound + 16 * NB - 1) / (16 * NB));
  const int G = (int)(most < num_cus() ? most : num_cus());
  if (G <= 0) return;
  hipLaunchKernelGGL((ring_ffn_kernel<SW, SY, KS, NB, kGateUp, kDense>), dim3(G), dim3(kRThreads), 0,
                     s, static_cast<const typename SW::T*>(w), wscale,
                     static_cast<const uint16_t*>(xs), rm, H, I, wk, act,
                     static_cast<typename SY::T*>(y), ksplit > 1 ? part : nullptr, rm.sorted_ids,
                     rm.counts, rm.offsets);
}

template <class SW, class SY, bool kGateUp, bool kDense>
void ring_nb(const void* w, const float* wscale, const void* xs, const RowMap& rm, int E, int H,
             int I, int64_t T, int tok_blocks, int ksplit, uint16_t* act, void* y, float* part,
             hipStream_t s) {
  if constexpr (SW::kBytes == 1) {
    if (ring_stage_k(kDtFP8, tok_blocks, kGateUp ? H : I) == 256) {
      if (tok_blocks <= 1)
        ring_go<SW, SY, 256, 1, kGateUp, kDense>(w, wscale, xs, rm, E, H, I, ksplit, T, act, y, part, s);
      else
        ring_go<SW, SY, 256, 2, kGateUp, kDense>(w, wscale, xs, rm, E, H, I, ksplit, T, act, y, part, s);
      return;
    }
  }
  if (tok_blocks <= 1) {
    ring_go<SW, SY, 128, 1, kGateUp, kDense>(w, wscale, xs, rm, E, H, I, ksplit, T, act, y, part, s);
  } else if (tok_blocks == 2) {
    ring_go<SW, SY, 128, 2, kGateUp, kDense>(w, wscale, xs, rm, E, H, I, ksplit, T, act, y, part, s);
  } else {
    ring_go<SW, SY, 128, 4, kGateUp, kDense>(w, wscale, xs, rm, E, H, I, ksplit, T, act, y, part, s);
  }
}

template <class SW>
hipError_t ring_gate_up(const void* x, const void* w13, const float* w13_scale, const RowMap& rm,
                        int E, int H, int I, int64_t T, int tok_blocks, int splits, uint16_t* act,
                        float* part, hipStream_t s) {
  const bool dense = rm.counts == nullptr;
  if (dense)
    ring_nb<SW, BF16, true, true>(w13, w13_scale, x, rm, E, H, I, T, tok_blocks, splits, act,
                                  nullptr, part, s);
  else
    ring_nb<SW, BF16, true, false>(w13, w13_scale, x, rm, E, H, I, T, tok_blocks, splits, act,
                                   nullptr, part, s);
  hipError_t e = hipGetLastError();
  // grouped partial sums are per pair: the finish writes each to its alignment row
  if (e == hipSuccess && splits > 1)
    e = dense ? launch_finish_gate_up(part, splits, rm.dense_rows, I, act, s)
              : launch_finish_gate_up(part, splits, T * rm.K, I, act, s, rm.inv_pos);
  return e;
}

template <class SW>
hipError_t ring_down(const void* w2, const float* w2_scale, const uint16_t* act, const RowMap& rm,
                     int E, int H, int I, int64_t T, int tok_blocks, int splits, void* y, int ydt,
                     float* part, hipStream_t s) {
  const bool dense = rm.counts == nullptr;
  if (ydt == kDtF32) {
    if (dense)
      ring_nb<SW, F32, false, true>(w2, w2_scale, act, rm, E, H, I, T, tok_blocks, splits, nullptr,
                                    y, part, s);
    else
      ring_nb<SW, F32, false, false>(w2, w2_scale, act, rm, E, H, I, T, tok_blocks, splits,
                                     nullptr, y, part, s);
  } else {
    if (dense)
      ring_nb<SW, BF16, false, true>(w2, w2_scale, act, rm, E, H, I, T, tok_blocks, splits,
                                     nullptr, y, part, s);
    else
      ring_nb<SW, BF16, false, false>(w2, w2_scale, act, rm, E, H, I, T, tok_blocks, splits,
                                      nullptr, y, part, s);
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && splits > 1)
    e = dense ? launch_finish_down(part, splits, rm.dense_rows, H, y, ydt, s)
              : launch_finish_down(part, splits, T * rm.K, H, y, ydt, s, rm.inv_pos);
  return e;
}

}  // namespace

bool ring_gate_up_ok(int xdt, int wdt, int H, int I) {
  return xdt == kDtBF16 && (wdt == kDtBF16 || wdt == kDtFP8) && H % kRK == 0 &&
         I % (wdt == kDtFP8 ? kRK : 64) == 0;
}

bool ring_down_ok(int wdt, int H, int I) {
  return (wdt == kDtBF16 || wdt == kDtFP8) && H % kRRows == 0 && I % kRK == 0;
}

// (sized for 256 CUs, MI355X's count, so that workspace sizes do not depend on
// the device queried)
int ring_gate_up_splits(int64_t rows, int H, int I, int ks) {
  return ring_splits(I / 64, H / ks, rows, 2 * I, 256);
}

int ring_down_splits(int64_t rows, int H, int I, int ks) {
  return ring_splits(H / kRRows, I / ks, rows, H, 256);
}

// Whole units are dealt to the workgroups, so with a slab per workgroup or
// more a split can still even out the rounds (Qwen2 at one token: 320 gate/up
// slabs, two rounds for some; split in 4, 1280 units are 5 each).  There it
// is taken only when the model gains a quarter: measured on MI355X, gains of
// 12% (Mixtral at one and two tokens) came out 4-8% slower, while Qwen2's 37%
// gave 16%.
int ring_grouped_splits(int64_t pairs, int64_t experts, int H, int I, bool gate_up, int ks) {
  const int64_t slabs = experts * (gate_up ? I / 64 : H / kRRows);
  if (slabs > (int64_t)1 << 20) return 1;
  const int nks = (gate_up ? H : I) / ks;
  const int outdim = gate_up ? 2 * I : H;
  const int s = ring_splits((int)slabs, nks, pairs, outdim, 256);
  if (slabs < 256 || s == 1) return s;
  const double t1 = (double)((slabs + 255) / 256) * nks;
  const double ts = (double)((slabs * s + 255) / 256) * ((nks + s - 1) / s) +
                    3.0 * 2.0 * s * pairs * outdim * 4 / ((double)kRRows * 256 * 256);
  return ts < 0.75 * t1 ? s : 1;
}

// (four token blocks of 256 k would leave two stages; measured slower than 128 k
// with five)
int ring_stage_k(int wdt, int tok_blocks, int kdim) {
  return wdt == kDtFP8 && tok_blocks <= 2 && kdim % 256 == 0 ? 256 : kRK;
}

hipError_t launch_ring_gate_up(const void* x, int wdt, const void* w13, const float* w13_scale,
                               const RowMap& rm, int E, int H, int I, int64_t T, int tok_blocks,
                               int splits, uint16_t* act, float* part, hipStream_t s) {
  if (wdt == kDtFP8)
    return ring_gate_up<FP8>(x, w13, w13_scale, rm, E, H, I, T, tok_blocks, splits, act, part, s);
  return ring_gate_up<BF16>(x, w13, nullptr, rm, E, H, I, T, tok_blocks, splits, act, part, s);
}

hipError_t launch_ring_down(const void* w2, int wdt, const float* w2_scale, const uint16_t* act,
                            const RowMap& rm, int E, int H, int I, int64_t T, int tok_blocks,
                            int splits, void* y, int ydt, float* part, hipStream_t s) {
  if (wdt == kDtFP8)
    return ring_down<FP8>(w2, w2_scale, act, rm, E, H, I, T, tok_blocks, splits, y, ydt, part, s);
  return ring_down<BF16>(w2, nullptr, act, rm, E, H, I, T, tok_blocks, splits, y, ydt, part, s);
}

}  // namespace moe
