// LDS-tiled grouped SwiGLU FFN on gfx950 (the MFMA-bound, prefill-shape
// schedule).
//
// In prefill each expert holds hundreds of tokens, and the grouped GEMM is
// bound by matrix-core throughput reduced by the per-expert split of the
// batch and by block padding (Serving-tax notes, Table 1 rows "GroupGEMM" and
// "padding"; the TEMPO page's grouped GEMM rounds the token dimension to
// 128-row tiles).  One workgroup computes a tile of 128 weight rows x one
// alignment block of BN tokens (BN = the plan's block, 64 or 128; every block
// belongs to one expert), over the whole contraction in steps of 64:
//
//   * weights (MFMA A, M = weight rows) and token rows (MFMA B, N = tokens,
//     gathered through the alignment for the gate/up half) go from HBM to
//     registers to LDS, double-buffered, one barrier per step; the next
//     step's global loads are in flight while the current one is multiplied;
//   * LDS rows are padded by 16 bytes, so the 16 rows one fragment read
//     touches fall in distinct banks;
//   * 4 wavefronts in 2 x 2, each 64 x BN/2 with 16x16x32 bf16 MFMAs;
//   * gate/up half: the tile's 16-row groups alternate gate and up rows of
//     the same intermediate columns, so each lane holds matching gate and up
//     sums and applies the SwiGLU in registers; down half: the rows are 128
//     output features and results go straight to the pair's output row.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kTileThreads = 256;
constexpr int kBM = 128;            // weight rows per workgroup
constexpr int kBK = 64;             // contraction per step
constexpr int kLdsRow = kBK + 8;    // bf16 elements per LDS row (16-byte pad)

template <int BN>
struct TileSmem {
  uint16_t a[2][kBM * kLdsRow];
  uint16_t b[2][BN * kLdsRow];
  int tok[BN];
  int dst[BN];
};

// kGateUp: A rows are pair-interleaved gate/up rows of w13[e]; B rows are x
// rows of the block's tokens.  Otherwise A rows are w2[e] rows h0.., B rows
// are the block's activation rows.
template <class SW, class SX, class SY, int BN, bool kGateUp>
__global__ __launch_bounds__(kTileThreads, 2) void tile_ffn_kernel(
    const typename SW::T* __restrict__ w, const typename SX::T* __restrict__ xs, RowMap rm,
    int H, int I, uint16_t* __restrict__ act, typename SY::T* __restrict__ y) {
  __shared__ TileSmem<BN> sm;
  constexpr int TN = BN / 2 / 16;   // 16-token tiles per wavefront
  const int blk = blockIdx.y;
  const bool dense = rm.counts == nullptr;
  int e, row0, nvalid;
  if (dense) {
    e = 0;
    row0 = blk * BN;
    nvalid = min(BN, (int)(rm.dense_rows - row0));
  } else {
    e = rm.block_expert[blk];
    if (e < 0) return;  // past the padded total
    // experts outside min_rows..max_rows are another launch's (or have no tokens)
    if (rm.counts[e] < rm.min_rows || rm.counts[e] > rm.max_rows) return;
    row0 = blk * BN;
    nvalid = min(BN, rm.offsets[e] + rm.counts[e] - row0);
  }
  const int Kdim = kGateUp ? H : I;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave >> 1, wn = wave & 1;
  const int m = lane & 15, g = lane >> 4;

  // rows of the block: token (gate/up) or activation row (down), and output row
  for (int j = tid; j < BN; j += kTileThreads) {
    const int jj = j < nvalid ? j : 0;  // rows past the bucket reuse its first row
    const int row = row0 + jj;
    if (kGateUp) {
      // (a block of padding rows only, as max padding makes, reads token 0)
      sm.tok[j] = dense ? row : (nvalid > 0 ? rm.sorted_ids[row] / rm.K : 0);
    } else {
      sm.tok[j] = row;
      sm.dst[j] = dense ? row : rm.sorted_ids[row];
    }
  }
  __syncthreads();

  // this thread's 16-byte pieces of each step: rows (tid/8) + 32*j, segment tid%8
  constexpr int APieces = kBM * kBK / 8 / kTileThreads;   // 4
  constexpr int BPieces = BN * kBK / 8 / kTileThreads;    // 4 or 2
  const int seg = tid & 7;
  const typename SW::T* arow[APieces];
  const int i0 = blockIdx.x * (kGateUp ? 64 : kBM);
  const typename SW::T* wexp = w + (size_t)e * (kGateUp ? 2 * (size_t)I * H : (size_t)H * I);
#pragma unroll
  for (int j = 0; j < APieces; ++j) {
    const int r = tid / 8 + 32 * j;
    size_t wr;
    if (kGateUp) {
      const int q = r >> 4;                       // 16-row group: even = gate, odd = up
      const int i = i0 + 16 * (q >> 1) + (r & 15);
      wr = (q & 1) ? (size_t)(I + i) : (size_t)i;
    } else {
      wr = (size_t)(i0 + r);
    }
    arow[j] = wexp + wr * Kdim + seg * 8;
  }
  const typename SX::T* brow[BPieces];
#pragma unroll
  for (int j = 0; j < BPieces; ++j) {
    const int r = tid / 8 + 32 * j;
    brow[j] = xs + (size_t)sm.tok[r] * Kdim + seg * 8;
  }

  u32x4 ra[APieces], rb[BPieces];
  auto gload = [&](int ks) {
    const int k = ks * kBK;
#pragma unroll
    for (int j = 0; j < APieces; ++j) ra[j] = load8<SW>(arow[j] + k);
#pragma unroll
    for (int j = 0; j < BPieces; ++j) rb[j] = load8<SX>(brow[j] + k);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < APieces; ++j)
      *reinterpret_cast<u32x4*>(&sm.a[buf][(tid / 8 + 32 * j) * kLdsRow + seg * 8]) = ra[j];
#pragma unroll
    for (int j = 0; j < BPieces; ++j)
      *reinterpret_cast<u32x4*>(&sm.b[buf][(tid / 8 + 32 * j) * kLdsRow + seg * 8]) = rb[j];
  };

  f32x4 acc[4][TN];
#pragma unroll
  for (int tm = 0; tm < 4; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = Kdim / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) gload(ks + 1);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 fa[4], fb[TN];
#pragma unroll
      for (int tm = 0; tm < 4; ++tm)
        fa[tm] = *reinterpret_cast<const u32x4*>(
            &sm.a[buf][(wm * 64 + tm * 16 + m) * kLdsRow + s * 32 + g * 8]);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        fb[tn] = *reinterpret_cast<const u32x4*>(
            &sm.b[buf][(wn * (BN / 2) + tn * 16 + m) * kLdsRow + s * 32 + g * 8]);
#pragma unroll
      for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = mfma16x16x32(fa[tm], fb[tn], acc[tm][tn]);
    }
    if (ks + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 4g..4g+3 of each 16-row tile, for token column m of each tile
  if (kGateUp) {
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int j = wn * (BN / 2) + tn * 16 + m;
        if (j < nvalid) {
          const f32x4 gs = acc[2 * p][tn], us = acc[2 * p + 1][tn];
          const int i = i0 + 16 * (wm * 2 + p) + 4 * g;
          uint2 v;
          v.x = pack_bf16x2(silu(gs.x) * us.x, silu(gs.y) * us.y);
          v.y = pack_bf16x2(silu(gs.z) * us.z, silu(gs.w) * us.w);
          *reinterpret_cast<uint2*>(act + (size_t)(row0 + j) * I + i) = v;
        }
      }
  } else {
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int j = wn * (BN / 2) + tn * 16 + m;
        if (j < nvalid) {
          const int h = i0 + wm * 64 + tm * 16 + 4 * g;
          typename SY::T* o = y + (size_t)sm.dst[j] * H + h;
          const f32x4 v = acc[tm][tn];
          store_out4<SY>(o, v);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Second-generation tile for bf16 storage: BM weight rows (256, or 128 for the
// grouped gate/up half at 64-token blocks) x BN tokens per workgroup (BN =
// block_m: 64 or 128, or 256 for dense rows), NW wavefronts in an NW/2 x 2
// grid, each owning a (BM / (NW/2)) x BN/2 register tile, and an
// ST-stage LDS ring filled by direct global->LDS loads
// (global_load_lds_dwordx4), so ST-1 steps of loads are in flight while one is
// multiplied without spending registers on staging.  8 wavefronts (2 per
// SIMD) measure faster than 4, which leave one wave per SIMD to hide the load
// latency.  Measured and not kept: 32-deep steps with four stages for
// 256-token blocks, and 256-token workgroups over two 128-row blocks of one
// expert (both 5-15 % slower than 64-deep steps over 128-token blocks).
//
// A direct load writes its 64 lanes' 16 bytes contiguously, so instead of
// padding, the 16-byte segments of each 128-byte LDS row are permuted:
// segment s of row r sits in slot s ^ (r & 7), which makes the fragment reads
// free of bank conflicts (measured with the LDS bank-conflict counter; 16-byte
// row padding costs 2 conflict cycles per read on gfx950, no permutation 6).
// 16-token tiles that hold only padding rows skip their matrix ops.
//
// Work order: a 1-D grid of (weight tile, token block) items, token block
// fastest, dealt to the 8 XCDs in contiguous runs (workgroup b runs on XCD
// b % 8), so the blocks that share a weight tile (those of one expert) run
// together on one XCD and read the tile through that XCD's L2 once.

#ifndef MOE_TILE_WAVES
#define MOE_TILE_WAVES 8
#endif

constexpr int kT2BM = 256;
constexpr int kRowBytes = kBK * 2;   // 128 bytes of one row per step

// AROW: bytes of a weight row per step (128 for bf16, 64 for FP8 codes); BM:
// weight rows of a tile
template <int BN, int ST, int AROW, int BM>
struct Tile2Smem {
  uint8_t a[ST][BM * AROW];
  uint8_t b[ST][BN * kRowBytes];
  int tok[BN];
  int dst[BN];
};

// stages that fit the 160 KB of LDS next to the token arrays (at most 6 for
// the 128-row tile, whose stages are smaller)
template <class SW, int BN, int BM>
constexpr int tile2_stages() {
  if constexpr (BM == 256) return SW::kBytes == 1 ? (BN >= 256 ? 3 : 4) : (BN >= 256 ? 2 : 3);
  constexpr int st = (160 * 1024 - 8 * BN) / (BM * 64 * SW::kBytes + BN * 128);
  return st > 6 ? 6 : st;
}

// byte offset of (row, 16-byte segment) in a stage of 64-byte FP8 weight rows:
// segments permuted by bits 2..3 of the row, so the 16 rows of a fragment read
// cover 16 different 16-byte bank groups
__device__ __forceinline__ int lds8_off(int row, int seg) {
  return row * 64 + ((seg ^ ((row >> 2) & 3)) << 4);
}

__device__ __forceinline__ int swz(int row) { return row & 7; }

// byte offset of (row, 16-byte segment) inside a stage buffer
__device__ __forceinline__ int lds_off(int row, int seg) {
  return row * kRowBytes + ((seg ^ swz(row)) << 4);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void lds_direct16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds_base, 16, 0, 0);
}
// The same with the non-temporal hint, for data read by one workgroup only
__device__ __forceinline__ void lds_direct16_nt(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds_base, 16, 0, 2);
}

// Workgroup barrier without the memory fence __syncthreads() adds (which would
// wait for every load in flight, draining the LDS ring).  The "memory" clobber
// keeps the compiler from moving LDS accesses across it; the loads a wave
// needs are waited for explicitly with wait_vmcnt before it.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// SW: weight storage, BF16 or FP8 E4M3 codes with fp32 row scales (wscale
// [E][2I] for gate/up, [E][H] for down): the codes are expanded exactly to
// bf16 as the fragments are read, and the row scales multiply the sums.
template <class SW, class SY, int BN, bool kGateUp, int NW, int BM = kT2BM>
__global__ __launch_bounds__(NW * kWave, 1) void tile2_ffn_kernel(
    const typename SW::T* __restrict__ w, const float* __restrict__ wscale,
    const uint16_t* __restrict__ xs, RowMap rm, int H, int I,
    uint16_t* __restrict__ act, typename SY::T* __restrict__ y, int ntiles, int nblocks,
    int ksplit, float* __restrict__ part, int64_t prows, int nfull) {
  constexpr bool kF8 = SW::kBytes == 1;
  constexpr int AROW = kF8 ? 64 : kRowBytes;               // weight row bytes per step
  constexpr int ASEG = AROW / 16;                          // lanes per weight row in a direct load
  constexpr int ST = tile2_stages<SW, BN, BM>();
  constexpr int NT = NW * kWave;
  constexpr int WM = NW / 2;                              // wavefront rows
  constexpr int TM = BM / WM / 16;                        // 16-row tiles per wavefront
  constexpr int TN = BN / 2 / 16;                         // 16-token tiles per wavefront
  constexpr int AInst = BM * AROW / 1024 / NW;            // direct loads per wave per step
  constexpr int BInst = BN * kRowBytes / 1024 / NW;
  constexpr int kLoads = AInst + BInst;
  static_assert(BInst >= 1 && kLoads * (ST - 1) < 64, "load counts");
  static_assert(AInst >= 1 && TM >= 2 && TM % 2 == 0, "tile rows");
  __shared__ Tile2Smem<BN, ST, AROW, BM> sm;
  int zk, tile, blk, slices;
  if (nfull > 0) {
    // one block of dense rows: tiles 0..nfull-1 whole (the first workgroups,
    // dispatched first: full rounds of the CUs), then each later tile's
    // contraction in ksplit slices, which fill the last round
    const int item0 = (int)blockIdx.x;
    blk = 0;
    if (item0 < nfull) {
      tile = item0;
      zk = 0;
      slices = 1;
    } else {
      const int r = item0 - nfull;
      if (r >= (ntiles - nfull) * ksplit) return;
      tile = nfull + r / ksplit;
      zk = r % ksplit;
      slices = ksplit;
    }
  } else {
    // XCD-aware work item: XCD b % 8 takes items [xcd * per, (xcd + 1) * per)
    const int per = (int)(gridDim.x / 8);
    const int item0 = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (item0 >= ksplit * ntiles * nblocks) return;
    zk = item0 / (ntiles * nblocks);   // slice of a split contraction (dense rows only)
    const int item = item0 % (ntiles * nblocks);
    tile = item / nblocks;
    blk = item % nblocks;
    slices = ksplit;
  }
  // split items write fp32 partial sums of the tiles past the whole ones: the
  // gate/up columns from c0 = nfull * BM / 2 (2 (I - c0) a row: gate, then up),
  // the down features from h0 = nfull * BM (H - h0 a row)
  float* const psum = slices > 1 ? part : nullptr;
  const bool dense = rm.counts == nullptr;
  int e, row0, nvalid;
  if (dense) {
    e = 0;
    row0 = blk * BN;
    nvalid = min(BN, (int)(rm.dense_rows - row0));
  } else {
    e = rm.block_expert[blk];
    if (e < 0) return;
    if (rm.counts[e] < rm.min_rows || rm.counts[e] > rm.max_rows) return;
    row0 = blk * BN;
    nvalid = min(BN, rm.offsets[e] + rm.counts[e] - row0);
  }
  const int Kdim = kGateUp ? H : I;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave-uniform, so that the per-wavefront tile counts below stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave >> 1, wn = wave & 1;
  const int m = lane & 15, g = lane >> 4;

  for (int j = tid; j < BN; j += NT) {
    const int jj = j < nvalid ? j : 0;  // rows past the bucket reuse its first row
    const int row = row0 + jj;
    if (kGateUp) {
      // (a block of padding rows only, as max padding makes, reads token 0)
      sm.tok[j] = dense ? row : (nvalid > 0 ? rm.sorted_ids[row] / rm.K : 0);
      // partial sums of a split contraction go to the row's pair (grouped rows)
      if (part) sm.dst[j] = dense ? row : rm.sorted_ids[row];
    } else {
      sm.tok[j] = row;
      sm.dst[j] = dense ? row : rm.sorted_ids[row];
    }
  }
  __syncthreads();

  // Direct loads: instruction i of a stage fills 1 KB of LDS rows; for bf16
  // weights rows 8i..8i+7, lane l filling row 8i + l/8, slot l%8, which holds
  // global segment (l%8) ^ swz(row); for FP8 weights rows 16i..16i+15, lane l
  // filling row 16i + l/4, slot l%4, global segment (l%4) ^ ((row >> 2) & 3).
  const int i0 = tile * (kGateUp ? BM / 2 : BM);
  const uint8_t* wexp = reinterpret_cast<const uint8_t*>(w) +
                        (size_t)e * (kGateUp ? 2 * (size_t)I * H : (size_t)H * I) * SW::kBytes;
  const uint8_t* asrc[AInst];
#pragma unroll
  for (int j = 0; j < AInst; ++j) {
    const int r = (1024 / AROW) * (wave * AInst + j) + lane / ASEG;
    size_t wr;
    if (kGateUp) {
      const int q = r >> 4;                       // 16-row group: even = gate, odd = up
      const int i = i0 + 16 * (q >> 1) + (r & 15);
      wr = (q & 1) ? (size_t)(I + i) : (size_t)i;
    } else {
      wr = (size_t)(i0 + r);
    }
    const int aslot = kF8 ? ((lane & 3) ^ ((r >> 2) & 3)) : ((lane & 7) ^ swz(r));
    asrc[j] = wexp + wr * Kdim * SW::kBytes + (aslot << 4);
  }
  const uint8_t* bsrc[BInst];
#pragma unroll
  for (int j = 0; j < BInst; ++j) {
    const int r = 8 * (wave * BInst + j) + lane / 8;
    bsrc[j] = reinterpret_cast<const uint8_t*>(xs + (size_t)sm.tok[r] * Kdim) +
              (((lane & 7) ^ swz(r)) << 4);
  }

  // this workgroup's steps [k0, k0 + nk) of the contraction.  Workgroups that
  // start together read the same offset of their weight rows at the same
  // time, and where a row is a whole number of 4 KB those reads pile onto the
  // same HBM channels; there each (expert, weight tile) starts 3 steps further
  // round its steps, taking k0 + rot .. k0 + nk - 1 and then k0 .. k0 + rot - 1
  // (one start per weight tile, so token blocks sharing a tile through L2 stay
  // in step).  Elsewhere the tiles stay in step: they share the token rows,
  // which they then read from L2 together.  Measured on MI355X (us, bf16):
  // Mixtral-shaped (8 KB gate/up rows, 28 KB down rows) DenseFA at 128 tokens
  // 176 -> 163, grouped down at 512 / 2048 tokens 283 -> 277 / 617 -> 604;
  // DeepSeek-V3-shaped grouped down (4 KB rows, Zipf routing) 344 -> 335; its
  // 14 KB gate/up rows rotated measured no gain.  Costs: Mixtral-shaped DenseFA
  // at 512 tokens 392 -> 399 and the grouped down at 128 tokens 176 -> 179.
  const int nk_all = Kdim / kBK;
  const int k0 = zk * nk_all / slices;
  const int nk = (zk + 1) * nk_all / slices - k0;
  const bool rotate = !kF8 && ((int64_t)Kdim * SW::kBytes) % 4096 == 0 && nk > 0;
  const int rot = rotate ? 3 * (tile + e * ntiles) % nk : 0;
  auto issue = [&](int ks, auto nt) {
    const int st = ks % ST;
    const int kp = ks + rot < nk ? ks + rot : ks + rot - nk;
    const size_t kb = (size_t)(k0 + kp) * kRowBytes;
#pragma unroll
    for (int j = 0; j < AInst; ++j) {
      const uint8_t* src = asrc[j] + (size_t)(k0 + kp) * AROW;
      if constexpr (decltype(nt)::value) lds_direct16_nt(src, &sm.a[st][(wave * AInst + j) * 1024]);
      else lds_direct16(src, &sm.a[st][(wave * AInst + j) * 1024]);
    }
#pragma unroll
    for (int j = 0; j < BInst; ++j)
      lds_direct16(bsrc[j] + kb, &sm.b[st][(wave * BInst + j) * 1024]);
  };

  // this wavefront's 16-token tiles that hold at least one token
  const int tn_live = min(TN, max(0, (nvalid - wn * (BN / 2) + 15) / 16));

  f32x4 acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One step's matrix ops on the stage in slot `slot`.  With registers to
  // spare (TN <= 4) the fragments of both 32-deep halves are read up front, so
  // the second half's reads are in flight while the first half's ops issue
  // (with TN = 8 that spills registers).  `masked` skips the 16-token tiles
  // past the block's tokens.
  constexpr int NB2 = TN <= 4 ? 2 : 1;
  auto step = [&](int slot, auto masked) {
    const uint8_t* A = sm.a[slot];
    const uint8_t* Bt = sm.b[slot];
#pragma unroll
    for (int h = 0; h < 2 / NB2; ++h) {
      u32x4 fa[NB2][TM], fb[NB2][TN];
#pragma unroll
      for (int q = 0; q < NB2; ++q) {
        const int s2 = h * NB2 + q;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const int r = wm * (TM * 16) + tm * 16 + m;
          if constexpr (kF8)   // 8 codes at k = 32 s2 + 8 g: half (g & 1) of segment 2 s2 + g / 2
            fa[q][tm] = fp8x8_to_bf16(*reinterpret_cast<const uint2*>(
                A + lds8_off(r, 2 * s2 + (g >> 1)) + 8 * (g & 1)));
          else
            fa[q][tm] = *reinterpret_cast<const u32x4*>(A + lds_off(r, s2 * 4 + g));
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          fb[q][tn] = *reinterpret_cast<const u32x4*>(
              Bt + lds_off(wn * (BN / 2) + tn * 16 + m, s2 * 4 + g));
      }
#pragma unroll
      for (int q = 0; q < NB2; ++q)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          if (!decltype(masked)::value || tn < tn_live) {
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
              acc[tm][tn] = mfma16x16x32(fa[q][tm], fb[q][tn], acc[tm][tn]);
          }
      if (NB2 == 2 && !decltype(masked)::value) {
        // order of the branch-free step: the first half's reads, then the
        // second half's reads one between each of the first ops, then the
        // rest; at most 15 reads are ever outstanding (the counter's limit),
        // so each op waits only for its own operands
        constexpr int NR = TM + TN;
        __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);   // DS reads
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * TM * TN - NR, 0);
      }
    }
  };
  // The k loop, in a copy per path so that the steady-state body (wait for
  // stage ks, barrier, issue stage ks + ST - 1, the step) is one basic block
  // and the waits inside it count only the reads an op needs.
  auto run = [&](auto masked, auto nt) {
#pragma unroll
    for (int s0 = 0; s0 < ST - 1; ++s0)
      if (s0 < nk) issue(s0, nt);
    int ks = 0;
    for (; ks + ST - 1 < nk; ++ks) {
      // stage ks must be in LDS: the ST-2 stages issued after it may stay in flight
      wait_vmcnt<(ST - 2) * kLoads>();
      barrier_no_fence();  // stage ks is in LDS for every wave; stage ks-1 is no longer read
      issue(ks + ST - 1, nt);
      step(ks % ST, masked);
    }
    for (; ks < nk; ++ks) {   // the last ST - 1 steps: nothing left to issue
      wait_vmcnt<0>();
      barrier_no_fence();
      step(ks % ST, masked);
    }
  };
  // The weight tile's loads carry the non-temporal hint where no other
  // workgroup reads the same rows: dense rows in one token block, or an expert
  // whose bucket is one block.  Where several token blocks share a weight tile
  // they run side by side and meet in L2, which the hint would defeat.  bf16
  // only (FP8 rows are 64-byte pieces a step, which the hint slows).  Measured
  // on MI355X (us): Mixtral-shaped layer at 128 tokens 535 -> 485 (its DenseFA
  // 166 -> 145), DeepSeek-V3-shaped DenseFA at 128 tokens 192 -> 173, Qwen2-
  // shaped gate/up at 256 tokens 409 -> 395; with the hint on every tile the
  // shared tiles lost up to 14% (Mixtral-shaped gate/up at 512 tokens 446 -> 510).
  const bool single = dense ? nblocks == 1 : rm.offsets[e + 1] - rm.offsets[e] <= BN;
  const bool live = NB2 == 2 && tn_live == TN;
  if constexpr (!kF8) {
    if (single) {
      if (live) run(std::false_type{}, std::true_type{});
      else run(std::true_type{}, std::true_type{});
    } else {
      if (live) run(std::false_type{}, std::false_type{});
      else run(std::true_type{}, std::false_type{});
    }
  } else {
    if (live) run(std::false_type{}, std::false_type{});
    else run(std::true_type{}, std::false_type{});
  }

  // epilogue: lane holds rows 4g..4g+3 of each 16-row tile, for token column m of each tile
  if (kGateUp) {
#pragma unroll
    for (int p = 0; p < TM / 2; ++p)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int j = wn * (BN / 2) + tn * 16 + m;
        if (j < nvalid) {
          f32x4 gs = acc[2 * p][tn], us = acc[2 * p + 1][tn];
          const int i = i0 + 16 * (wm * (TM / 2) + p) + 4 * g;
          if constexpr (kF8) {   // row scales of the lane's 4 gate and 4 up rows
            const float* se = wscale + (size_t)e * 2 * I;
            gs = gs * *reinterpret_cast<const f32x4*>(se + i);
            us = us * *reinterpret_cast<const f32x4*>(se + I + i);
          }
          if (psum) {  // split contraction: this slice's fp32 sums, SwiGLU in the finish kernel
            const int c0 = nfull * (BM / 2), wt = I - c0;
            float* pr = psum + ((size_t)zk * prows + sm.dst[j]) * (2 * (size_t)wt);
            *reinterpret_cast<f32x4*>(pr + (i - c0)) = gs;
            *reinterpret_cast<f32x4*>(pr + wt + (i - c0)) = us;
            continue;
          }
          uint2 v;
          v.x = pack_bf16x2(silu(gs.x) * us.x, silu(gs.y) * us.y);
          v.y = pack_bf16x2(silu(gs.z) * us.z, silu(gs.w) * us.w);
          *reinterpret_cast<uint2*>(act + (size_t)(row0 + j) * I + i) = v;
        }
      }
  } else {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int j = wn * (BN / 2) + tn * 16 + m;
        if (j < nvalid) {
          const int h = i0 + wm * (TM * 16) + tm * 16 + 4 * g;
          f32x4 v = acc[tm][tn];
          if constexpr (kF8) v = v * *reinterpret_cast<const f32x4*>(wscale + (size_t)e * H + h);
          if (psum) {  // split contraction: fp32 slice, summed in slice order by the finish kernel
            const int h0 = nfull * BM;
            *reinterpret_cast<f32x4*>(psum + ((size_t)zk * prows + sm.dst[j]) * (H - h0) +
                                      (h - h0)) = v;
          } else {
            typename SY::T* o = y + (size_t)sm.dst[j] * H + h;
            store_out4<SY>(o, v);
          }
        }
      }
  }
}

template <class S, int BN>
static void gu_launch(const void* x, const void* w13, const RowMap& rm, int64_t nblocks, int H,
                      int I, uint16_t* act, hipStream_t s) {
  hipLaunchKernelGGL((tile_ffn_kernel<S, S, BF16, BN, true>), dim3(I / 64, (unsigned)nblocks),
                     dim3(kTileThreads), 0, s, static_cast<const typename S::T*>(w13),
                     static_cast<const typename S::T*>(x), rm, H, I, act, (uint16_t*)nullptr);
}

template <class SW, class SY, int BN>
static void dn_launch(const void* w2, const uint16_t* act, const RowMap& rm, int64_t nblocks,
                      int H, int I, void* y, hipStream_t s) {
  hipLaunchKernelGGL((tile_ffn_kernel<SW, BF16, SY, BN, false>), dim3(H / kBM, (unsigned)nblocks),
                     dim3(kTileThreads), 0, s, static_cast<const typename SW::T*>(w2), act, rm, H,
                     I, (uint16_t*)nullptr, static_cast<typename SY::T*>(y));
}

// 1-D grid of tiles x blocks items, rounded up to a multiple of the 8 XCDs
static unsigned xcd_grid(int64_t items) { return (unsigned)((items + 7) / 8 * 8); }


// ---------------------------------------------------------------------------
// Wide gate/up tile for experts holding several 128-token blocks: a workgroup
// of 8 wavefronts computes 512 weight rows (256 gate/up column pairs) x one
// 128-token block, each wavefront 128 rows x 64 tokens (4 x 2), over steps of
// 32 of the contraction (64-byte rows: 40 KB a stage, 3 stages in LDS).  Per
// matrix op it moves 17% fewer bytes into LDS and reads 25% fewer out of it
// than the 256-row tile, and the next step's fragments are read while the
// current step's ops issue.  Measured on MI355X it is faster once experts
// average 4 blocks (Mixtral-shaped experts at 512 tokens each: 1.10 vs 1.25
// ms for the gate/up GEMM) and slower with fewer blocks, where 512-row tiles
// leave too few workgroups per weight column.
//
// Pipeline at step t (stage t's fragments already in registers): wait for
// this wavefront's loads of stage t+1, barrier (stage t+1 in LDS for every
// wavefront; every wavefront has finished reading stage t's slot), load
// stage t+3 into stage t's slot, then the ops on stage t with the fragment
// reads of stage t+1 in flight.  Loads run two steps ahead.
constexpr int kWBM = 512;           // weight rows per workgroup
constexpr int kWBN = 128;           // tokens per workgroup (the alignment block)
constexpr int kWRow = 64;           // bytes of a row per step (32 bf16)
constexpr int kWST = 3;             // stages
constexpr int kWWaves = 8;

// byte offset of (row, 16-byte segment) in a stage of 64-byte rows: a 16-byte
// fragment read is served 8 lanes (8 consecutive rows, one segment) at a
// time from 128 bytes of banks, which hold two 64-byte rows; permuting the
// segments by bits 1..2 of the row puts the 8 reads in 8 different places
// (0 bank-conflict cycles measured; bits 2..3 gave a 2-way conflict)
__device__ __forceinline__ int ldsw_off(int row, int seg) {
  return row * kWRow + ((seg ^ ((row >> 1) & 3)) << 4);
}

struct WideSmem {
  uint8_t a[kWST][kWBM * kWRow];
  uint8_t b[kWST][kWBN * kWRow];
  int tok[kWBN];
};

template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(N >= 0 && N < 16, "lgkmcnt");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (0x7 << 4) | (N << 8));
}

__global__ __launch_bounds__(kWWaves * kWave, 1) void wide_gate_up_kernel(
    const uint16_t* __restrict__ w, const uint16_t* __restrict__ xs, RowMap rm, int H, int I,
    uint16_t* __restrict__ act, int ntiles, int nblocks) {
  constexpr int TM = 8, TN = 4;                          // 16-row / 16-token tiles per wavefront
  constexpr int AInst = kWBM * kWRow / 1024 / kWWaves;   // direct loads per wavefront per stage
  constexpr int BInst = kWBN * kWRow / 1024 / kWWaves;
  constexpr int kLoads = AInst + BInst;
  __shared__ WideSmem sm;
  const int per = (int)(gridDim.x / 8);
  const int item = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (item >= ntiles * nblocks) return;
  const int tile = item / nblocks;
  const int blk = item % nblocks;
  const bool dense = rm.counts == nullptr;
  int e, row0, nvalid;
  if (dense) {
    e = 0;
    row0 = blk * kWBN;
    nvalid = min(kWBN, (int)(rm.dense_rows - row0));
  } else {
    e = rm.block_expert[blk];
    if (e < 0) return;
    if (rm.counts[e] < rm.min_rows || rm.counts[e] > rm.max_rows) return;
    row0 = blk * kWBN;
    nvalid = min(kWBN, rm.offsets[e] + rm.counts[e] - row0);
  }
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave >> 1, wn = wave & 1;
  const int m = lane & 15, g = lane >> 4;

  for (int j = tid; j < kWBN; j += kWWaves * kWave) {
    const int row = row0 + (j < nvalid ? j : 0);   // rows past the bucket reuse its first row
    sm.tok[j] = dense ? row : (nvalid > 0 ? rm.sorted_ids[row] / rm.K : 0);
  }
  __syncthreads();

  // Direct loads: instruction n of a stage fills LDS rows 16n..16n+15 (1 KB),
  // lane l filling row 16n + l/4, slot l%4 with the row's global segment
  // (l%4) ^ ((row >> 1) & 3).  Weight instruction n is 16-row group n of the
  // tile: even groups are gate rows, odd groups the up rows of the same 16
  // columns.  Weight addresses are a wave-uniform row offset per instruction
  // plus one 32-bit lane offset (an expert's matrix is below 4 GB).
  const int i0 = tile * (kWBM / 2);
  const uint8_t* wexp = reinterpret_cast<const uint8_t*>(w) + (size_t)e * 2 * (size_t)I * H * 2;
  const int lrow = lane >> 2;
  const int lseg = (lane & 3) ^ ((lrow >> 1) & 3);
  const uint32_t alane = (uint32_t)lrow * (uint32_t)H * 2u + (uint32_t)(lseg << 4);
  uint32_t arow[AInst];
#pragma unroll
  for (int j = 0; j < AInst; ++j) {
    const int q = wave * AInst + j;
    const int i = i0 + 16 * (q >> 1);
    arow[j] = (uint32_t)((q & 1) ? I + i : i) * (uint32_t)H * 2u;
  }
  const uint8_t* bsrc[BInst];
#pragma unroll
  for (int j = 0; j < BInst; ++j) {
    const int r = 16 * (wave * BInst + j) + lrow;
    bsrc[j] = reinterpret_cast<const uint8_t*>(xs + (size_t)sm.tok[r] * H) + (lseg << 4);
  }
  const int nk = H / 32;
  auto issue = [&](int ks) {
    const int st = ks % kWST;
    const uint32_t kb = (uint32_t)ks * kWRow;
#pragma unroll
    for (int j = 0; j < AInst; ++j)
      lds_direct16(wexp + (arow[j] + kb + alane), &sm.a[st][(wave * AInst + j) * 1024]);
#pragma unroll
    for (int j = 0; j < BInst; ++j)
      lds_direct16(bsrc[j] + kb, &sm.b[st][(wave * BInst + j) * 1024]);
  };

  // this wavefront's 16-token tiles that hold at least one token
  const int tn_live = min(TN, max(0, (nvalid - wn * (kWBN / 2) + 15) / 16));
  f32x4 acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragments of a stage: lane (m, g) reads k-group g of row 16 tm + m; the
  // masked path skips the 16-token tiles past the block's tokens
  auto read = [&](int slot, u32x4 (&fa)[TM], u32x4 (&fb)[TN], auto masked) {
    const uint8_t* A = sm.a[slot];
    const uint8_t* Bt = sm.b[slot];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
      fa[tm] = *reinterpret_cast<const u32x4*>(A + ldsw_off(wm * 128 + tm * 16 + m, g));
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
      if (!decltype(masked)::value || tn < tn_live)
        fb[tn] = *reinterpret_cast<const u32x4*>(Bt + ldsw_off(wn * (kWBN / 2) + tn * 16 + m, g));
  };
  auto ops = [&](const u32x4 (&fa)[TM], const u32x4 (&fb)[TN], auto masked) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
      if (!decltype(masked)::value || tn < tn_live) {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) acc[tm][tn] = mfma16x16x32(fa[tm], fb[tn], acc[tm][tn]);
      }
  };
  // step t on fragments (ca, cb), reading stage t+1's into (na, nb); the
  // steady form (t + 3 < nk) has no conditions, so it is one basic block
  auto body = [&](int t, u32x4 (&ca)[TM], u32x4 (&cb)[TN], u32x4 (&na)[TM], u32x4 (&nb)[TN],
                  auto steady, auto masked) {
    if constexpr (decltype(steady)::value) {
      wait_vmcnt<kLoads>();
      wait_lgkmcnt<0>();
      barrier_no_fence();
      issue(t + 3);
      read((t + 1) % kWST, na, nb, masked);   // completes while the ops issue
      ops(ca, cb, masked);
    } else {
      if (t + 2 < nk) wait_vmcnt<kLoads>();
      else wait_vmcnt<0>();
      wait_lgkmcnt<0>();
      barrier_no_fence();
      if (t + 3 < nk) issue(t + 3);
      if (t + 1 < nk) read((t + 1) % kWST, na, nb, masked);
      ops(ca, cb, masked);
    }
  };
  auto run = [&](auto masked) {
    u32x4 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
#pragma unroll
    for (int s0 = 0; s0 < kWST; ++s0)
      if (s0 < nk) issue(s0);
    // stage 0 landed (the later stages may stay in flight)
    if (nk >= 3) wait_vmcnt<2 * kLoads>();
    else wait_vmcnt<0>();
    barrier_no_fence();
    read(0, fa0, fb0, masked);
    int t = 0;
    for (; t + 4 < nk; t += 2) {
      body(t, fa0, fb0, fa1, fb1, std::true_type{}, masked);
      body(t + 1, fa1, fb1, fa0, fb0, std::true_type{}, masked);
    }
    for (; t < nk; t += 2) {
      body(t, fa0, fb0, fa1, fb1, std::false_type{}, masked);
      if (t + 1 < nk) body(t + 1, fa1, fb1, fa0, fb0, std::false_type{}, masked);
    }
  };
  if (tn_live == TN)
    run(std::false_type{});
  else
    run(std::true_type{});

  // epilogue: lane holds rows 4g..4g+3 of each 16-row tile, for token column m
  // of each tile; tile pair (2p, 2p+1) is the gate and up of 16 columns
#pragma unroll
  for (int p = 0; p < TM / 2; ++p)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int j = wn * (kWBN / 2) + tn * 16 + m;
      if (j < nvalid) {
        const f32x4 gs = acc[2 * p][tn], us = acc[2 * p + 1][tn];
        const int i = i0 + 16 * (wm * (TM / 2) + p) + 4 * g;
        uint2 v;
        v.x = pack_bf16x2(silu(gs.x) * us.x, silu(gs.y) * us.y);
        v.y = pack_bf16x2(silu(gs.z) * us.z, silu(gs.w) * us.w);
        *reinterpret_cast<uint2*>(act + (size_t)(row0 + j) * I + i) = v;
      }
    }
}

bool tile_wide_ok(int block_m, int H, int I) {
  return block_m == kWBN && I % (kWBM / 2) == 0 && H % 32 == 0 && H >= 32 &&
         (int64_t)2 * I * H * 2 < ((int64_t)1 << 32);
}

hipError_t launch_tile_gate_up_wide(const void* x, const void* w13, const RowMap& rm,
                                    int64_t nblocks, int H, int I, uint16_t* act, hipStream_t s) {
  if (!tile_wide_ok(rm.block_m, H, I)) return hipErrorInvalidValue;
  const int ntiles = I / (kWBM / 2);
  hipLaunchKernelGGL(wide_gate_up_kernel, dim3(xcd_grid((int64_t)ntiles * nblocks)),
                     dim3(kWWaves * kWave), 0, s, static_cast<const uint16_t*>(w13),
                     static_cast<const uint16_t*>(x), rm, H, I, act, ntiles, (int)nblocks);
  return hipGetLastError();
}

// Rows of one slice of partial sums: the dense rows, or the pairs (T*K) of
// grouped rows, whose partial sums are indexed by pair.
static int64_t part_rows(const RowMap& rm, int64_t pairs) {
  return rm.counts == nullptr ? rm.dense_rows : pairs;
}

// Workgroups of a launch: with nfull whole tiles (one block of dense rows),
// nfull + (ntiles - nfull) * ksplit in order; else the XCD-aware grid
static unsigned tile2_grid(int ntiles, int64_t nblocks, int ksplit, int nfull) {
  if (nfull > 0) return (unsigned)(nfull + (int64_t)(ntiles - nfull) * ksplit);
  return xcd_grid((int64_t)ksplit * ntiles * nblocks);
}

template <int BN, class SW = BF16, int BM = kT2BM>
static void gu2_launch(const void* x, const void* w13, const RowMap& rm, int64_t nblocks, int H,
                       int I, uint16_t* act, hipStream_t s, const float* wscale = nullptr,
                       int ksplit = 1, float* part = nullptr, int64_t prows = 0, int nfull = 0) {
  const int ntiles = I / (BM / 2);
  hipLaunchKernelGGL((tile2_ffn_kernel<SW, BF16, BN, true, MOE_TILE_WAVES, BM>),
                     dim3(tile2_grid(ntiles, nblocks, ksplit, nfull)),
                     dim3(MOE_TILE_WAVES * kWave), 0, s,
                     static_cast<const typename SW::T*>(w13), wscale,
                     static_cast<const uint16_t*>(x), rm, H, I, act, (uint16_t*)nullptr, ntiles,
                     (int)nblocks, ksplit, ksplit > 1 ? part : (float*)nullptr, prows, nfull);
}

template <class SY, int BN, class SW = BF16, int BM = kT2BM>
static void dn2_launch(const void* w2, const uint16_t* act, const RowMap& rm, int64_t nblocks,
                       int H, int I, void* y, int ksplit, float* part, hipStream_t s,
                       const float* wscale = nullptr, int64_t prows = 0) {
  const int ntiles = H / BM;
  hipLaunchKernelGGL((tile2_ffn_kernel<SW, SY, BN, false, MOE_TILE_WAVES, BM>),
                     dim3(tile2_grid(ntiles, nblocks, ksplit, 0)),
                     dim3(MOE_TILE_WAVES * kWave), 0, s, static_cast<const typename SW::T*>(w2),
                     wscale, act, rm, H, I, (uint16_t*)nullptr, static_cast<typename SY::T*>(y),
                     ntiles, (int)nblocks, ksplit, ksplit > 1 ? part : (float*)nullptr, prows, 0);
}

// the finish of a split launch: slices added in order; grouped partial sums
// (per pair) go to the pair's alignment row (gate/up) or pair row (down)
static hipError_t finish_gu(const float* part, int ksplit, const RowMap& rm, int64_t prows, int I,
                            uint16_t* act, hipStream_t s) {
  return rm.counts == nullptr ? launch_finish_gate_up(part, ksplit, prows, I, act, s)
                              : launch_finish_gate_up(part, ksplit, prows, I, act, s, rm.inv_pos);
}

static hipError_t finish_dn(const float* part, int ksplit, const RowMap& rm, int64_t prows, int H,
                            void* y, int ydt, hipStream_t s) {
  return rm.counts == nullptr ? launch_finish_down(part, ksplit, prows, H, y, ydt, s)
                              : launch_finish_down(part, ksplit, prows, H, y, ydt, s, rm.inv_pos);
}

hipError_t launch_tile_gate_up(const void* x, int xdt, const void* w13, const RowMap& rm,
                               int64_t nblocks, int H, int I, uint16_t* act, hipStream_t s,
                               int ksplit, float* part, int64_t pairs, int nfull) {
  if (nfull > 0) {   // one block of dense rows, 128-row tiles, the last round split
    if (xdt != kDtBF16 || rm.counts != nullptr || rm.block_m != 128 || nblocks != 1 ||
        I % 64 != 0 || nfull >= I / 64 || (ksplit > 1 && part == nullptr))
      return hipErrorInvalidValue;
    gu2_launch<128, BF16, 128>(x, w13, rm, 1, H, I, act, s, nullptr, ksplit, part,
                               rm.dense_rows, nfull);
    if (ksplit > 1) return launch_finish_gate_up(part, ksplit, rm.dense_rows, I, act, s, nullptr,
                                                 nfull * 64);
    return hipGetLastError();
  }
  if (xdt == kDtBF16 && I % (kT2BM / 2) == 0) {
    const int64_t prows = part_rows(rm, pairs);
    if (rm.block_m == 256) gu2_launch<256>(x, w13, rm, nblocks, H, I, act, s, nullptr, ksplit, part, prows);
    else if (rm.block_m == 128) gu2_launch<128>(x, w13, rm, nblocks, H, I, act, s, nullptr, ksplit, part, prows);
    // grouped 64-token blocks of every expert (mid-size batches, HBM-bound):
    // 128-row tiles, whose 24 KB stages keep five in flight where the 256-row
    // tile's 40 KB keep two.  Measured on MI355X (us, 256 -> 128 rows):
    // Mixtral-shaped T=96 gate/up 369 -> 356, T=128 346 -> 340; as the down
    // projection 1-4.5% slower.  Not for the launch of the busy experts only
    // (min_rows > 1), which is empty under even routing and then costs its
    // grid's dispatch: twice the workgroups measured 18.8 against 11.1 us
    else if (rm.counts && rm.min_rows <= 1)
      gu2_launch<64, BF16, 128>(x, w13, rm, nblocks, H, I, act, s, nullptr, ksplit, part, prows);
    else gu2_launch<64>(x, w13, rm, nblocks, H, I, act, s, nullptr, ksplit, part, prows);
    if (ksplit > 1) return finish_gu(part, ksplit, rm, prows, I, act, s);
    return hipGetLastError();
  }
  if (rm.block_m == 64) {
    if (xdt == kDtF32) gu_launch<F32, 64>(x, w13, rm, nblocks, H, I, act, s);
    else gu_launch<BF16, 64>(x, w13, rm, nblocks, H, I, act, s);
  } else {
    if (xdt == kDtF32) gu_launch<F32, 128>(x, w13, rm, nblocks, H, I, act, s);
    else gu_launch<BF16, 128>(x, w13, rm, nblocks, H, I, act, s);
  }
  return hipGetLastError();
}

template <class SW, int BN>
static void dn_by_out(const void* w2, const uint16_t* act, const RowMap& rm, int64_t nblocks,
                      int H, int I, void* y, int ydt, hipStream_t s) {
  if (ydt == kDtF32) dn_launch<SW, F32, BN>(w2, act, rm, nblocks, H, I, y, s);
  else dn_launch<SW, BF16, BN>(w2, act, rm, nblocks, H, I, y, s);
}

hipError_t launch_tile_down(const void* w2, int wdt, const uint16_t* act, const RowMap& rm,
                            int64_t nblocks, int H, int I, void* y, int ydt, int ksplit,
                            float* part, hipStream_t s, int64_t pairs) {
  if (wdt == kDtBF16 && H % kT2BM == 0) {
    const int64_t pr = part_rows(rm, pairs);
    if (rm.block_m == 256) {
      if (ydt == kDtF32) dn2_launch<F32, 256>(w2, act, rm, nblocks, H, I, y, ksplit, part, s, nullptr, pr);
      else dn2_launch<BF16, 256>(w2, act, rm, nblocks, H, I, y, ksplit, part, s, nullptr, pr);
    } else if (rm.block_m == 128) {
      if (ydt == kDtF32) dn2_launch<F32, 128>(w2, act, rm, nblocks, H, I, y, ksplit, part, s, nullptr, pr);
      else dn2_launch<BF16, 128>(w2, act, rm, nblocks, H, I, y, ksplit, part, s, nullptr, pr);
    } else {
      if (ydt == kDtF32) dn2_launch<F32, 64>(w2, act, rm, nblocks, H, I, y, ksplit, part, s, nullptr, pr);
      else dn2_launch<BF16, 64>(w2, act, rm, nblocks, H, I, y, ksplit, part, s, nullptr, pr);
    }
    if (ksplit > 1) return finish_dn(part, ksplit, rm, pr, H, y, ydt, s);
    return hipGetLastError();
  }
  if (rm.block_m == 64) {
    if (wdt == kDtF32) dn_by_out<F32, 64>(w2, act, rm, nblocks, H, I, y, ydt, s);
    else dn_by_out<BF16, 64>(w2, act, rm, nblocks, H, I, y, ydt, s);
  } else {
    if (wdt == kDtF32) dn_by_out<F32, 128>(w2, act, rm, nblocks, H, I, y, ydt, s);
    else dn_by_out<BF16, 128>(w2, act, rm, nblocks, H, I, y, ydt, s);
  }
  return hipGetLastError();
}

bool tile_fp8_ok(int H, int I, int block_m) {
  return H % kT2BM == 0 && I % (kT2BM / 2) == 0 &&
         (block_m == 64 || block_m == 128 || block_m == 256);
}

hipError_t launch_tile_gate_up_fp8(const void* x, const void* w13, const float* w13_scale,
                                   const RowMap& rm, int64_t nblocks, int H, int I, uint16_t* act,
                                   hipStream_t s, int ksplit, float* part) {
  if (rm.block_m == 256)
    gu2_launch<256, FP8>(x, w13, rm, nblocks, H, I, act, s, w13_scale, ksplit, part, rm.dense_rows);
  else if (rm.block_m == 128)
    gu2_launch<128, FP8>(x, w13, rm, nblocks, H, I, act, s, w13_scale, ksplit, part, rm.dense_rows);
  else
    gu2_launch<64, FP8>(x, w13, rm, nblocks, H, I, act, s, w13_scale, ksplit, part, rm.dense_rows);
  if (ksplit > 1) return launch_finish_gate_up(part, ksplit, rm.dense_rows, I, act, s);
  return hipGetLastError();
}

hipError_t launch_tile_down_fp8(const void* w2, const float* w2_scale, const uint16_t* act,
                                const RowMap& rm, int64_t nblocks, int H, int I, void* y, int ydt,
                                int ksplit, float* part, hipStream_t s) {
  auto go = [&](auto bn) {
    constexpr int BN = decltype(bn)::value;
    if (ydt == kDtF32)
      dn2_launch<F32, BN, FP8>(w2, act, rm, nblocks, H, I, y, ksplit, part, s, w2_scale,
                               rm.dense_rows);
    else
      dn2_launch<BF16, BN, FP8>(w2, act, rm, nblocks, H, I, y, ksplit, part, s, w2_scale,
                                rm.dense_rows);
  };
  if (rm.block_m == 256) go(std::integral_constant<int, 256>{});
  else if (rm.block_m == 128) go(std::integral_constant<int, 128>{});
  else go(std::integral_constant<int, 64>{});
  if (ksplit > 1) return launch_finish_down(part, ksplit, rm.dense_rows, H, y, ydt, s);
  return hipGetLastError();
}

}  // namespace moe
