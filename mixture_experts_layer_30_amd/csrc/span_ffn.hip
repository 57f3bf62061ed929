// Prefill-shape grouped SwiGLU FFN on gfx950: each weight tile streamed once
// per span of up to 256 of an expert's tokens.
//
// In prefill each expert holds hundreds of tokens; the grouped GEMM is bound by
// matrix-core throughput, lowered by the per-expert split of the batch and by
// padding to the M-tile (Serving-tax notes, Table 1 rows "GroupGEMM" and
// "padding"; prefill-phase section).  A tile that covers one 128-token block
// streams the expert's weights once per block: measured on MI355X, the L2
// catches few of those repeats (HBM fetch 2.0x the weight bytes at 2 blocks an
// expert, 3.1x at 4), and a grid of fixed tiles leaves its last round of the
// 256 CUs part-empty.
//
// Here the work item is (expert, 256-row weight tile, span): a span is a run
// of up to 256 of the expert's rows of the alignment (expert e's span s is
// rows offsets[e] + 256 s ..), so an expert's weight tile is streamed once
// per 256 of its tokens, whatever the padding block.  Workgroups are
// persistent, one per CU: the items (expert-major, then tile, span fastest)
// are cut into 8 contiguous runs, one per XCD (workgroup b runs on XCD b % 8),
// and the workgroups of an XCD take its run round-robin, so the spans that
// share a weight tile run side by side on one XCD and share its L2.
//
// A workgroup is 8 wavefronts in 2 (weight rows) x 4 (tokens); each owns 128
// rows x 64 tokens with 16x16x32 bf16 MFMAs (32 accumulators).  Wavefront wn
// takes the span's 16-token tiles wn, wn+4, wn+8, wn+12, so a short span
// still spreads its tiles over the 4 token columns; tiles past the span's
// tokens skip their matrix ops, and the token rows of 16-row groups past the
// span's end are not loaded.  An expert of 257 to 384 tokens gets two spans
// of equal length instead of 256 and a short rest, so that its items weigh the
// same (measured on MI355X, Mixtral-shaped T=1024 gate/up: 773 -> 729 us;
// equal spans for every split expert made T=2048 3% slower and skewed loads
// slower, as each wavefront's busiest token column sets an item's time).  The contraction goes in steps of 32 (64-byte
// rows: 32 KB a stage) through a 4-stage LDS ring filled by direct
// global->LDS loads, three stages ahead of the matrix ops; a step's fragments
// are read from LDS while the previous step's ops issue.
//
//   gate/up: tile rows alternate 16 gate and 16 up rows of the same
//            intermediate columns (128 columns a tile), so each lane holds
//            matching gate and up sums and applies the SwiGLU in registers;
//            act rows are the alignment rows.
//   down:    tile rows are 256 output features; each token's sums go to its
//            pair's output row.  An expert of 193 to 256 tokens gets two
//            spans of equal length here too: the down items carry the I-long
//            contraction, and an expert's H/256 tiles each read its
//            activation rows again, so one span an expert (Mixtral T=1024:
//            128 items for 256 CUs) leaves CUs idle while the launch is
//            bound by those re-reads from HBM.  The two spans of a tile run
//            side by side on one XCD and read its weights through L2
//            (measured on MI355X: Mixtral-shaped T=1024 down 400 -> 339-343
//            us; a two-way contraction split of the long spans instead,
//            with fp32 partial sums and a finish launch, 352-358).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kPRows = 256;                 // weight rows of an item
constexpr int kPTok = 256;                  // tokens of a span
constexpr int kPRow = 64;                   // bytes of a row per step (32 bf16)
constexpr int kPST = 4;                     // stages
constexpr int kPWaves = 8;
constexpr int kPThreads = kPWaves * kWave;
constexpr int kPMaxE = kPThreads;           // experts the in-kernel scan covers

struct SpanSmem {
  uint8_t a[kPST][kPRows * kPRow];
  uint8_t b[kPST][kPTok * kPRow];
  int tok[kPTok];
  int dst[kPTok];
  int pre[kPMaxE + 1];     // items before expert e
  int wsum[kPWaves];
};

// byte offset of (row, 16-byte segment) in a stage of 64-byte rows: a 16-byte
// fragment read is served 8 lanes (8 consecutive rows, one segment) at a time
// from 128 bytes of banks, which hold two rows; permuting the segments by bits
// 1..2 of the row puts the 8 reads in 8 different places
__device__ __forceinline__ int span_off(int row, int seg) {
  return row * kPRow + ((seg ^ ((row >> 1) & 3)) << 4);
}

// Spans of an expert's n rows: runs of 256 and a shorter last one; the down
// projection halves an expert of 193..256 rows (its length rule below)
template <bool kGateUp>
__device__ __forceinline__ int span_count(int n) {
  const int s = (n + kPTok - 1) / kPTok;
  return (!kGateUp && s == 1 && n > 3 * kPTok / 4) ? 2 : s;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void span_load16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 16, 0, 0);
}

__device__ __forceinline__ void span_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void span_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void span_wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (0x7 << 4) | (0 << 8));
}

// w: w13 [E][2I][H] (gate/up) or w2 [E][H][I] (down); xs: x [T][H] (gate/up)
// or act [rows][I] (down).  Writes act [rows][I] (gate/up) or y [pairs][H] at
// each row's pair (down; dense rows: y [T][H]).
template <class SY, bool kGateUp>
__global__ __launch_bounds__(kPThreads, 1) void span_ffn_kernel(
    const uint16_t* __restrict__ w, const uint16_t* __restrict__ xs, RowMap rm, int E, int H,
    int I, uint16_t* __restrict__ act, typename SY::T* __restrict__ y) {
  __shared__ __attribute__((aligned(1024))) SpanSmem sm;
  constexpr int TM = 8, TN = 4;
  const bool dense = rm.counts == nullptr;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave-uniform, so that the indices derived from it stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave >> 2, wn = wave & 3;
  const int m = lane & 15, g = lane >> 4;
  const int Kdim = kGateUp ? H : I;
  const int ntiles = kGateUp ? I / (kPRows / 2) : H / kPRows;
  const int nexp = dense ? 1 : E;

  // items per expert (tiles x spans of the experts within min_rows..max_rows),
  // scanned across the workgroup into pre[]
  {
    int u = 0;
    if (tid < nexp) {
      const int n = dense ? (int)rm.dense_rows : rm.counts[tid];
      if (dense || (n >= rm.min_rows && n <= rm.max_rows)) u = ntiles * span_count<kGateUp>(n);
    }
    int incl = u;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int v = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += v;
    }
    if (lane == kWave - 1) sm.wsum[wave] = incl;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int v = 0; v < kPWaves; ++v) before += v < wave ? sm.wsum[v] : 0;
    if (tid < nexp) sm.pre[tid + 1] = before + incl;
    if (tid == 0) sm.pre[0] = 0;
    __syncthreads();
  }
  const int total = __builtin_amdgcn_readfirstlane(sm.pre[nexp]);
  // this workgroup's items: XCD x = b % 8 owns items [x * per, (x + 1) * per)
  const int nc = (int)gridDim.x / 8;
  const int xcd = (int)blockIdx.x % 8, c = (int)blockIdx.x / 8;
  const int per = (total + 7) / 8;
  const int hi = min(total, (xcd + 1) * per);

  const int lrow = lane >> 2;   // row of a direct load within its 16
  for (int it = xcd * per + c; it < hi; it += nc) {
    // expert of item `it`: the last e with pre[e] <= it
    // (every value below is the same in all lanes: kept in scalar registers)
    int lo = 0, up = nexp;
    while (up - lo > 1) {
      const int mid = (lo + up) >> 1;
      if (__builtin_amdgcn_readfirstlane(sm.pre[mid]) <= it) lo = mid;
      else up = mid;
    }
    const int e = lo;
    const int n = dense ? (int)rm.dense_rows : __builtin_amdgcn_readfirstlane(rm.counts[e]);
    // spans of 256 rows and a shorter last one; an expert of 257..384 rows gets
    // two spans of equal length (within one row) instead, so that its items
    // weigh about the same rather than one full and one near-empty (the down
    // projection: from 193 rows)
    const int spans = span_count<kGateUp>(n);
    const int l = it - __builtin_amdgcn_readfirstlane(sm.pre[e]);
    const int tile = l / spans, span = l - tile * spans;
    const int slen = (spans == 2 && n <= 3 * kPTok / 2) ? (n + 1) / 2 : kPTok;
    const int row0 =
        (dense ? 0 : __builtin_amdgcn_readfirstlane(rm.offsets[e])) + span * slen;
    const int nvalid = min(slen, n - span * slen);

    __syncthreads();   // the previous item's epilogue has read dst[]
    if (tid < kPTok) {
      const int row = row0 + (tid < nvalid ? tid : 0);   // rows past the span repeat its first
      if (kGateUp) {
        sm.tok[tid] = dense ? row : rm.sorted_ids[row] / rm.K;
      } else {
        sm.tok[tid] = row;
        sm.dst[tid] = dense ? row : rm.sorted_ids[row];
      }
    }
    __syncthreads();

    // Direct loads: load n of a stage fills LDS rows 16n..16n+15 (1 KB), lane l
    // filling row 16n + l/4, slot l%4 with the row's global segment
    // (l%4) ^ ((row >> 1) & 3).  Wave w issues weight loads 2w, 2w+1 and token
    // loads 2w, 2w+1.
    // Addresses: a scalar base plus a 32-bit lane offset (an expert's weight
    // matrix and the token matrix are below 4 GB, which span_ok checks).
    const int i0 = tile * (kGateUp ? kPRows / 2 : kPRows);
    const uint8_t* wexp = reinterpret_cast<const uint8_t*>(w) +
                          (size_t)e * (kGateUp ? 2 * (size_t)I * H : (size_t)H * I) * 2;
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(xs);
    uint32_t aoff[2], boff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 16 * (2 * wave + j) + lrow;
      const uint32_t seg = (uint32_t)((lane & 3) ^ ((r >> 1) & 3));
      uint32_t wr;
      if (kGateUp) {
        const int q = r >> 4;                           // 16-row group: even gate, odd up
        const int col = i0 + 16 * (q >> 1) + (r & 15);
        wr = (uint32_t)((q & 1) ? I + col : col);
      } else {
        wr = (uint32_t)(i0 + r);
      }
      aoff[j] = wr * (uint32_t)Kdim * 2u + (seg << 4);
      boff[j] = (uint32_t)sm.tok[r] * (uint32_t)Kdim * 2u + (seg << 4);
    }
    const int nk = Kdim / 32;
    // token loads of this wavefront that hold tokens (16-row groups 2w, 2w+1
    // below the span's end); the others are skipped, and the ring's waits
    // count the wavefront's own loads per stage, 2 + lb
    // (a full span, nvalid == 256, takes the unconditional path: lb == 2)
    const int lb = min(2, max(0, (nvalid + 15) / 16 - 2 * wave));
    auto issue = [&](int ks, auto skip) {
      const int st = ks % kPST;
      const uint32_t kb = (uint32_t)ks * kPRow;
#pragma unroll
      for (int j = 0; j < 2; ++j) span_load16(wexp + (aoff[j] + kb), &sm.a[st][(2 * wave + j) * 1024]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (!decltype(skip)::value || j < lb)
          span_load16(xb + (boff[j] + kb), &sm.b[st][(2 * wave + j) * 1024]);
    };
    // wait until at most S stages' loads of this wavefront are in flight
    auto wait_stages = [&](auto S, auto skip) {
      constexpr int n = decltype(S)::value;
      if (!decltype(skip)::value || lb == 2) span_wait_vm<4 * n>();
      else if (lb == 1) span_wait_vm<3 * n>();
      else span_wait_vm<2 * n>();
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;

    // this wavefront's live 16-token tiles: wn, wn + 4, ... below the span's tiles
    const int nt = (nvalid + 15) / 16;
    const int tn_live = nt > wn ? min(TN, (nt - wn + 3) / 4) : 0;
    f32x4 acc[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto read = [&](int slot, u32x4 (&fa)[TM], u32x4 (&fb)[TN], auto masked) {
      const uint8_t* A = sm.a[slot];
      const uint8_t* Bt = sm.b[slot];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        fa[tm] = *reinterpret_cast<const u32x4*>(A + span_off(wm * 128 + tm * 16 + m, g));
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        if (!decltype(masked)::value || tn < tn_live)
          fb[tn] = *reinterpret_cast<const u32x4*>(Bt + span_off((wn + 4 * tn) * 16 + m, g));
    };
    auto ops = [&](const u32x4 (&fa)[TM], const u32x4 (&fb)[TN], auto masked) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        if (!decltype(masked)::value || tn < tn_live) {
#pragma unroll
          for (int tm = 0; tm < TM; ++tm)
            acc[tm][tn] = mfma16x16x32(fa[tm], fb[tn], acc[tm][tn]);
        }
    };
    // step t on fragments (ca, cb), reading stage t+1's into (na, nb).  Before
    // the barrier: stage t+1 has landed (the loads of the stages after it may
    // stay in flight) and this wavefront's reads of stage t are done; after it
    // stage t's slot is free for stage t+4.  The steady form (t + 4 < nk) has
    // no conditions, so it is one basic block.
    auto body = [&](int t, u32x4 (&ca)[TM], u32x4 (&cb)[TN], u32x4 (&na)[TM], u32x4 (&nb)[TN],
                    auto steady, auto skip, auto masked) {
      if constexpr (decltype(steady)::value) {
        wait_stages(S2{}, skip);
        span_wait_lgkm0();
        span_barrier();
        issue(t + 4, skip);
        read((t + 1) % kPST, na, nb, masked);   // completes while the ops issue
        ops(ca, cb, masked);
        if constexpr (!decltype(masked)::value) {
          // issue order: the stage's direct loads, then the fragment reads one
          // between each of the first ops, then the remaining ops -- and none of
          // the ops moved past the next barrier, whose wait for the reads would
          // then find the matrix pipe empty
          if constexpr (!decltype(skip)::value)
            __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);       // VMEM
#pragma unroll
          for (int i = 0; i < TM + TN; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);       // DS read
          }
          __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - TM - TN, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        if (t + 3 < nk) wait_stages(S2{}, skip);
        else if (t + 2 < nk) wait_stages(S1{}, skip);
        else wait_stages(S0{}, skip);
        span_wait_lgkm0();
        span_barrier();
        if (t + 4 < nk) issue(t + 4, skip);
        if (t + 1 < nk) read((t + 1) % kPST, na, nb, masked);
        ops(ca, cb, masked);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // skip: a partial span (its token loads limited to the groups holding
    // tokens); masked: this wavefront has token tiles past the span's end
    auto run = [&](auto skip, auto masked) {
      u32x4 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
#pragma unroll
      for (int s0 = 0; s0 < kPST; ++s0)
        if (s0 < nk) issue(s0, skip);
      // stage 0 landed (the stages issued after it may stay in flight)
      if (nk >= 4) wait_stages(S3{}, skip);
      else if (nk == 3) wait_stages(S2{}, skip);
      else if (nk == 2) wait_stages(S1{}, skip);
      else wait_stages(S0{}, skip);
      span_barrier();
      read(0, fa0, fb0, masked);
      int t = 0;
      for (; t + 5 < nk; t += 2) {
        body(t, fa0, fb0, fa1, fb1, std::true_type{}, skip, masked);
        body(t + 1, fa1, fb1, fa0, fb0, std::true_type{}, skip, masked);
      }
      for (; t < nk; t += 2) {
        body(t, fa0, fb0, fa1, fb1, std::false_type{}, skip, masked);
        if (t + 1 < nk) body(t + 1, fa1, fb1, fa0, fb0, std::false_type{}, skip, masked);
      }
    };
    if (nt == kPTok / 16)   // every 16-row group holds tokens: nothing to skip
      run(std::false_type{}, std::false_type{});
    else if (tn_live == TN)
      run(std::true_type{}, std::false_type{});
    else
      run(std::true_type{}, std::true_type{});

    // epilogue: lane holds rows 4g..4g+3 of each 16-row tile for token column
    // m of each of its token tiles
    if constexpr (kGateUp) {
#pragma unroll
      for (int p = 0; p < TM / 2; ++p)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int j = (wn + 4 * tn) * 16 + m;
          if (j < nvalid) {
            const f32x4 gs = acc[2 * p][tn], us = acc[2 * p + 1][tn];
            const int i = i0 + 16 * (4 * wm + p) + 4 * g;
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
          const int j = (wn + 4 * tn) * 16 + m;
          if (j < nvalid) {
            const int h = i0 + wm * 128 + tm * 16 + 4 * g;
            store_out4<SY>(y + (size_t)sm.dst[j] * H + h, acc[tm][tn]);
          }
        }
    }
  }
}

// compute units of the device current at the first call, as a multiple of the
// 8 XCDs (a static initialised once, so concurrent first calls do not race)
int span_workgroups() {
  static const int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 8)
      cus = 256;
    return cus / 8 * 8;
  }();
  return n;
}

// workgroups for at most `items` items: a multiple of 8, at most one per CU
unsigned span_grid(int64_t items) {
  const int64_t g = (items + 7) / 8 * 8;
  return (unsigned)(g < span_workgroups() ? (g < 8 ? 8 : g) : span_workgroups());
}

// items of a launch: tiles x the spans of the rows, at most rows/256 + one per
// expert (gate/up) or rows/192 + one per expert (down, whose experts of 193..256
// rows take two spans)
int64_t span_items(const RowMap& rm, int E, int64_t rows_bound, int ntiles, bool gate_up) {
  const int64_t per = gate_up ? kPTok : 3 * kPTok / 4;
  const int64_t spans = rm.counts == nullptr ? rm.dense_rows / per + 1 : rows_bound / per + E;
  return spans * ntiles;
}

}  // namespace

bool span_ok(int E, int H, int I, int64_t x_rows, int64_t act_rows) {
  const int64_t lim = (int64_t)1 << 32;
  return E >= 1 && E <= kPMaxE && H % kPRows == 0 && I % (kPRows / 2) == 0 &&
         (int64_t)2 * I * H * 2 < lim && x_rows * H * 2 < lim && act_rows * I * 2 < lim;
}

hipError_t launch_span_gate_up(const void* x, const void* w13, const RowMap& rm, int E, int H,
                               int I, int64_t x_rows, int64_t rows_bound, uint16_t* act,
                               hipStream_t s) {
  if (!span_ok(rm.counts == nullptr ? 1 : E, H, I, x_rows, rows_bound)) return hipErrorInvalidValue;
  const int ntiles = I / (kPRows / 2);
  const int64_t items = span_items(rm, E, rows_bound, ntiles, true);
  if (items <= 0) return hipSuccess;
  hipLaunchKernelGGL((span_ffn_kernel<BF16, true>), dim3(span_grid(items)), dim3(kPThreads), 0, s,
                     static_cast<const uint16_t*>(w13), static_cast<const uint16_t*>(x), rm, E, H,
                     I, act, (uint16_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_span_down(const void* w2, const uint16_t* act, const RowMap& rm, int E, int H,
                            int I, int64_t act_rows, int64_t rows_bound, void* y, int ydt,
                            hipStream_t s) {
  if (!span_ok(rm.counts == nullptr ? 1 : E, H, I, 0, act_rows)) return hipErrorInvalidValue;
  const int ntiles = H / kPRows;
  const int64_t items = span_items(rm, E, rows_bound, ntiles, false);
  if (items <= 0) return hipSuccess;
  if (ydt == kDtF32)
    hipLaunchKernelGGL((span_ffn_kernel<F32, false>), dim3(span_grid(items)), dim3(kPThreads), 0,
                       s, static_cast<const uint16_t*>(w2), act, rm, E, H, I, (uint16_t*)nullptr,
                       static_cast<float*>(y));
  else
    hipLaunchKernelGGL((span_ffn_kernel<BF16, false>), dim3(span_grid(items)), dim3(kPThreads), 0,
                       s, static_cast<const uint16_t*>(w2), act, rm, E, H, I, (uint16_t*)nullptr,
                       static_cast<uint16_t*>(y));
  return hipGetLastError();
}

}  // namespace moe
