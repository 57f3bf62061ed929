// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Records the message moe_last_error() returns on this thread; returns status.
int set_last_error(int status, const char* fmt, ...);

constexpr int kDtF32 = 0;
constexpr int kDtBF16 = 1;
constexpr int kDtFP8 = 2;   // weights only: OCP E4M3 codes with fp32 row scales

// k_tok (nullable): per-token budgets, clamped to [0, K]; unused slots get -1 / 0
hipError_t launch_route(const float* logits, int64_t T, int E, int K, const int32_t* k_tok,
                        int32_t* ids, float* w, hipStream_t s);

// max_pad: 0 block-wise padding, 1 max padding (every expert ceil(max N / B) * B rows)
hipError_t launch_align(const int32_t* ids, int64_t T, int K, int E, int B, int64_t cap,
                        int max_pad, int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* inv_pos, hipStream_t s);

hipError_t launch_combine(const void* y, int ydt, const float* w, const void* shared, int sdt,
                          int64_t T, int K, int H, void* out, int odt, hipStream_t s);

// Token rows of a grouped (or dense) GEMM.  Grouped: expert e owns the rows
// offsets[e] .. offsets[e] + counts[e] - 1 of the alignment; row r holds pair
// sorted_ids[r], i.e. token sorted_ids[r] / K.  Dense (counts == nullptr): one
// "expert" whose row r is token r, for r < dense_rows.
//
// min_rows / max_rows (grouped rows; 1 and INT32_MAX by default) restrict every
// grouped kernel to the experts with min_rows <= count <= max_rows: the LDS-ring
// kernel takes the experts whose tokens fit its passes and the register-
// streaming or the tiled kernel the rest.
struct RowMap {
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* inv_pos;   // grouped: alignment row of each pair (-1: pair unused)
  int K;
  int64_t dense_rows;
  int block_m;
  int min_rows, max_rows;
};

// Weight-streaming schedule.  tok_blocks: 16-token MFMA blocks per pass over
// the weights (1, 2 or 4); E: grid extent over experts (1 for dense).
// splits > 1 (dense rows only) cuts the contraction into that many slices
// whose fp32 sums go to `part` ([splits][rows][2I] for gate/up, [splits][rows][H]
// for down) and are added in slice order by a finish kernel.
hipError_t launch_stream_gate_up(const void* x, int xdt, const void* w13, const RowMap& rm, int E,
                                 int H, int I, int tok_blocks, int splits, uint16_t* act,
                                 float* part, hipStream_t s);
hipError_t launch_stream_down(const void* w2, int wdt, const uint16_t* act, const RowMap& rm,
                              int E, int H, int I, int tok_blocks, int splits, void* y, int ydt,
                              float* part, hipStream_t s);

// LDS-tiled MFMA schedule: one workgroup per (block_m-row token block, 128 weight rows).
// ksplit > 1 (bf16, I % 128 == 0 only): the contraction in slices whose fp32 gate and
// up sums go to part [ksplit][rows][2I] -- rows the dense rows, or for grouped rows
// the `pairs` (T*K) pairs, indexed by pair -- the SwiGLU applied by the finish kernel
// after adding them in slice order (grouped: into each pair's alignment row).
// nfull > 0 (bf16 dense rows in one 128-token block, I % 64 == 0, nfull < I/64):
// 128-row tiles, tiles 0..nfull-1 whole and each later tile's contraction in ksplit
// slices, whose sums go to part [ksplit][rows][2 (I - 64 nfull)] (columns from
// 64 nfull: gate, then up); hipErrorInvalidValue for other shapes.
hipError_t launch_tile_gate_up(const void* x, int xdt, const void* w13, const RowMap& rm,
                               int64_t nblocks, int H, int I, uint16_t* act, hipStream_t s,
                               int ksplit = 1, float* part = nullptr, int64_t pairs = 0,
                               int nfull = 0);
// The gate/up tile of 512 weight rows x 128 tokens for bf16 experts that hold
// several 128-token blocks: block_m 128, I % 256 == 0, H % 32 == 0 and an
// expert's gate/up matrix below 4 GB (tile_wide_ok); hipErrorInvalidValue else.
bool tile_wide_ok(int block_m, int H, int I);
hipError_t launch_tile_gate_up_wide(const void* x, const void* w13, const RowMap& rm,
                                    int64_t nblocks, int H, int I, uint16_t* act, hipStream_t s);
// ksplit > 1 (bf16, H % 256 == 0 only) splits the contraction into slices whose
// fp32 sums go to part [ksplit][rows][H] (rows: the dense rows, or the `pairs` pairs
// of grouped rows), added in order by a finish kernel.
hipError_t launch_tile_down(const void* w2, int wdt, const uint16_t* act, const RowMap& rm,
                            int64_t nblocks, int H, int I, void* y, int ydt, int ksplit,
                            float* part, hipStream_t s, int64_t pairs = 0);

// The tiled schedule with FP8 E4M3 weights and fp32 row scales (w13_scale
// [E][2I], w2_scale [E][H]) and bf16 tokens; needs H % 256 == 0, I % 128 == 0 and
// block_m 64, 128 or 256 (tile_fp8_ok).  ksplit as for launch_tile_gate_up and
// launch_tile_down.
bool tile_fp8_ok(int H, int I, int block_m);
hipError_t launch_tile_gate_up_fp8(const void* x, const void* w13, const float* w13_scale,
                                   const RowMap& rm, int64_t nblocks, int H, int I, uint16_t* act,
                                   hipStream_t s, int ksplit = 1, float* part = nullptr);
hipError_t launch_tile_down_fp8(const void* w2, const float* w2_scale, const uint16_t* act,
                                const RowMap& rm, int64_t nblocks, int H, int I, void* y, int ydt,
                                int ksplit, float* part, hipStream_t s);

// Prefill-shape schedule with each 256-row weight tile streamed once per span
// of up to 256 of an expert's tokens (dense rows: of the T rows), by persistent
// workgroups: bf16 weights and tokens, E <= 512, H % 256 == 0, I % 128 == 0,
// and an expert's gate/up matrix, the x_rows x H tokens and the act_rows x I
// activations each below 4 GB (span_ok; hipErrorInvalidValue else).
// rows_bound bounds the grouped rows (T * K; the plan's cap for the act rows);
// only experts with min_rows..max_rows tokens are computed.
bool span_ok(int E, int H, int I, int64_t x_rows, int64_t act_rows);
hipError_t launch_span_gate_up(const void* x, const void* w13, const RowMap& rm, int E, int H,
                               int I, int64_t x_rows, int64_t rows_bound, uint16_t* act,
                               hipStream_t s);
hipError_t launch_span_down(const void* w2, const uint16_t* act, const RowMap& rm, int E, int H,
                            int I, int64_t act_rows, int64_t rows_bound, void* y, int ydt,
                            hipStream_t s);

// act[o][col0 + i] = silu(g) * u for i < W = I - col0, with g, u the in-order sums
// over z < splits of part[z][r][i] and part[z][r][W + i], o = out_row[r] (r when
// out_row is null; rows with out_row[r] < 0 are skipped).
hipError_t launch_finish_gate_up(const float* part, int splits, int64_t rows, int I,
                                 uint16_t* act, hipStream_t s, const int32_t* out_row = nullptr,
                                 int col0 = 0);

// y[r][h] = sum over z < splits (in order) of part[z][r][h], rounded to ydt
// (rows with skip[r] < 0 left untouched when skip is not null).
hipError_t launch_finish_down(const float* part, int splits, int64_t rows, int H, void* y,
                              int ydt, hipStream_t s, const int32_t* skip = nullptr);

// LDS-ring variant of the weight-streaming schedule: bf16 tokens, bf16 or FP8
// weights, 128-row weight slabs streamed in stages of ring_stage_k contraction
// elements by persistent workgroups (one per CU).  *_ok tells whether a shape
// qualifies; *_splits is the contraction split it uses for `rows` dense rows at
// ks elements per stage (part holds [splits][rows][2I] resp. [splits][rows][H]
// fp32).
bool ring_gate_up_ok(int xdt, int wdt, int H, int I);
bool ring_down_ok(int wdt, int H, int I);
int ring_gate_up_splits(int64_t rows, int H, int I, int ks = 128);
int ring_down_splits(int64_t rows, int H, int I, int ks = 128);
// the same for grouped rows: `pairs` partial-sum rows, at most `experts`
// experts with tokens (each within one pass)
int ring_grouped_splits(int64_t pairs, int64_t experts, int H, int I, bool gate_up, int ks = 128);
// contraction elements per stage for weights wdt, tok_blocks blocks per pass and
// contraction length kdim: 128, or 256 for FP8 weights with at most 2 blocks
int ring_stage_k(int wdt, int tok_blocks, int kdim);
// T bounds the rows of any expert; tok_blocks (1, 2, 4) is the 16-token blocks
// per pass over the weights (an expert with more tokens takes more passes).
// wdt: kDtBF16, or kDtFP8 with the row scales w13_scale [E][2I] / w2_scale [E][H].
hipError_t launch_ring_gate_up(const void* x, int wdt, const void* w13, const float* w13_scale,
                               const RowMap& rm, int E, int H, int I, int64_t T, int tok_blocks,
                               int splits, uint16_t* act, float* part, hipStream_t s);
hipError_t launch_ring_down(const void* w2, int wdt, const float* w2_scale, const uint16_t* act,
                            const RowMap& rm, int E, int H, int I, int64_t T, int tok_blocks,
                            int splits, void* y, int ydt, float* part, hipStream_t s);

}  // namespace moe
