/*
 * moe_layer.h -- C ABI of the MI355X (gfx950) forward pass of one
 * Mixture-of-Experts feed-forward layer, and of its FLOP-matched dense
 * baseline (DenseFA).
 *
 * The layer pass is five stream-ordered calls:
 *
 *   moe_route        router logits -> top-K expert ids and combine weights
 *                    (moe_route_var: a routing budget per token)
 *   moe_align        (token, slot) pairs -> expert buckets padded to the tile
 *   moe_grouped_ffn  per-expert SwiGLU: gate/up GEMM + SwiGLU, then down GEMM
 *                    (also callable as its two halves, moe_grouped_gate_up and
 *                    moe_grouped_down)
 *   moe_combine      weighted sum of each token's K expert rows (+ shared)
 *   dense_ffn_fa     one dense SwiGLU FFN over all tokens: the DenseFA
 *                    baseline, and the shared experts of a layer
 *
 * Sources for what each call computes are cited at the call.  "Serving-tax
 * notes" below means the talk notes on "Demystifying the Mixture of Experts
 * Serving Tax" (MLSys 2026); "TEMPO page" means the article on TEMPO
 * (makespan-aware expert-parallel load balancing).
 *
 * Conventions (all calls):
 *  - Every buffer is device memory owned by the caller; the library never
 *    allocates or frees memory.  The state it keeps between calls is the
 *    per-thread message of moe_last_error() and the per-GPU workspace array of
 *    moe_grouped_ffn_noalloc (with its device address); every other call is
 *    thread-safe.
 *  - Tensors are dense row-major; base pointers are 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    on it and the call returns without waiting; results are valid once the
 *    stream has reached that point.  No call synchronises with the host.
 *  - Arguments are checked before anything is launched; on error nothing is
 *    enqueued and no output is touched.  T = 0 is a successful no-op.
 *  - A failed launch returns MOE_EHIP.  moe_last_error() returns a message
 *    for the last failure on the calling thread.
 *  - Limits: 1 <= K <= E <= 256; H and the intermediate sizes multiples of 64;
 *    T * K < 2^31; alignment block 1..1024.  Storage dtypes are fp32 or bf16;
 *    GEMM operands are rounded to bf16 and accumulated in fp32.
 */
#ifndef MOE_LAYER_H
#define MOE_LAYER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = 1,        /* null/misaligned pointer, negative size, K outside [1, E], ... */
    MOE_EUNSUPPORTED = 2,  /* shape or dtype outside the limits above */
    MOE_ECAPACITY = 3,     /* plan capacity or workspace smaller than required */
    MOE_EHIP = 4           /* a HIP launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Schedules of the grouped FFN (and of the dense FFN). */
typedef enum {
    MOE_SCHED_AUTO = 0,    /* TILE once experts average 24 tokens (T*K >= 24*E), T > 32
                              and block_m allows it; below that RING where it applies,
                              chosen per expert on the device (two regimes per expert,
                              TEMPO page): experts whose tokens fit a ring pass (every
                              token up to T = 32; 16 or 32 beyond) streamed, busier ones
                              tiled when block_m allows it, else streamed by STREAM; else
                              STREAM; SPAN instead of TILE where it applies, once experts
                              average 256 tokens (T*K >= 256*E), with n = ceil(T*K/256):
                              for the gate/up half when (I/128)*n >= 768, for the down half
                              when (H/256)*n >= 128 and (H/256)*(T*K/256 + E) <= 256;
                              else the bf16 gate/up tile is 512 weight rows wide
                              once experts average 512 tokens (T*K >= 512*E, block_m 128,
                              I % 256 == 0); dense rows: TILE above 32
                              tokens (a gate/up grid, (I/128) x ceil(T/block), of fewer
                              than 128 tiles, or a down grid of fewer than 256, splits
                              its contraction in fp32 slices added in slice order), else
                              streamed */
    MOE_SCHED_STREAM = 1,  /* weight-streaming: each active expert's weights read once per
                              pass of up to 64 tokens, straight into MFMA operand registers;
                              any supported shape and dtype; for HBM-bound (decode) shapes */
    MOE_SCHED_TILE = 2,    /* MFMA tiles of block_m tokens x 128 to 512 weight rows
                              staged through LDS (a ring of direct loads for bf16 and FP8
                              weights, registers for fp32); for MFMA-bound
                              (prefill) shapes; needs block_m 64 or 128 */
    MOE_SCHED_RING = 3,    /* weight-streaming through an LDS ring filled by whole-line
                              direct loads, one persistent workgroup per CU; needs bf16,
                              H % 128 == 0 and I % 64 == 0 (gate/up), I % 128 == 0 (down) */
    MOE_SCHED_SPAN = 4     /* MFMA tiles of 256 weight rows x spans of up to 256 of one
                              expert's tokens, any block_m: each weight tile streamed once
                              per span, by persistent workgroups (one per CU) that cut the
                              items into one run per XCD; for MFMA-bound (prefill) shapes;
                              needs bf16, E <= 512, H % 256 == 0, I % 128 == 0 and an
                              expert's gate/up matrix, x and the activations each below
                              4 GB (else MOE_EUNSUPPORTED) */
} moe_schedule;

/*
 * The alignment produced by moe_align and read by the grouped FFN.  All
 * arrays are int32 device memory owned by the caller:
 *   expert_counts  [E]        N_e, pairs routed to expert e
 *   expert_offsets [E+1]      exclusive prefix sum of P_e = ceil(N_e/B)*B;
 *                             expert_offsets[E] = num_padded
 *   sorted_ids     [cap]      pair index p = t*K + k of each row; bucket e is
 *                             rows expert_offsets[e] .. +N_e-1 in ascending p;
 *                             every other row holds the sentinel T*K
 *   block_expert   [cap/B]    expert of each B-row block; -1 past num_padded
 *   inv_pos        [T*K]      row holding pair p
 *   block_m        B, the padding block (the GEMM M-tile)
 *   cap            rows of sorted_ids; a multiple of B and at least
 *                  moe_align_capacity(T, K, E, B)
 */
typedef struct {
    int32_t *expert_counts;
    int32_t *expert_offsets;
    int32_t *sorted_ids;
    int32_t *block_expert;
    int32_t *inv_pos;
    int32_t block_m;
    int64_t cap;
} moe_plan;

/* Message for the last failed call on this thread ("" if none). */
const char *moe_last_error(void);
const char *moe_status_string(moe_status s);

/*
 * Rows the alignment may need: the padded total sum_e ceil(N_e/B)*B is at
 * most T*K + min(E, T*K)*(B-1) (each non-empty bucket adds fewer than B rows
 * of padding), rounded up to a multiple of B.  Returns -1 on bad arguments.
 */
int64_t moe_align_capacity(int64_t T, int K, int E, int block_m);

/* Padding schemes of the alignment (Serving-tax notes, "Padding model (Section 5.1)"). */
typedef enum {
    MOE_PAD_BLOCK = 0,   /* each expert on its own: P = sum_i ceil(N_i/B)*B */
    MOE_PAD_MAX = 1      /* every expert the busiest one's slot: P = E*ceil(max_i N_i/B)*B */
} moe_padding;

/*
 * Rows an alignment with padding `pad` may need: moe_align_capacity for
 * MOE_PAD_BLOCK; E * ceil(T/B)*B for MOE_PAD_MAX (no expert holds more than T
 * pairs, its tokens' K experts being distinct).  Returns -1 on bad arguments.
 */
int64_t moe_align_capacity_ex(int64_t T, int K, int E, int block_m, moe_padding pad);

/* Workspace bytes moe_grouped_ffn needs: the SwiGLU activations, [cap][I] bf16. */
int64_t moe_ffn_workspace_bytes(int64_t cap, int I);

/*
 * Workspace bytes with which moe_grouped_ffn (and its halves, bf16 and FP8)
 * may also split the contraction of a launch across workgroups: a
 * weight-streaming launch when few experts can be active (T*K or E small:
 * their weight slabs alone would leave compute units idle), and the tiled
 * bf16 down projection when its token blocks would (sized where MOE_SCHED_AUTO
 * tiles: T > 32 and T*K >= 24*E).  The workspace holds the activations, then
 * fp32 partial sums per pair added in a fixed order by a second kernel.  A
 * workspace of at least this size selects the split wherever it applies; one
 * of moe_ffn_workspace_bytes never splits.  The two give results that differ
 * only in fp32 rounding; each is deterministic.  Returns -1 on bad arguments.
 */
int64_t moe_ffn_workspace_bytes_ex(int64_t cap, int64_t T, int K, int E, int H, int I);

/* Workspace bytes dense_ffn_fa needs: the activations of T tokens (bf16) and,
 * when the contraction is split across workgroups, the fp32 partial sums.
 * Returns -1 on unsupported sizes. */
int64_t dense_ffn_workspace_bytes(int64_t T, int H, int I_fa);

/*
 * Routing (Serving-tax notes, Table 1 row "auxiliary kernels": routing and
 * top-K; finding 5 / Fig. 5).  The pages leave the gating function open; it
 * is softmax over the E logits, the K largest, renormalised to sum to one:
 *   selected: the K experts with the largest logits, ties to the lower id;
 *   slot order: logit descending, then id ascending;
 *   topk_w[t][j] = p_{e_j} / sum_i p_{e_i},  p = softmax(logits[t]).
 * logits   [T][E] fp32 (finite)          topk_ids [T][K] int32 (out)
 * topk_w   [T][K] fp32 (out)
 * Errors: MOE_EINVAL (null/misaligned, T < 0, K outside [1, E]),
 *         MOE_EUNSUPPORTED (E > 256).
 */
moe_status moe_route(const float *logits, int64_t T, int E, int K, int32_t *topk_ids,
                     float *topk_w, void *stream);

/*
 * Routing with a per-token budget (MoE-Prism page: the routing top-k is a
 * runtime knob chosen per request, so one batch mixes budgets).  Token t takes
 * k_t = k_tok[t] experts, clamped to [0, Kmax], selected and renormalised as
 * by moe_route with K = k_t; its slots k_t .. Kmax-1 get id -1 and weight 0.
 * The rest of the pass runs with K = Kmax: moe_align leaves the unused slots
 * out (no row, inv_pos -1), the grouped FFN never sees them, moe_combine
 * skips their zero weights; a token with k_t = 0 gets only the shared experts.
 * k_tok [T] int32 device memory.  Errors: as moe_route (Kmax for K).
 */
moe_status moe_route_var(const float *logits, int64_t T, int E, int Kmax, const int32_t *k_tok,
                         int32_t *topk_ids, float *topk_w, void *stream);

/*
 * Alignment with block-wise padding (Serving-tax notes, "Padding model
 * (Section 5.1)": every expert's token count rounded up to a multiple of the
 * block B, P = sum_i ceil(N_i/B)*B; the 128-row grouped-GEMM tile of the
 * TEMPO page is the prefill choice of B).  Fills every array of `plan` (see
 * moe_plan) over its whole length.  Deterministic: buckets hold their pairs in
 * ascending p.  topk_ids [T][K] int32 in [0, E), or negative for an unused
 * slot (moe_route_var): such a pair gets no row and inv_pos -1.
 * Errors: MOE_EINVAL, MOE_EUNSUPPORTED (E > 256), MOE_ECAPACITY (cap too small).
 */
moe_status moe_align(const int32_t *topk_ids, int64_t T, int K, int E, const moe_plan *plan,
                     void *stream);

/*
 * moe_align with a choice of padding scheme (Section 5.1 of the Serving-tax
 * notes): MOE_PAD_BLOCK is moe_align; MOE_PAD_MAX gives every expert, empty
 * ones included, ceil(max_i N_i/B)*B rows (offsets[e] = e times that), the
 * layout of a grouped GEMM with one fixed-size slot per expert.  Buckets hold
 * the same pairs in the same order as with block-wise padding.  plan->cap must
 * be at least moe_align_capacity_ex(T, K, E, block_m, pad).  Every grouped-FFN
 * schedule reads either layout.
 * Errors: as moe_align; MOE_EINVAL for an unknown scheme.
 */
moe_status moe_align_ex(const int32_t *topk_ids, int64_t T, int K, int E, const moe_plan *plan,
                        moe_padding pad, void *stream);

/*
 * moe_route (k_tok NULL) or moe_route_var (k_tok [T] int32 budgets), then
 * moe_align_ex, with the same arguments and the same results bit for bit: the
 * Table 1 auxiliary kernels of the Serving-tax notes at decode, where each is a
 * few microseconds of work.  While T*K <= 4096 and one workgroup routes the
 * batch in one pass (T <= 128, 64, 32 or 16 for E <= 8, 16, 32, or more) both
 * run in one launch of one workgroup (the ids it routes stay in LDS for the
 * alignment); otherwise the two launches.  topk_ids / topk_w are written as by moe_route; the plan as by
 * moe_align_ex.
 * Errors: those of moe_route and moe_align_ex.
 */
moe_status moe_route_align(const float *logits, int64_t T, int E, int K, const int32_t *k_tok,
                           int32_t *topk_ids, float *topk_w, const moe_plan *plan,
                           moe_padding pad, void *stream);

/*
 * Grouped expert FFN (Serving-tax notes, Table 1 row "GroupGEMM": the batch
 * is split per expert; Table 2 gives the MoE intermediate size).  The expert
 * body is a bias-free SwiGLU.  For each valid row r of the plan (pair
 * p = sorted_ids[r], token t = p / K, expert e):
 *   a = silu(W1_e x_t) * (W3_e x_t),   y_pairs[p] = W2_e a
 * x        [T][H]       dtype dt
 * w13      [E][2I][H]   dtype dt; rows 0..I-1 of each expert are W1 (gate),
 *                       rows I..2I-1 are W3 (up)
 * w2       [E][H][I]    dtype dt (down projection, out x in)
 * workspace            >= moe_ffn_workspace_bytes(plan->cap, I) bytes (the
 *                      _ex size also allows a contraction split, see there)
 * y_pairs  [T*K][H]     dtype dt (out), row p = t*K + k
 * Rows of experts with no tokens are never read: an unused expert's weights
 * cost no HBM traffic.
 * Errors: MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ECAPACITY.
 */
moe_status moe_grouped_ffn(const void *x, moe_dtype dt, int64_t T, int H, int I, int E, int K,
                           const void *w13, const void *w2, const moe_plan *plan,
                           void *workspace, int64_t workspace_bytes, void *y_pairs,
                           void *stream);

/*
 * Allocation-free variant of moe_grouped_ffn, for callers that cannot allocate
 * device memory: code under HIP graph capture, serving loops and harnesses
 * that forbid allocation.  It computes what moe_grouped_ffn computes, with the
 * same kernels and schedules as moe_grouped_ffn given a workspace of
 * MOE_NOALLOC_SCRATCH_BYTES bytes, but that workspace is a device array held
 * by the library: one array of MOE_NOALLOC_SCRATCH_BYTES on each GPU the
 * library runs on, from when its code is loaded there until the process ends.
 * The caller passes the inputs, the plan and y_pairs as for moe_grouped_ffn;
 * the call allocates and frees no device memory.
 * Every call on one GPU shares that GPU's array and finds the last call's
 * contents in it; no part of it needs to start at zero (rows of the array
 * that hold no token may be read by the tiled schedule, but their products
 * are never stored).  Calls that overlap on one GPU race (two streams, or two
 * host threads whose calls are not ordered on one stream): their results are
 * undefined.  Calls ordered on one stream are safe.
 * Errors: as moe_grouped_ffn; MOE_ECAPACITY when moe_ffn_workspace_bytes(
 * plan->cap, I) exceeds MOE_NOALLOC_SCRATCH_BYTES, checked before any device
 * call.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((int64_t)128 << 20)
moe_status moe_grouped_ffn_noalloc(const void *x, moe_dtype dt, int64_t T, int H, int I, int E,
                                   int K, const void *w13, const void *w2, const moe_plan *plan,
                                   void *y_pairs, void *stream);

/* First half of moe_grouped_ffn: writes a = silu(W1 x) * (W3 x) as bf16 into
 * workspace row r, columns 0..I-1, for every valid row r. */
moe_status moe_grouped_gate_up(const void *x, moe_dtype dt, int64_t T, int H, int I, int E, int K,
                               const void *w13, const moe_plan *plan, void *workspace,
                               int64_t workspace_bytes, moe_schedule sched, void *stream);

/* Second half of moe_grouped_ffn: y_pairs[sorted_ids[r]] = W2_e a_r for every valid row r.
 * Reads the activations from the workspace; with a workspace of the _ex size
 * it may write partial sums past them. */
moe_status moe_grouped_down(const void *w2, moe_dtype dt, int64_t T, int H, int I, int E, int K,
                            const moe_plan *plan, void *workspace, int64_t workspace_bytes,
                            void *y_pairs, moe_schedule sched, void *stream);

/*
 * Combine, the "local sum" of finding 5 (Serving-tax notes):
 *   out[t] = sum_{k = 0..K-1, in slot order} topk_w[t][k] * y_pairs[t*K + k]  (+ shared[t])
 * accumulated in fp32, rounded once to odt.  No atomics: bit-identical on
 * every run.  shared may be NULL (a layer with no shared experts).  Slots of
 * weight 0 are skipped and their rows not read (the unused slots of
 * moe_route_var have no row).
 * y_pairs [T*K][H] ydt; topk_w [T][K] fp32; shared [T][H] sdt; out [T][H] odt.
 */
moe_status moe_combine(const void *y_pairs, moe_dtype ydt, const float *topk_w, const void *shared,
                       moe_dtype sdt, int64_t T, int K, int H, void *out, moe_dtype odt,
                       void *stream);

/*
 * Dense SwiGLU FFN over all T tokens: out = W2 (silu(W1 x) * (W3 x)).
 * As DenseFA (Serving-tax notes, section "定義", Eq. 1: tau = T(MoE, b) /
 * T(DenseFA, b)) its width is I_fa = K*I + I_s, the MoE layer's per-token
 * FLOPs; it also computes a layer's shared experts (width I_s, weight 1).
 * x [T][H] dt; w13 [2*I_fa][H] dt (gate rows then up rows); w2 [H][I_fa] dt;
 * workspace >= dense_ffn_workspace_bytes(T, H, I_fa); out [T][H] odt.
 * Deterministic: when the contraction is split across workgroups the partial
 * sums are added in a fixed order by a second kernel, never with atomics.
 * MOE_SCHED_AUTO streams up to 32 tokens and tiles above; its gate/up half
 * takes the span schedule (bf16, span shape conditions) where that gives
 * (I_fa/128) * ceil(T/256) >= 384 work items.
 */
moe_status dense_ffn_fa(const void *x, moe_dtype dt, int64_t T, int H, int I_fa, const void *w13,
                        const void *w2, void *workspace, int64_t workspace_bytes, void *out,
                        moe_dtype odt, moe_schedule sched, void *stream);

/*
 * FP8 weights: weight quantization, the notes' decode-phase remedy (Serving-tax
 * notes, "デコード最適化": it cuts the bytes that weight amplification makes the
 * step read).  Weights are OCP FP8 E4M3 codes (1 sign bit, 4 exponent bits
 * with bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN) with one fp32
 * scale per matrix row: W[r][c] = value(code[r][c]) * scale[r].  x, the
 * activations and y_pairs are bf16; the codes are expanded to bf16 exactly,
 * multiplied on bf16 MFMA with fp32 accumulation, and each row's scale is
 * applied to its accumulators.  The LDS-ring weight-streaming schedule runs
 * the experts in passes of up to 32 of an expert's tokens (busier experts take
 * several passes); once experts average 24 tokens (T*K >= 24*E, T > 32) the
 * tiled schedule takes every expert when block_m is 64 or 128, H % 256 == 0
 * and I % 128 == 0.  Dense rows are streamed up to 32 tokens and tiled above
 * (same shape conditions, and the contraction splits of dense_ffn_fa's tiled
 * schedule; else streamed).
 * Shapes: H % 128 == 0 and I % 128 == 0.  Pointers: codes 16-byte aligned,
 * scales 4-byte aligned.  Same plan and workspace as the bf16 calls.
 *   moe_grouped_gate_up_fp8: w13 [E][2I][H] codes, w13_scale [E][2I] fp32
 *   moe_grouped_down_fp8:    w2 [E][H][I] codes,  w2_scale [E][H] fp32
 *   dense_ffn_fp8:           w13 [2I][H], w13_scale [2I], w2 [H][I], w2_scale [H]
 * Errors: as their bf16 counterparts; MOE_EUNSUPPORTED for other shapes.
 */
moe_status moe_grouped_gate_up_fp8(const void *x, int64_t T, int H, int I, int E, int K,
                                   const uint8_t *w13, const float *w13_scale,
                                   const moe_plan *plan, void *workspace, int64_t workspace_bytes,
                                   void *stream);
moe_status moe_grouped_down_fp8(const uint8_t *w2, const float *w2_scale, int64_t T, int H, int I,
                                int E, int K, const moe_plan *plan, void *workspace,
                                int64_t workspace_bytes, void *y_pairs, void *stream);
moe_status dense_ffn_fp8(const void *x, int64_t T, int H, int I, const uint8_t *w13,
                         const float *w13_scale, const uint8_t *w2, const float *w2_scale,
                         void *workspace, int64_t workspace_bytes, void *out, moe_dtype odt,
                         void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LAYER_H */
