// C ABI of the MoE layer library: argument checks, schedule choice, launches.
// What each call computes is documented in include/moe_layer.h.
#include "moe_layer.h"

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kernels.h"
#include "route_align.h"

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

moe_status ok() {
  g_err[0] = 0;
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

constexpr int kMaxExperts = 256;

bool valid_dtype(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }
size_t dt_bytes(int dt) { return dt == MOE_F32 ? 4 : 2; }

int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

moe_status check_route_shape(int64_t T, int E, int K) {
  if (T < 0) return fail(MOE_EINVAL, "T = %lld < 0", (long long)T);
  if (E < 1 || K < 1 || K > E) return fail(MOE_EINVAL, "need 1 <= K <= E (K = %d, E = %d)", K, E);
  if (E > kMaxExperts) return fail(MOE_EUNSUPPORTED, "E = %d > %d", E, kMaxExperts);
  if (T * K >= (int64_t)1 << 31) return fail(MOE_EUNSUPPORTED, "T*K must be < 2^31");
  return MOE_OK;
}

moe_status check_plan(const moe_plan* plan, int64_t T, int K, int E,
                      moe_padding pad = MOE_PAD_BLOCK) {
  if (!plan) return fail(MOE_EINVAL, "plan is NULL");
  if (plan->block_m < 1 || plan->block_m > 1024)
    return fail(MOE_EUNSUPPORTED, "block_m = %d outside 1..1024", plan->block_m);
  const int32_t* arrs[5] = {plan->expert_counts, plan->expert_offsets, plan->sorted_ids,
                            plan->block_expert, plan->inv_pos};
  const char* names[5] = {"expert_counts", "expert_offsets", "sorted_ids", "block_expert",
                          "inv_pos"};
  for (int i = 0; i < 5; ++i)
    if (!arrs[i] || !aligned(arrs[i], 4))
      return fail(MOE_EINVAL, "plan->%s is NULL or misaligned", names[i]);
  if (plan->cap % plan->block_m != 0)
    return fail(MOE_EINVAL, "plan->cap = %lld is not a multiple of block_m = %d",
                (long long)plan->cap, plan->block_m);
  const int64_t need = moe_align_capacity_ex(T, K, E, plan->block_m, pad);
  if (plan->cap < need)
    return fail(MOE_ECAPACITY, "plan->cap = %lld < %lld required", (long long)plan->cap,
                (long long)need);
  if (plan->cap >= (int64_t)1 << 31) return fail(MOE_EUNSUPPORTED, "plan->cap must be < 2^31");
  return MOE_OK;
}

moe_status check_ffn_dims(int H, int I) {
  if (H < 64 || H % 64 != 0) return fail(MOE_EUNSUPPORTED, "H = %d must be a positive multiple of 64", H);
  if (I < 64 || I % 64 != 0) return fail(MOE_EUNSUPPORTED, "I = %d must be a positive multiple of 64", I);
  return MOE_OK;
}

// 16-token MFMA blocks per weight pass of the streaming schedule.  Each
// expert holds at most T rows (a token's K experts are distinct), so T bounds
// the largest bucket.
int stream_tok_blocks(int64_t max_rows) {
  if (max_rows <= 16) return 1;
  if (max_rows <= 32) return 2;
  return 4;
}

// Token blocks per pass of the LDS-ring schedule, whose LDS holds the pass's
// token rows next to the weights (more blocks, fewer stages in flight): the
// expected load of an expert, lam = T*K/E, with a margin.  An expert above 16
// times that takes several passes.  With whole_pass (bf16 weights) a pass
// takes every token up to 32, so no expert is left to a second launch
// (measured on MI355X: Qwen2 at T=32 with Zipf routing, expected load 4 tokens
// per expert, 0.508 -> 0.461 ms); bf16 uses 2*lam + 8 above that.  FP8
// weights, whose busy experts stay in the ring launch for more passes, take
// lam + 8: their 256-element stages hold 512-byte token rows, so a second
// token block costs a whole stage (3 in flight instead of 4), which a rare
// second pass costs less than (Mixtral at T=32, 8 tokens per expert: one
// block, 0.281 -> 0.249 ms per FP8 pass; Qwen2 at T=64 Zipf 0.421 -> 0.397 ms;
// one pass for every token measured 0.342 against 0.308 ms for Qwen2 at T=32).
int ring_tok_blocks(int64_t T, int K, int E, bool whole_pass = true) {
  const int64_t lam = (T * K + E - 1) / E;
  int64_t want = whole_pass ? 2 * lam + 8 : lam + 8;
  if (want > T || (whole_pass && T <= 32)) want = T;
  // four blocks would leave room for only three stages (measured slower than
  // handing the busier experts to the register-streaming kernel)
  return stream_tok_blocks(want < 32 ? want : 32);
}

// Contraction split of the grouped ring launches: only while every expert fits
// one pass (no busy experts handed to the register kernel) and the slabs of
// the experts that can have tokens, min(E, T*K), leave compute units idle.
// The fp32 partial sums, [split][T*K][2I] resp. [split][T*K][H], follow the
// activations in the workspace.
struct GroupedSplit {
  int gu, dn;
  int64_t part_bytes;
};

GroupedSplit grouped_split(int64_t T, int K, int E, int H, int I, int ks, bool whole_pass = true) {
  GroupedSplit g{1, 1, 0};
  const int nb = ring_tok_blocks(T, K, E, whole_pass);
  if (T <= 0 || T > 16 * nb || H % 128 || I % 128) return g;
  const int64_t pairs = T * K;
  const int64_t experts = pairs < E ? pairs : E;
  g.gu = moe::ring_grouped_splits(pairs, experts, H, I, true, ks);
  g.dn = moe::ring_grouped_splits(pairs, experts, H, I, false, ks);
  const int64_t a = g.gu > 1 ? g.gu * pairs * 2 * I * 4 : 0, b = g.dn > 1 ? g.dn * pairs * H * 4 : 0;
  g.part_bytes = a > b ? a : b;
  return g;
}

int64_t grouped_part_offset(int64_t cap, int I) { return round_up(cap * (int64_t)I * 2, 256); }

// The split a grouped call uses: the plan's (at the weights' stage length ks,
// at most the bf16 plan's, which sized the workspace), or none when the
// caller's workspace has no room for the partial sums.
// (A split needs every expert within one pass; the pass of whole_pass = false
// is never longer, so the bf16 sizing of the workspace covers it.)
GroupedSplit grouped_split_for(int64_t T, int K, int E, int H, int I, int ks, int64_t cap,
                               int64_t workspace_bytes, bool whole_pass = true) {
  GroupedSplit g = grouped_split(T, K, E, H, I, 128, whole_pass);
  if (workspace_bytes < grouped_part_offset(cap, I) + g.part_bytes) return GroupedSplit{1, 1, 0};
  if (ks != 128) {
    const GroupedSplit f = grouped_split(T, K, E, H, I, ks, whole_pass);
    g.gu = f.gu < g.gu ? f.gu : g.gu;
    g.dn = f.dn < g.dn ? f.dn : g.dn;
  }
  return g;
}

// Dense FFN plan: workgroups per streaming launch are slabs x splits; the
// contraction is split (deterministically, partial sums added in slice order)
// until about 1024 workgroups exist, keeping at least 2 chunks per wavefront.
struct DensePlan {
  int tok_blocks, split_gu, split_dn;  // streaming schedule
  int tile_block, tile_split;          // tiled schedule: token block and down-projection split
  int tile_split_gu;                   // and gate/up split
  int tile_full_gu, tile_tail_gu;      // gate/up in 128-row tiles: whole tiles, tail split
  bool ring_gu, ring_dn;               // LDS-ring streaming applies to the half
  int ring_split_gu, ring_split_dn;    // and the contraction split it uses
  int64_t act_bytes, part_bytes;
};

int pick_splits(int slabs, int nch) {
  const int target = 1024;
  int s = (target + slabs - 1) / slabs;
  const int most = nch / 8 > 1 ? nch / 8 : 1;
  return s < 1 ? 1 : (s > most ? most : s);
}

// Contraction split of a tiled launch over dense rows: `tiles` output tiles per
// token block, `nb` blocks, contraction kdim, T tokens.  The 512-thread
// workgroups run one per CU, so the grid goes in rounds of 256; split s gives
// each workgroup 1/s of a tile's contraction (at least 8 steps of 64) and adds
// fp32 partial sums (s x T x rows, written, then read by the finish kernel).
// In units of one unsplit tile's time the s in 1..most minimising
//   rounds(s) * (1/s + 3*64/kdim) + [s > 1] * 4*s*T/kdim * tiles/256
// is taken: the first term counts the rounds with the pipeline fill of each
// (three steps), the second prices the partials against the weight bytes the
// full chip streams in one round.  Measured on MI355X: a narrow FFN (the
// shared expert of DeepSeek-V3, I = 2048, at 128 tokens: 16 gate/up tiles)
// runs 2.3x faster split 14 ways, while a split that spills a few workgroups
// into a second round (144 gate/up tiles split in 2) is 5-15% slower.
int tile_splits(int64_t tiles, int64_t nb, int kdim, int64_t T) {
  const int64_t items = tiles * nb;
  if (items <= 0 || kdim <= 0) return 1;
  const int most = kdim / 64 / 8 > 1 ? kdim / 64 / 8 : 1;
  int best = 1;
  double best_cost = 0.0;
  for (int s = 1; s <= most; ++s) {
    const double rounds = (double)((items * s + 255) / 256);
    double c = rounds * (1.0 / s + 192.0 / kdim);
    if (s > 1) c += 4.0 * s * (double)T / kdim * (double)tiles / 256.0;
    if (s == 1 || c < best_cost) {
      best = s;
      best_cost = c;
    }
  }
  return best;
}

// Contraction split of the grouped 256-row tile's down projection (bf16, block
// 64 or 128): the rounds model above over the token blocks the experts hold,
// estimated for even routing with a margin for its spread -- E_act =
// min(E, T*K) experts of lambda + 2 sqrt(lambda) pairs each, lambda = T*K /
// E_act -- with fp32 partial sums per pair (T*K rows) added by the finish
// kernel.  Measured on MI355X (Mixtral-shaped, us): at T=128 (8 experts of
// one 64-token block: 128 down items for 256 CUs) the down projection split
// in 2 runs 177 against 210; the same split of gate/up ran 391 against 344
// (its partial sums are 2I wide) and is not taken; at T=512 an estimate
// without the margin split a down projection whose experts mostly hold two
// blocks (301 against 283).
struct TileSplit {
  int gu, dn;
  int64_t part_bytes;
};

TileSplit grouped_tile_split(int64_t T, int K, int E, int H, int I, int block_m) {
  TileSplit t{1, 1, 0};
  if ((block_m != 64 && block_m != 128) || H % 256 || I % 128 || T <= 0) return t;
  const int64_t pairs = T * K;
  const int64_t eact = pairs < E ? pairs : E;
  const double lambda = (double)pairs / (double)eact;
  const int64_t per = (int64_t)ceil(lambda + 2.0 * sqrt(lambda));
  const int64_t nb = eact * ((per + block_m - 1) / block_m);
  t.dn = tile_splits(H / 256, nb, I, pairs);
  t.part_bytes = t.dn > 1 ? t.dn * pairs * H * 4 : 0;
  return t;
}

// Modelled time of tile_splits' choice s for `tiles` output tiles (one token
// block), in units of one unsplit 256-row tile
double tile_split_cost(int64_t tiles, int s, int kdim, int64_t T) {
  double c = (double)((tiles * s + 255) / 256) * (1.0 / s + 192.0 / kdim);
  if (s > 1) c += 4.0 * s * (double)T / kdim * (double)tiles / 256.0;
  return c;
}

// Gate/up of dense rows in one 128-token block in 128-row tiles (n = I/64 of
// them): the first nfull = 256 floor(n/256) whole, in full rounds of the CUs,
// and the remaining r tiles' contraction split s ways to fill the last round,
// their fp32 partial sums (s x T x 128 columns each) added by the finish
// kernel.  In the units above a 128-row tile weighs 1/2:
//   0.5 [nfull/256 (1 + f) + rounds(r s) (1/s + f)] + [s > 1] 0.5 * 4 s T/H * r/256,
// f = 192/H the pipeline fill; s in 1..H/512.  Taken where it beats the uniform
// split of 256-row tiles.  Measured on MI355X (DeepSeek-V3-shaped DenseFA, 128
// tokens: 288 tiles = 256 whole + 32 split 8 ways, in place of 144 tiles of 256
// rows split 3 ways into 432 workgroups).
struct TailPlan {
  int nfull, s;
  double cost;
};

TailPlan dense_tail_split(int64_t T, int H, int I) {
  TailPlan t{0, 1, 1e30};
  if (T > 128 || I % 64 || H % 64) return t;
  const int64_t n = I / 64;
  const int64_t nfull = n / 256 * 256, r = n - nfull;
  if (nfull == 0 || r == 0) return t;
  const double f = 192.0 / H;
  const int most = H / 64 / 8 > 1 ? H / 64 / 8 : 1;
  for (int s = 1; s <= most; ++s) {
    double c = 0.5 * ((double)nfull / 256 * (1 + f) + (double)((r * s + 255) / 256) * (1.0 / s + f));
    if (s > 1) c += 0.5 * 4.0 * s * (double)T / H * (double)r / 256.0;
    if (c < t.cost) {
      t.nfull = (int)nfull;
      t.s = s;
      t.cost = c;
    }
  }
  return t;
}

DensePlan dense_plan(int64_t T, int H, int I, int dt) {
  DensePlan p;
  p.tok_blocks = stream_tok_blocks(T);
  p.split_gu = pick_splits(I / 32, H / 64);
  p.split_dn = pick_splits(H / 64, I / 64);
  // tiled: 256-token blocks where the 256-row bf16 tile covers both halves and more than
  // 128 rows come (each weight tile then read once per 256 tokens; measured faster than
  // 128-token blocks from 192 rows up); the contraction splits of the down projection
  // (H/256 tiles per block) and of gate/up (I/128 tiles per block) by the rounds model above
  const bool tile2 = dt == MOE_BF16 && I % 128 == 0 && H % 256 == 0;
  p.tile_block = (tile2 && T > 128) ? 256 : 128;
  p.tile_split = 1;
  p.tile_split_gu = 1;
  p.tile_full_gu = 0;
  p.tile_tail_gu = 1;
  if (tile2) {
    const int64_t nb = (T + p.tile_block - 1) / p.tile_block;
    p.tile_split = tile_splits(H / 256, nb, I, T);
    p.tile_split_gu = tile_splits(I / 128, nb, H, T);
    const TailPlan tp = dense_tail_split(T, H, I);
    if (nb == 1 && tp.nfull > 0 && tp.cost < tile_split_cost(I / 128, p.tile_split_gu, H, T)) {
      p.tile_full_gu = tp.nfull;
      p.tile_tail_gu = tp.s;
    }
  }
  p.ring_gu = moe::ring_gate_up_ok(dt, dt, H, I);
  p.ring_dn = moe::ring_down_ok(dt, H, I);
  p.ring_split_gu = p.ring_gu ? moe::ring_gate_up_splits(T, H, I) : 1;
  p.ring_split_dn = p.ring_dn ? moe::ring_down_splits(T, H, I) : 1;
  p.act_bytes = round_up(round_up(T, 128) * (int64_t)I * 2, 256);
  // partial sums of whichever split schedule runs: the largest of them
  const int64_t cand[7] = {p.split_gu > 1 ? (int64_t)p.split_gu * T * 2 * I * 4 : 0,
                           p.split_dn > 1 ? (int64_t)p.split_dn * T * H * 4 : 0,
                           p.tile_split > 1 ? (int64_t)p.tile_split * T * H * 4 : 0,
                           p.tile_split_gu > 1 ? (int64_t)p.tile_split_gu * T * 2 * I * 4 : 0,
                           p.ring_split_gu > 1 ? (int64_t)p.ring_split_gu * T * 2 * I * 4 : 0,
                           p.ring_split_dn > 1 ? (int64_t)p.ring_split_dn * T * H * 4 : 0,
                           p.tile_full_gu > 0 && p.tile_tail_gu > 1
                               ? (int64_t)p.tile_tail_gu * T * 2 * (I - 64 * (int64_t)p.tile_full_gu) * 4
                               : 0};
  p.part_bytes = 0;
  for (int64_t c : cand) p.part_bytes = c > p.part_bytes ? c : p.part_bytes;
  return p;
}

// The tiled schedule needs tiles that hold one expert's rows (block 64 or 128)
// and 128-row output tiles of the down projection (H a multiple of 128).  Auto
// picks it once experts average kTileFrom tokens: measured on MI355X, from
// there one pass of a tile over each weight tile beats the weight-streaming
// schedules, whose passes hold at most 32 (ring) or 64 (register) tokens.
constexpr int kTileFrom = 24;
bool tile_ok(int block_m, int H) { return (block_m == 64 || block_m == 128) && H % 128 == 0; }

// The 512-row gate/up tile once experts average 4 blocks of 128 tokens
// (T*K >= 512*E): measured on MI355X, 12% faster than the 256-row tile for
// Mixtral-shaped experts at 512 tokens each, 6-7% slower at 128-256 tokens
// each (too few workgroups per weight column), even with Qwen2's at 256.
bool wide_gate_up(moe_dtype dt, int64_t T, int K, int E, int block_m, int H, int I) {
  return dt == MOE_BF16 && T * K >= (int64_t)512 * E && moe::tile_wide_ok(block_m, H, I);
}

// The span schedule: bf16, E <= 512, H % 256 == 0, I % 128 == 0 and 32-bit
// offsets into an expert's gate/up matrix, x (T rows) and act (act_rows rows).
bool span_shape_ok(moe_dtype dt, int E, int H, int I, int64_t T, int64_t act_rows) {
  return dt == MOE_BF16 && moe::span_ok(E, H, I, T, act_rows);
}

// AUTO takes the span schedule where its items fill the CUs several times over
// (a span kernel's workgroups each take whole items, a weight tile's whole
// contraction).  With n = ceil(T*K / 256), a lower bound on the spans:
//   gate/up: experts average 256 tokens (T*K >= 256*E) and (I/128) * n >= 768
//            items, three rounds of MI355X's 256 CUs;
//   down:    the same average, (H/256) * n >= 128 and at most one round,
//            (H/256) * (T*K/256 + E) <= 256: its items carry the I-long
//            contraction (3.5x a gate/up item for Mixtral), so a second,
//            mostly idle round of them costs more than the re-reads saved.
// Measured on MI355X (us, tile -> span): Mixtral-shaped T=1024 gate/up 750 ->
// 708, down 439 -> 405; T=2048 gate/up 1130 -> 997 (against the 512-row
// tile), down 631 -> 774 (two rounds: left tiled); Qwen2-shaped T=2048
// gate/up 876 -> 849; T=256 (32 tokens an expert) 398 -> 520; one
// Mixtral-shaped expert at 256 tokens (112 gate/up and 16 down items) 329 ->
// 509 for the pair, hence the item floors.
bool span_auto_gate_up(moe_dtype dt, int64_t T, int K, int E, int H, int I, int64_t cap) {
  const int64_t n = (T * K + 255) / 256;
  return T * K >= (int64_t)256 * E && (int64_t)(I / 128) * n >= 768 &&
         span_shape_ok(dt, E, H, I, T, cap);
}

bool span_auto_down(moe_dtype dt, int64_t T, int K, int E, int H, int I, int64_t cap) {
  const int64_t n = (T * K + 255) / 256;
  return T * K >= (int64_t)256 * E && (int64_t)(H / 256) * n >= 128 &&
         (int64_t)(H / 256) * (T * K / 256 + E) <= 256 && span_shape_ok(dt, E, H, I, T, cap);
}

moe_status span_unsupported(const char* what) {
  return fail(MOE_EUNSUPPORTED, "%s: span schedule needs bf16, E <= 512, H %% 256 == 0, "
              "I %% 128 == 0 and an expert's gate/up matrix, x and the activations each "
              "below 4 GB", what);
}

moe_status pick_schedule(moe_schedule req, int64_t T, int K, int E, int block_m, int H,
                         moe_schedule* out) {
  if (req == MOE_SCHED_TILE) {
    if (!tile_ok(block_m, H))
      return fail(MOE_EUNSUPPORTED, "tile schedule needs block_m 64 or 128 and H %% 128 == 0 "
                  "(block_m = %d, H = %d)", block_m, H);
    *out = MOE_SCHED_TILE;
  } else if (req == MOE_SCHED_STREAM || req == MOE_SCHED_RING || req == MOE_SCHED_SPAN) {
    *out = req;
  } else if (req == MOE_SCHED_AUTO) {
    // (T <= 32: every expert fits one streaming pass, which beats a tile)
    *out = (tile_ok(block_m, H) && T * K >= kTileFrom * (int64_t)E && T > 32) ? MOE_SCHED_TILE
                                                                     : MOE_SCHED_STREAM;
  } else {
    return fail(MOE_EINVAL, "schedule %d", (int)req);
  }
  return MOE_OK;
}

// The streaming schedules of one half: an explicit RING request needs a shape
// the ring kernel takes (ring_ok); AUTO upgrades STREAM to RING where it also
// expects it to be faster (auto_ok).
moe_status pick_stream(moe_schedule req, bool ring_ok, bool auto_ok, const char* what,
                       moe_schedule* use) {
  if (*use == MOE_SCHED_RING && !ring_ok)
    return fail(MOE_EUNSUPPORTED, "%s: ring schedule needs bf16, H %% 128 == 0 and "
                "I %% 64 == 0 (gate/up) or I %% 128 == 0 (down)", what);
  if (*use == MOE_SCHED_STREAM && req == MOE_SCHED_AUTO && ring_ok && auto_ok)
    *use = MOE_SCHED_RING;
  return MOE_OK;
}

}  // namespace

namespace moe {

int set_last_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

}  // namespace moe

extern "C" {

const char* moe_last_error(void) { return g_err; }

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ECAPACITY: return "capacity or workspace too small";
    case MOE_EHIP: return "HIP launch failed";
  }
  return "unknown status";
}

int64_t moe_align_capacity(int64_t T, int K, int E, int block_m) {
  if (T < 0 || K < 1 || E < 1 || block_m < 1) return -1;
  const int64_t TK = T * K;
  const int64_t active = TK < E ? TK : E;
  return round_up(TK + active * (block_m - 1), block_m);
}

int64_t moe_align_capacity_ex(int64_t T, int K, int E, int block_m, moe_padding pad) {
  if (pad == MOE_PAD_BLOCK) return moe_align_capacity(T, K, E, block_m);
  if (pad != MOE_PAD_MAX || T < 0 || K < 1 || E < 1 || block_m < 1) return -1;
  return (int64_t)E * round_up(T, block_m);
}

int64_t moe_ffn_workspace_bytes(int64_t cap, int I) {
  if (cap < 0 || I < 0) return -1;
  return cap * (int64_t)I * 2;
}

int64_t moe_ffn_workspace_bytes_ex(int64_t cap, int64_t T, int K, int E, int H, int I) {
  if (cap < 0 || T < 0 || K < 1 || E < 1 || H < 1 || I < 1) return -1;
  const GroupedSplit g = grouped_split(T, K, E, H, I, 128);
  int64_t part = g.part_bytes;
  // the tiled down projection's split where AUTO tiles (at either block the
  // tiles take); a call with a smaller workspace runs unsplit
  if (T > 32 && T * K >= kTileFrom * (int64_t)E) {
    for (int b : {64, 128}) {
      const TileSplit t = grouped_tile_split(T, K, E, H, I, b);
      part = t.part_bytes > part ? t.part_bytes : part;
    }
  }
  return grouped_part_offset(cap, I) + part;
}

int64_t dense_ffn_workspace_bytes(int64_t T, int H, int I_fa) {
  if (T < 0 || H < 64 || I_fa < 64 || H % 64 || I_fa % 64) return -1;
  // sized for the larger of the two storage dtypes' plans
  const DensePlan a = dense_plan(T, H, I_fa, MOE_BF16), b = dense_plan(T, H, I_fa, MOE_F32);
  const int64_t pa = a.act_bytes + a.part_bytes, pb = b.act_bytes + b.part_bytes;
  return pa > pb ? pa : pb;
}

moe_status moe_route(const float* logits, int64_t T, int E, int K, int32_t* topk_ids,
                     float* topk_w, void* stream) {
  moe_status st = check_route_shape(T, E, K);
  if (st) return st;
  if (T == 0) return ok();
  if (!logits || !topk_ids || !topk_w || !aligned(logits, 4) || !aligned(topk_ids, 4) ||
      !aligned(topk_w, 4))
    return fail(MOE_EINVAL, "moe_route: NULL or misaligned pointer");
  return hip_status(moe::launch_route(logits, T, E, K, nullptr, topk_ids, topk_w,
                                     (hipStream_t)stream),
                    "moe_route");
}

moe_status moe_route_var(const float* logits, int64_t T, int E, int Kmax, const int32_t* k_tok,
                         int32_t* topk_ids, float* topk_w, void* stream) {
  moe_status st = check_route_shape(T, E, Kmax);
  if (st) return st;
  if (T == 0) return ok();
  if (!logits || !k_tok || !topk_ids || !topk_w || !aligned(logits, 4) || !aligned(k_tok, 4) ||
      !aligned(topk_ids, 4) || !aligned(topk_w, 4))
    return fail(MOE_EINVAL, "moe_route_var: NULL or misaligned pointer");
  return hip_status(moe::launch_route(logits, T, E, Kmax, k_tok, topk_ids, topk_w,
                                     (hipStream_t)stream),
                    "moe_route_var");
}

moe_status moe_align_ex(const int32_t* topk_ids, int64_t T, int K, int E, const moe_plan* plan,
                        moe_padding pad, void* stream) {
  moe_status st = check_route_shape(T, E, K);
  if (st) return st;
  if (pad != MOE_PAD_BLOCK && pad != MOE_PAD_MAX)
    return fail(MOE_EINVAL, "moe_align_ex: padding scheme %d", (int)pad);
  if (T > 0 && (!topk_ids || !aligned(topk_ids, 4)))
    return fail(MOE_EINVAL, "moe_align: topk_ids NULL or misaligned");
  st = check_plan(plan, T, K, E, pad);
  if (st) return st;
  return hip_status(moe::launch_align(topk_ids, T, K, E, plan->block_m, plan->cap,
                                      pad == MOE_PAD_MAX ? 1 : 0, plan->expert_counts,
                                      plan->expert_offsets, plan->sorted_ids, plan->block_expert,
                                      plan->inv_pos, (hipStream_t)stream),
                    "moe_align");
}

moe_status moe_align(const int32_t* topk_ids, int64_t T, int K, int E, const moe_plan* plan,
                     void* stream) {
  return moe_align_ex(topk_ids, T, K, E, plan, MOE_PAD_BLOCK, stream);
}

moe_status moe_route_align(const float* logits, int64_t T, int E, int K, const int32_t* k_tok,
                           int32_t* topk_ids, float* topk_w, const moe_plan* plan,
                           moe_padding pad, void* stream) {
  moe_status st = check_route_shape(T, E, K);
  if (st) return st;
  if (pad != MOE_PAD_BLOCK && pad != MOE_PAD_MAX)
    return fail(MOE_EINVAL, "moe_route_align: padding scheme %d", (int)pad);
  if (T > 0 && (!logits || !topk_ids || !topk_w || !aligned(logits, 4) || !aligned(topk_ids, 4) ||
                !aligned(topk_w, 4) || (k_tok && !aligned(k_tok, 4))))
    return fail(MOE_EINVAL, "moe_route_align: NULL or misaligned pointer");
  st = check_plan(plan, T, K, E, pad);
  if (st) return st;
  if (T == 0)   // the plan of an empty batch: the alignment alone
    return moe_align_ex(topk_ids, T, K, E, plan, pad, stream);
  return hip_status(moe::launch_route_align(logits, T, E, K, k_tok, topk_ids, topk_w,
                                            plan->block_m, plan->cap, pad == MOE_PAD_MAX ? 1 : 0,
                                            plan->expert_counts, plan->expert_offsets,
                                            plan->sorted_ids, plan->block_expert, plan->inv_pos,
                                            (hipStream_t)stream),
                    "moe_route_align");
}

static moe_status check_grouped(const void* x, moe_dtype dt, int64_t T, int H, int I, int E, int K,
                                const moe_plan* plan, int64_t workspace_bytes) {
  moe_status st = check_route_shape(T, E, K);
  if (st) return st;
  if (!valid_dtype(dt)) return fail(MOE_EUNSUPPORTED, "dtype %d", (int)dt);
  st = check_ffn_dims(H, I);
  if (st) return st;
  st = check_plan(plan, T, K, E);
  if (st) return st;
  if (workspace_bytes < moe_ffn_workspace_bytes(plan->cap, I))
    return fail(MOE_ECAPACITY, "workspace %lld bytes < %lld required", (long long)workspace_bytes,
                (long long)moe_ffn_workspace_bytes(plan->cap, I));
  (void)x;
  return MOE_OK;
}

// The grouped tile's split for this call: bf16 only, and none when the
// caller's workspace has no room for the partial sums.
static TileSplit grouped_tile_split_for(moe_dtype dt, int64_t T, int K, int E, int H, int I,
                                        const moe_plan* plan, int64_t workspace_bytes) {
  TileSplit t = grouped_tile_split(T, K, E, H, I, plan->block_m);
  if (dt != MOE_BF16 || workspace_bytes < grouped_part_offset(plan->cap, I) + t.part_bytes)
    return TileSplit{1, 1, 0};
  return t;
}

static moe::RowMap grouped_rows(const moe_plan* plan, int K) {
  moe::RowMap rm;
  rm.counts = plan->expert_counts;
  rm.offsets = plan->expert_offsets;
  rm.sorted_ids = plan->sorted_ids;
  rm.block_expert = plan->block_expert;
  rm.K = K;
  rm.dense_rows = 0;
  rm.inv_pos = plan->inv_pos;
  rm.block_m = plan->block_m;
  rm.min_rows = 1;
  rm.max_rows = INT32_MAX;
  return rm;
}

moe_status moe_grouped_gate_up(const void* x, moe_dtype dt, int64_t T, int H, int I, int E, int K,
                               const void* w13, const moe_plan* plan, void* workspace,
                               int64_t workspace_bytes, moe_schedule sched, void* stream) {
  moe_status st = check_grouped(x, dt, T, H, I, E, K, plan, workspace_bytes);
  if (st) return st;
  if (T == 0) return ok();
  if (!x || !w13 || !workspace || !aligned(x, 16) || !aligned(w13, 16) || !aligned(workspace, 16))
    return fail(MOE_EINVAL, "moe_grouped_gate_up: NULL or misaligned pointer");
  moe_schedule use;
  st = pick_schedule(sched, T, K, E, plan->block_m, H, &use);
  if (st) return st;
  const bool ring = moe::ring_gate_up_ok(dt, dt, H, I);
  st = pick_stream(sched, ring, ring, "moe_grouped_gate_up", &use);
  if (st) return st;
  if (sched == MOE_SCHED_AUTO && use == MOE_SCHED_TILE &&
      span_auto_gate_up(dt, T, K, E, H, I, plan->cap))
    use = MOE_SCHED_SPAN;
  // automatic below kTileFrom tokens per expert: experts that fit a ring pass
  // are streamed, busier ones tiled where the plan's block allows (two regimes
  // per expert, TEMPO page).  From kTileFrom on every expert is tiled: two
  // launches that each leave part of the GPU idle measured slower.
  const bool hot_tiled = sched == MOE_SCHED_AUTO && tile_ok(plan->block_m, H);
  const moe::RowMap rm = grouped_rows(plan, K);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (use == MOE_SCHED_SPAN) {
    if (!span_shape_ok(dt, E, H, I, T, plan->cap)) return span_unsupported("moe_grouped_gate_up");
    e = moe::launch_span_gate_up(x, w13, rm, E, H, I, T, T * K, (uint16_t*)workspace, s);
  } else if (use == MOE_SCHED_TILE && wide_gate_up(dt, T, K, E, plan->block_m, H, I))
    e = moe::launch_tile_gate_up_wide(x, w13, rm, plan->cap / plan->block_m, H, I,
                                      (uint16_t*)workspace, s);
  else if (use == MOE_SCHED_TILE) {
    const TileSplit ts = grouped_tile_split_for(dt, T, K, E, H, I, plan, workspace_bytes);
    float* part = (float*)((char*)workspace + grouped_part_offset(plan->cap, I));
    e = moe::launch_tile_gate_up(x, dt, w13, rm, plan->cap / plan->block_m, H, I,
                                 (uint16_t*)workspace, s, ts.gu, part, T * K);
  }
  else if (use == MOE_SCHED_RING) {
    // experts whose tokens fit one ring pass go to the ring kernel, busier ones
    // (possible only when T exceeds a pass) to the register-streaming kernel
    const int nb = ring_tok_blocks(T, K, E);
    moe::RowMap cold = rm, hot = rm;
    cold.max_rows = 16 * nb;
    hot.min_rows = 16 * nb + 1;
    const GroupedSplit g = grouped_split_for(T, K, E, H, I, 128, plan->cap, workspace_bytes);
    float* part = (float*)((char*)workspace + grouped_part_offset(plan->cap, I));
    e = moe::launch_ring_gate_up(x, dt, w13, nullptr, cold, E, H, I, T, nb, g.gu,
                                 (uint16_t*)workspace, part, s);
    if (e == hipSuccess && T > 16 * nb)
      e = hot_tiled ? moe::launch_tile_gate_up(x, dt, w13, hot, plan->cap / plan->block_m, H, I,
                                               (uint16_t*)workspace, s)
                    : moe::launch_stream_gate_up(x, dt, w13, hot, E, H, I, stream_tok_blocks(T), 1,
                                                 (uint16_t*)workspace, nullptr, s);
  }
  else
    e = moe::launch_stream_gate_up(x, dt, w13, rm, E, H, I, stream_tok_blocks(T), 1,
                                   (uint16_t*)workspace, nullptr, s);
  return hip_status(e, "moe_grouped_gate_up");
}

moe_status moe_grouped_down(const void* w2, moe_dtype dt, int64_t T, int H, int I, int E, int K,
                            const moe_plan* plan, void* workspace, int64_t workspace_bytes,
                            void* y_pairs, moe_schedule sched, void* stream) {
  moe_status st = check_grouped(w2, dt, T, H, I, E, K, plan, workspace_bytes);
  if (st) return st;
  if (T == 0) return ok();
  if (!w2 || !workspace || !y_pairs || !aligned(w2, 16) || !aligned(workspace, 16) ||
      !aligned(y_pairs, 16))
    return fail(MOE_EINVAL, "moe_grouped_down: NULL or misaligned pointer");
  moe_schedule use;
  st = pick_schedule(sched, T, K, E, plan->block_m, H, &use);
  if (st) return st;
  const bool ring = moe::ring_down_ok(dt, H, I);
  st = pick_stream(sched, ring, ring, "moe_grouped_down", &use);
  if (st) return st;
  if (sched == MOE_SCHED_AUTO && use == MOE_SCHED_TILE &&
      span_auto_down(dt, T, K, E, H, I, plan->cap))
    use = MOE_SCHED_SPAN;
  const bool hot_tiled = sched == MOE_SCHED_AUTO && tile_ok(plan->block_m, H);
  const moe::RowMap rm = grouped_rows(plan, K);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (use == MOE_SCHED_SPAN) {
    if (!span_shape_ok(dt, E, H, I, T, plan->cap)) return span_unsupported("moe_grouped_down");
    e = moe::launch_span_down(w2, (const uint16_t*)workspace, rm, E, H, I, plan->cap, T * K,
                              y_pairs, dt, s);
  } else if (use == MOE_SCHED_TILE) {
    const TileSplit ts = grouped_tile_split_for(dt, T, K, E, H, I, plan, workspace_bytes);
    float* part = (float*)((char*)workspace + grouped_part_offset(plan->cap, I));
    e = moe::launch_tile_down(w2, dt, (const uint16_t*)workspace, rm, plan->cap / plan->block_m,
                              H, I, y_pairs, dt, ts.dn, part, s, T * K);
  }
  else if (use == MOE_SCHED_RING) {
    const int nb = ring_tok_blocks(T, K, E);
    moe::RowMap cold = rm, hot = rm;
    cold.max_rows = 16 * nb;
    hot.min_rows = 16 * nb + 1;
    const GroupedSplit g = grouped_split_for(T, K, E, H, I, 128, plan->cap, workspace_bytes);
    float* part = (float*)((char*)workspace + grouped_part_offset(plan->cap, I));
    e = moe::launch_ring_down(w2, dt, nullptr, (const uint16_t*)workspace, cold, E, H, I, T, nb,
                              g.dn, y_pairs, dt, part, s);
    if (e == hipSuccess && T > 16 * nb)
      e = hot_tiled ? moe::launch_tile_down(w2, dt, (const uint16_t*)workspace, hot,
                                            plan->cap / plan->block_m, H, I, y_pairs, dt, 1,
                                            nullptr, s)
                    : moe::launch_stream_down(w2, dt, (const uint16_t*)workspace, hot, E, H, I,
                                              stream_tok_blocks(T), 1, y_pairs, dt, nullptr, s);
  }
  else
    e = moe::launch_stream_down(w2, dt, (const uint16_t*)workspace, rm, E, H, I,
                                stream_tok_blocks(T), 1, y_pairs, dt, nullptr, s);
  return hip_status(e, "moe_grouped_down");
}

moe_status moe_grouped_ffn(const void* x, moe_dtype dt, int64_t T, int H, int I, int E, int K,
                           const void* w13, const void* w2, const moe_plan* plan, void* workspace,
                           int64_t workspace_bytes, void* y_pairs, void* stream) {
  moe_status st = moe_grouped_gate_up(x, dt, T, H, I, E, K, w13, plan, workspace, workspace_bytes,
                                      MOE_SCHED_AUTO, stream);
  if (st) return st;
  return moe_grouped_down(w2, dt, T, H, I, E, K, plan, workspace, workspace_bytes, y_pairs,
                          MOE_SCHED_AUTO, stream);
}

moe_status moe_combine(const void* y_pairs, moe_dtype ydt, const float* topk_w, const void* shared,
                       moe_dtype sdt, int64_t T, int K, int H, void* out, moe_dtype odt,
                       void* stream) {
  if (T < 0 || K < 1) return fail(MOE_EINVAL, "moe_combine: T = %lld, K = %d", (long long)T, K);
  if (!valid_dtype(ydt) || !valid_dtype(sdt) || !valid_dtype(odt))
    return fail(MOE_EUNSUPPORTED, "moe_combine: dtype");
  if (H < 8 || H % 8 != 0) return fail(MOE_EUNSUPPORTED, "moe_combine: H = %d must be a multiple of 8", H);
  if (T * K >= (int64_t)1 << 31) return fail(MOE_EUNSUPPORTED, "T*K must be < 2^31");
  if (T == 0) return ok();
  if (!y_pairs || !topk_w || !out || !aligned(y_pairs, 16) || !aligned(topk_w, 4) ||
      !aligned(out, 16) || (shared && !aligned(shared, 16)))
    return fail(MOE_EINVAL, "moe_combine: NULL or misaligned pointer");
  return hip_status(moe::launch_combine(y_pairs, ydt, topk_w, shared, sdt, T, K, H, out, odt,
                                        (hipStream_t)stream),
                    "moe_combine");
}

moe_status dense_ffn_fa(const void* x, moe_dtype dt, int64_t T, int H, int I_fa, const void* w13,
                        const void* w2, void* workspace, int64_t workspace_bytes, void* out,
                        moe_dtype odt, moe_schedule sched, void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "dense_ffn_fa: T < 0");
  if (T >= (int64_t)1 << 31) return fail(MOE_EUNSUPPORTED, "dense_ffn_fa: T must be < 2^31");
  if (!valid_dtype(dt) || !valid_dtype(odt)) return fail(MOE_EUNSUPPORTED, "dense_ffn_fa: dtype");
  moe_status st = check_ffn_dims(H, I_fa);
  if (st) return st;
  if (workspace_bytes < dense_ffn_workspace_bytes(T, H, I_fa))
    return fail(MOE_ECAPACITY, "dense_ffn_fa: workspace %lld bytes < %lld required",
                (long long)workspace_bytes, (long long)dense_ffn_workspace_bytes(T, H, I_fa));
  if (T == 0) return ok();
  if (!x || !w13 || !w2 || !workspace || !out || !aligned(x, 16) || !aligned(w13, 16) ||
      !aligned(w2, 16) || !aligned(workspace, 16) || !aligned(out, 16))
    return fail(MOE_EINVAL, "dense_ffn_fa: NULL or misaligned pointer");
  moe::RowMap rm;
  memset(&rm, 0, sizeof rm);
  rm.K = 1;
  rm.dense_rows = T;
  rm.block_m = 128;
  rm.min_rows = 1;
  rm.max_rows = INT32_MAX;
  hipStream_t s = (hipStream_t)stream;
  // dense rows form one expert; auto: the LDS ring up to 32 rows (one pass of
  // two token blocks), the tiled schedule above (measured: from 48 rows it
  // reads the weights once where the streaming passes would read them twice)
  moe_schedule use;
  st = pick_schedule(sched, T, 1, 1, 128, H, &use);
  if (st) return st;
  const DensePlan dp = dense_plan(T, H, I_fa, dt);
  if (sched == MOE_SCHED_AUTO)
    use = (T <= 32 || !tile_ok(128, H)) ? MOE_SCHED_STREAM : MOE_SCHED_TILE;
  if (use == MOE_SCHED_SPAN) {
    if (!span_shape_ok(dt, 1, H, I_fa, T, T)) return span_unsupported("dense_ffn_fa");
    uint16_t* act = (uint16_t*)workspace;
    hipError_t e = moe::launch_span_gate_up(x, w13, rm, 1, H, I_fa, T, T, act, s);
    if (e != hipSuccess) return hip_status(e, "dense_ffn_fa gate/up");
    e = moe::launch_span_down(w2, act, rm, 1, H, I_fa, T, T, out, odt, s);
    return hip_status(e, "dense_ffn_fa down");
  }
  if (use == MOE_SCHED_TILE) {
    uint16_t* act = (uint16_t*)workspace;
    float* part = (float*)((char*)workspace + dp.act_bytes);
    rm.block_m = dp.tile_block;
    const int64_t nblocks = (T + rm.block_m - 1) / rm.block_m;
    // AUTO: the gate/up half on the span schedule where its (I/128) x ceil(T/256)
    // items fill the CUs 1.5 times over, the down half tiled (its H/256 tiles a
    // span are too few items).  Measured on MI355X (us, tiled -> span gate/up):
    // DenseFA Mixtral-shaped at T=512 (448 items) 417-418 -> 380-385, T=1024
    // 778-788 -> 721-726, T=2048 1359-1369 -> 1248-1254, T=4096 2635-2645 ->
    // 2472-2480; Qwen2's shared experts at T=2048 915-934 -> 841-846.  The span
    // writes act rows 0..T-1; the tiles' rows past T feed only outputs that are
    // never stored.
    const bool span_gu = sched == MOE_SCHED_AUTO && span_shape_ok(dt, 1, H, I_fa, T, T) &&
                         (int64_t)(I_fa / 128) * ((T + 255) / 256) >= 384;
    hipError_t e = span_gu ? moe::launch_span_gate_up(x, w13, rm, 1, H, I_fa, T, T, act, s)
                 : dp.tile_full_gu > 0
                       ? moe::launch_tile_gate_up(x, dt, w13, rm, nblocks, H, I_fa, act, s,
                                                  dp.tile_tail_gu, part, 0, dp.tile_full_gu)
                       : moe::launch_tile_gate_up(x, dt, w13, rm, nblocks, H, I_fa, act, s,
                                                  dp.tile_split_gu, part);
    if (e != hipSuccess) return hip_status(e, "dense_ffn_fa gate/up");
    e = moe::launch_tile_down(w2, dt, act, rm, nblocks, H, I_fa, out, odt, dp.tile_split, part, s);
    return hip_status(e, "dense_ffn_fa down");
  }
  moe_schedule use_gu = use, use_dn = use;
  // (AUTO: the ring kernel while a pass of at most 32 rows covers every token;
  // past that its four-block layout is the slower one)
  st = pick_stream(sched, dp.ring_gu, T <= 32, "dense_ffn_fa gate/up", &use_gu);
  if (st) return st;
  st = pick_stream(sched, dp.ring_dn, T <= 32, "dense_ffn_fa down", &use_dn);
  if (st) return st;
  uint16_t* act = (uint16_t*)workspace;
  float* part = (float*)((char*)workspace + dp.act_bytes);
  hipError_t e =
      use_gu == MOE_SCHED_RING
          ? moe::launch_ring_gate_up(x, dt, w13, nullptr, rm, 1, H, I_fa, T, dp.tok_blocks,
                                     dp.ring_split_gu, act, part, s)
          : moe::launch_stream_gate_up(x, dt, w13, rm, 1, H, I_fa, dp.tok_blocks, dp.split_gu, act,
                                       part, s);
  if (e != hipSuccess) return hip_status(e, "dense_ffn_fa gate/up");
  e = use_dn == MOE_SCHED_RING
          ? moe::launch_ring_down(w2, dt, nullptr, act, rm, 1, H, I_fa, T, dp.tok_blocks,
                                  dp.ring_split_dn, out, odt, part, s)
          : moe::launch_stream_down(w2, dt, act, rm, 1, H, I_fa, dp.tok_blocks, dp.split_dn, out,
                                    odt, part, s);
  return hip_status(e, "dense_ffn_fa down");
}

// FP8 ring passes of one token block leave experts with more than 16 tokens
// to several passes, each streaming the expert's weights again; past 64 tokens
// those experts go to a second ring launch of two-block passes instead
// (measured on MI355X: DeepSeek-V3 at T=128 with Zipf routing 0.842 -> 0.783
// ms; at 32-64 tokens the second launch cost as much as it saved, or more).
bool fp8_hot_pass(int64_t T, int nb) { return nb == 1 && T > 64; }

// FP8 experts are tiled once they average kTileFrom tokens (as the bf16
// automatic schedule does) and the shape allows; below that every expert
// streams through the ring, the busier ones in several passes (measured on
// MI355X: cheaper than a second tiled launch for them, whose workgroups for
// the other experts' blocks still have to start and exit)
bool fp8_tiled(int64_t T, int K, int E, int H, int I, int block_m) {
  return T > 32 && T * K >= kTileFrom * (int64_t)E && moe::tile_fp8_ok(H, I, block_m) &&
         block_m <= 128;
}

static moe_status check_fp8_weights(const void* w, const float* scale, int H, int I,
                                    const char* what) {
  if (H % 128 != 0 || I % 128 != 0)
    return fail(MOE_EUNSUPPORTED, "%s: FP8 weights need H %% 128 == 0 and I %% 128 == 0 "
                "(H = %d, I = %d)", what, H, I);
  if (!w || !aligned(w, 16) || !scale || !aligned(scale, 4))
    return fail(MOE_EINVAL, "%s: NULL or misaligned weights or scales", what);
  return MOE_OK;
}

moe_status moe_grouped_gate_up_fp8(const void* x, int64_t T, int H, int I, int E, int K,
                                   const uint8_t* w13, const float* w13_scale,
                                   const moe_plan* plan, void* workspace, int64_t workspace_bytes,
                                   void* stream) {
  moe_status st = check_grouped(x, MOE_BF16, T, H, I, E, K, plan, workspace_bytes);
  if (st) return st;
  st = check_fp8_weights(w13, w13_scale, H, I, "moe_grouped_gate_up_fp8");
  if (st) return st;
  if (T == 0) return ok();
  if (!x || !workspace || !aligned(x, 16) || !aligned(workspace, 16))
    return fail(MOE_EINVAL, "moe_grouped_gate_up_fp8: NULL or misaligned pointer");
  const moe::RowMap rm = grouped_rows(plan, K);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (fp8_tiled(T, K, E, H, I, plan->block_m)) {
    e = moe::launch_tile_gate_up_fp8(x, w13, w13_scale, rm, plan->cap / plan->block_m, H, I,
                                     (uint16_t*)workspace, s);
  } else {
    const int nb = ring_tok_blocks(T, K, E, false);
    const GroupedSplit g = grouped_split_for(T, K, E, H, I,
                                             moe::ring_stage_k(moe::kDtFP8, nb, H), plan->cap,
                                             workspace_bytes, false);
    float* part = (float*)((char*)workspace + grouped_part_offset(plan->cap, I));
    if (fp8_hot_pass(T, nb)) {
      moe::RowMap cold = rm, hot = rm;
      cold.max_rows = 16;
      hot.min_rows = 17;
      e = moe::launch_ring_gate_up(x, moe::kDtFP8, w13, w13_scale, cold, E, H, I, T, 1, 1,
                                   (uint16_t*)workspace, part, s);
      if (e == hipSuccess)
        e = moe::launch_ring_gate_up(x, moe::kDtFP8, w13, w13_scale, hot, E, H, I, T, 2, 1,
                                     (uint16_t*)workspace, part, s);
    } else {
      e = moe::launch_ring_gate_up(x, moe::kDtFP8, w13, w13_scale, rm, E, H, I, T, nb, g.gu,
                                   (uint16_t*)workspace, part, s);
    }
  }
  return hip_status(e, "moe_grouped_gate_up_fp8");
}

moe_status moe_grouped_down_fp8(const uint8_t* w2, const float* w2_scale, int64_t T, int H, int I,
                                int E, int K, const moe_plan* plan, void* workspace,
                                int64_t workspace_bytes, void* y_pairs, void* stream) {
  moe_status st = check_grouped(w2, MOE_BF16, T, H, I, E, K, plan, workspace_bytes);
  if (st) return st;
  st = check_fp8_weights(w2, w2_scale, H, I, "moe_grouped_down_fp8");
  if (st) return st;
  if (T == 0) return ok();
  if (!workspace || !y_pairs || !aligned(workspace, 16) || !aligned(y_pairs, 16))
    return fail(MOE_EINVAL, "moe_grouped_down_fp8: NULL or misaligned pointer");
  const moe::RowMap rm = grouped_rows(plan, K);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (fp8_tiled(T, K, E, H, I, plan->block_m)) {
    e = moe::launch_tile_down_fp8(w2, w2_scale, (const uint16_t*)workspace, rm,
                                  plan->cap / plan->block_m, H, I, y_pairs, moe::kDtBF16, 1,
                                  nullptr, s);
  } else {
    const int nb = ring_tok_blocks(T, K, E, false);
    const GroupedSplit g = grouped_split_for(T, K, E, H, I,
                                             moe::ring_stage_k(moe::kDtFP8, nb, I), plan->cap,
                                             workspace_bytes, false);
    float* part = (float*)((char*)workspace + grouped_part_offset(plan->cap, I));
    if (fp8_hot_pass(T, nb)) {
      moe::RowMap cold = rm, hot = rm;
      cold.max_rows = 16;
      hot.min_rows = 17;
      e = moe::launch_ring_down(w2, moe::kDtFP8, w2_scale, (const uint16_t*)workspace, cold, E, H,
                                I, T, 1, 1, y_pairs, moe::kDtBF16, part, s);
      if (e == hipSuccess)
        e = moe::launch_ring_down(w2, moe::kDtFP8, w2_scale, (const uint16_t*)workspace, hot, E,
                                  H, I, T, 2, 1, y_pairs, moe::kDtBF16, part, s);
    } else {
      e = moe::launch_ring_down(w2, moe::kDtFP8, w2_scale, (const uint16_t*)workspace, rm, E, H,
                                I, T, nb, g.dn, y_pairs, moe::kDtBF16, part, s);
    }
  }
  return hip_status(e, "moe_grouped_down_fp8");
}

moe_status dense_ffn_fp8(const void* x, int64_t T, int H, int I, const uint8_t* w13,
                         const float* w13_scale, const uint8_t* w2, const float* w2_scale,
                         void* workspace, int64_t workspace_bytes, void* out, moe_dtype odt,
                         void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "dense_ffn_fp8: T < 0");
  if (T >= (int64_t)1 << 31) return fail(MOE_EUNSUPPORTED, "dense_ffn_fp8: T must be < 2^31");
  if (!valid_dtype(odt)) return fail(MOE_EUNSUPPORTED, "dense_ffn_fp8: dtype");
  moe_status st = check_ffn_dims(H, I);
  if (st) return st;
  st = check_fp8_weights(w13, w13_scale, H, I, "dense_ffn_fp8");
  if (st) return st;
  st = check_fp8_weights(w2, w2_scale, H, I, "dense_ffn_fp8");
  if (st) return st;
  if (workspace_bytes < dense_ffn_workspace_bytes(T, H, I))
    return fail(MOE_ECAPACITY, "dense_ffn_fp8: workspace %lld bytes < %lld required",
                (long long)workspace_bytes, (long long)dense_ffn_workspace_bytes(T, H, I));
  if (T == 0) return ok();
  if (!x || !workspace || !out || !aligned(x, 16) || !aligned(workspace, 16) || !aligned(out, 16))
    return fail(MOE_EINVAL, "dense_ffn_fp8: NULL or misaligned pointer");
  moe::RowMap rm;
  memset(&rm, 0, sizeof rm);
  rm.K = 1;
  rm.dense_rows = T;
  rm.block_m = 128;
  rm.min_rows = 1;
  rm.max_rows = INT32_MAX;
  const DensePlan dp = dense_plan(T, H, I, MOE_BF16);
  hipStream_t s = (hipStream_t)stream;
  if (T > 32 && moe::tile_fp8_ok(H, I, dp.tile_block)) {
    // past one streaming pass: the tiled schedule reads each weight tile once
    // per token block (the streaming passes would read all weights again)
    uint16_t* act = (uint16_t*)workspace;
    float* part = (float*)((char*)workspace + dp.act_bytes);
    rm.block_m = dp.tile_block;
    const int64_t nblocks = (T + rm.block_m - 1) / rm.block_m;
    hipError_t e = moe::launch_tile_gate_up_fp8(x, w13, w13_scale, rm, nblocks, H, I, act, s,
                                                dp.tile_split_gu, part);
    if (e != hipSuccess) return hip_status(e, "dense_ffn_fp8 gate/up");
    e = moe::launch_tile_down_fp8(w2, w2_scale, act, rm, nblocks, H, I, out, odt, dp.tile_split,
                                  part, s);
    return hip_status(e, "dense_ffn_fp8 down");
  }
  // contraction splits at the FP8 stage length, within the bf16 plan's (which
  // sized the workspace's partial sums)
  const int ks_gu = moe::ring_stage_k(moe::kDtFP8, dp.tok_blocks, H);
  const int ks_dn = moe::ring_stage_k(moe::kDtFP8, dp.tok_blocks, I);
  int split_gu = moe::ring_gate_up_splits(T, H, I, ks_gu);
  int split_dn = moe::ring_down_splits(T, H, I, ks_dn);
  split_gu = split_gu < dp.ring_split_gu ? split_gu : dp.ring_split_gu;
  split_dn = split_dn < dp.ring_split_dn ? split_dn : dp.ring_split_dn;
  uint16_t* act = (uint16_t*)workspace;
  float* part = (float*)((char*)workspace + dp.act_bytes);
  hipError_t e = moe::launch_ring_gate_up(x, moe::kDtFP8, w13, w13_scale, rm, 1, H, I, T,
                                          dp.tok_blocks, split_gu, act, part, s);
  if (e != hipSuccess) return hip_status(e, "dense_ffn_fp8 gate/up");
  e = moe::launch_ring_down(w2, moe::kDtFP8, w2_scale, act, rm, 1, H, I, T, dp.tok_blocks,
                            split_dn, out, odt, part, s);
  return hip_status(e, "dense_ffn_fp8 down");
}

}  // extern "C"
