"""One MoE feed-forward layer pass on the GPU, as five library calls.

Buffers are allocated once, when the runner is built; a pass then only
enqueues the library's kernels on the current stream:

  moe_route -> moe_align -> moe_grouped_gate_up -> moe_grouped_down -> moe_combine

with the shared experts (one dense_ffn_fa call, which needs no routing) on a
second stream of the runner's, forked from the current stream at the start of
the pass and joined before the combine.  Both halves are bound by HBM
bandwidth; running them side by side fills the other half's ramp-up and tail
(measured on MI355X: Qwen2-shaped layer at 1 / 32 / 256 / 2048 tokens 4-9%
faster, results bit-identical).

The DenseFA baseline is one dense_ffn_fa call (DensePA, the dense FFN
with the MoE's parameter count, another one of width E*I + I_s).  The tax of
the Serving-tax notes (section "定義", Eq. 1) is tau = T(MoE, b) / T(DenseFA, b).
"""
import torch

from . import binding as B
from .debug import check_plan, debug_enabled


def default_block_m(T, K, E):
    """Padding block: 16 (one MFMA token block) while every expert fits a pass
    of the streaming schedules (T <= 32); else 64 or 128, the tile's token
    block, so that the busy experts can be tiled: 128 once experts average 96
    tokens, or from 192 tokens on (measured on MI355X: skewed routing puts
    hundreds of tokens on the busiest experts, whose weight tiles are then read
    once per 128 tokens instead of per 64 -- DeepSeek-V3 at 256 / 512 tokens
    with Zipf routing 1.35 / 1.79 -> 1.28 / 1.60 ms, Qwen2 at 512 1.10 -> 1.00 ms,
    Mixtral at 256 0.615 -> 0.596 ms; within 1% either way for uniform routing)."""
    if T * K >= 96 * E or T >= 192:
        return 128
    return 64 if T > 32 or T * K >= 24 * E else 16


class MoELayer:
    def __init__(self, shape, inputs, block_m=None, sched=B.SCHED_AUTO, out_dtype=None,
                 pad=B.PAD_BLOCK, fp8=False, k_tok=None, debug=None):
        """fp8: run the experts, shared experts and DenseFA on the FP8 E4M3 codes
        and row scales of the inputs (keys q13/s13, q2/s2, qs13/ss13, qs2/ss2,
        qfa13/sfa13, qfa2/sfa2; see synth.add_fp8_weights).  k_tok: per-token
        routing budgets [T] int32 on the device (moe_route_var; K is then the
        largest budget allowed).  debug (default: the MOE_DEBUG environment
        variable): check every alignment's invariants on the host
        (debug.check_plan), raising debug.PlanError on a violation."""
        self.debug = debug_enabled(debug)
        x = inputs["x"]
        if fp8 and x.dtype != torch.bfloat16:
            raise B.MoEError(B.MOE_EUNSUPPORTED, f"FP8 weights need bf16 tokens, got {x.dtype}")
        self.fp8 = fp8
        self.k_tok = k_tok
        self.shape, self.inputs, self.sched = shape, inputs, sched
        self.T = T = x.shape[0]
        H, I, E, K = shape.hidden, shape.inter, shape.experts, shape.topk
        dev = x.device
        self.block_m = block_m or default_block_m(T, K, E)
        self.topk_ids = torch.empty(T, K, dtype=torch.int32, device=dev)
        self.topk_w = torch.empty(T, K, dtype=torch.float32, device=dev)
        self.pad = pad
        self.plan = B.Plan(T, K, E, self.block_m, dev, pad=pad)
        # with room for the contraction split of few-expert decode launches
        ws = B.moe_ffn_workspace_bytes_ex(self.plan.cap, T, K, E, H, I)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        self.y_pairs = torch.empty(max(T * K, 1), H, dtype=x.dtype, device=dev)
        self.out = torch.empty(T, H, dtype=out_dtype or x.dtype, device=dev)
        self.has_shared = inputs.get("qs13" if fp8 else "ws13") is not None
        if self.has_shared:
            self.side = torch.cuda.Stream(device=dev)   # default priority
            self.shared_out = torch.empty(T, H, dtype=torch.float32, device=dev)
            self.shared_ws = torch.empty(max(B.dense_ffn_workspace_bytes(T, H, shape.shared_inter), 16),
                                         dtype=torch.uint8, device=dev)
        if inputs.get("qfa13" if fp8 else "wfa13") is not None:
            self.fa_out = torch.empty(T, H, dtype=out_dtype or x.dtype, device=dev)
            self.fa_ws = torch.empty(max(B.dense_ffn_workspace_bytes(T, H, shape.dense_fa_inter), 16),
                                     dtype=torch.uint8, device=dev)
        if inputs.get("wpa13") is not None:
            self.pa_out = torch.empty(T, H, dtype=out_dtype or x.dtype, device=dev)
            self.pa_ws = torch.empty(max(B.dense_ffn_workspace_bytes(T, H, shape.dense_pa_inter), 16),
                                     dtype=torch.uint8, device=dev)

    # the five steps, callable one by one (the benchmark times them separately)
    def route(self):
        if self.k_tok is not None:
            B.moe_route_var(self.inputs["logits"], self.shape.topk, self.k_tok, self.topk_ids,
                            self.topk_w)
        else:
            B.moe_route(self.inputs["logits"], self.shape.topk, self.topk_ids, self.topk_w)

    def align(self):
        if self.pad == B.PAD_BLOCK:
            B.moe_align(self.topk_ids, self.shape.experts, self.plan)
        else:
            B.moe_align_ex(self.topk_ids, self.shape.experts, self.plan, self.pad)
        self._debug_plan()

    def route_align(self):
        """route() then align() in one call (one launch for small batches)."""
        B.moe_route_align(self.inputs["logits"], self.shape.topk, self.topk_ids, self.topk_w,
                          self.plan, self.pad, self.k_tok)
        self._debug_plan()

    def _debug_plan(self):
        if self.debug:
            check_plan(self.plan.arrays(), self.topk_ids, self.shape.experts, self.block_m,
                       self.plan.cap, "block" if self.pad == B.PAD_BLOCK else "max")

    def gate_up(self):
        d = self.inputs
        if self.fp8:
            B.moe_grouped_gate_up_fp8(d["x"], d["q13"], d["s13"], self.shape.topk, self.plan,
                                      self.workspace)
        else:
            B.moe_grouped_gate_up(d["x"], d["w13"], self.shape.topk, self.plan, self.workspace,
                                  self.sched)

    def down(self):
        d = self.inputs
        if self.fp8:
            B.moe_grouped_down_fp8(d["q2"], d["s2"], self.T, self.shape.topk, self.plan,
                                   self.workspace, self.y_pairs)
        else:
            B.moe_grouped_down(d["w2"], self.T, self.shape.topk, self.plan, self.workspace,
                               self.y_pairs, self.sched)

    def shared(self):
        if self.has_shared:
            d = self.inputs
            if self.fp8:
                B.dense_ffn_fp8(d["x"], d["qs13"], d["ss13"], d["qs2"], d["ss2"], self.shared_ws,
                                self.shared_out)
            else:
                B.dense_ffn_fa(d["x"], d["ws13"], d["ws2"], self.shared_ws, self.shared_out,
                               self.sched)

    def combine(self):
        B.moe_combine(self.y_pairs, self.topk_w, self.out,
                      self.shared_out if self.has_shared else None)

    def forward(self, gate_up_events=None):
        """One pass; gate_up_events = (a, b): HIP events recorded on the current
        stream just before and after the grouped gate/up launch (the benchmark
        times the dominant kernel inside the pass with them)."""
        cur = torch.cuda.current_stream()
        if self.has_shared:
            fork = torch.cuda.Event()
            fork.record(cur)         # after the previous pass's combine read shared_out
            self.side.wait_event(fork)
            with torch.cuda.stream(self.side):
                self.shared()
            join = torch.cuda.Event()
            join.record(self.side)
        if self.has_shared:
            # the shared experts' ring, forked first, holds every CU's LDS while it
            # streams; the routing kernel (no LDS) still runs beside it, a fused
            # routing + alignment launch would wait (measured on MI355X: Qwen2-shaped
            # T = 1 pass 190 -> 192-206 us fused; Mixtral-shaped T = 1, no shared
            # experts, 142 -> 135)
            self.route()
            self.align()
        else:
            self.route_align()
        if gate_up_events:
            gate_up_events[0].record(cur)
        self.gate_up()
        if gate_up_events:
            gate_up_events[1].record(cur)
        self.down()
        if self.has_shared:
            cur.wait_event(join)
        self.combine()
        return self.out

    def dense_fa(self):
        d = self.inputs
        if self.fp8:
            B.dense_ffn_fp8(d["x"], d["qfa13"], d["sfa13"], d["qfa2"], d["sfa2"], self.fa_ws,
                            self.fa_out)
        else:
            B.dense_ffn_fa(d["x"], d["wfa13"], d["wfa2"], self.fa_ws, self.fa_out, self.sched)
        return self.fa_out

    def dense_pa(self):
        B.dense_ffn_fa(self.inputs["x"], self.inputs["wpa13"], self.inputs["wpa2"], self.pa_ws,
                       self.pa_out, self.sched)
        return self.pa_out
