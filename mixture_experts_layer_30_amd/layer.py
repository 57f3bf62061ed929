"""One MoE feed-forward layer pass on the GPU, as five library calls.

Buffers are allocated once, when the runner is built; a pass then only
enqueues the library's kernels on the current stream:

  moe_route -> moe_align -> moe_grouped_gate_up -> moe_grouped_down
  [-> dense_ffn_fa for the shared experts] -> moe_combine

and the DenseFA baseline is one dense_ffn_fa call (DensePA, the dense FFN
with the MoE's parameter count, another one of width E*I + I_s).  The tax of
the Serving-tax notes (section "定義", Eq. 1) is tau = T(MoE, b) / T(DenseFA, b).
"""
import torch

from . import binding as B


def default_block_m(T, K, E):
    """Padding block: 16 (one MFMA token block) for the streaming schedules,
    64 or 128 (the tile's token block) once experts average 24 tokens, the
    tiled schedule's range; 128 from 96 tokens on average (measured crossover)."""
    if T * K >= 96 * E:
        return 128
    return 64 if T * K >= 24 * E else 16


class MoELayer:
    def __init__(self, shape, inputs, block_m=None, sched=B.SCHED_AUTO, out_dtype=None,
                 pad=B.PAD_BLOCK):
        x = inputs["x"]
        self.shape, self.inputs, self.sched = shape, inputs, sched
        self.T = T = x.shape[0]
        H, I, E, K = shape.hidden, shape.inter, shape.experts, shape.topk
        dev = x.device
        self.block_m = block_m or default_block_m(T, K, E)
        self.topk_ids = torch.empty(T, K, dtype=torch.int32, device=dev)
        self.topk_w = torch.empty(T, K, dtype=torch.float32, device=dev)
        self.pad = pad
        self.plan = B.Plan(T, K, E, self.block_m, dev, pad=pad)
        ws = B.moe_ffn_workspace_bytes(self.plan.cap, I)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        self.y_pairs = torch.empty(max(T * K, 1), H, dtype=x.dtype, device=dev)
        self.out = torch.empty(T, H, dtype=out_dtype or x.dtype, device=dev)
        self.has_shared = inputs.get("ws13") is not None
        if self.has_shared:
            self.shared_out = torch.empty(T, H, dtype=torch.float32, device=dev)
            self.shared_ws = torch.empty(max(B.dense_ffn_workspace_bytes(T, H, shape.shared_inter), 16),
                                         dtype=torch.uint8, device=dev)
        if inputs.get("wfa13") is not None:
            self.fa_out = torch.empty(T, H, dtype=out_dtype or x.dtype, device=dev)
            self.fa_ws = torch.empty(max(B.dense_ffn_workspace_bytes(T, H, shape.dense_fa_inter), 16),
                                     dtype=torch.uint8, device=dev)
        if inputs.get("wpa13") is not None:
            self.pa_out = torch.empty(T, H, dtype=out_dtype or x.dtype, device=dev)
            self.pa_ws = torch.empty(max(B.dense_ffn_workspace_bytes(T, H, shape.dense_pa_inter), 16),
                                     dtype=torch.uint8, device=dev)

    # the five steps, callable one by one (the benchmark times them separately)
    def route(self):
        B.moe_route(self.inputs["logits"], self.shape.topk, self.topk_ids, self.topk_w)

    def align(self):
        if self.pad == B.PAD_BLOCK:
            B.moe_align(self.topk_ids, self.shape.experts, self.plan)
        else:
            B.moe_align_ex(self.topk_ids, self.shape.experts, self.plan, self.pad)

    def gate_up(self):
        B.moe_grouped_gate_up(self.inputs["x"], self.inputs["w13"], self.shape.topk, self.plan,
                              self.workspace, self.sched)

    def down(self):
        B.moe_grouped_down(self.inputs["w2"], self.T, self.shape.topk, self.plan, self.workspace,
                           self.y_pairs, self.sched)

    def shared(self):
        if self.has_shared:
            B.dense_ffn_fa(self.inputs["x"], self.inputs["ws13"], self.inputs["ws2"], self.shared_ws,
                           self.shared_out, self.sched)

    def combine(self):
        B.moe_combine(self.y_pairs, self.topk_w, self.out,
                      self.shared_out if self.has_shared else None)

    def forward(self):
        self.route()
        self.align()
        self.gate_up()
        self.down()
        self.shared()
        self.combine()
        return self.out

    def dense_fa(self):
        B.dense_ffn_fa(self.inputs["x"], self.inputs["wfa13"], self.inputs["wfa2"], self.fa_ws,
                       self.fa_out, self.sched)
        return self.fa_out

    def dense_pa(self):
        B.dense_ffn_fa(self.inputs["x"], self.inputs["wpa13"], self.inputs["wpa2"], self.pa_ws,
                       self.pa_out, self.sched)
        return self.pa_out
