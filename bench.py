"""Benchmark of one MoE feed-forward layer pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config mixtral] [--T 32]
                    [--routing uniform] [--all] [--no-cpu]

A step is one whole layer pass over one batch of synthetic tokens: route,
align, grouped gate/up + SwiGLU, grouped down, shared experts (if any) and
combine.  W untimed steps, then exactly K timed steps between two device
synchronisations.  Prints one JSON line with tokens/s (the layer's T tokens
per step), the roofline of the dominant kernel (the grouped gate/up GEMM,
timed live with HIP events on the stream it runs on), the tax tau against the
FLOP-matched dense FFN (DenseFA) timed the same way (and against DensePA, the
parameter-matched one), the analytic tax model's prediction with MI355X
constants, and the CPU oracle timed on the host's cores on a bounded sample of
the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from mixture_experts_layer_30_amd import configs, synth, taxmodel  # noqa: E402
from mixture_experts_layer_30_amd import binding as B  # noqa: E402
from mixture_experts_layer_30_amd.layer import MoELayer  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3
PROFILES = os.path.join(ROOT, "profiles")
METRIC = "MoE-layer tokens/s at 1 GPU, % HBM/MFMA roofline, tax τ vs DenseFA"

# the largest workload that fits one GPU: a DeepSeek-V3-shaped layer (22.5 GB of routed
# weights resident) at the decode batch where the notes place DeepSeek's peak tax (128)
HEADLINE = [("deepseek_v3", 128, "uniform")]
ALL = [("tiny", 64, "uniform"), ("mixtral", 32, "uniform"), ("mixtral", 1024, "uniform"),
       ("qwen2", 1, "zipf"), ("qwen2", 32, "zipf"), ("qwen2", 256, "zipf"), ("qwen2", 2048, "zipf"),
       ("deepseek_v3", 128, "uniform"), ("deepseek_v3", 128, "zipf")] + \
      [("mixtral_sweep", T, "uniform") for T in (1, 8, 128, 512, 2048)]


def source_hash(files):
    """Hash of the kernel sources a counter measurement was taken with."""
    h = hashlib.sha256()
    for f in files:
        p = os.path.join(ROOT, "mixture_experts_layer_30_amd", "csrc", f)
        h.update(open(p, "rb").read() if os.path.exists(p) else b"")
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per gate/up launch from the committed rocprofv3 counter runs
    (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter reads for a copy
    of known size), or None once the kernel sources have changed since."""
    p = os.path.join(PROFILES, "hbm_traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p)).get("workloads", {}).get(workload)
    if not rec or rec.get("source_hash") != source_hash(rec.get("sources", [])):
        return None
    return rec.get("bytes_per_launch")


def gate_up_kernel(shape, T, block_m):
    """The kernel(s) the library's automatic schedule runs for the gate/up half
    (mirrors the choice made in the C ABI; for the record only)."""
    H, I, K, E = shape.hidden, shape.inter, shape.topk, shape.experts
    tile = block_m in (64, 128) and H % 128 == 0
    if tile and T * K >= 24 * E and T > 32:
        if (shape.dtype == "bf16" and T * K >= 256 * E and E <= 512 and H % 256 == 0
                and I % 128 == 0 and (I // 128) * ((T * K + 255) // 256) >= 768):
            return "span_ffn_kernel (256-row MFMA tiles over 256-token spans, persistent)"
        if (shape.dtype == "bf16" and block_m == 128 and T * K >= 512 * E and I % 256 == 0
                and H % 32 == 0):
            return "wide_gate_up_kernel (512-row MFMA tiles through an LDS ring)"
        return "tile2_ffn_kernel (MFMA tiles through an LDS ring)"
    if shape.dtype == "bf16" and H % 128 == 0 and I % 64 == 0:
        if T <= 32:
            return "ring_ffn_kernel (LDS-ring weight streaming, gate/up + SwiGLU)"
        return ("ring_ffn_kernel (experts within a ring pass) + "
                + ("tile2_ffn_kernel" if tile else "stream_gate_up_kernel") + " (busier experts)")
    return "stream_gate_up_kernel (register weight streaming, gate/up + SwiGLU)"


def algorithmic(shape, T, e_active):
    """Unpadded algorithmic bytes and flops (weights of active experts read once)."""
    H, I, K, Is = shape.hidden, shape.inter, shape.topk, shape.shared_inter
    eb = 4 if shape.dtype == "f32" else 2
    gu_bytes = e_active * 2 * I * H * eb + T * H * eb + T * K * I * 2
    layer_bytes = (e_active * 3 * I * H * eb + 3 * H * Is * eb + T * H * eb * 2
                   + T * shape.experts * 4)
    gu_flops = 2 * T * K * H * 2 * I
    layer_flops = 6 * T * K * H * I + 6 * T * H * Is
    fa_bytes = 3 * H * shape.dense_fa_inter * eb + 2 * T * H * eb
    fa_flops = 6 * T * H * shape.dense_fa_inter
    pa_bytes = 3 * H * shape.dense_pa_inter * eb + 2 * T * H * eb
    pa_flops = 6 * T * H * shape.dense_pa_inter
    return dict(gu_bytes=gu_bytes, layer_bytes=layer_bytes, gu_flops=gu_flops,
                layer_flops=layer_flops, fa_bytes=fa_bytes, fa_flops=fa_flops,
                pa_bytes=pa_bytes, pa_flops=pa_flops)


def time_steps(fn, steps, warmup, mid=None):
    """Time exactly `steps` calls of fn between device syncs; with `mid` = (before, after)
    callables, HIP events on the current stream bracket the dominant kernel live."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [] if mid else None
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        if mid:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            fn(a, b, stream)
            evs.append((a, b))
        else:
            fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(end)
    kern_ms = None
    if evs:
        kern_ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    return gpu_ms / steps, wall * 1e3 / steps, kern_ms


def time_flushed(fn, steps):
    """Per-call device times (HIP events) with a 512 MiB write between calls,
    outside the events, so no call finds its weights in the 256 MB Infinity
    Cache; returns median, p10 and p90 in ms."""
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    fn()
    torch.cuda.synchronize()
    pairs = []
    for i in range(steps):
        scratch.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in pairs])
    del scratch
    return {"median_ms": round(float(np.median(ms)), 4), "p10_ms": round(float(np.percentile(ms, 10)), 4),
            "p90_ms": round(float(np.percentile(ms, 90)), 4)}


def breakdown(layer, reps=10):
    """Per-call device time (HIP events), a Fig. 5-style split of the pass."""
    names = ["route", "align", "gate_up", "down", "shared", "combine"]
    out = {}
    torch.cuda.synchronize()
    for n in names:
        fn = getattr(layer, n)
        tot = 0.0
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            tot += a.elapsed_time(b)
        out[n] = round(tot / reps * 1e3, 2)
    return out


def cpu_baseline(shape, dev_inputs, T, budget_s=20.0, min_s=10.0, host_bytes=8 << 30):
    """The oracle (as it is) on the host cores, on a bounded sample of the batch:
    at most budget_s of estimated work per pass, and no more tokens than keep
    the host copy of the experts they use within host_bytes."""
    import oracle
    x = dev_inputs["x"].cpu()
    logits = dev_inputs["logits"].cpu()
    ids, _ = oracle.route(logits, shape.topk)
    # estimate the cost of one token (expert MACs in fp64) and size the sample
    macs_tok = 3 * shape.hidden * (shape.topk * shape.inter + shape.shared_inter)
    threads = oracle.max_threads()
    n = int(max(1, min(T, budget_s * 0.4e9 * threads / macs_tok)))
    tokens = np.linspace(0, T - 1, n).round().astype(np.int64)
    tokens = np.unique(tokens)
    w13d, w2d = dev_inputs["w13"], dev_inputs["w2"]
    per_expert = w13d[0].numel() * w13d.element_size() + w2d[0].numel() * w2d.element_size()
    keep, used = [], set()
    for t in tokens:
        more = used | set(ids[t].tolist())
        if keep and len(more) * per_expert > host_bytes:
            break
        keep.append(int(t))
        used = more
    tokens = np.array(keep, dtype=np.int64)
    used = sorted(used)
    # only the experts the sample routes to are copied; the others are never read
    # (torch.empty leaves their pages untouched)
    E = shape.experts
    w13 = torch.empty((E,) + tuple(w13d.shape[1:]), dtype=w13d.dtype)
    w2 = torch.empty((E,) + tuple(w2d.shape[1:]), dtype=w2d.dtype)
    for e in used:
        w13[e] = dev_inputs["w13"][e].cpu()
        w2[e] = dev_inputs["w2"][e].cpu()
    ws13 = dev_inputs["ws13"].cpu() if dev_inputs.get("ws13") is not None else None
    ws2 = dev_inputs["ws2"].cpu() if dev_inputs.get("ws2") is not None else None
    # the sample is passed repeatedly until about min_s seconds of CPU work are timed
    # (a whole small batch takes well under a second)
    xs, ls = x[tokens], logits[tokens]
    reps, dt = 0, 0.0
    while reps == 0 or dt < min_s:
        t0 = time.perf_counter()
        oracle.moe_layer(xs, ls, w13, w2, shape.topk, ws13, ws2)
        dt += time.perf_counter() - t0
        reps += 1
    return {"value": round(reps * len(tokens) / dt, 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(tokens)} of the {T} tokens of the same batch ({len(used)} experts' "
                      f"weights bf16 on host, fp64 accumulation), {reps} pass{'es' if reps > 1 else ''}, "
                      f"{dt:.2f} s wall"}


def run_workload(name, T, routing, steps, warmup, do_cpu):
    shape = configs.CONFIGS[name]
    torch.manual_seed(0)
    d = synth.layer_inputs(shape, T, routing, seed=0, device="cuda", dense=True, densepa=True)
    layer = MoELayer(shape, d)
    layer.forward()
    torch.cuda.synchronize()
    ids = layer.topk_ids.cpu().numpy()
    e_active = int(len(np.unique(ids)))
    num_padded = int(layer.plan.expert_offsets[-1].item())
    alg = algorithmic(shape, T, e_active)

    def step(a=None, b=None, stream=None):
        # the layer pass, events around its gate/up launch on the current stream
        layer.forward((a, b) if a is not None else None)

    ms, wall_ms, gu_ms = time_steps(step, steps, warmup, mid=True)
    # the gate/up launch alone, back to back (nothing else on the GPU: the number a
    # kernel trace of it reports; in the pass the shared experts stream beside it)
    gu_alone_ms, _, _ = time_steps(layer.gate_up, steps, warmup)
    fa_ms, _, _ = time_steps(layer.dense_fa, steps, warmup)
    pa_ms, _, _ = time_steps(layer.dense_pa, steps, warmup)
    bd = breakdown(layer)
    fl_moe = time_flushed(layer.forward, steps)
    fl_fa = time_flushed(layer.dense_fa, steps)
    model = taxmodel.tax(shape, T, e_active=e_active)
    model_uniform = taxmodel.tax(shape, T)

    dtype = "f32" if shape.dtype == "f32" else "bf16"
    gu_s = gu_ms * 1e-3
    ai = alg["gu_flops"] / alg["gu_bytes"]
    peak_flops = FP32_PEAK_TFLOPS if dtype == "f32" else BF16_PEAK_TFLOPS
    ridge = peak_flops * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": round(alg["gu_bytes"] / gu_s / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(alg["gu_flops"] / gu_s / 1e12, 1),
                "peak": peak_flops, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    workload = f"{name} T={T} {routing}"
    traffic = measured_traffic(workload)
    roof["traffic"] = traffic
    # not counted in this run: read from the committed counter record, and only while
    # the kernel's sources are the ones the counters were taken with
    roof["traffic_source"] = ("profiles/hbm_traffic.json: rocprofv3 FETCH_SIZE and WRITE_SIZE runs "
                              "of the same kernel sources, scaled by a device copy's counts"
                              if traffic is not None else None)
    roof["kernel"] = gate_up_kernel(shape, T, layer.block_m)
    roof["algorithmic_bytes"] = alg["gu_bytes"]
    roof["algorithmic_flops"] = alg["gu_flops"]
    roof["avg_launch_us"] = round(gu_ms * 1e3, 2)
    roof["isolated_avg_launch_us"] = round(gu_alone_ms * 1e3, 2)
    roof["isolated_frac"] = round((alg["gu_bytes"] / (gu_alone_ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
                                  if roof["bound"] == "hbm" else
                                  (alg["gu_flops"] / (gu_alone_ms * 1e-3) / 1e12 / peak_flops), 4)

    layer_s = ms * 1e-3
    rec = {
        "metric": METRIC,
        "value": round(T * steps / (ms * steps * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": workload, "hidden": shape.hidden, "inter": shape.inter,
                   "experts": shape.experts, "topk": shape.topk,
                   "shared_inter": shape.shared_inter, "tokens": T, "routing": routing,
                   "block_m": layer.block_m, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "layer": {"achieved_GBps": round(alg["layer_bytes"] / layer_s / 1e9, 1),
                  "achieved_TFLOPs": round(alg["layer_flops"] / layer_s / 1e12, 2),
                  "hbm_frac": round(alg["layer_bytes"] / layer_s / 1e9 / HBM_PEAK_GBS, 4),
                  "mfma_frac": round(alg["layer_flops"] / layer_s / 1e12 / peak_flops, 4),
                  "e_active": e_active, "padding_eta": round(num_padded / (T * shape.topk), 4),
                  "breakdown_us": bd, "wall_ms_per_step": round(wall_ms, 4)},
        "tau": round(ms / fa_ms, 4),
        "dense_fa": {"ms": round(fa_ms, 4), "inter": shape.dense_fa_inter,
                     "achieved_GBps": round(alg["fa_bytes"] / (fa_ms * 1e-3) / 1e9, 1),
                     "achieved_TFLOPs": round(alg["fa_flops"] / (fa_ms * 1e-3) / 1e12, 2),
                     "hbm_frac": round(alg["fa_bytes"] / (fa_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "mfma_frac": round(alg["fa_flops"] / (fa_ms * 1e-3) / 1e12 / peak_flops, 4)},
        "tau_pa": round(ms / pa_ms, 4),
        "dense_pa": {"ms": round(pa_ms, 4), "inter": shape.dense_pa_inter,
                     "achieved_GBps": round(alg["pa_bytes"] / (pa_ms * 1e-3) / 1e9, 1),
                     "achieved_TFLOPs": round(alg["pa_flops"] / (pa_ms * 1e-3) / 1e12, 2)},
        "per_call_flushed": {"moe_layer": fl_moe, "dense_fa": fl_fa,
                             "tau_median": round(fl_moe["median_ms"] / fl_fa["median_ms"], 4)},
        "tax_model": {"constants": {"hbm_GBps": taxmodel.MI355X_HBM_BPS / 1e9,
                                    "bf16_TFLOPs": taxmodel.MI355X_BF16_FLOPS / 1e12,
                                    "eta": model["eta"]},
                      "e_active_measured": e_active,
                      "e_active_uniform": round(model_uniform["e_active"], 3),
                      "regime": model["regime"],
                      "tau_fa_pred": round(model["tau_fa"], 4),
                      "tau_fa_pred_uniform": round(model_uniform["tau_fa"], 4),
                      "tau_pa_pred": round(model["tau_pa"], 4),
                      "tau_fa_rel_err": round(model["tau_fa"] / (ms / fa_ms) - 1, 4),
                      "t_moe_pred_ms": round(model["t_moe_s"] * 1e3, 4),
                      "t_densefa_pred_ms": round(model["t_densefa_s"] * 1e3, 4)},
    }
    if do_cpu:
        rec["cpu_baseline"] = cpu_baseline(shape, d, T)
    del d, layer
    torch.cuda.empty_cache()
    return rec


def run_only(name, T, routing, what, steps, fp8=False):
    """Runs one piece of the pass `steps` times with nothing else on the GPU in
    between (for hardware-counter runs of a single kernel); fp8: with FP8 E4M3
    weights."""
    if what == "copy":
        # a plain device copy of known size, to calibrate the byte counters
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"only": "copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                          "steps": steps}))
        return
    shape = configs.CONFIGS[name]
    if what == "vendor_gemm":
        # the vendor library's GEMM (torch.mm: hipBLASLt) on one expert's gate/up at
        # the batch's average load, T*K/E tokens x 2I outputs x H: a reference for
        # the grouped prefill kernels' counters, not a step of the pass
        H, I = shape.hidden, shape.inter
        m = T * shape.topk // shape.experts
        x = synth.tokens(m, H, "bf16", seed=1, device="cuda")
        w = synth.swiglu_weights(I, H, "bf16", seed=2, device="cuda")[0]
        out = torch.empty(m, 2 * I, dtype=torch.bfloat16, device="cuda")
        wt = w.t()
        torch.mm(x, wt, out=out)
        torch.cuda.synchronize()
        for _ in range(steps):
            torch.mm(x, wt, out=out)
        torch.cuda.synchronize()
        print(json.dumps({"only": what, "workload": f"{name} T={T}: one expert's gate/up, {m} tokens",
                          "steps": steps, "flops_per_launch": 2 * m * H * 2 * I}))
        return
    d = synth.layer_inputs(shape, T, routing, seed=0, device="cuda", dense=(what == "dense_fa"))
    if fp8:
        synth.add_fp8_weights(d, drop_bf16=True)
    layer = MoELayer(shape, d, fp8=fp8)
    layer.route()
    layer.align()
    layer.gate_up()
    torch.cuda.synchronize()
    ids = layer.topk_ids.cpu().numpy()
    e_active = int(len(np.unique(ids)))
    fn = {"gate_up": layer.gate_up, "down": layer.down, "dense_fa": layer.dense_fa,
          "layer": layer.forward}[what]
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    alg = algorithmic(shape, T, e_active)
    if fp8:  # 1-byte codes plus fp32 row scales
        H, I, K = shape.hidden, shape.inter, shape.topk
        alg["gu_bytes"] = e_active * 2 * I * (H + 4) + T * H * 2 + T * K * I * 2
    print(json.dumps({"only": what, "workload": f"{name} T={T} {routing}", "steps": steps,
                      "fp8": fp8, "e_active": e_active, "gate_up_algorithmic_bytes": alg["gu_bytes"],
                      "gate_up_algorithmic_flops": alg["gu_flops"],
                      "dense_fa_algorithmic_flops": alg["fa_flops"]}))


def padding_sweep(steps):
    """Padding model of the Serving-tax notes (Section 5.1): the padded rows P
    and the padding factor eta = P / (T*K) of block-wise and max padding for
    B in 16..256, and the tiled gate/up kernel's time against P (B = 64, 128)
    with a least-squares line per B; one JSON line per point, then the fits."""
    shape = configs.CONFIGS["qwen2"]
    E, K = shape.experts, shape.topk
    points = []
    for T in (256, 512, 1024, 2048):
        for routing in ("uniform", "zipf"):
            d = synth.layer_inputs(shape, T, routing, seed=0, device="cuda", dense=False)
            for bm in (16, 32, 64, 128, 256):
                for pad, pname in ((B.PAD_BLOCK, "block"), (B.PAD_MAX, "max")):
                    tiled = bm in (64, 128)
                    layer = MoELayer(shape, d, block_m=bm, pad=pad,
                                     sched=B.SCHED_TILE if tiled else B.SCHED_STREAM)
                    layer.route()
                    layer.align()
                    torch.cuda.synchronize()
                    P = int(layer.plan.expert_offsets[-1].item())
                    rec = {"padding_sweep": f"qwen2 T={T} {routing}", "block_m": bm, "padding": pname,
                           "P_rows": P, "eta": round(P / (T * K), 4)}
                    if tiled:
                        us, _, _ = time_steps(layer.gate_up, steps, 2)
                        rec["gate_up_us"] = round(us * 1e3, 2)
                        points.append((bm, P, us * 1e3))
                    print(json.dumps(rec), flush=True)
                    del layer
            del d
            torch.cuda.empty_cache()
    for bm in (64, 128):
        xs = np.array([p for b, p, _ in points if b == bm], dtype=np.float64)
        ys = np.array([t for b, _, t in points if b == bm], dtype=np.float64)
        slope, icpt = np.polyfit(xs, ys, 1)
        pred = slope * xs + icpt
        r2 = 1.0 - ((ys - pred) ** 2).sum() / ((ys - ys.mean()) ** 2).sum()
        print(json.dumps({"padding_fit": f"tiled gate/up time vs padded rows, qwen2 shape, block_m={bm}",
                          "points": len(xs), "us_per_row": round(slope, 6),
                          "intercept_us": round(icpt, 2), "r2": round(float(r2), 5)}), flush=True)


# expert shapes of the cost profile and the replica counts swept (up to the
# experts a GPU holds at 8-way expert parallelism, and at most the layer's E)
COST_REPLICAS = {"mixtral": [1, 2, 4, 8], "qwen2": [1, 2, 4, 8], "deepseek_v3": [1, 2, 4, 8, 16, 32]}
COST_TOKENS = [1, 2, 4, 8, 16, 32, 48, 64, 96, 128, 160, 192, 224, 256, 320, 384, 512, 768, 1024]


def cost_profile(names, steps):
    """Per-expert cost profile of the TEMPO page (section "Dwa reżimy, jeden
    próg"): the time of the grouped expert FFN (gate/up + down, the library's
    automatic schedule) for N tokens shared evenly by G replicas of one expert
    (distinct weight copies, so each replica streams its own weights), cache
    flushed before every call; then the max-affine fit t = max(a + bG, c + beta*N)
    and the threshold n*(G).  One JSON line per expert shape."""
    import dataclasses
    from mixture_experts_layer_30_amd.costprofile import fit_max_affine
    for name in names:
        base = configs.CONFIGS[name]
        gs = COST_REPLICAS[name]
        shp = dataclasses.replace(base, experts=max(gs), topk=1, shared_inter=0)
        d = synth.layer_inputs(shp, max(COST_TOKENS), "uniform", seed=0, device="cuda", dense=False)
        pts = []
        for G in gs:
            sg = dataclasses.replace(shp, experts=G)
            row = []
            for N in COST_TOKENS:
                if N < G:
                    continue
                logits = torch.zeros(N, G, dtype=torch.float32, device="cuda")
                logits[torch.arange(N), torch.arange(N) % G] = 1.0   # token n -> replica n mod G
                inp = {"x": d["x"][:N], "logits": logits, "w13": d["w13"][:G], "w2": d["w2"][:G],
                       "ws13": None, "ws2": None}
                # the automatic schedule, then the weight-streaming and the tiled
                # schedules forced (the tile needs 64- or 128-row blocks)
                us = {}
                for key, kw in (("auto", {}), ("stream", {"sched": B.SCHED_RING}),
                                ("tile", {"sched": B.SCHED_TILE,
                                          "block_m": 128 if N >= 128 * G else 64})):
                    layer = MoELayer(sg, inp, **kw)
                    layer.route()
                    layer.align()

                    def fn():
                        layer.gate_up()
                        layer.down()

                    us[key] = round(time_flushed(fn, steps)["median_ms"] * 1e3, 2)
                pts.append((G, N, us["auto"], us["stream"], us["tile"]))
                row.append(f"{N}:{us['auto']:.0f}/{us['stream']:.0f}/{us['tile']:.0f}")
            print(f"[cost profile] {name} G={G} (auto/stream/tile us): " + " ".join(row),
                  file=sys.stderr, flush=True)
        G, N, t_auto, t_str, t_tile = (np.array([p[i] for p in pts], dtype=np.float64)
                                       for i in range(5))

        def fit_rec(t):
            f = fit_max_affine(G, N, t)
            return {"a": round(f.a, 3), "b": round(f.b, 3), "c": round(f.c, 3), "beta": round(f.beta, 5),
                    "r2": round(f.r2, 5), "max_rel_err": round(f.max_rel_err, 4),
                    "points_memory": f.n_memory, "points_compute": f.n_compute,
                    "n_star": {str(g): (None if f.n_star(g) is None else round(f.n_star(g), 1))
                               for g in gs}}

        t_best = np.minimum(t_str, t_tile)

        def per_replicas(t):
            """For each G: the flat (weight-streaming) level m, the first N whose
            time exceeds 1.25 m, the marginal cost per token over the three
            largest N (least squares) and the token count at which that cost
            alone would reach m (the threshold if the compute regime were
            proportional to the tokens)."""
            out = {}
            for g in gs:
                sel = G == g
                n, tt = N[sel], t[sel]
                m = float(np.median(tt[n <= max(g, 16)]))
                over = n[tt > 1.25 * m]
                tail = np.argsort(n)[-3:]
                slope = float(np.polyfit(n[tail], tt[tail], 1)[0])
                out[str(g)] = {"flat_us": round(m, 1),
                               "flat_ends_at_N": None if len(over) == 0 else int(over.min()),
                               "tail_us_per_token": round(slope, 4),
                               "n_star_marginal": round(m / slope, 1) if slope > 0 else None}
            return out

        rec = {"cost_profile": name, "hidden": base.hidden, "inter": base.inter, "dtype": base.dtype,
               "unit": "us", "steps": steps,
               "fit_auto": fit_rec(t_auto),
               "fit_best": fit_rec(t_best),
               "per_replicas_best": per_replicas(t_best),
               "per_replicas_auto": per_replicas(t_auto),
               "expert_weight_bytes": 3 * base.hidden * base.inter * 2,
               # tokens per replica at which an expert's flops at the bf16 MFMA peak take as
               # long as reading its weights at the HBM peak (1 flop per weight byte per token)
               "n_star_roofline": round(BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9), 1),
               "points": {"columns": ["G", "N", "auto_us", "stream_us", "tile_us"],
                          "rows": [list(p) for p in pts]}}
        print(json.dumps(rec), flush=True)
        del d
        torch.cuda.empty_cache()


# routing budgets of the per-token-K workload: a decode batch of requests that
# each chose their own top-k (MoE-Prism page), uniform over these levels
VAR_K_LEVELS = {"qwen2": [2, 4, 6, 8], "deepseek_v3": [2, 4, 6, 8]}
VAR_K_WORK = [("qwen2", 32, "zipf"), ("deepseek_v3", 128, "uniform"), ("deepseek_v3", 128, "zipf")]


def run_var_k(name, T, routing, steps, warmup):
    """Per-token routing budgets (MoE-Prism page: the routing top-k as a
    per-request knob): one pass over the mixed batch (moe_route_var), against
    serving every token at the largest budget ("over-serving") and against one
    pass per budget tier (split batches).  Reports tokens/s of each."""
    import dataclasses
    shape = configs.CONFIGS[name]
    levels = VAR_K_LEVELS[name]
    d = synth.layer_inputs(shape, T, routing, seed=0, device="cuda", dense=False)
    k_tok = synth.budgets(T, levels, seed=0, device="cuda")
    var = MoELayer(shape, d, k_tok=k_tok)
    var.forward()
    torch.cuda.synchronize()
    ids = var.topk_ids.cpu().numpy()
    e_var = int(len(np.unique(ids[ids >= 0])))
    ms_var, _, _ = time_steps(var.forward, steps, warmup)
    fl_var = time_flushed(var.forward, steps)
    full = MoELayer(shape, d)
    full.forward()
    torch.cuda.synchronize()
    e_full = int(len(np.unique(full.topk_ids.cpu().numpy())))
    ms_full, _, _ = time_steps(full.forward, steps, warmup)
    fl_full = time_flushed(full.forward, steps)
    del full
    # split batches: one layer pass per budget tier over its tokens
    kt = k_tok.cpu()
    tiers = []
    for k in sorted(set(kt.tolist())):
        idx = torch.nonzero(kt == k).flatten().to("cuda")
        sub = dict(d, x=d["x"][idx].contiguous(), logits=d["logits"][idx].contiguous())
        tiers.append(MoELayer(dataclasses.replace(shape, topk=k), sub))

    def split_pass():
        for lay in tiers:
            lay.forward()

    split_pass()
    torch.cuda.synchronize()
    ms_split, _, _ = time_steps(split_pass, steps, warmup)
    fl_split = time_flushed(split_pass, steps)
    H, I, Is = shape.hidden, shape.inter, shape.shared_inter
    pairs = int(kt.sum())
    layer_bytes = e_var * 3 * H * I * 2 + 3 * H * Is * 2 + 2 * T * H * 2 + T * shape.experts * 4
    rec = {"metric": "MoE-layer tokens/s at 1 GPU with per-token routing budgets",
           "value": round(T / (ms_var * 1e-3), 2), "unit": "tokens/s", "ms_per_step": round(ms_var, 4),
           "steps": steps, "warmup": warmup, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"{name} T={T} {routing}", "budgets": levels,
                      "pairs": pairs, "pairs_at_max_k": T * shape.topk,
                      "e_active": e_var, "e_active_at_max_k": e_full},
           "layer": {"achieved_GBps": round(layer_bytes / (ms_var * 1e-3) / 1e9, 1),
                     "hbm_frac": round(layer_bytes / (ms_var * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
           "over_serving": {"ms_per_step": round(ms_full, 4), "tokens_per_s": round(T / (ms_full * 1e-3), 2)},
           "split_batches": {"ms_per_step": round(ms_split, 4), "tokens_per_s": round(T / (ms_split * 1e-3), 2),
                             "passes": len(tiers)},
           "flushed_median_ms": {"mixed": fl_var["median_ms"], "over_serving": fl_full["median_ms"],
                                 "split_batches": fl_split["median_ms"]},
           "speedup_vs_over_serving": round(ms_full / ms_var, 4),
           "speedup_vs_split_batches": round(ms_split / ms_var, 4)}
    del d, var, tiers
    torch.cuda.empty_cache()
    return rec


def run_fp8(name, T, routing, steps, warmup):
    """The same pass with FP8 E4M3 expert, shared and DenseFA weights (row scales,
    bf16 activations): the notes' weight-quantization remedy for the decode tax.
    Reports tokens/s, the gate/up kernel against the HBM roofline on the FP8
    bytes, tau against the FP8 DenseFA, and the speed-up over the bf16 pass."""
    shape = configs.CONFIGS[name]
    d = synth.layer_inputs(shape, T, routing, seed=0, device="cuda", dense=True)
    bf = MoELayer(shape, d)
    bf.forward()
    torch.cuda.synchronize()
    e_active = int(len(np.unique(bf.topk_ids.cpu().numpy())))
    ms_bf, _, _ = time_steps(bf.forward, steps, warmup)
    del bf
    synth.add_fp8_weights(d, drop_bf16=True)
    torch.cuda.empty_cache()
    layer = MoELayer(shape, d, fp8=True)
    layer.forward()
    torch.cuda.synchronize()

    def step(a=None, b=None, stream=None):
        # the layer pass, events around its gate/up launch on the current stream
        layer.forward((a, b) if a is not None else None)

    ms, _, gu_ms = time_steps(step, steps, warmup, mid=True)
    fa_ms, _, _ = time_steps(layer.dense_fa, steps, warmup)
    H, I, K, Is = shape.hidden, shape.inter, shape.topk, shape.shared_inter
    # FP8 bytes: codes (1 B) plus fp32 row scales; tokens and activations bf16
    gu_bytes = e_active * 2 * I * H + e_active * 2 * I * 4 + T * H * 2 + T * K * I * 2
    layer_bytes = (e_active * 3 * I * H + e_active * (2 * I + H) * 4 + 3 * H * Is + (2 * Is + H) * 4
                   * (Is > 0) + 2 * T * H * 2 + T * shape.experts * 4)
    fa_bytes = 3 * H * shape.dense_fa_inter + (2 * shape.dense_fa_inter + H) * 4 + 2 * T * H * 2
    rec = {"metric": "MoE-layer tokens/s at 1 GPU with FP8 E4M3 weights", "value": round(T / (ms * 1e-3), 2),
           "unit": "tokens/s", "ms_per_step": round(ms, 4), "steps": steps, "warmup": warmup,
           "dtype": "fp8-e4m3 weights (fp32 row scales), bf16 activations, fp32 accumulation",
           "config": {"workload": f"{name} T={T} {routing}", "e_active": e_active},
           "roofline": {"bound": "hbm", "kernel": "ring_ffn_kernel<FP8, ...> (gate/up + SwiGLU)",
                        "achieved": round(gu_bytes / (gu_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gu_bytes / (gu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "avg_launch_us": round(gu_ms * 1e3, 2), "algorithmic_bytes": gu_bytes,
                        "traffic": measured_traffic(f"{name} T={T} {routing} fp8")},
           "layer": {"achieved_GBps": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
           "tau_fp8": round(ms / fa_ms, 4),
           "dense_fa_fp8": {"ms": round(fa_ms, 4), "achieved_GBps": round(fa_bytes / (fa_ms * 1e-3) / 1e9, 1)},
           "speedup_vs_bf16": round(ms_bf / ms, 4), "bf16_ms_per_step": round(ms_bf, 4)}
    del d, layer
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=None)
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--routing", default=None)
    ap.add_argument("--all", action="store_true", help="one line per workload of every config")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", choices=["gate_up", "down", "dense_fa", "layer", "copy", "vendor_gemm"],
                    help="run one piece `--steps` times, untimed (for counter runs)")
    ap.add_argument("--fp8", action="store_true",
                    help="also time the decode workloads with FP8 E4M3 weights (one line each)")
    ap.add_argument("--var-k", action="store_true",
                    help="per-token routing budgets vs max-budget and split-batch passes (MoE-Prism)")
    ap.add_argument("--cost-profile", action="store_true",
                    help="per-expert time vs tokens and replicas, max-affine fit and n* (TEMPO page)")
    ap.add_argument("--padding-sweep", action="store_true",
                    help="padded rows, eta and tiled gate/up time vs padded rows (Section 5.1)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer is built and timed on a single MI355X; "
              "runs on more than one GPU are not part of this library", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.padding_sweep:
        padding_sweep(args.steps)
        return
    if args.cost_profile:
        cost_profile([args.config] if args.config else list(COST_REPLICAS), args.steps)
        return
    if args.var_k:
        for name, T, routing in VAR_K_WORK:
            if args.config in (None, name):
                print(json.dumps(run_var_k(name, T, routing, args.steps, args.warmup)), flush=True)
        return
    if args.only:
        shape = configs.CONFIGS[args.config or "mixtral"]
        run_only(args.config or "mixtral", args.T or shape.tokens[0],
                 args.routing or shape.routing[0], args.only, args.steps, fp8=args.fp8)
        return
    if args.all:
        work = ALL
    elif args.config:
        shape = configs.CONFIGS[args.config]
        work = [(args.config, args.T or shape.tokens[0], args.routing or shape.routing[0])]
    else:
        work = HEADLINE
    for i, (name, T, routing) in enumerate(work):
        rec = run_workload(name, T, routing, args.steps, args.warmup,
                           do_cpu=(not args.no_cpu) and (i == 0))
        print(json.dumps(rec), flush=True)
    if args.fp8:
        shapes = [(n, T, r) for n, T, r in work
                  if configs.CONFIGS[n].dtype == "bf16" and configs.CONFIGS[n].hidden % 128 == 0
                  and configs.CONFIGS[n].inter % 128 == 0 and T * configs.CONFIGS[n].topk
                  < 24 * configs.CONFIGS[n].experts]
        for name, T, routing in shapes:
            print(json.dumps(run_fp8(name, T, routing, args.steps, args.warmup)), flush=True)


if __name__ == "__main__":
    main()
