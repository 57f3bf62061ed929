"""Seeded synthetic inputs for the MoE layer and the DenseFA baseline.

Both the HIP path and the CPU oracle are fed from here; this module holds none
of the method's arithmetic, only the input distributions:

* x ~ N(0, 1), router logits ~ N(0, 1) (fp32);
* "zipf" routing adds a log-Zipf expert prior: l[t, e] = n[t, e] - s * ln(e + 1),
  so expert 0 is the hottest (the normaliser of the Zipf law is dropped: a
  constant shift of all logits of a token does not change softmax);
* every weight W ~ N(0, std = 1/sqrt(fan_in)), fan_in = H for the gate/up
  matrices and the intermediate width for the down matrix;
* values are rounded once to the storage dtype (bf16 round-to-nearest-even).

Each tensor draws from its own generator seeded from (seed, tensor name), so
adding a tensor never shifts another.  Generation happens on `device`; tests
that need the same values on the host copy the device tensors back.
"""
import math
import zlib

import torch

_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1000003 + zlib.crc32(name.encode())) & 0x7FFFFFFFFFFFFFFF)
    return g


def _normal(shape, std, dtype, seed, name, device, chunk_dim0=None):
    """N(0, std^2) rounded to dtype; generated in slices of dim 0 to bound the fp32 temporary."""
    out = torch.empty(shape, dtype=dtype, device=device)
    g = _gen(seed, name, device)
    n0 = shape[0]
    step = chunk_dim0 or n0
    for a in range(0, n0, step):
        b = min(n0, a + step)
        t = torch.randn((b - a,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        out[a:b].copy_(t)
        del t
    return out


def router_logits(T, E, routing="uniform", zipf_s=1.2, seed=0, device="cpu", name="logits"):
    l = _normal((T, E), 1.0, torch.float32, seed, name, device)
    if routing == "zipf":
        prior = torch.log(torch.arange(1, E + 1, dtype=torch.float64, device=device)) * zipf_s
        l = (l.double() - prior[None, :]).float()
    elif routing != "uniform":
        raise ValueError(f"unknown routing {routing!r}")
    return l.contiguous()


def budgets(T, levels, seed=0, device="cpu", name="k_tok"):
    """Per-token routing budgets [T] int32, each drawn uniformly from `levels`
    (a batch of decode requests with their own top-k, as on the MoE-Prism
    page; one token per request)."""
    g = _gen(seed, name, "cpu")
    lv = torch.tensor(list(levels), dtype=torch.int32)
    return lv[torch.randint(0, len(lv), (T,), generator=g)].to(device)


def tokens(T, H, dtype="bf16", seed=0, device="cpu", name="x"):
    return _normal((T, H), 1.0, _DT[dtype], seed, name, device)


def swiglu_weights(n_out_inter, H, dtype="bf16", seed=0, device="cpu", prefix="w", experts=None):
    """Gate/up matrix [.., 2*I, H] (rows 0..I-1 gate, I..2I-1 up) and down matrix [.., H, I]."""
    I = n_out_inter
    dt = _DT[dtype]
    if experts is None:
        w13 = _normal((2 * I, H), 1.0 / math.sqrt(H), dt, seed, prefix + "13", device, chunk_dim0=4096)
        w2 = _normal((H, I), 1.0 / math.sqrt(I), dt, seed, prefix + "2", device, chunk_dim0=4096)
    else:
        w13 = _normal((experts, 2 * I, H), 1.0 / math.sqrt(H), dt, seed, prefix + "13", device, chunk_dim0=1)
        w2 = _normal((experts, H, I), 1.0 / math.sqrt(I), dt, seed, prefix + "2", device, chunk_dim0=1)
    return w13, w2


FP8_MAX = 448.0   # largest finite FP8 E4M3 value


def quantize_fp8_rows(w, chunk_rows=8192):
    """FP8 E4M3 weight codes and fp32 row scales for a [..., rows, cols] matrix:
    scale = max |w[row]| / 448 (1 for an all-zero row), code = w / scale rounded
    to the nearest E4M3 value (torch's float8_e4m3fn conversion).  Returns
    (uint8 codes of w's shape, float32 scales of shape [..., rows]).  An input
    transform (weight quantization, the notes' decode-phase remedy); the layer
    consumes codes and scales as given."""
    q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    sc = torch.empty(w.shape[:-1], dtype=torch.float32, device=w.device)
    flat_w = w.reshape(-1, w.shape[-1])
    flat_q = q.view(-1, w.shape[-1])
    flat_s = sc.view(-1)
    for r0 in range(0, flat_w.shape[0], chunk_rows):
        blk = flat_w[r0:r0 + chunk_rows].float()
        amax = blk.abs().amax(dim=1)
        s_ = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
        flat_s[r0:r0 + chunk_rows] = s_
        flat_q[r0:r0 + chunk_rows] = (blk / s_[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return q, sc


def layer_inputs(shape, T, routing=None, seed=0, device="cpu", dense=True, moe=True,
                 densepa=False):
    """All inputs of one MoE layer pass (and its DenseFA / DensePA baselines) for a LayerShape."""
    routing = routing or shape.routing[0]
    d = {"T": T, "routing": routing}
    d["x"] = tokens(T, shape.hidden, shape.dtype, seed, device)
    d["logits"] = router_logits(T, shape.experts, routing, shape.zipf_s, seed, device)
    if moe:
        d["w13"], d["w2"] = swiglu_weights(shape.inter, shape.hidden, shape.dtype, seed, device,
                                           "expert_w", experts=shape.experts)
        if shape.shared_inter:
            d["ws13"], d["ws2"] = swiglu_weights(shape.shared_inter, shape.hidden, shape.dtype, seed,
                                                 device, "shared_w")
        else:
            d["ws13"] = d["ws2"] = None
    if dense:
        d["wfa13"], d["wfa2"] = swiglu_weights(shape.dense_fa_inter, shape.hidden, shape.dtype, seed,
                                               device, "densefa_w")
    if densepa:
        d["wpa13"], d["wpa2"] = swiglu_weights(shape.dense_pa_inter, shape.hidden, shape.dtype, seed,
                                               device, "densepa_w")
    return d


# weight tensors of layer_inputs and the keys of their FP8 codes and row scales
FP8_KEYS = {"w13": ("q13", "s13"), "w2": ("q2", "s2"), "ws13": ("qs13", "ss13"),
            "ws2": ("qs2", "ss2"), "wfa13": ("qfa13", "sfa13"), "wfa2": ("qfa2", "sfa2")}


def add_fp8_weights(d, drop_bf16=False):
    """Adds FP8 E4M3 codes and row scales of every weight tensor of layer_inputs'
    dict d (see quantize_fp8_rows); with drop_bf16 the bf16 tensors are released."""
    for k, (qk, sk) in FP8_KEYS.items():
        if d.get(k) is not None:
            d[qk], d[sk] = quantize_fp8_rows(d[k])
            if drop_bf16:
                d[k] = None
        elif k in d:
            d[qk] = d[sk] = None
    return d
