"""GPU parity at the full layer shapes of Table 2 (talk notes on "Demystifying
the Mixture of Experts Serving Tax", section "評価対象モデル (Table 2)"),
through the C ABI, against the CPU oracle.

Routing ids and every alignment array are compared bit-exact for every token.
Outputs are compared within max|gpu - ref| / max|ref| <= 1e-2:

* decode batches (up to 128 tokens): every token of the batch;
* prefill batches: a stratified sample -- at least one token from every
  (expert, alignment block) pair, so that every tile of every expert is
  checked, plus every token of the busiest expert's first and last block.

The oracle is fed one expert at a time: each expert that the compared tokens
use is copied to the host, run over all of its (token, slot) rows and
dropped, so a DeepSeek-V3-shaped layer's 22.5 GB of weights never sit in host
memory together.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_30_amd import binding as B
from mixture_experts_layer_30_amd import configs, synth
from mixture_experts_layer_30_amd.layer import MoELayer

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()  # the HIP library must be there: fail loudly, never fall back
    oracle.lib()


def rel_err(gpu, ref):
    g = gpu.detach().float().cpu().double().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(g - ref).max() / max(np.abs(ref).max(), 1e-30))


def oracle_out(dev, shape, tokens, k_tok=None, fp8=False):
    """The oracle's layer output for the given tokens (host index array): its
    routing of them, each expert they use run once over all of its rows with
    that expert's weights copied to the host for the call only, the shared
    experts, the combine.  k_tok: per-token budgets [T] (host) or None.
    Returns (out [n, H] float64, ids [n, K])."""
    tsel = torch.from_numpy(np.asarray(tokens, dtype=np.int64))
    x = dev["x"].index_select(0, tsel.to(dev["x"].device)).cpu()
    logits = dev["logits"].index_select(0, tsel.to(DEV)).cpu()
    K, H = shape.topk, shape.hidden
    if k_tok is None:
        ids, w = oracle.route(logits, K)
    else:
        ids, w = oracle.route_var(logits, K, np.asarray(k_tok)[tokens])
    y = np.zeros((len(tokens) * K, H))
    for e in np.unique(ids[ids >= 0]):
        sel = np.argwhere(ids == e)
        xe = x[torch.from_numpy(sel[:, 0])]
        if fp8:
            ye = oracle.swiglu_fp8(xe, dev["q13"][e].cpu(), dev["s13"][e].cpu(), dev["q2"][e].cpu(),
                                   dev["s2"][e].cpu())
        else:
            ye = oracle.swiglu(xe, dev["w13"][e].cpu(), dev["w2"][e].cpu())
        y[sel[:, 0] * K + sel[:, 1]] = ye
    s = None
    if shape.shared_inter:
        if fp8:
            s = oracle.swiglu_fp8(x, dev["qs13"].cpu(), dev["ss13"].cpu(), dev["qs2"].cpu(),
                                  dev["ss2"].cpu())
        else:
            s = oracle.swiglu(x, dev["ws13"].cpu(), dev["ws2"].cpu())
    return oracle.combine(y, w, s), ids


def stratified_tokens(ids, E, block, seed):
    """Tokens covering every (expert, block) pair of the block-wise alignment
    (bucket e holds its pairs p = t*K + k in ascending p, cut into blocks of
    `block` rows): one token drawn from each pair's rows, plus every token of
    the busiest expert's first and last block."""
    rng = np.random.default_rng(seed)
    K = ids.shape[1]
    flat = ids.ravel()
    chosen = set()
    for e in range(E):
        pairs = np.flatnonzero(flat == e)
        for b0 in range(0, len(pairs), block):
            blk = pairs[b0:b0 + block]
            chosen.add(int(blk[rng.integers(len(blk))]) // K)
    hot = np.flatnonzero(flat == np.bincount(flat[flat >= 0], minlength=E).argmax())
    last = (len(hot) - 1) // block * block
    chosen.update((hot[:block] // K).tolist())
    chosen.update((hot[last:] // K).tolist())
    return np.array(sorted(chosen), dtype=np.int64)


def dense_tokens(T, block, seed):
    """Dense rows: one token per `block` rows, plus every token of the first and last block."""
    if T <= 128:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    chosen = {int(b0 + rng.integers(min(block, T - b0))) for b0 in range(0, T, block)}
    chosen.update(range(block))
    chosen.update(range((T - 1) // block * block, T))
    return np.array(sorted(chosen), dtype=np.int64)


def check_routing_and_plan(layer, dev, shape, k_tok=None):
    """Routing and every alignment array, bit-exact over the whole batch."""
    if k_tok is None:
        rids, rw = oracle.route(dev["logits"].cpu(), shape.topk)
    else:
        rids, rw = oracle.route_var(dev["logits"].cpu(), shape.topk, k_tok)
    assert (layer.topk_ids.cpu().numpy() == rids).all()
    assert np.abs(layer.topk_w.cpu().numpy() - rw).max() <= 1e-5
    got = {k: v.cpu().numpy() for k, v in layer.plan.arrays().items()}
    ra = oracle.align(rids, shape.experts, layer.block_m, layer.plan.cap)
    for k in ra:
        assert (got[k] == ra[k]).all(), k
    return rids


# (workload, T, routing, decode): decode batches are compared on every token
FULL_CASES = [
    ("mixtral", 1, "uniform", True),       # two experts: the down projection splits its contraction
    ("mixtral", 32, "uniform", True),
    ("qwen2", 1, "zipf", True),
    ("qwen2", 32, "zipf", True),
    ("deepseek_v3", 128, "uniform", True),
    ("deepseek_v3", 128, "zipf", True),
    ("mixtral", 128, "uniform", True),     # 64-token tiles, the down projection's contraction split
    ("mixtral", 1024, "uniform", False),   # span schedule on both halves (one or two spans an expert)
    ("mixtral", 2048, "uniform", False),   # span gate/up (two or three spans an expert), tiled down
    ("qwen2", 256, "zipf", False),
    ("qwen2", 2048, "zipf", False),        # span gate/up with skewed spans, tiled down
    ("mixtral", 4096, "uniform", False),   # 1024 tokens per expert: four spans each, 8 blocks
    ("deepseek_v3", 4096, "zipf", False),  # 32 768 pairs over 256 experts, skewed, tiled at block 128
]


@pytest.mark.parametrize("name,T,routing,decode", FULL_CASES)
def test_layer_parity_full_size(name, T, routing, decode):
    shape = configs.CONFIGS[name]
    dense = name == "mixtral"
    print(f"\n[full-size parity] {name} T={T} {routing}", flush=True)
    dev = synth.layer_inputs(shape, T, routing, seed=0, device=DEV, dense=dense,
                             densepa=(name == "mixtral" and T == 32))
    layer = MoELayer(shape, dev)
    out = layer.forward()
    torch.cuda.synchronize()
    rids = check_routing_and_plan(layer, dev, shape)
    tokens = np.arange(T) if decode else stratified_tokens(rids, shape.experts, layer.block_m, T)
    print(f"  comparing {len(tokens)} of {T} tokens", flush=True)
    ref, ids = oracle_out(dev, shape, tokens)
    assert (ids == rids[tokens]).all()
    tsel = torch.from_numpy(tokens).to(DEV)
    assert rel_err(out.index_select(0, tsel), ref) <= TOL
    if dense:
        fa = layer.dense_fa()
        torch.cuda.synchronize()
        ft = dense_tokens(T, 128, T + 1)
        fsel = torch.from_numpy(ft).to(DEV)
        ref_fa = oracle.dense_ffn(dev["x"].index_select(0, fsel).cpu(), dev["wfa13"].cpu(),
                                  dev["wfa2"].cpu())
        assert rel_err(fa.index_select(0, fsel), ref_fa) <= TOL
    if "wpa13" in dev:   # DensePA: the dense FFN of width E*I holding the MoE's parameter count
        pa = layer.dense_pa()
        torch.cuda.synchronize()
        ref_pa = oracle.dense_ffn(dev["x"].cpu(), dev["wpa13"].cpu(), dev["wpa2"].cpu())
        assert rel_err(pa, ref_pa) <= TOL
    del dev, layer, out
    torch.cuda.empty_cache()


# DenseFA (I_fa = K*I + I_s) on its own, every token: the DeepSeek-V3 shape at 128 tokens
# (tiled, both contractions split), the Mixtral sweep's 8 tokens and Qwen2's 32 tokens
# (LDS ring, contractions split by the ring's rounds model)
@pytest.mark.parametrize("name,T", [("deepseek_v3", 128), ("mixtral_sweep", 8), ("qwen2", 32)])
def test_dense_fa_full_size(name, T):
    shape = configs.CONFIGS[name]
    print(f"\n[full-size DenseFA parity] {name} T={T}", flush=True)
    x = synth.tokens(T, shape.hidden, "bf16", seed=T + 5, device=DEV)
    w13, w2 = synth.swiglu_weights(shape.dense_fa_inter, shape.hidden, "bf16", seed=6,
                                   device=DEV)
    ws = torch.empty(B.dense_ffn_workspace_bytes(T, shape.hidden, shape.dense_fa_inter),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty(T, shape.hidden, dtype=torch.bfloat16, device=DEV)
    B.dense_ffn_fa(x, w13, w2, ws, out)
    torch.cuda.synchronize()
    ref = oracle.dense_ffn(x.cpu(), w13.cpu(), w2.cpu())
    assert rel_err(out, ref) <= TOL
    del w13, w2, ws
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,T,routing,levels", [("qwen2", 32, "zipf", [0, 2, 4, 8]),
                                                   ("deepseek_v3", 128, "uniform", [2, 4, 6, 8])])
def test_layer_parity_var_k_full_size(name, T, routing, levels):
    """Per-token routing budgets (MoE-Prism page) at full size, every token."""
    shape = configs.CONFIGS[name]
    print(f"\n[var-K full-size parity] {name} T={T} {routing} budgets {levels}", flush=True)
    dev = synth.layer_inputs(shape, T, routing, seed=0, device=DEV, dense=False)
    k_tok = synth.budgets(T, levels, seed=1)
    layer = MoELayer(shape, dev, k_tok=k_tok.to(DEV))
    out = layer.forward()
    torch.cuda.synchronize()
    kt = k_tok.numpy()
    check_routing_and_plan(layer, dev, shape, k_tok=kt)
    tokens = np.arange(T)
    ref, _ = oracle_out(dev, shape, tokens, k_tok=kt)
    assert rel_err(out, ref) <= TOL
    del dev, layer, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,T,routing", [("mixtral", 1, "uniform"), ("mixtral", 32, "uniform"),
                                            ("qwen2", 32, "zipf"), ("deepseek_v3", 128, "zipf")])
def test_layer_parity_fp8_full_size(name, T, routing):
    """FP8 E4M3 expert and shared weights with row scales at full size, every token."""
    shape = configs.CONFIGS[name]
    print(f"\n[fp8 full-size parity] {name} T={T} {routing}", flush=True)
    dev = synth.layer_inputs(shape, T, routing, seed=0, device=DEV, dense=False)
    synth.add_fp8_weights(dev, drop_bf16=True)
    layer = MoELayer(shape, dev, fp8=True)
    out = layer.forward()
    torch.cuda.synchronize()
    rids = check_routing_and_plan(layer, dev, shape)
    ref, ids = oracle_out(dev, shape, np.arange(T), fp8=True)
    assert (ids == rids).all()
    assert rel_err(out, ref) <= TOL
    del dev, layer, out
    torch.cuda.empty_cache()
