"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments with the documented status before launching
anything (every call here returns during argument checking)."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_30_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_layer.h")

FAKE = 0x10000  # an aligned, never dereferenced address
NULL = None


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from mixture_experts_layer_30_amd import build
        build.build()
    return B.lib()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\([^;{]*\)\s*;", src)))


def test_exports_every_declared_function(L):
    names = header_functions()
    assert set(names) == set(B.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    assert L.moe_status_string(0) == b"ok"
    assert L.moe_status_string(3) == b"capacity or workspace too small"


def test_align_capacity_bound(L):
    # T*K + min(E, T*K)*(B-1), rounded up to B
    assert B.moe_align_capacity(128, 8, 256, 16) == 1024 + 256 * 15
    assert B.moe_align_capacity(2048, 8, 64, 128) == 16384 + 64 * 127 + 64
    assert B.moe_align_capacity(1, 2, 8, 128) == 256
    assert B.moe_align_capacity(0, 2, 8, 16) == 0
    assert B.moe_align_capacity(-1, 2, 8, 16) == -1
    assert B.moe_ffn_workspace_bytes(4864, 2048) == 4864 * 2048 * 2
    # max padding: E slots of ceil(T/B)*B rows (no expert holds more than T pairs)
    assert B.moe_align_capacity_ex(128, 8, 256, 16, B.PAD_BLOCK) == B.moe_align_capacity(128, 8, 256, 16)
    assert B.moe_align_capacity_ex(100, 2, 8, 64, B.PAD_MAX) == 8 * 128
    assert B.moe_align_capacity_ex(100, 2, 8, 64, 7) == -1
    # grouped FFN with room for a contraction split: the activations (256-byte
    # rounded) plus fp32 partial sums per pair, only where few experts can have
    # tokens (Mixtral at one token: 2 experts x 32 down slabs) ...
    cap = B.moe_align_capacity(1, 2, 8, 16)
    ex = B.moe_ffn_workspace_bytes_ex(cap, 1, 2, 8, 4096, 14336)
    assert ex > B.moe_ffn_workspace_bytes(cap, 14336)
    assert (ex - cap * 14336 * 2) % (2 * 4096 * 4) == 0   # whole [split][pairs][H] fp32 slices
    # ... and not once the experts' slabs fill the GPU or a pass cannot hold the tokens
    cap = B.moe_align_capacity(32, 2, 8, 16)
    assert B.moe_ffn_workspace_bytes_ex(cap, 32, 2, 8, 4096, 14336) == cap * 14336 * 2
    cap = B.moe_align_capacity(2048, 8, 64, 128)
    assert B.moe_ffn_workspace_bytes_ex(cap, 2048, 8, 64, 3584, 2560) == cap * 2560 * 2
    assert B.moe_ffn_workspace_bytes_ex(cap, 2048, 0, 64, 3584, 2560) == -1
    assert B.moe_ffn_workspace_bytes_ex(-1, 1, 2, 8, 4096, 14336) == -1
    # activations (128-row rounded) plus split-K partial sums
    assert B.dense_ffn_workspace_bytes(1, 128, 512) >= 128 * 512 * 2
    assert B.dense_ffn_workspace_bytes(1, 100, 512) == -1
    assert B.dense_ffn_workspace_bytes(0, 4096, 28672) >= 0   # empty batch


def st(r):
    return int(r)


def route(L, T=4, E=8, K=2, logits=FAKE, ids=FAKE, w=FAKE):
    return st(L.moe_route(logits, T, E, K, ids, w, None))


def test_route_argument_checks(L):
    assert route(L, K=9) == B.MOE_EINVAL
    assert route(L, K=0) == B.MOE_EINVAL
    assert route(L, T=-1) == B.MOE_EINVAL
    assert route(L, E=300, K=2) == B.MOE_EUNSUPPORTED
    assert route(L, logits=NULL) == B.MOE_EINVAL
    assert route(L, ids=FAKE + 2) == B.MOE_EINVAL
    assert b"NULL or misaligned" in L.moe_last_error()
    assert route(L, T=0, logits=NULL, ids=NULL, w=NULL) == B.MOE_OK  # empty batch: no-op


def test_route_var_argument_checks(L):
    def rv(T=4, E=8, K=2, logits=FAKE, k=FAKE, ids=FAKE, w=FAKE):
        return st(L.moe_route_var(logits, T, E, K, k, ids, w, None))
    assert rv(K=9) == B.MOE_EINVAL
    assert rv(K=0) == B.MOE_EINVAL
    assert rv(E=300, K=2) == B.MOE_EUNSUPPORTED
    assert rv(k=NULL) == B.MOE_EINVAL
    assert rv(k=FAKE + 2) == B.MOE_EINVAL
    assert b"moe_route_var" in L.moe_last_error()
    assert rv(T=0, logits=NULL, k=NULL, ids=NULL, w=NULL) == B.MOE_OK  # empty batch: no-op


def plan(cap=4864, block_m=16, ptr=FAKE):
    return B.moe_plan(ptr, ptr, ptr, ptr, ptr, block_m, cap)


def test_align_argument_checks(L):
    small = plan(cap=4848)
    assert st(L.moe_align(FAKE, 128, 8, 256, ctypes.byref(small), None)) == B.MOE_ECAPACITY
    odd = plan(cap=4865)
    assert st(L.moe_align(FAKE, 128, 8, 256, ctypes.byref(odd), None)) == B.MOE_EINVAL
    nullp = plan(ptr=0)
    assert st(L.moe_align(FAKE, 128, 8, 256, ctypes.byref(nullp), None)) == B.MOE_EINVAL
    assert st(L.moe_align(FAKE, 128, 8, 256, None, None)) == B.MOE_EINVAL
    bad_b = plan(block_m=0)
    assert st(L.moe_align(FAKE, 128, 8, 256, ctypes.byref(bad_b), None)) == B.MOE_EUNSUPPORTED
    # max padding needs E * ceil(T/B)*B rows; an unknown scheme is refused
    assert st(L.moe_align_ex(FAKE, 128, 8, 256, ctypes.byref(plan(cap=4864)), B.PAD_MAX,
                             None)) == B.MOE_ECAPACITY
    assert st(L.moe_align_ex(FAKE, 128, 8, 256, ctypes.byref(plan(cap=4864)), 5,
                             None)) == B.MOE_EINVAL


def test_grouped_ffn_argument_checks(L):
    p = plan(cap=4864)
    ws = B.moe_ffn_workspace_bytes(4864, 2048)
    args = lambda **kw: dict(dict(x=FAKE, dt=B.MOE_BF16, T=128, H=7168, I=2048, E=256, K=8,  # noqa: E731
                                  w13=FAKE, w2=FAKE, ws=ws, y=FAKE), **kw)

    def call(a):
        return st(L.moe_grouped_ffn(a["x"], a["dt"], a["T"], a["H"], a["I"], a["E"], a["K"],
                                    a["w13"], a["w2"], ctypes.byref(p), FAKE, a["ws"], a["y"], None))
    assert call(args(H=7000)) == B.MOE_EUNSUPPORTED
    assert call(args(I=2050)) == B.MOE_EUNSUPPORTED
    assert call(args(dt=7)) == B.MOE_EUNSUPPORTED
    assert call(args(ws=ws - 1)) == B.MOE_ECAPACITY
    assert call(args(x=NULL)) == B.MOE_EINVAL
    assert call(args(w13=FAKE + 8)) == B.MOE_EINVAL
    assert call(args(K=9, E=8)) == B.MOE_EINVAL
    assert call(args(T=0)) == B.MOE_OK


def test_fp8_argument_checks(L):
    p = plan(cap=4864)
    ws = B.moe_ffn_workspace_bytes(4864, 2048)
    # H not a multiple of 128
    assert st(L.moe_grouped_gate_up_fp8(FAKE, 128, 192, 2048, 256, 8, FAKE, FAKE, ctypes.byref(p), FAKE,
                                        ws, None)) == B.MOE_EUNSUPPORTED
    # missing scales
    assert st(L.moe_grouped_gate_up_fp8(FAKE, 128, 7168, 2048, 256, 8, FAKE, NULL, ctypes.byref(p), FAKE,
                                        ws, None)) == B.MOE_EINVAL
    assert st(L.moe_grouped_down_fp8(FAKE, NULL, 128, 7168, 2048, 256, 8, ctypes.byref(p), FAKE, ws, FAKE,
                                     None)) == B.MOE_EINVAL
    # workspace too small
    assert st(L.moe_grouped_down_fp8(FAKE, FAKE, 128, 7168, 2048, 256, 8, ctypes.byref(p), FAKE, ws - 1,
                                     FAKE, None)) == B.MOE_ECAPACITY
    assert st(L.dense_ffn_fp8(FAKE, 4, 4096, 14400, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, FAKE,
                              B.MOE_BF16, None)) == B.MOE_EUNSUPPORTED
    # empty batch: no-op
    assert st(L.dense_ffn_fp8(NULL, 0, 4096, 14336, FAKE, FAKE, FAKE, FAKE, NULL, 1 << 30, NULL,
                              B.MOE_BF16, None)) == B.MOE_OK


def test_combine_and_dense_argument_checks(L):
    assert st(L.moe_combine(FAKE, B.MOE_BF16, FAKE, None, B.MOE_F32, 4, 2, 100, FAKE, B.MOE_BF16,
                            None)) == B.MOE_EUNSUPPORTED
    assert st(L.moe_combine(FAKE, B.MOE_BF16, NULL, None, B.MOE_F32, 4, 2, 128, FAKE, B.MOE_BF16,
                            None)) == B.MOE_EINVAL
    assert st(L.moe_combine(FAKE, B.MOE_BF16, FAKE, FAKE + 4, B.MOE_F32, 4, 2, 128, FAKE,
                            B.MOE_BF16, None)) == B.MOE_EINVAL
    ws = B.dense_ffn_workspace_bytes(32, 4096, 28672)
    assert st(L.dense_ffn_fa(FAKE, B.MOE_BF16, 32, 4096, 28672, FAKE, FAKE, FAKE, ws - 2, FAKE,
                             B.MOE_BF16, 0, None)) == B.MOE_ECAPACITY
    assert st(L.dense_ffn_fa(FAKE, B.MOE_BF16, 32, 4096, 28600, FAKE, FAKE, FAKE, ws, FAKE,
                             B.MOE_BF16, 0, None)) == B.MOE_EUNSUPPORTED
    assert st(L.dense_ffn_fa(FAKE, B.MOE_BF16, -1, 4096, 28672, FAKE, FAKE, FAKE, ws, FAKE,
                             B.MOE_BF16, 0, None)) == B.MOE_EINVAL


def test_binding_refuses_to_run_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(ImportError):
        B.lib()


def test_fp8_binding_rejects_other_activation_dtypes(L):
    """The FP8 entry points take no dtype for x and y_pairs (bf16 by definition):
    the binding refuses other dtypes before calling the library."""
    import torch
    x32 = torch.zeros(4, 128)
    q = torch.zeros(2, 256, 128, dtype=torch.uint8)
    s = torch.ones(2, 256)
    p = B.Plan(4, 1, 2, 16, "cpu")
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    with pytest.raises(B.MoEError) as e:
        B.moe_grouped_gate_up_fp8(x32, q, s, 1, p, ws)
    assert e.value.status == B.MOE_EUNSUPPORTED
    with pytest.raises(B.MoEError):   # scales must be fp32
        B.moe_grouped_gate_up_fp8(x32.bfloat16(), q, s.double(), 1, p, ws)
    q2 = torch.zeros(2, 128, 128, dtype=torch.uint8)
    with pytest.raises(B.MoEError):
        B.moe_grouped_down_fp8(q2, torch.ones(2, 128), 4, 1, p, ws, torch.zeros(4, 128))
    with pytest.raises(B.MoEError):
        B.dense_ffn_fp8(x32, q[0], s[0], q2[0], torch.ones(128), ws, torch.zeros(4, 128))


def test_layer_rejects_fp8_with_fp32_tokens():
    import torch
    from mixture_experts_layer_30_amd.configs import LayerShape
    from mixture_experts_layer_30_amd.layer import MoELayer
    shape = LayerShape("t", 128, 128, 2, 1, 0, "f32", (4,), ("uniform",))
    with pytest.raises(B.MoEError):
        MoELayer(shape, {"x": torch.zeros(4, 128), "logits": torch.zeros(4, 2)}, fp8=True)


def test_noalloc_argument_checks(L):
    """moe_grouped_ffn_noalloc checks its plan against the library's array before
    any device call; an empty batch returns without touching the device."""
    assert st(L.moe_grouped_ffn_noalloc(FAKE, B.MOE_BF16, 32, 4096, 14336, 8, 2, FAKE, FAKE, None,
                                        FAKE, None)) == B.MOE_EINVAL
    big = plan(cap=33792)   # 33792 rows x 14336 x 2 B of activations: far above the array
    assert B.moe_ffn_workspace_bytes(33792, 14336) > B.NOALLOC_SCRATCH_BYTES
    assert st(L.moe_grouped_ffn_noalloc(FAKE, B.MOE_BF16, 16384, 4096, 14336, 8, 2, FAKE, FAKE,
                                        ctypes.byref(big), FAKE, None)) == B.MOE_ECAPACITY
    assert "allocation-free" in L.moe_last_error().decode()
    small = plan(cap=192)
    assert st(L.moe_grouped_ffn_noalloc(NULL, B.MOE_BF16, 0, 4096, 14336, 8, 2, FAKE, FAKE,
                                        ctypes.byref(small), NULL, None)) == B.MOE_OK
