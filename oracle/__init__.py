"""CPU oracle of one MoE feed-forward layer pass -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The library's compute path never calls it; it shares no
code with the HIP kernels (the C source is compiled with gcc on its own).

Thin ctypes marshalling around ``moe_oracle.c``; every step of the arithmetic
is in that file.  Inputs are torch CPU tensors or numpy arrays, fp32 or bf16
(weights also FP8 E4M3 codes as uint8 with fp32 row scales); results are
float64 numpy arrays (routing ids and alignment arrays int32).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "moe_oracle.c")
LIB = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "libmoe_oracle.so")

F32, BF16, FP8 = 0, 1, 2
_lib = None


def build(force=True):
    """Compile the oracle with gcc (plain -O2, no fast-math, OpenMP)."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
                           "-Wextra", "-Wno-unused-parameter", SRC, "-o", tmp, "-lm"])
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        vp, i64, i32, dp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.orc_route.argtypes = [vp, i64, i32, i32, vp, vp]
        L.orc_route.restype = i32
        L.orc_route_var.argtypes = [vp, i64, i32, i32, vp, vp, vp]
        L.orc_route_var.restype = i32
        L.orc_align.argtypes = [vp, i64, i32, i32, i32, i64, vp, vp, vp, vp, vp]
        L.orc_align.restype = i32
        L.orc_align_mode.argtypes = [vp, i64, i32, i32, i32, i64, i32, vp, vp, vp, vp, vp]
        L.orc_align_mode.restype = i32
        L.orc_swiglu.argtypes = [vp, i32, i64, i32, i32, vp, vp, i32, dp]
        L.orc_swiglu.restype = i32
        L.orc_swiglu_s.argtypes = [vp, i32, i64, i32, i32, vp, vp, i32, vp, vp, dp]
        L.orc_swiglu_s.restype = i32
        L.orc_fp8_e4m3.argtypes = [ctypes.c_uint8]
        L.orc_fp8_e4m3.restype = ctypes.c_double
        L.orc_combine.argtypes = [dp, dp, dp, i64, i32, i32, dp]
        L.orc_combine.restype = None
        L.orc_moe_layer.argtypes = [vp, i32, vp, i64, i32, i32, i32, i32, vp, vp, i32, i32, vp, vp,
                                    vp, dp, dp]
        L.orc_moe_layer.restype = i32
        L.orc_moe_layer_s.argtypes = [vp, i32, vp, i64, i32, i32, i32, i32, vp, vp, i32, vp, vp, i32,
                                      vp, vp, vp, vp, vp, dp, dp]
        L.orc_moe_layer_s.restype = i32
        L.orc_moe_layer_k.argtypes = [vp, i32, vp, vp, i64, i32, i32, i32, i32, vp, vp, i32, vp, vp,
                                      i32, vp, vp, vp, vp, vp, dp, dp]
        L.orc_moe_layer_k.restype = i32
        L.orc_set_threads.argtypes = [i32]
        L.orc_max_threads.restype = i32
        _lib = L
    return _lib


def _arr(t):
    """(contiguous numpy array, dtype code) for fp32/bf16 torch tensors or numpy arrays."""
    if t is None:
        return None, F32
    if isinstance(t, np.ndarray):
        a = np.ascontiguousarray(t)
        if a.dtype == np.float32:
            return a, F32
        if a.dtype == np.uint16:
            return a, BF16
        if a.dtype == np.uint8:
            return a, FP8
        raise TypeError(f"unsupported numpy dtype {a.dtype}")
    import torch
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.float32:
        return t.numpy(), F32
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16), BF16
    if t.dtype == torch.uint8:
        return t.numpy(), FP8
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _scales(t):
    """fp32 row scales as a contiguous numpy array (or None)."""
    if t is None:
        return None
    if not isinstance(t, np.ndarray):
        t = t.detach().to("cpu").contiguous().numpy()
    a = np.ascontiguousarray(t, dtype=np.float32)
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    """Raises for a nonzero oracle return code (-3: a host allocation failed)."""
    if rc == -3:
        raise MemoryError(f"{what}: out of host memory")
    if rc:
        raise ValueError(f"{what}: bad arguments (code {rc})")


def set_threads(n):
    lib().orc_set_threads(int(n))


def max_threads():
    return lib().orc_max_threads()


def route(logits, K):
    """Softmax top-K routing; returns (ids int32 [T,K], w float64 [T,K])."""
    l, dt = _arr(logits)
    assert dt == F32, "router logits are fp32"
    T, E = l.shape
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float64)
    _check(lib().orc_route(_p(l), T, E, K, _p(ids), _p(w)), f"orc_route (E={E}, K={K})")
    return ids, w


def _budget(k_tok, T):
    k = np.ascontiguousarray(np.asarray(k_tok, dtype=np.int32).reshape(-1))
    assert k.shape == (T,), "one budget per token"
    return k


def route_var(logits, Kmax, k_tok):
    """Routing with a per-token budget k_t (clamped to [0, Kmax]): token t's
    first k_t slots as route(..., K=k_t), the rest id -1 and weight 0; returns
    (ids int32 [T,Kmax], w float64 [T,Kmax])."""
    l, dt = _arr(logits)
    assert dt == F32, "router logits are fp32"
    T, E = l.shape
    k = _budget(k_tok, T)
    ids = np.empty((T, Kmax), np.int32)
    w = np.empty((T, Kmax), np.float64)
    _check(lib().orc_route_var(_p(l), T, E, Kmax, _p(k), _p(ids), _p(w)),
           f"orc_route_var (E={E}, Kmax={Kmax})")
    return ids, w


PAD_MODES = {"block": 0, "max": 1}


def align(ids, E, B, cap, mode="block"):
    """Padded alignment of the T*K pairs (block-wise or max padding, Section 5.1
    of the Serving-tax notes); returns a dict of int32 arrays."""
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
    T, K = ids.shape
    out = dict(expert_counts=np.empty(E, np.int32), expert_offsets=np.empty(E + 1, np.int32),
               sorted_ids=np.empty(cap, np.int32), block_expert=np.empty(cap // B, np.int32),
               inv_pos=np.empty(T * K, np.int32))
    rc = lib().orc_align_mode(_p(ids), T, K, E, B, cap, PAD_MODES[mode], _p(out["expert_counts"]),
                              _p(out["expert_offsets"]), _p(out["sorted_ids"]),
                              _p(out["block_expert"]), _p(out["inv_pos"]))
    if rc == -2:
        raise ValueError("orc_align: padded total exceeds capacity")
    _check(rc, "orc_align")
    return out


def swiglu(x, w13, w2):
    """y = W2 (silu(W1 x) * (W3 x)) per row; w13 [2I,H], w2 [H,I]."""
    xa, xdt = _arr(x)
    a13, wdt = _arr(w13)
    a2, wdt2 = _arr(w2)
    assert wdt == wdt2
    n, H = xa.shape
    I = a13.shape[0] // 2
    assert a13.shape == (2 * I, H) and a2.shape == (H, I)
    y = np.empty((n, H), np.float64)
    _check(lib().orc_swiglu(_p(xa), xdt, n, H, I, _p(a13), _p(a2), wdt, _p(y)), "orc_swiglu")
    return y


dense_ffn = swiglu


def fp8_e4m3(code):
    """Value of one FP8 E4M3 code (0..255)."""
    return lib().orc_fp8_e4m3(int(code))


def swiglu_fp8(x, q13, s13, q2, s2):
    """SwiGLU with FP8 E4M3 weights (uint8 codes) times fp32 row scales:
    W13 = q13 * s13[:, None] ([2I,H], [2I]), W2 = q2 * s2[:, None] ([H,I], [H])."""
    xa, xdt = _arr(x)
    a13, wdt = _arr(q13)
    a2, wdt2 = _arr(q2)
    assert wdt == FP8 and wdt2 == FP8
    n, H = xa.shape
    I = a13.shape[0] // 2
    sc13, sc2 = _scales(s13), _scales(s2)
    assert a13.shape == (2 * I, H) and a2.shape == (H, I) and sc13.shape == (2 * I,) and sc2.shape == (H,)
    y = np.empty((n, H), np.float64)
    _check(lib().orc_swiglu_s(_p(xa), xdt, n, H, I, _p(a13), _p(a2), wdt, _p(sc13), _p(sc2), _p(y)),
           "orc_swiglu_s")
    return y


def moe_layer_fp8(x, logits, q13, s13, q2, s2, K, qs13=None, ss13=None, qs2=None, ss2=None):
    """Whole layer with FP8 E4M3 weights and fp32 row scales (routed experts
    q13 [E,2I,H] / s13 [E,2I], q2 [E,H,I] / s2 [E,H]; shared experts likewise);
    returns (out float64 [T,H], ids int32 [T,K], w float64 [T,K])."""
    xa, xdt = _arr(x)
    la, _ = _arr(logits)
    a13, wdt = _arr(q13)
    a2, _ = _arr(q2)
    assert wdt == FP8
    T, H = xa.shape
    E = a13.shape[0]
    I = a13.shape[1] // 2
    sc13, sc2 = _scales(s13), _scales(s2)
    assert a13.shape == (E, 2 * I, H) and a2.shape == (E, H, I) and la.shape == (T, E)
    assert sc13.shape == (E, 2 * I) and sc2.shape == (E, H)
    b13, _ = _arr(qs13)
    b2, _ = _arr(qs2)
    Is = 0 if b13 is None else b13.shape[0] // 2
    out = np.empty((T, H), np.float64)
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float64)
    rc = lib().orc_moe_layer_s(_p(xa), xdt, _p(la), T, H, I, E, K, _p(a13), _p(a2), wdt, _p(sc13),
                               _p(sc2), Is, _p(b13), _p(b2), _p(_scales(ss13)), _p(_scales(ss2)),
                               _p(ids), _p(w), _p(out))
    _check(rc, "orc_moe_layer")
    return out, ids, w


def combine(y, w, s=None):
    """out[t] = sum_k w[t,k] y[t*K+k] (+ s[t]); slots of weight 0 skipped."""
    w = np.ascontiguousarray(w, dtype=np.float64)
    T, K = w.shape
    y = np.ascontiguousarray(y, dtype=np.float64).reshape(T * K, -1)
    H = y.shape[1]
    s = None if s is None else np.ascontiguousarray(s, dtype=np.float64)
    out = np.empty((T, H), np.float64)
    lib().orc_combine(_p(y), _p(w), _p(s), T, K, H, _p(out))
    return out


def moe_layer_var(x, logits, w13, w2, Kmax, k_tok, ws13=None, ws2=None):
    """Whole layer with a per-token routing budget k_tok [T] (see route_var);
    returns (out float64 [T,H], ids int32 [T,Kmax], w float64 [T,Kmax])."""
    xa, xdt = _arr(x)
    la, _ = _arr(logits)
    a13, wdt = _arr(w13)
    a2, _ = _arr(w2)
    T, H = xa.shape
    E = a13.shape[0]
    I = a13.shape[1] // 2
    assert a13.shape == (E, 2 * I, H) and a2.shape == (E, H, I) and la.shape == (T, E)
    k = _budget(k_tok, T)
    s13, _ = _arr(ws13)
    s2, _ = _arr(ws2)
    Is = 0 if s13 is None else s13.shape[0] // 2
    out = np.empty((T, H), np.float64)
    ids = np.empty((T, Kmax), np.int32)
    w = np.empty((T, Kmax), np.float64)
    rc = lib().orc_moe_layer_k(_p(xa), xdt, _p(la), _p(k), T, H, I, E, Kmax, _p(a13), _p(a2), wdt,
                               None, None, Is, _p(s13), _p(s2), None, None, _p(ids), _p(w), _p(out))
    _check(rc, "orc_moe_layer_k")
    return out, ids, w


def moe_layer(x, logits, w13, w2, K, ws13=None, ws2=None):
    """Whole layer; returns (out float64 [T,H], ids int32 [T,K], w float64 [T,K])."""
    xa, xdt = _arr(x)
    la, _ = _arr(logits)
    a13, wdt = _arr(w13)
    a2, _ = _arr(w2)
    T, H = xa.shape
    E = a13.shape[0]
    I = a13.shape[1] // 2
    assert a13.shape == (E, 2 * I, H) and a2.shape == (E, H, I) and la.shape == (T, E)
    s13, _ = _arr(ws13)
    s2, _ = _arr(ws2)
    Is = 0 if s13 is None else s13.shape[0] // 2
    out = np.empty((T, H), np.float64)
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float64)
    rc = lib().orc_moe_layer(_p(xa), xdt, _p(la), T, H, I, E, K, _p(a13), _p(a2), wdt, Is,
                             _p(s13), _p(s2), _p(ids), _p(w), _p(out))
    _check(rc, "orc_moe_layer")
    return out, ids, w
