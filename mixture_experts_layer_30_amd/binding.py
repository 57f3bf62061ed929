"""ctypes binding of libmoe_layer.so: one Python function per C entry point,
same names, argument marshalling only (device pointers from torch tensors,
the current HIP stream).  Every step of the layer runs in the library's HIP
kernels; if the library is missing this module raises instead of computing
anything another way.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_layer.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ECAPACITY, MOE_EHIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
SCHED_AUTO, SCHED_STREAM, SCHED_TILE, SCHED_RING, SCHED_SPAN = 0, 1, 2, 3, 4
PAD_BLOCK, PAD_MAX = 0, 1

# every function the C header declares
EXPORTS = ["moe_last_error", "moe_status_string", "moe_align_capacity", "moe_align_capacity_ex",
           "moe_ffn_workspace_bytes", "moe_ffn_workspace_bytes_ex", "dense_ffn_workspace_bytes",
           "moe_route", "moe_route_var", "moe_align", "moe_align_ex", "moe_route_align", "moe_grouped_ffn", "moe_grouped_gate_up", "moe_grouped_down",
           "moe_combine", "dense_ffn_fa", "moe_grouped_gate_up_fp8", "moe_grouped_down_fp8",
           "dense_ffn_fp8", "moe_grouped_ffn_noalloc"]

# workspace bytes held per GPU by moe_grouped_ffn_noalloc (MOE_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 128 << 20


class MoEError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class moe_plan(ctypes.Structure):
    _fields_ = [("expert_counts", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p),
                ("sorted_ids", ctypes.c_void_p), ("block_expert", ctypes.c_void_p),
                ("inv_pos", ctypes.c_void_p), ("block_m", ctypes.c_int32), ("cap", ctypes.c_int64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m mixture_experts_layer_30_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        P = ctypes.POINTER(moe_plan)
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [i32]
        L.moe_align_capacity.restype = i64
        L.moe_align_capacity.argtypes = [i64, i32, i32, i32]
        L.moe_align_capacity_ex.restype = i64
        L.moe_align_capacity_ex.argtypes = [i64, i32, i32, i32, i32]
        L.moe_ffn_workspace_bytes.restype = i64
        L.moe_ffn_workspace_bytes.argtypes = [i64, i32]
        L.moe_ffn_workspace_bytes_ex.restype = i64
        L.moe_ffn_workspace_bytes_ex.argtypes = [i64, i64, i32, i32, i32, i32]
        L.dense_ffn_workspace_bytes.restype = i64
        L.dense_ffn_workspace_bytes.argtypes = [i64, i32, i32]
        L.moe_route.restype = i32
        L.moe_route.argtypes = [vp, i64, i32, i32, vp, vp, vp]
        L.moe_route_var.restype = i32
        L.moe_route_var.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp]
        L.moe_align.restype = i32
        L.moe_align.argtypes = [vp, i64, i32, i32, P, vp]
        L.moe_align_ex.restype = i32
        L.moe_align_ex.argtypes = [vp, i64, i32, i32, P, i32, vp]
        L.moe_route_align.restype = i32
        L.moe_route_align.argtypes = [vp, i64, i32, i32, vp, vp, vp, P, i32, vp]
        L.moe_grouped_ffn.restype = i32
        L.moe_grouped_ffn.argtypes = [vp, i32, i64, i32, i32, i32, i32, vp, vp, P, vp, i64, vp, vp]
        L.moe_grouped_ffn_noalloc.restype = i32
        L.moe_grouped_ffn_noalloc.argtypes = [vp, i32, i64, i32, i32, i32, i32, vp, vp, P, vp, vp]
        L.moe_grouped_gate_up.restype = i32
        L.moe_grouped_gate_up.argtypes = [vp, i32, i64, i32, i32, i32, i32, vp, P, vp, i64, i32, vp]
        L.moe_grouped_down.restype = i32
        L.moe_grouped_down.argtypes = [vp, i32, i64, i32, i32, i32, i32, P, vp, i64, vp, i32, vp]
        L.moe_combine.restype = i32
        L.moe_combine.argtypes = [vp, i32, vp, vp, i32, i64, i32, i32, vp, i32, vp]
        L.dense_ffn_fa.restype = i32
        L.dense_ffn_fa.argtypes = [vp, i32, i64, i32, i32, vp, vp, vp, i64, vp, i32, i32, vp]
        L.moe_grouped_gate_up_fp8.restype = i32
        L.moe_grouped_gate_up_fp8.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, P, vp, i64, vp]
        L.moe_grouped_down_fp8.restype = i32
        L.moe_grouped_down_fp8.argtypes = [vp, vp, i64, i32, i32, i32, i32, P, vp, i64, vp, vp]
        L.dense_ffn_fp8.restype = i32
        L.dense_ffn_fp8.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, vp, i64, vp, i32, vp]
        _lib = L
    return _lib


def _check(status):
    if status != MOE_OK:
        raise MoEError(status, lib().moe_last_error().decode())


def _dt(t):
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise MoEError(MOE_EUNSUPPORTED, f"dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def moe_align_capacity(T, K, E, block_m):
    return lib().moe_align_capacity(T, K, E, block_m)


def moe_align_capacity_ex(T, K, E, block_m, pad):
    return lib().moe_align_capacity_ex(T, K, E, block_m, pad)


def moe_ffn_workspace_bytes(cap, I):
    return lib().moe_ffn_workspace_bytes(cap, I)


def moe_ffn_workspace_bytes_ex(cap, T, K, E, H, I):
    return lib().moe_ffn_workspace_bytes_ex(cap, T, K, E, H, I)


def dense_ffn_workspace_bytes(T, H, I):
    return lib().dense_ffn_workspace_bytes(T, H, I)


class Plan:
    """Device arrays of one alignment (see moe_plan in include/moe_layer.h)."""

    def __init__(self, T, K, E, block_m, device, cap=None, pad=PAD_BLOCK):
        self.T, self.K, self.E, self.block_m, self.pad = T, K, E, block_m, pad
        self.cap = moe_align_capacity_ex(T, K, E, block_m, pad) if cap is None else cap
        i32 = torch.int32
        self.expert_counts = torch.empty(E, dtype=i32, device=device)
        self.expert_offsets = torch.empty(E + 1, dtype=i32, device=device)
        self.sorted_ids = torch.empty(max(self.cap, 1), dtype=i32, device=device)
        self.block_expert = torch.empty(max(self.cap // block_m, 1), dtype=i32, device=device)
        self.inv_pos = torch.empty(max(T * K, 1), dtype=i32, device=device)
        self.c = moe_plan(self.expert_counts.data_ptr(), self.expert_offsets.data_ptr(),
                          self.sorted_ids.data_ptr(), self.block_expert.data_ptr(),
                          self.inv_pos.data_ptr(), block_m, self.cap)

    def arrays(self):
        return dict(expert_counts=self.expert_counts, expert_offsets=self.expert_offsets,
                    sorted_ids=self.sorted_ids[:self.cap], block_expert=self.block_expert[:self.cap // self.block_m],
                    inv_pos=self.inv_pos[:self.T * self.K])


def moe_route(logits, K, topk_ids, topk_w, stream=None):
    T, E = logits.shape
    _check(lib().moe_route(_ptr(logits), T, E, K, _ptr(topk_ids), _ptr(topk_w), _stream(stream)))


def moe_route_var(logits, Kmax, k_tok, topk_ids, topk_w, stream=None):
    """Routing with a per-token budget k_tok [T] int32 (device)."""
    T, E = logits.shape
    _check(lib().moe_route_var(_ptr(logits), T, E, Kmax, _ptr(k_tok), _ptr(topk_ids), _ptr(topk_w),
                               _stream(stream)))


def moe_align(topk_ids, E, plan, stream=None):
    T, K = topk_ids.shape
    _check(lib().moe_align(_ptr(topk_ids), T, K, E, ctypes.byref(plan.c), _stream(stream)))


def moe_align_ex(topk_ids, E, plan, pad, stream=None):
    T, K = topk_ids.shape
    _check(lib().moe_align_ex(_ptr(topk_ids), T, K, E, ctypes.byref(plan.c), pad, _stream(stream)))


def moe_route_align(logits, K, topk_ids, topk_w, plan, pad=None, k_tok=None, stream=None):
    """moe_route (or moe_route_var with budgets k_tok) then moe_align_ex, in one
    launch for small batches."""
    T, E = logits.shape
    _check(lib().moe_route_align(_ptr(logits), T, E, K, _ptr(k_tok) if k_tok is not None else None,
                                 _ptr(topk_ids), _ptr(topk_w), ctypes.byref(plan.c),
                                 PAD_BLOCK if pad is None else pad, _stream(stream)))


def moe_grouped_ffn(x, w13, w2, K, plan, workspace, y_pairs, stream=None):
    T, H = x.shape
    E, I2, _ = w13.shape
    _check(lib().moe_grouped_ffn(_ptr(x), _dt(x), T, H, I2 // 2, E, K, _ptr(w13), _ptr(w2),
                                 ctypes.byref(plan.c), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _ptr(y_pairs), _stream(stream)))


def moe_grouped_ffn_noalloc(x, w13, w2, K, plan, y_pairs, stream=None):
    """moe_grouped_ffn with the library's own per-GPU workspace (no workspace argument)."""
    T, H = x.shape
    E, I2, _ = w13.shape
    _check(lib().moe_grouped_ffn_noalloc(_ptr(x), _dt(x), T, H, I2 // 2, E, K, _ptr(w13), _ptr(w2),
                                         ctypes.byref(plan.c), _ptr(y_pairs), _stream(stream)))


def moe_grouped_gate_up(x, w13, K, plan, workspace, sched=SCHED_AUTO, stream=None):
    T, H = x.shape
    E, I2, _ = w13.shape
    _check(lib().moe_grouped_gate_up(_ptr(x), _dt(x), T, H, I2 // 2, E, K, _ptr(w13),
                                     ctypes.byref(plan.c), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), sched, _stream(stream)))


def moe_grouped_down(w2, T, K, plan, workspace, y_pairs, sched=SCHED_AUTO, stream=None):
    E, H, I = w2.shape
    _check(lib().moe_grouped_down(_ptr(w2), _dt(w2), T, H, I, E, K, ctypes.byref(plan.c),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _ptr(y_pairs), sched, _stream(stream)))


def moe_combine(y_pairs, topk_w, out, shared=None, stream=None):
    T, K = topk_w.shape
    H = out.shape[1]
    sdt = _dt(shared) if shared is not None else MOE_F32
    _check(lib().moe_combine(_ptr(y_pairs), _dt(y_pairs), _ptr(topk_w), _ptr(shared), sdt, T, K, H,
                             _ptr(out), _dt(out), _stream(stream)))


def dense_ffn_fa(x, w13, w2, workspace, out, sched=SCHED_AUTO, stream=None):
    T, H = x.shape
    I = w2.shape[1]
    _check(lib().dense_ffn_fa(_ptr(x), _dt(x), T, H, I, _ptr(w13), _ptr(w2), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _ptr(out), _dt(out),
                              sched, _stream(stream)))


def _need(t, dtype, what):
    """The FP8 entry points take no dtype argument for these tensors: check here."""
    if t.dtype != dtype:
        raise MoEError(MOE_EUNSUPPORTED, f"{what} must be {dtype}, got {t.dtype}")


def _fp8_weights(q, s, what):
    _need(q, torch.uint8, what + " codes")
    _need(s, torch.float32, what + " row scales")


def moe_grouped_gate_up_fp8(x, q13, s13, K, plan, workspace, stream=None):
    """FP8 E4M3 expert weights: q13 uint8 [E,2I,H] codes, s13 fp32 [E,2I] row scales; x bf16."""
    _need(x, torch.bfloat16, "x")
    _fp8_weights(q13, s13, "w13")
    T, H = x.shape
    E, I2, _ = q13.shape
    _check(lib().moe_grouped_gate_up_fp8(_ptr(x), T, H, I2 // 2, E, K, _ptr(q13), _ptr(s13),
                                         ctypes.byref(plan.c), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_grouped_down_fp8(q2, s2, T, K, plan, workspace, y_pairs, stream=None):
    """q2 uint8 [E,H,I] codes, s2 fp32 [E,H] row scales; y_pairs bf16."""
    _need(y_pairs, torch.bfloat16, "y_pairs")
    _fp8_weights(q2, s2, "w2")
    E, H, I = q2.shape
    _check(lib().moe_grouped_down_fp8(_ptr(q2), _ptr(s2), T, H, I, E, K, ctypes.byref(plan.c),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _ptr(y_pairs), _stream(stream)))


def dense_ffn_fp8(x, q13, s13, q2, s2, workspace, out, stream=None):
    """x bf16 [T,H]; q13/s13, q2/s2 FP8 codes and row scales; out bf16 or fp32."""
    _need(x, torch.bfloat16, "x")
    _fp8_weights(q13, s13, "w13")
    _fp8_weights(q2, s2, "w2")
    T, H = x.shape
    I = q2.shape[1]
    _check(lib().dense_ffn_fp8(_ptr(x), T, H, I, _ptr(q13), _ptr(s13), _ptr(q2), _ptr(s2),
                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _ptr(out), _dt(out), _stream(stream)))

