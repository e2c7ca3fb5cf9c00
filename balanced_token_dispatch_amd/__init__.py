"""Python binding of libmoe.so: the one-rank hot path of a redundant-expert MoE layer.

Argument marshalling only.  Every step runs in the HIP kernels of
libmoe.so (see include/moe.h for each call's contract); this module turns
torch tensors into device pointers and torch's current stream into a
hipStream_t.  Importing it fails loudly when the library is not built.
"""
import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is not built; build it with `python balanced_token_dispatch_amd/_build.py`")

_lib = ctypes.CDLL(_LIB_PATH)

MOE_OK, MOE_EINVAL, MOE_ENOSPACE, MOE_EHIP = 0, 1, 2, 3
DEV_BAD_EXPERT_ID, DEV_SLOT_OVERFLOW = 1, 2
F32, BF16 = 0, 1
GEMM_FWD, GEMM_DGRAD, GEMM_WGRAD = 0, 1, 2

EXPORTS = ("moe_status_string", "moe_plan_words", "moe_plan_workspace_bytes", "moe_plan",
           "moe_dispatch_layout_workspace_bytes", "moe_dispatch_layout", "moe_prefetch",
           "moe_permute", "moe_group_gemm", "moe_combine", "moe_replica_grad_fold",
           "moe_unpermute_reduce", "moe_combine_weight_grad", "moe_group_gemm_swiglu",
           "moe_swiglu_backward", "moe_group_gemm_workspace_bytes", "moe_plan_noalloc",
           "moe_group_gemm_gather")

PLAN_NOALLOC_SCRATCH_BYTES = 4 << 20   # MOE_PLAN_NOALLOC_SCRATCH_BYTES in moe.h


class MoeDims(ctypes.Structure):
    _fields_ = [("R", ctypes.c_int32), ("S", ctypes.c_int32), ("K", ctypes.c_int32),
                ("E", ctypes.c_int32), ("B", ctypes.c_int32)]


_P = ctypes.c_void_p
_D = ctypes.POINTER(MoeDims)
_I32, _I64, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t

_lib.moe_status_string.restype = ctypes.c_char_p
_lib.moe_status_string.argtypes = [ctypes.c_int]
for _n in ("moe_plan_words", "moe_plan_workspace_bytes", "moe_dispatch_layout_workspace_bytes"):
    getattr(_lib, _n).restype = _SZ
    getattr(_lib, _n).argtypes = [_D]
_lib.moe_plan.argtypes = [_D, _P, _P, _P, _P, _P, _SZ, _P]
_lib.moe_plan_noalloc.argtypes = [_D, _P, _P, _P, _P, _P]
_lib.moe_dispatch_layout.argtypes = [_D, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]
_lib.moe_prefetch.argtypes = [_D, _I32, _P, _P, _I64, _P]
_lib.moe_permute.argtypes = [_D, ctypes.c_int, _I64, _P, _P, _P, _P, _P]
_lib.moe_group_gemm_workspace_bytes.restype = _SZ
_lib.moe_group_gemm_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
_lib.moe_group_gemm.argtypes = [ctypes.c_int, ctypes.c_int, _I32, _I32, _I32, _I32, _P, _P, _P,
                                _P, _P, _SZ, _P]
_lib.moe_group_gemm_gather.argtypes = [ctypes.c_int, ctypes.c_int, _I32, _I32, _I32, _I32, _P, _I64,
                                       _P, _I32, _P, _P, _P, _P, _SZ, _P]
_lib.moe_combine.argtypes = [_D, ctypes.c_int, _I64, _I32, _P, _P, _P, _P, _P]
_lib.moe_replica_grad_fold.argtypes = [_D, _I32, _P, _P, _I64, _P]
_lib.moe_unpermute_reduce.argtypes = [_D, ctypes.c_int, _I64, _I32, _P, _P, _P, _P]
_lib.moe_combine_weight_grad.argtypes = [_D, ctypes.c_int, _I64, _I32, _P, _P, _P, _P, _P]
_lib.moe_group_gemm_swiglu.argtypes = [ctypes.c_int, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P,
                                       _P, _SZ, _P]
_lib.moe_swiglu_backward.argtypes = [ctypes.c_int, _I64, _I64, _P, _P, _P, _P]
for _n in EXPORTS[3:]:
    if _n.endswith("_bytes"):
        continue
    getattr(_lib, _n).restype = ctypes.c_int


class MoeError(RuntimeError):
    pass


def library():
    """The loaded ctypes library (for tests that call the C ABI directly)."""
    return _lib


def dims(R, S, K, E, B):
    return MoeDims(R, S, K, E, B)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc, name):
    if rc != MOE_OK:
        raise MoeError(f"{name}: {_lib.moe_status_string(rc).decode()} (status {rc})")


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise MoeError(f"unsupported dtype {t.dtype}")


def plan_words(d):
    return int(_lib.moe_plan_words(ctypes.byref(d)))


def plan_workspace_bytes(d):
    return int(_lib.moe_plan_workspace_bytes(ctypes.byref(d)))


def dispatch_layout_workspace_bytes(d):
    return int(_lib.moe_dispatch_layout_workspace_bytes(ctypes.byref(d)))


def moe_plan(d, topk_idx, counts, plan, dev_status, ws, stream=None):
    _check(_lib.moe_plan(ctypes.byref(d), _ptr(topk_idx), _ptr(counts), _ptr(plan),
                         _ptr(dev_status), _ptr(ws), ws.numel() * ws.element_size(),
                         _stream(stream)), "moe_plan")


def moe_plan_noalloc(d, topk_idx, counts, plan, dev_status, stream=None):
    """moe_plan without a workspace: the library's static per-GPU scratch (see moe.h)."""
    _check(_lib.moe_plan_noalloc(ctypes.byref(d), _ptr(topk_idx), _ptr(counts), _ptr(plan),
                                 _ptr(dev_status), _stream(stream)), "moe_plan_noalloc")


def moe_dispatch_layout(d, rank, topk_idx, plan, cu_seqlens, dest_pos, src_flat, ws, stream=None):
    _check(_lib.moe_dispatch_layout(ctypes.byref(d), rank, _ptr(topk_idx), _ptr(plan),
                                    _ptr(cu_seqlens), _ptr(dest_pos), _ptr(src_flat), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)),
           "moe_dispatch_layout")


def moe_prefetch(d, rank, plan, w, stream=None):
    row_bytes = w[0].numel() * w.element_size()
    _check(_lib.moe_prefetch(ctypes.byref(d), rank, _ptr(plan), _ptr(w), row_bytes,
                             _stream(stream)), "moe_prefetch")


def moe_permute(d, x_all, src_flat, xp, row_scale=None, stream=None):
    _check(_lib.moe_permute(ctypes.byref(d), _dtype(x_all), x_all.shape[1], _ptr(x_all),
                            _ptr(src_flat), _ptr(row_scale), _ptr(xp), _stream(stream)),
           "moe_permute")


def group_gemm_workspace_bytes(op, dtype=BF16):
    return _lib.moe_group_gemm_workspace_bytes(op, dtype)


def _ws(ws):
    return (None, 0) if ws is None else (_ptr(ws), ws.numel() * ws.element_size())


def moe_group_gemm(op, a, b, cu_seqlens, out, Kd, N, ws=None, stream=None):
    """ws: optional scratch tensor of at least group_gemm_workspace_bytes(op) bytes."""
    G = cu_seqlens.numel() - 1
    wp, wn = _ws(ws)
    _check(_lib.moe_group_gemm(op, _dtype(a), G, a.shape[0], Kd, N, _ptr(a), _ptr(b),
                               _ptr(cu_seqlens), _ptr(out), wp, wn, _stream(stream)),
           "moe_group_gemm")


def moe_group_gemm_gather(op, x_src, gather, gather_div, b, cu_seqlens, out, Kd, N, ws=None,
                          stream=None):
    """moe_group_gemm (FWD or WGRAD) with row m of the row operand read from token row
    x_src[gather[m] // gather_div]: the permute fused into the GEMM."""
    G = cu_seqlens.numel() - 1
    wp, wn = _ws(ws)
    _check(_lib.moe_group_gemm_gather(op, _dtype(x_src), G, gather.numel(), Kd, N, _ptr(x_src),
                                      x_src.shape[0], _ptr(gather), gather_div, _ptr(b),
                                      _ptr(cu_seqlens), _ptr(out), wp, wn, _stream(stream)),
           "moe_group_gemm_gather")


def moe_group_gemm_swiglu(a, b, cu_seqlens, z, h, Kd, N, ws=None, stream=None):
    """Gated up-projection: z = silu(gate) * up over (gate, up) column pairs of W; h optional."""
    G = cu_seqlens.numel() - 1
    wp, wn = _ws(ws)
    _check(_lib.moe_group_gemm_swiglu(_dtype(a), G, a.shape[0], Kd, N, _ptr(a), _ptr(b),
                                      _ptr(cu_seqlens), _ptr(z), _ptr(h), wp, wn,
                                      _stream(stream)),
           "moe_group_gemm_swiglu")


def moe_swiglu_backward(h, dz, dh, stream=None):
    _check(_lib.moe_swiglu_backward(_dtype(h), dz.shape[0], dz.shape[1], _ptr(h), _ptr(dz),
                                    _ptr(dh), _stream(stream)), "moe_swiglu_backward")


def moe_combine(d, rank, y_all, dest_pos, topk_w, out, stream=None):
    _check(_lib.moe_combine(ctypes.byref(d), _dtype(y_all), y_all.shape[1], rank, _ptr(y_all),
                            _ptr(dest_pos), _ptr(topk_w), _ptr(out), _stream(stream)),
           "moe_combine")


def moe_unpermute_reduce(d, rank, dxp_all, dest_pos, dx, stream=None):
    _check(_lib.moe_unpermute_reduce(ctypes.byref(d), _dtype(dxp_all), dxp_all.shape[1], rank,
                                     _ptr(dxp_all), _ptr(dest_pos), _ptr(dx), _stream(stream)),
           "moe_unpermute_reduce")


def moe_combine_weight_grad(d, rank, y_all, dest_pos, dout, dw, stream=None):
    _check(_lib.moe_combine_weight_grad(ctypes.byref(d), _dtype(y_all), y_all.shape[1], rank,
                                        _ptr(y_all), _ptr(dest_pos), _ptr(dout), _ptr(dw),
                                        _stream(stream)), "moe_combine_weight_grad")


def moe_replica_grad_fold(d, rank, plan, dw, stream=None):
    _check(_lib.moe_replica_grad_fold(ctypes.byref(d), rank, _ptr(plan), _ptr(dw),
                                      dw[0].numel(), _stream(stream)), "moe_replica_grad_fold")
