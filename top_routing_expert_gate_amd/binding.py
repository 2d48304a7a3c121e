"""ctypes binding of libmoe (include/moe.h): argument marshalling only.

Every function here has the name and argument order of its C entry point.
Tensor arguments are torch tensors on the GPU (or raw device addresses as
ints, or None for NULL); ``stream`` defaults to torch's current stream.
Statuses 1-4 and 6 raise ValueError, status 5 raises RuntimeError.  All compute
runs in the HIP kernels of libmoe; there is no fallback of any kind: if the
library is missing this module raises on first use.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; MOE_LIBRARY may point at another build of the same ABI
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(_PKG, "libmoe.so")
# the same library built with the routing check inside moe_dispatch
DEBUG_LIB_PATH = os.path.join(_PKG, "libmoe_debug.so")

# enums of include/moe.h
(MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP,
 MOE_ERR_TOO_LARGE) = range(7)
MOE_F32, MOE_BF16 = 0, 1
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID, MOE_SCORE_SOFTMAX_ALL = 0, 1, 2
MOE_EXPERT_SILU_MLP, MOE_EXPERT_SWIGLU, MOE_EXPERT_GELU_MLP = 0, 1, 2
MOE_DROP_ZERO, MOE_DROP_RESIDUAL = 0, 1
MOE_MAX_EXPERTS = 256

EXPORTS = ["moe_capacity", "moe_routed_rows_max", "moe_workspace_size", "moe_status_str",
           "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_balance_stats",
           "moe_forward", "moe_forward_noalloc", "moe_scratch_bytes", "moe_check_routing",
           "moe_debug_checks"]


class MoeDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("score_fn", ctypes.c_int32), ("expert_kind", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("d_ff_shared", ctypes.c_int32),
                ("drop_policy", ctypes.c_int32), ("capacity", ctypes.c_int64)]


_WEIGHT_FIELDS = ["w_router", "router_bias", "sel_bias", "w_act", "w_lin", "w_down", "b_act",
                  "b_down", "ws_act", "ws_lin", "ws_down", "bs_act", "bs_down"]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WEIGHT_FIELDS]


_AUX_FIELDS = ["logits", "topk_idx", "topk_w", "counts_assigned", "counts_kept", "n_dropped",
               "balance", "p_mean"]


class MoeForwardAux(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _AUX_FIELDS] + [("balance_coef", ctypes.c_float)]


_lib = None
_debug_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built in-tree); raise if it is not there."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def debug_lib() -> ctypes.CDLL:
    """Load libmoe_debug.so, the build whose moe_dispatch checks its routing
    (same ABI; its entry points are called through the returned handle)."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = _load(DEBUG_LIB_PATH)
    return _debug_lib


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m top_routing_expert_gate_amd.build`")
    if True:
        L = ctypes.CDLL(path)
        vp, P = ctypes.c_void_p, ctypes.POINTER
        L.moe_capacity.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_double]
        L.moe_capacity.restype = ctypes.c_int64
        L.moe_routed_rows_max.argtypes = [P(MoeDesc)]
        L.moe_routed_rows_max.restype = ctypes.c_int64
        L.moe_workspace_size.argtypes = [P(MoeDesc)]
        L.moe_workspace_size.restype = ctypes.c_size_t
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_route.argtypes = [P(MoeDesc), P(MoeWeights), vp, vp, vp, vp, vp, vp]
        L.moe_dispatch.argtypes = [P(MoeDesc), vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.moe_expert_ffn.argtypes = [P(MoeDesc), P(MoeWeights), vp, vp, vp, vp, vp,
                                     ctypes.c_size_t, vp]
        L.moe_combine.argtypes = [P(MoeDesc), vp, vp, vp, vp, vp, vp, vp]
        L.moe_balance_stats.argtypes = [P(MoeDesc), vp, vp, ctypes.c_float, vp, vp, vp,
                                        ctypes.c_size_t, vp]
        L.moe_forward.argtypes = [P(MoeDesc), P(MoeWeights), vp, vp, P(MoeForwardAux), vp,
                                  ctypes.c_size_t, vp]
        L.moe_forward_noalloc.argtypes = [P(MoeDesc), P(MoeWeights), vp, vp, P(MoeForwardAux), vp]
        L.moe_scratch_bytes.argtypes = []
        L.moe_scratch_bytes.restype = ctypes.c_size_t
        L.moe_check_routing.argtypes = [P(MoeDesc), vp, vp, vp]
        L.moe_debug_checks.argtypes = []
        for f in ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine",
                  "moe_balance_stats", "moe_forward", "moe_forward_noalloc", "moe_check_routing",
                  "moe_debug_checks"):
            getattr(L, f).restype = ctypes.c_int
    return L


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int) -> None:
    if status == MOE_OK:
        return
    msg = lib().moe_status_str(status).decode()
    if status == MOE_ERR_HIP:
        raise RuntimeError(f"libmoe: {msg}")
    raise ValueError(f"libmoe status {status}: {msg}")


def make_desc(T: int, d_model: int, d_ff: int, E: int, k: int, dtype: int, score_fn: int,
              expert_kind: int, n_shared: int = 0, capacity: int = -1,
              d_ff_shared: Optional[int] = None, drop_policy: int = MOE_DROP_ZERO) -> MoeDesc:
    return MoeDesc(T=T, d_model=d_model, d_ff=d_ff, E=E, k=k, dtype=dtype, score_fn=score_fn,
                   expert_kind=expert_kind, n_shared=n_shared,
                   d_ff_shared=d_ff if d_ff_shared is None else d_ff_shared,
                   drop_policy=drop_policy, capacity=capacity)


def make_weights(**tensors) -> MoeWeights:
    """MoeWeights from keyword tensors named like the C struct members.  The
    returned struct keeps references to the tensors."""
    unknown = set(tensors) - set(_WEIGHT_FIELDS)
    if unknown:
        raise TypeError(f"unknown weight names {sorted(unknown)}")
    w = MoeWeights(**{n: _ptr(t) for n, t in tensors.items()})
    w._keep = dict(tensors)
    return w


def make_aux(balance_coef: float = 0.0, **tensors) -> MoeForwardAux:
    unknown = set(tensors) - set(_AUX_FIELDS)
    if unknown:
        raise TypeError(f"unknown aux names {sorted(unknown)}")
    a = MoeForwardAux(balance_coef=balance_coef, **{n: _ptr(t) for n, t in tensors.items()})
    a._keep = dict(tensors)
    return a


# ---------------------------------------------------------------------------
# entry points (names and argument order of include/moe.h)
# ---------------------------------------------------------------------------

def moe_capacity(T: int, E: int, capacity_factor: float) -> int:
    return int(lib().moe_capacity(T, E, capacity_factor))


def moe_routed_rows_max(desc: MoeDesc) -> int:
    return int(lib().moe_routed_rows_max(ctypes.byref(desc)))


def moe_workspace_size(desc: MoeDesc) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(desc)))


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def moe_route(desc, weights, x, logits_in, logits_out, topk_idx, topk_w, stream=None) -> None:
    w = ctypes.byref(weights) if weights is not None else None
    _check(lib().moe_route(ctypes.byref(desc), w, _ptr(x), _ptr(logits_in), _ptr(logits_out),
                           _ptr(topk_idx), _ptr(topk_w), _stream(stream)))


def moe_dispatch(desc, topk_idx, counts_assigned, counts_kept, offsets, sorted_token, row_of,
                 n_dropped, ws, stream=None) -> None:
    _check(lib().moe_dispatch(ctypes.byref(desc), _ptr(topk_idx), _ptr(counts_assigned),
                              _ptr(counts_kept), _ptr(offsets), _ptr(sorted_token), _ptr(row_of),
                              _ptr(n_dropped), _ptr(ws), _nbytes(ws) if ws is not None else 0,
                              _stream(stream)))


def moe_expert_ffn(desc, weights, x, offsets, sorted_token, Y, ws, stream=None) -> None:
    _check(lib().moe_expert_ffn(ctypes.byref(desc), ctypes.byref(weights), _ptr(x),
                                _ptr(offsets), _ptr(sorted_token), _ptr(Y), _ptr(ws),
                                _nbytes(ws) if ws is not None else 0, _stream(stream)))


def moe_combine(desc, Y, Y_shared, x, row_of, topk_w, out, stream=None) -> None:
    _check(lib().moe_combine(ctypes.byref(desc), _ptr(Y), _ptr(Y_shared), _ptr(x), _ptr(row_of),
                             _ptr(topk_w), _ptr(out), _stream(stream)))


def moe_balance_stats(desc, logits, counts_assigned, coef, p_mean, stats, ws, stream=None) -> None:
    _check(lib().moe_balance_stats(ctypes.byref(desc), _ptr(logits), _ptr(counts_assigned),
                                   float(coef), _ptr(p_mean), _ptr(stats), _ptr(ws),
                                   _nbytes(ws) if ws is not None else 0, _stream(stream)))


def moe_forward(desc, weights, x, out, aux, ws, stream=None) -> None:
    a = ctypes.byref(aux) if aux is not None else None
    _check(lib().moe_forward(ctypes.byref(desc), ctypes.byref(weights), _ptr(x), _ptr(out), a,
                             _ptr(ws), _nbytes(ws) if ws is not None else 0, _stream(stream)))


def moe_forward_noalloc(desc, weights, x, out, aux, stream=None) -> None:
    a = ctypes.byref(aux) if aux is not None else None
    _check(lib().moe_forward_noalloc(ctypes.byref(desc), ctypes.byref(weights), _ptr(x),
                                     _ptr(out), a, _stream(stream)))


def moe_scratch_bytes() -> int:
    return int(lib().moe_scratch_bytes())


def moe_check_routing(desc, topk_idx, n_bad, stream=None) -> None:
    _check(lib().moe_check_routing(ctypes.byref(desc), _ptr(topk_idx), _ptr(n_bad),
                                   _stream(stream)))


def moe_debug_checks() -> int:
    return int(lib().moe_debug_checks())
