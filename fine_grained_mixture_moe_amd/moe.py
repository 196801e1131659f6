"""Thin ctypes binding of libmoe.so (include/moe.h) -- argument marshalling only.

Each function has the name of the C entry point it wraps and takes torch
tensors on the GPU (or None for nullable pointers); it passes their device
pointers and the current HIP stream, and raises MoEError on a non-zero
status.  No layer arithmetic happens here: every step runs in the HIP
kernels.  There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_STALLED = 0, -1, -2, -3, -4, -5
MOE_F32, MOE_BF16 = 0, 1


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {moe_status_str(status)} ({status})")
        self.status = status


class moe_problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("n_routed", ctypes.c_int32), ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]

    @classmethod
    def make(cls, T, d, n_shared, n_routed, top_k, inter, dtype) -> "moe_problem":
        dt = dtype if isinstance(dtype, int) else {"f32": MOE_F32, "bf16": MOE_BF16}[dtype]
        return cls(T, d, n_shared, n_routed, top_k, inter, dt)

    def __repr__(self):
        return (f"moe_problem(T={self.T}, d={self.d}, n_shared={self.n_shared}, n_routed={self.n_routed}, "
                f"top_k={self.top_k}, inter={self.inter}, dtype={self.dtype})")


class moe_layer_io(ctypes.Structure):
    """The pointer struct of moe_layer_forward (include/moe.h), field by field."""
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x", "centroids", "bias", "w1_routed", "w3_routed", "w2_routed", "w1_shared", "w3_shared", "w2_shared",
        "idx", "gate", "probs", "counts", "prob_sum", "offsets", "sorted_token", "slot_of",
        "y_routed", "y_shared", "h", "f", "P", "f_dev", "P_dev", "exp_bal", "dev_bal")]


_lib = None
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_pp = ctypes.POINTER(moe_problem)


def lib() -> ctypes.CDLL:
    """Load libmoe.so (raises OSError when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is missing: run __graft_entry__.build() (hipcc, gfx950) first")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_version.restype = ctypes.c_char_p
        L.moe_workspace_size.argtypes = [_pp, ctypes.POINTER(_sz)]
        L.moe_route.argtypes = [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.moe_route_noalloc.argtypes = [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.moe_permute.argtypes = [_pp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.moe_expert_ffn.argtypes = [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _sz, _vp]
        L.moe_expert_ffn_status.argtypes = [_pp, _vp, _sz, _vp]
        L.moe_expert_ffn_kernel.argtypes = [_pp, ctypes.c_int]
        L.moe_expert_ffn_kernel.restype = ctypes.c_char_p
        L.moe_expert_up.argtypes = [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.moe_expert_down.argtypes = [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.moe_combine.argtypes = [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.moe_balance_stats.argtypes = [_pp, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.moe_route_ablate.argtypes = [_pp, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.moe_route_hash.argtypes = [_pp, _vp, _vp, _vp, _vp, _vp]
        L.moe_layer_forward.argtypes = [_pp, ctypes.c_int32, ctypes.POINTER(moe_layer_io), _vp, _sz, _vp]
        L.moe_backward_workspace_size.argtypes = [_pp, ctypes.POINTER(_sz)]
        L.moe_combine_backward.argtypes = [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.moe_expert_ffn_backward.argtypes = [_pp] + [_vp] * 20 + [_sz, _vp]
        L.moe_route_backward.argtypes = [_pp, ctypes.c_int32, ctypes.c_float, ctypes.c_float] + [_vp] * 13 + [_sz, _vp]
        for fn in ("moe_workspace_size", "moe_route", "moe_route_noalloc", "moe_permute", "moe_expert_ffn", "moe_expert_ffn_status",
                   "moe_expert_up",
                   "moe_expert_down", "moe_combine", "moe_balance_stats", "moe_backward_workspace_size",
                   "moe_combine_backward", "moe_expert_ffn_backward", "moe_route_backward", "moe_route_ablate",
                   "moe_route_hash", "moe_layer_forward"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoEError(fn, status)


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def moe_version() -> str:
    return lib().moe_version().decode()


def moe_workspace_size(p: moe_problem) -> int:
    n = _sz(0)
    _check("moe_workspace_size", lib().moe_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def moe_route(p, x, centroids, bias, idx, gate, probs, counts, prob_sum, ws, ws_bytes, stream=None):
    _check("moe_route", lib().moe_route(ctypes.byref(p), _ptr(x), _ptr(centroids), _ptr(bias), _ptr(idx),
                                        _ptr(gate), _ptr(probs), _ptr(counts), _ptr(prob_sum), _ptr(ws),
                                        ws_bytes, _stream(stream)))


def moe_route_noalloc(p, x, centroids, bias, idx, gate, probs, counts, prob_sum, stream=None):
    _check("moe_route_noalloc", lib().moe_route_noalloc(ctypes.byref(p), _ptr(x), _ptr(centroids), _ptr(bias),
                                                        _ptr(idx), _ptr(gate), _ptr(probs), _ptr(counts),
                                                        _ptr(prob_sum), _stream(stream)))


def moe_route_ablate(p, disabled_top, x, centroids, bias, idx, gate, probs, counts, prob_sum, ws, ws_bytes,
                     stream=None):
    _check("moe_route_ablate", lib().moe_route_ablate(ctypes.byref(p), int(disabled_top), _ptr(x), _ptr(centroids),
                                                      _ptr(bias), _ptr(idx), _ptr(gate), _ptr(probs), _ptr(counts),
                                                      _ptr(prob_sum), _ptr(ws), ws_bytes, _stream(stream)))


def moe_route_hash(p, token_ids, idx, gate, counts, stream=None):
    _check("moe_route_hash", lib().moe_route_hash(ctypes.byref(p), _ptr(token_ids), _ptr(idx), _ptr(gate),
                                                  _ptr(counts), _stream(stream)))


def moe_permute(p, idx, offsets, sorted_token, slot_of, ws, ws_bytes, stream=None):
    _check("moe_permute", lib().moe_permute(ctypes.byref(p), _ptr(idx), _ptr(offsets), _ptr(sorted_token),
                                            _ptr(slot_of), _ptr(ws), ws_bytes, _stream(stream)))


def moe_expert_ffn(p, x, offsets, sorted_token, w1_routed, w3_routed, w2_routed, w1_shared, w3_shared,
                   w2_shared, y_routed, y_acc, gate, slot_of, ws, ws_bytes, stream=None):
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        ctypes.byref(p), _ptr(x), _ptr(offsets), _ptr(sorted_token), _ptr(w1_routed), _ptr(w3_routed),
        _ptr(w2_routed), _ptr(w1_shared), _ptr(w3_shared), _ptr(w2_shared), _ptr(y_routed), _ptr(y_acc),
        _ptr(gate), _ptr(slot_of), _ptr(ws), ws_bytes, _stream(stream)))


def moe_expert_ffn_status(p, ws, ws_bytes, stream=None) -> int:
    """Status word of the last moe_expert_ffn on ws (synchronises the stream); returned, not raised."""
    return lib().moe_expert_ffn_status(ctypes.byref(p), _ptr(ws), ws_bytes, _stream(stream))


def moe_expert_ffn_kernel(p, accumulate: bool = False) -> str:
    name = lib().moe_expert_ffn_kernel(ctypes.byref(p), int(bool(accumulate)))
    if name is None:
        raise MoEError("moe_expert_ffn_kernel", MOE_ERR_INVALID_ARG)
    return name.decode()


def moe_expert_up(p, x, offsets, sorted_token, w1_routed, w3_routed, w1_shared, w3_shared, ws, ws_bytes,
                  stream=None):
    _check("moe_expert_up", lib().moe_expert_up(
        ctypes.byref(p), _ptr(x), _ptr(offsets), _ptr(sorted_token), _ptr(w1_routed), _ptr(w3_routed),
        _ptr(w1_shared), _ptr(w3_shared), _ptr(ws), ws_bytes, _stream(stream)))


def moe_expert_down(p, offsets, w2_routed, w2_shared, y_routed, y_shared, ws, ws_bytes, stream=None):
    _check("moe_expert_down", lib().moe_expert_down(
        ctypes.byref(p), _ptr(offsets), _ptr(w2_routed), _ptr(w2_shared), _ptr(y_routed), _ptr(y_shared),
        _ptr(ws), ws_bytes, _stream(stream)))


def moe_combine(p, x, y_routed, y_acc, gate, slot_of, h, stream=None):
    _check("moe_combine", lib().moe_combine(ctypes.byref(p), _ptr(x), _ptr(y_routed), _ptr(y_acc),
                                            _ptr(gate), _ptr(slot_of), _ptr(h), _stream(stream)))


def moe_balance_stats(p, groups, counts, prob_sum, f, P, f_dev, P_dev, exp_bal, dev_bal, stream=None):
    _check("moe_balance_stats", lib().moe_balance_stats(
        ctypes.byref(p), int(groups), _ptr(counts), _ptr(prob_sum), _ptr(f), _ptr(P), _ptr(f_dev),
        _ptr(P_dev), _ptr(exp_bal), _ptr(dev_bal), _stream(stream)))


# -- backward pass ------------------------------------------------------------

def moe_backward_workspace_size(p: moe_problem) -> int:
    n = _sz(0)
    _check("moe_backward_workspace_size", lib().moe_backward_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def moe_combine_backward(p, dh, y_routed, gate, slot_of, dy_routed, dgate, stream=None):
    _check("moe_combine_backward", lib().moe_combine_backward(ctypes.byref(p), _ptr(dh), _ptr(y_routed),
                                                              _ptr(gate), _ptr(slot_of), _ptr(dy_routed),
                                                              _ptr(dgate), _stream(stream)))


def moe_expert_ffn_backward(p, x, offsets, sorted_token, slot_of, w1_routed, w3_routed, w2_routed, w1_shared,
                            w3_shared, w2_shared, dh, dy_routed, dx_ffn, dw1_routed, dw3_routed, dw2_routed,
                            dw1_shared, dw3_shared, dw2_shared, ws, ws_bytes, stream=None):
    _check("moe_expert_ffn_backward", lib().moe_expert_ffn_backward(
        ctypes.byref(p), _ptr(x), _ptr(offsets), _ptr(sorted_token), _ptr(slot_of), _ptr(w1_routed),
        _ptr(w3_routed), _ptr(w2_routed), _ptr(w1_shared), _ptr(w3_shared), _ptr(w2_shared), _ptr(dh),
        _ptr(dy_routed), _ptr(dx_ffn), _ptr(dw1_routed), _ptr(dw3_routed), _ptr(dw2_routed), _ptr(dw1_shared),
        _ptr(dw3_shared), _ptr(dw2_shared), _ptr(ws), ws_bytes, _stream(stream)))


def moe_route_backward(p, groups, alpha1, alpha2, x, centroids, probs, idx, dgate, f, f_dev, dh, dx_ffn, dx,
                       dcentroids, dbias, ws, ws_bytes, stream=None):
    _check("moe_route_backward", lib().moe_route_backward(
        ctypes.byref(p), int(groups), float(alpha1), float(alpha2), _ptr(x), _ptr(centroids), _ptr(probs),
        _ptr(idx), _ptr(dgate), _ptr(f), _ptr(f_dev), _ptr(dh), _ptr(dx_ffn), _ptr(dx), _ptr(dcentroids),
        _ptr(dbias), _ptr(ws), ws_bytes, _stream(stream)))


def moe_layer_forward(p, groups, io: dict, ws, ws_bytes, stream=None):
    """io: the moe_layer_io fields by name (tensors or None)."""
    s = moe_layer_io(**{k: _ptr(v) for k, v in io.items()})
    _check("moe_layer_forward", lib().moe_layer_forward(ctypes.byref(p), groups, ctypes.byref(s), _ptr(ws), ws_bytes,
                                                        _stream(stream)))
