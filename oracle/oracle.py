"""ctypes front of liboracle.so -- the plain CPU oracle (test infrastructure only).

Every function takes and returns NumPy arrays; floating-point inputs are the
exact fp32 values (for bf16 workloads, the fp32 upcast of the same bf16 bits
the GPU receives).  See moe_oracle.c for the definitions and the passages of
the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_vp = ctypes.c_void_p
_i = ctypes.c_int


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_num_threads.restype = _i
        L.oracle_set_num_threads.argtypes = [_i]
        L.oracle_logits.argtypes = [_i, _i, _i, _f32p, _f32p, _vp, _f32p]
        L.oracle_route.argtypes = [_i, _i, _i, _i, _f32p, _f32p, _vp, _i32p, _f32p, _vp, _i32p, _f64p]
        L.oracle_permute.argtypes = [_i, _i, _i, _i32p, _i32p, _i32p, _i32p]
        L.oracle_permute.restype = _i
        L.oracle_expert_ffn.argtypes = [_i, _i, _f32p, _f32p, _f32p, _f32p, _f64p]
        L.oracle_layer_tokens.argtypes = [_i, _i32p, _i, _i, _i, _i, _i, _f32p, _i32p, _f32p,
                                          _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.oracle_balance_stats.argtypes = [_i, _i, _i, _i, _i32p, _f64p, _f32p, _f32p, _f32p, _f32p,
                                           _f32p, _f32p]
        L.oracle_balance_stats.restype = _i
        L.oracle_forward.argtypes = [_i, _i, _i, _i, _i, _i, _i, _f32p, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _vp, _vp, _f64p, _f32p, _f32p]
        L.oracle_forward.restype = _i
        L.oracle_route_ablate.argtypes = [_i, _i, _i, _i, _i, _f32p, _f32p, _vp, _i32p, _f32p, _vp, _i32p, _f64p]
        L.oracle_route_hash.argtypes = [_i, _i, _i32p, _i32p, _f32p, _i32p]
        _d = ctypes.c_double
        L.oracle_backward_tokens.argtypes = [_i, _i32p, _i, _i, _i, _i, _i, _i, _i, _d, _d, _f32p, _vp,
                                             _i32p, _f32p, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                             _f32p, _vp, _vp, _vp]
        L.oracle_backward_router.argtypes = [_i, _i, _i, _f32p, _f64p, _f64p, _f64p]
        L.oracle_backward_weight_rows.argtypes = [_i, _i, _i, _i, _i, _i, _f32p, _i32p, _f32p, _vp, _vp,
                                                  _vp, _vp, _vp, _vp, _f32p, _i, _i32p, _f64p, _f64p,
                                                  _i, _i32p, _f64p]
        _lib = L
    return _lib


def _c(a, dt=np.float32):
    return np.ascontiguousarray(a, dtype=dt)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


def logits(x, E, bias=None) -> np.ndarray:
    x, E = _c(x), _c(E)
    T, d = x.shape
    Nr = E.shape[0]
    b = None if bias is None else _c(bias)
    z = np.empty((T, Nr), np.float32)
    lib().oracle_logits(T, d, Nr, x, E, _ptr(b), z)
    return z


def route(x, E, top_k: int, bias=None, want_probs: bool = False):
    """-> dict(idx [T,K'] i32, gate [T,K'] f32, probs [T,N'] f32|None, counts [N'] i32, prob_sum [N'] f64)."""
    x, E = _c(x), _c(E)
    T, d = x.shape
    Nr = E.shape[0]
    b = None if bias is None else _c(bias)
    idx = np.empty((T, top_k), np.int32)
    gate = np.empty((T, top_k), np.float32)
    probs = np.empty((T, Nr), np.float32) if want_probs else None
    counts = np.empty(Nr, np.int32)
    psum = np.empty(Nr, np.float64)
    lib().oracle_route(T, d, Nr, top_k, x, E, _ptr(b), idx, gate, _ptr(probs), counts, psum)
    return dict(idx=idx, gate=gate, probs=probs, counts=counts, prob_sum=psum)


def route_ablate(x, E, top_k: int, skip: int, bias=None, want_probs: bool = False):
    """Routing with each token's `skip` top-ranked routed experts disabled (ranks skip..skip+K'-1 taken)."""
    x, E = _c(x), _c(E)
    T, d = x.shape
    Nr = E.shape[0]
    b = None if bias is None else _c(bias)
    idx = np.empty((T, top_k), np.int32)
    gate = np.empty((T, top_k), np.float32)
    probs = np.empty((T, Nr), np.float32) if want_probs else None
    counts = np.empty(Nr, np.int32)
    psum = np.empty(Nr, np.float64)
    lib().oracle_route_ablate(T, d, Nr, top_k, int(skip), x, E, _ptr(b), idx, gate, _ptr(probs), counts, psum)
    return dict(idx=idx, gate=gate, probs=probs, counts=counts, prob_sum=psum)


def route_hash(token_ids, n_routed: int):
    """Hash routing: idx [T,1] from a fixed multiplicative hash of the token ids, gate 1."""
    ids = _c(token_ids, np.int32)
    T = ids.shape[0]
    idx = np.empty((T, 1), np.int32)
    gate = np.empty((T, 1), np.float32)
    counts = np.empty(n_routed, np.int32)
    lib().oracle_route_hash(T, n_routed, ids if T else np.zeros(1, np.int32), idx, gate, counts)
    return dict(idx=idx, gate=gate, counts=counts)


def permute(idx, n_routed: int):
    """-> dict(offsets [N'+1], sorted_token [T*K'], slot_of [T,K']) (int32)."""
    idx = _c(idx, np.int32)
    T, K = idx.shape
    offsets = np.empty(n_routed + 1, np.int32)
    sorted_token = np.empty(max(T * K, 1), np.int32)
    slot_of = np.empty(max(T * K, 1), np.int32)
    if idx.size == 0:
        idx = np.zeros(1, np.int32)
    rc = lib().oracle_permute(T, n_routed, K, idx, offsets, sorted_token, slot_of)
    if rc != 0:
        raise ValueError("oracle_permute: expert index out of range or repeated within a token")
    return dict(offsets=offsets, sorted_token=sorted_token[:T * K], slot_of=slot_of[:T * K].reshape(T, K))


def expert_ffn(u, W1, W3, W2) -> np.ndarray:
    """One SwiGLU expert on one token: W2 (SiLU(W1 u) * (W3 u)), fp64 result [d]."""
    u, W1, W3, W2 = _c(u), _c(W1), _c(W3), _c(W2)
    w, d = W1.shape
    y = np.empty(d, np.float64)
    lib().oracle_expert_ffn(d, w, u, W1, W3, W2, y)
    return y


def layer_tokens(tokens, x, idx, gate, w1_s, w3_s, w2_s, w1_r, w3_r, w2_r,
                 want_y_routed: bool = False):
    """Layer output for the listed tokens.

    -> dict(y_shared [n,d], y_routed [n,K',d] (if asked), y [n,d], h [n,d]) in fp64.
    Shared weights [K_s, w, d]/[K_s, d, w]; routed weights [N', w, d]/[N', d, w].
    """
    tokens = _c(tokens, np.int32)
    x = _c(x)
    T, d = x.shape
    idx = _c(idx, np.int32).reshape(T, -1) if idx is not None and np.size(idx) else np.zeros((T, 0), np.int32)
    K = idx.shape[1]
    gate = _c(gate).reshape(T, K) if K else np.zeros((T, 0), np.float32)
    ws = [None if a is None or a.size == 0 else _c(a) for a in (w1_s, w3_s, w2_s)]
    wr = [None if a is None or a.size == 0 else _c(a) for a in (w1_r, w3_r, w2_r)]
    Ks = 0 if ws[0] is None else ws[0].shape[0]
    Nr = 0 if wr[0] is None else wr[0].shape[0]
    w = (ws[0] if Ks else wr[0]).shape[1]
    n = tokens.shape[0]
    y_shared = np.empty((n, d), np.float64)
    y_routed = np.empty((n, K, d), np.float64) if want_y_routed else None
    y = np.empty((n, d), np.float64)
    h = np.empty((n, d), np.float64)
    lib().oracle_layer_tokens(n, tokens, d, Ks, Nr, K, w, x, idx, gate,
                              *[_ptr(a) for a in ws], *[_ptr(a) for a in wr],
                              _ptr(y_shared), _ptr(y_routed), _ptr(y), _ptr(h))
    return dict(y_shared=y_shared, y_routed=y_routed, y=y, h=h)


def balance_stats(T: int, top_k: int, groups: int, counts, prob_sum):
    """-> dict(f [N'], P [N'], f_dev [D], P_dev [D], exp_bal, dev_bal) in fp32."""
    counts = _c(counts, np.int32)
    prob_sum = _c(prob_sum, np.float64)
    Nr = counts.shape[0]
    f = np.empty(Nr, np.float32)
    P = np.empty(Nr, np.float32)
    fd = np.empty(groups, np.float32)
    Pd = np.empty(groups, np.float32)
    eb = np.empty(1, np.float32)
    db = np.empty(1, np.float32)
    rc = lib().oracle_balance_stats(T, Nr, top_k, groups, counts, prob_sum, f, P, fd, Pd, eb, db)
    if rc != 0:
        raise ValueError("oracle_balance_stats: need 1 <= K' <= N', D | N'")
    return dict(f=f, P=P, f_dev=fd, P_dev=Pd, exp_bal=float(eb[0]), dev_bal=float(db[0]))


def forward(n_tok: int, x, E, bias, top_k: int, groups: int, w1_s, w3_s, w2_s, w1_r, w3_r, w2_r):
    """Whole layer pass on the first n_tok tokens (route, group, FFNs, sum, stats) -> h [n,d] fp64."""
    x = _c(x)
    d = x.shape[1]
    ws = [None if a is None or a.size == 0 else _c(a) for a in (w1_s, w3_s, w2_s)]
    wr = [None if a is None or a.size == 0 else _c(a) for a in (w1_r, w3_r, w2_r)]
    Ks = 0 if ws[0] is None else ws[0].shape[0]
    Nr = 0 if wr[0] is None else wr[0].shape[0]
    w = (ws[0] if Ks else wr[0]).shape[1]
    E = None if E is None or np.size(E) == 0 else _c(E)
    b = None if bias is None else _c(bias)
    h = np.empty((n_tok, d), np.float64)
    eb = np.zeros(1, np.float32)
    db = np.zeros(1, np.float32)
    rc = lib().oracle_forward(n_tok, d, Ks, Nr, top_k, w, groups, x, _ptr(E), _ptr(b),
                              *[_ptr(a) for a in ws], *[_ptr(a) for a in wr], h, eb, db)
    if rc != 0:
        raise ValueError("oracle_forward failed")
    return h, float(eb[0]), float(db[0])


# ---------------------------------------------------------------------------
# Backward pass (see moe_oracle.c for the chain-rule formulas and readings).
# ---------------------------------------------------------------------------

def _weights(w1_s, w3_s, w2_s, w1_r, w3_r, w2_r):
    ws = [None if a is None or np.size(a) == 0 else _c(a) for a in (w1_s, w3_s, w2_s)]
    wr = [None if a is None or np.size(a) == 0 else _c(a) for a in (w1_r, w3_r, w2_r)]
    Ks = 0 if ws[0] is None else ws[0].shape[0]
    Nr = 0 if wr[0] is None else wr[0].shape[0]
    w = (ws[0] if Ks else wr[0]).shape[1]
    return ws, wr, Ks, Nr, w


def backward_tokens(tokens, x, E, idx, gate, probs, f, f_dev, alpha1: float, alpha2: float, dh,
                    w1_s, w3_s, w2_s, w1_r, w3_r, w2_r):
    """Per-token backward for the listed tokens.

    -> dict(dgate [n,K'] fp64, dz [n,N'] fp64, dx [n,d] fp64).  probs [T,N'], f [N'], f_dev [D]
    are the forward's outputs; dh [T,d] the upstream gradient; alpha1/alpha2 weight ExpBal/DevBal.
    """
    tokens = _c(tokens, np.int32)
    x, dh = _c(x), _c(dh)
    T, d = x.shape
    ws, wr, Ks, Nr, w = _weights(w1_s, w3_s, w2_s, w1_r, w3_r, w2_r)
    n = tokens.shape[0]
    if Nr:
        idx = _c(idx, np.int32).reshape(T, -1)
        K = idx.shape[1]
        gate = _c(gate).reshape(T, K)
        probs, f, f_dev, E = _c(probs), _c(f), _c(f_dev), _c(E)
        D = f_dev.shape[0]
    else:
        K, D = 0, 1
        idx = np.zeros(1, np.int32)
        gate = np.zeros(1, np.float32)
    dgate = np.empty((n, max(K, 1)), np.float64)
    dz = np.empty((n, max(Nr, 1)), np.float64)
    dx = np.empty((n, d), np.float64)
    lib().oracle_backward_tokens(n, tokens, T, d, Ks, Nr, K, w, D, float(alpha1), float(alpha2), x,
                                 _ptr(E) if Nr else None, idx, gate,
                                 _ptr(probs) if Nr else None, _ptr(f) if Nr else None,
                                 _ptr(f_dev) if Nr else None,
                                 *[_ptr(a) for a in ws], *[_ptr(a) for a in wr], dh,
                                 _ptr(dgate), _ptr(dz), _ptr(dx))
    return dict(dgate=dgate[:, :K], dz=dz[:, :Nr], dx=dx)


def backward_router(x, dz):
    """dE [N',d] = dz^T x and dbias [N'] = column sums of dz, from dz [T,N'] of every token (fp64)."""
    x = _c(x)
    dz = _c(dz, np.float64)
    T, d = x.shape
    Nr = dz.shape[1]
    dE = np.empty((Nr, d), np.float64)
    db = np.empty(Nr, np.float64)
    lib().oracle_backward_router(T, d, Nr, x, dz, dE, db)
    return dE, db


def backward_weight_rows(e: int, x, idx, gate, dh, w1_s, w3_s, w2_s, w1_r, w3_r, w2_r,
                         rows_up, rows_down):
    """Selected rows of the weight gradients of global expert e (shared first).

    -> (dW1 [n1,d], dW3 [n1,d], dW2 [n2,w]) fp64 for rows_up of [w,d] and rows_down of [d,w].
    """
    x, dh = _c(x), _c(dh)
    T, d = x.shape
    ws, wr, Ks, Nr, w = _weights(w1_s, w3_s, w2_s, w1_r, w3_r, w2_r)
    if Nr:
        idx = _c(idx, np.int32).reshape(T, -1)
        K = idx.shape[1]
        gate = _c(gate).reshape(T, K)
    else:
        K = 0
        idx = np.zeros(1, np.int32)
        gate = np.zeros(1, np.float32)
    r1 = _c(rows_up, np.int32)
    r2 = _c(rows_down, np.int32)
    dW1 = np.empty((max(r1.size, 1), d), np.float64)
    dW3 = np.empty((max(r1.size, 1), d), np.float64)
    dW2 = np.empty((max(r2.size, 1), w), np.float64)
    lib().oracle_backward_weight_rows(int(e), T, d, Ks, K, w, x, idx, gate, *[_ptr(a) for a in ws],
                                      *[_ptr(a) for a in wr], dh, r1.size, r1, dW1, dW3, r2.size, r2, dW2)
    return dW1[:r1.size], dW3[:r1.size], dW2[:r2.size]
