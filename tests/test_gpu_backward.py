"""GPU parity of the backward pass: the three backward calls through the C ABI
against the oracle's fp64 backward (itself pinned by finite differences).

Bars, element-wise with a scale floor:  |got - ref| <= tol * (|ref| + rms(ref))
with tol 3e-2 for bf16 layers (the SwiGLU and dy intermediates are rounded to
bf16, as the forward rounds its activations) and 1e-4 for fp32 layers.  Small
cases compare every output; the full-size case compares sampled tokens,
sampled weight rows, and the invariants sum_r dcentroids_r = 0, sum dbias = 0.
"""
import numpy as np
import pytest

from oracle import oracle as O
from fine_grained_mixture_moe_amd import workloads as W
from fine_grained_mixture_moe_amd.layer import DeviceLayer
import parity as PT

pytestmark = pytest.mark.gpu

TOL = {"bf16": 3e-2, "f32": 1e-4}
ALPHA1, ALPHA2 = 0.01, 0.02


FAILS = []


def close(name, got, ref, tol, floor=0.0):
    """Record a failure of the bar (all outputs of a case are checked, then the case fails)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return
    scale = max(np.sqrt(np.mean(ref ** 2)), floor) + 1e-30
    err = np.abs(got - ref)
    bad = err > tol * (np.abs(ref) + scale)
    msg = f"{name}: {int(bad.sum())} of {bad.size} outside the bar; max err/rms {err.max() / scale:.3g}"
    PT.say(("  FAIL " if bad.any() else "  ok   ") + msg)
    if bad.any():
        FAILS.append(msg)


def make_dh(inp, seed=99):
    wl = inp.wl
    rng = np.random.default_rng(seed)
    dh = rng.standard_normal((wl.T, wl.d)).astype(np.float32)
    if wl.dtype == "bf16":
        dh = W.f32_from_bf16_bits(W.bf16_bits_from_f32(dh))
    return dh


def run_backward(inp, tokens=None, weight_experts=None, full_router=True, tag=""):
    wl = inp.wl
    FAILS.clear()
    PT.say(f"[bwd] {tag} {wl.name} T={wl.T} d={wl.d} Ks={wl.n_shared} Nr={wl.n_routed} K={wl.top_k} w={wl.inter} "
           f"{wl.dtype} groups={wl.groups}")
    dl = DeviceLayer(inp, want_probs=True)
    dl.forward()
    dh = make_dh(inp)
    dl.backward(dh, ALPHA1, ALPHA2)
    g = dl.backward_results()
    tol = TOL[wl.dtype]
    o = PT.oracle_routing(inp)
    st = o["stats"]
    sh, ro = inp.shared, inp.routed
    wts = (sh(inp.w1).f32, sh(inp.w3).f32, sh(inp.w2).f32, ro(inp.w1).f32, ro(inp.w3).f32, ro(inp.w2).f32)
    tok = np.arange(wl.T, dtype=np.int32) if tokens is None else np.asarray(tokens, np.int32)
    bt = O.backward_tokens(tok, inp.x.f32, inp.centroids, o["idx"], o["gate"], o["probs"], st["f"], st["f_dev"],
                           ALPHA1, ALPHA2, dh, *wts)
    close("dgate", g["dgate"][tok], bt["dgate"], tol)
    close("dx", g["dx"][tok], bt["dx"], tol)
    # the experts' part of dx on its own (the oracle's dx less the residual and the router part)
    dze = bt["dz"] @ inp.centroids.astype(np.float64) if wl.n_routed else 0.0
    close("dx_ffn", g["dx_ffn"][tok], bt["dx"] - dh[tok] - dze, tol)
    if wl.n_routed:
        # the router part alone: oracle dz E against the GPU dx - dx_ffn - dh (a difference of
        # fp32 values of the size of dx, so the bar's floor is the size of dx)
        close("dz E", g["dx"][tok] - g["dx_ffn"][tok] - dh[tok], bt["dz"] @ inp.centroids.astype(np.float64), tol,
              floor=float(np.sqrt(np.mean(bt["dx"] ** 2))))
    if full_router:
        dE, db = O.backward_router(inp.x.f32, bt["dz"])
        close("dcentroids", g["dcent"], dE, tol)
        close("dbias", g["dbias"], db, tol)
    else:
        scale = np.abs(g["dcent"]).max() + 1e-30
        assert np.abs(g["dcent"].sum(axis=0)).max() <= 1e-3 * scale * wl.n_routed
        assert abs(g["dbias"].sum()) <= 1e-3 * (np.abs(g["dbias"]).max() + 1e-30) * wl.n_routed
    experts = range(wl.n_shared + wl.n_routed) if weight_experts is None else weight_experts
    rng = np.random.default_rng(5)
    for e in experts:
        rows_up = np.arange(wl.inter, dtype=np.int32) if weight_experts is None else \
            np.sort(rng.choice(wl.inter, 8, replace=False)).astype(np.int32)
        rows_dn = np.arange(wl.d, dtype=np.int32) if weight_experts is None else \
            np.sort(rng.choice(wl.d, 8, replace=False)).astype(np.int32)
        dW1, dW3, dW2 = O.backward_weight_rows(e, inp.x.f32, o["idx"], o["gate"], dh, *wts, rows_up, rows_dn)
        if e < wl.n_shared:
            gw1, gw3, gw2 = g["dw1_s"][e], g["dw3_s"][e], g["dw2_s"][e]
        else:
            r = e - wl.n_shared
            gw1, gw3, gw2 = g["dw1_r"][r], g["dw3_r"][r], g["dw2_r"][r]
        # the bar's scale is the whole gradient of this expert (rows of an unused expert are zero)
        close(f"dW1[{e}]", gw1[rows_up], dW1, tol)
        close(f"dW3[{e}]", gw3[rows_up], dW3, tol)
        close(f"dW2[{e}]", gw2[rows_dn], dW2, tol)
    assert not FAILS, "; ".join(FAILS[:6])
    return dl, g


SMALL = [
    # (T, d, Ks, Nr, K, w, dtype, seed, zipf, groups)
    (300, 128, 1, 16, 4, 64, "f32", 1, None, 4),
    (300, 128, 1, 16, 4, 64, "bf16", 2, None, 2),
    (513, 256, 2, 64, 6, 128, "bf16", 3, 1.1, 4),
    (257, 128, 1, 100, 3, 128, "f32", 6, None, 5),
    (700, 128, 3, 2, 2, 192, "bf16", 7, None, 2),
    (200, 192, 0, 200, 16, 64, "bf16", 5, None, 8),
    (1, 64, 0, 8, 1, 64, "f32", 4, None, 1),
    (130, 64, 0, 1, 1, 64, "f32", 8, None, 1),
    # 256 x 256 bf16 tiles: most experts empty (their weight gradients must be exact zeros)
    (40, 128, 0, 64, 2, 128, "bf16", 9, None, 4),
    # W2 segments of width 320 straddle the 256-wide tiles of da and dW2; shared width 640
    (600, 192, 2, 8, 2, 320, "bf16", 10, None, 2),
    # 750 rows per expert: three row runs of 256, 256 and 238 rows for da and the dx rows
    (1500, 128, 1, 4, 2, 128, "bf16", 12, None, 2),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"T{c[0]}_d{c[1]}_s{c[2]}_r{c[3]}_k{c[4]}_w{c[5]}_{c[6]}" for c in SMALL])
def test_backward_small_cases(case):
    T, d, Ks, Nr, K, w, dt, seed, zipf, groups = case
    inp = W.make_random_case(T, d, Ks, Nr, K, w, dtype=dt, seed=seed, zipf_s=zipf, groups=groups, w_std=0.05)
    run_backward(inp, tag="small")


def test_backward_c1_full():
    run_backward(W.make_inputs(W.WORKLOADS["c1"]), tag="c1")


def test_backward_c2b_sampled():
    inp = W.make_c2_fine(independent_centroids=True)
    tokens = W.sample_tokens(inp.wl.T, 48)
    run_backward(inp, tokens=tokens, weight_experts=[0, 17, 63], full_router=False, tag="c2b")


def test_backward_skewed_shared_sampled():
    """Zipf(1.1)-skewed routing with two shared experts at T = 4096: many tiles per group, groups
    of very different sizes, shared dx-row tiles with twice the routed k extent."""
    inp = W.make_random_case(4096, 512, 2, 32, 4, 256, dtype="bf16", seed=21, zipf_s=1.1, groups=4, w_std=0.05)
    tokens = W.sample_tokens(inp.wl.T, 48)
    run_backward(inp, tokens=tokens, weight_experts=[0, 1, 2, 33], full_router=False, tag="skewed")


def test_backward_is_deterministic():
    inp = W.make_random_case(600, 128, 1, 32, 4, 128, dtype="bf16", seed=11)
    PT.say("[bwd] determinism")
    dl = DeviceLayer(inp, want_probs=True)
    dl.forward()
    dh = make_dh(inp)
    dl.backward(dh, ALPHA1, ALPHA2)
    a = dl.backward_results()
    dl.backward(dh, ALPHA1, ALPHA2)
    b = dl.backward_results()
    for k, v in a.items():
        if v is not None:
            assert np.array_equal(v, b[k]), k
