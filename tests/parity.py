"""Shared helpers of the GPU parity tests: run the oracle, run the HIP path,
compare them at the stated bars.

Bars: bit-exact for idx, counts, offsets, sorted_token, slot_of, f and f';
relative 1e-5 for gates, affinities, prob_sum, P, P', ExpBal, DevBal;
per-token-row infinity-norm relative error  max_t |got_t - ref_t|_inf /
|ref_t|_inf  below 2e-2 (bf16) or 1e-4 (fp32) for every expert output, the
expert sum y (without the residual) and h.
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import oracle as O
from fine_grained_mixture_moe_amd import workloads as W

TOL = {"bf16": 2e-2, "f32": 1e-4}
REL_ROUTE = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    if ref.size == 0:
        return 0.0
    num = np.abs(got - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max())


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    den = np.maximum(np.abs(ref), 1e-30)
    return float((np.abs(got - ref) / den).max())


def oracle_routing(inp: W.LayerInputs, want_probs: bool = True) -> dict:
    wl = inp.wl
    r = O.route(inp.x.f32, inp.centroids, wl.top_k, inp.bias, want_probs=want_probs)
    p = O.permute(r["idx"], wl.n_routed)
    s = O.balance_stats(wl.T, wl.top_k, wl.groups, r["counts"], r["prob_sum"]) if wl.T >= 0 else None
    r.update(p)
    r["stats"] = s
    return r


def oracle_outputs(inp: W.LayerInputs, idx, gate, tokens) -> dict:
    sh, ro = inp.shared, inp.routed
    return O.layer_tokens(tokens, inp.x.f32, idx, gate, sh(inp.w1).f32, sh(inp.w3).f32, sh(inp.w2).f32,
                          ro(inp.w1).f32, ro(inp.w3).f32, ro(inp.w2).f32, want_y_routed=True)


def check_routing(g: dict, o: dict, wl: W.Workload, probs: bool = True) -> None:
    assert np.array_equal(g["idx"], o["idx"]), "expert indices differ"
    assert np.array_equal(g["counts"], o["counts"]), "per-expert counts differ"
    assert rel_err(g["gate"], o["gate"]) < REL_ROUTE, rel_err(g["gate"], o["gate"])
    if probs and "probs" in g:
        assert rel_err(g["probs"], o["probs"]) < REL_ROUTE, rel_err(g["probs"], o["probs"])
    assert rel_err(g["prob_sum"], o["prob_sum"]) < REL_ROUTE, rel_err(g["prob_sum"], o["prob_sum"])


def check_grouping(g: dict, o: dict) -> None:
    assert np.array_equal(g["offsets"], o["offsets"]), "offsets differ"
    assert np.array_equal(g["sorted_token"], o["sorted_token"]), "sorted_token differs"
    assert np.array_equal(g["slot_of"], o["slot_of"]), "slot_of differs"


def check_stats(g: dict, s: dict) -> None:
    assert np.array_equal(g["f"], s["f"]), "f differs"
    assert np.array_equal(g["f_dev"], s["f_dev"]), "f' differs"
    assert rel_err(g["P"], s["P"]) < REL_ROUTE
    assert rel_err(g["P_dev"], s["P_dev"]) < REL_ROUTE
    assert rel_err([g["exp_bal"]], [s["exp_bal"]]) < REL_ROUTE
    assert rel_err([g["dev_bal"]], [s["dev_bal"]]) < REL_ROUTE


def check_outputs(g: dict, inp: W.LayerInputs, tokens: np.ndarray, ref: dict, tag: str = "") -> dict:
    """Compare expert outputs, y (no residual) and h on the listed tokens.

    g["y"] is the GPU's own expert sum: moe_combine run with an all-zero
    residual (DeviceLayer.expert_sum), so the combine kernel's gate-weighted
    sum is checked at the bar without the residual hiding it.  The grouped
    rows y_routed and the shared sum are checked where the mode keeps them
    (the accumulating expert FFN keeps neither)."""
    wl = inp.wl
    tol = TOL[wl.dtype]
    K = wl.top_k
    errs = {}
    if K and g.get("y_routed") is not None:
        slots = g["slot_of"][tokens]                          # [n, K]
        y_r = g["y_routed"][slots.reshape(-1)].reshape(len(tokens), K, wl.d)
        errs["y_routed"] = row_rel_err(y_r.reshape(-1, wl.d), ref["y_routed"].reshape(-1, wl.d))
    if wl.n_shared and g.get("y_shared") is not None:
        errs["y_shared"] = row_rel_err(g["y_shared"][tokens], ref["y_shared"])
    assert "y" in g, "the GPU expert sum is missing: call DeviceLayer.expert_sum() before results()"
    errs["y"] = row_rel_err(g["y"][tokens], ref["y"])
    errs["h"] = row_rel_err(g["h"][tokens], ref["h"])
    say(f"  {tag} {wl.name}: " + ", ".join(f"{k}={v:.3e}" for k, v in errs.items()) + f" (tol {tol:g})")
    for k, v in errs.items():
        assert v < tol, f"{k}: {v:.3e} >= {tol}"
    return errs
