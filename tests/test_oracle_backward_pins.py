"""Pins of the oracle's backward pass (CPU only).

The backward formulas in the oracle are checked against things other than
themselves:
  * central finite differences of the loss L = sum(dh * h) + a1*ExpBal + a2*DevBal
    (Top-K selection held fixed, the reading the backward documents), computed
    with an fp64 forward that is first matched to the oracle's own forward;
  * finite differences of the oracle's fp64 layer output (oracle.layer_tokens)
    for the expert weights and the gates;
  * invariants: softmax-backward rows sum to zero, dbias = column sums of dz,
    zero upstream gradient gives zero gradients.
Inputs live on a 2^-10 grid so that +-eps perturbations are exact in fp32.
"""
import numpy as np
import pytest

from oracle import oracle as O

EPS = 2.0 ** -10


def grid(rng, shape, scale):
    return (np.round(rng.standard_normal(shape) * scale / EPS) * EPS).astype(np.float32)


def make_case(seed=0, T=6, d=8, Ks=1, Nr=5, K=2, w=4, D=1):
    rng = np.random.default_rng(seed)
    c = dict(T=T, d=d, Ks=Ks, Nr=Nr, K=K, w=w, D=D)
    c["x"] = grid(rng, (T, d), 1.0)
    c["E"] = grid(rng, (Nr, d), 0.5)
    c["b"] = grid(rng, (Nr,), 0.5)
    c["w1_s"], c["w3_s"] = grid(rng, (Ks, w, d), 0.4), grid(rng, (Ks, w, d), 0.4)
    c["w2_s"] = grid(rng, (Ks, d, w), 0.4)
    c["w1_r"], c["w3_r"] = grid(rng, (Nr, w, d), 0.4), grid(rng, (Nr, w, d), 0.4)
    c["w2_r"] = grid(rng, (Nr, d, w), 0.4)
    c["dh"] = grid(rng, (T, d), 1.0)
    c["a1"], c["a2"] = 0.3, 0.7
    return c


def silu(v):
    return v / (1.0 + np.exp(-v))


def ffn64(u, W1, W3, W2):
    p = W1.astype(np.float64) @ u
    q = W3.astype(np.float64) @ u
    return W2.astype(np.float64) @ (silu(p) * q)


def forward64(c, idx):
    """fp64 layer forward with the Top-K selection idx held fixed -> (h, s, ExpBal, DevBal)."""
    x = c["x"].astype(np.float64)
    z = x @ c["E"].astype(np.float64).T + c["b"].astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    s = np.exp(z)
    s /= s.sum(axis=1, keepdims=True)
    T, d, Nr, K, D = c["T"], c["d"], c["Nr"], c["K"], c["D"]
    h = x.copy()
    for t in range(T):
        for e in range(c["Ks"]):
            h[t] += ffn64(x[t], c["w1_s"][e], c["w3_s"][e], c["w2_s"][e])
        for k in range(K):
            r = idx[t, k]
            h[t] += s[t, r] * ffn64(x[t], c["w1_r"][r], c["w3_r"][r], c["w2_r"][r])
    counts = np.bincount(idx.ravel(), minlength=Nr)
    f = Nr * counts / (K * T)
    P = s.mean(axis=0)
    g = Nr // D
    fdev = np.array([f[i * g:(i + 1) * g].mean() for i in range(D)])
    Pdev = np.array([P[i * g:(i + 1) * g].sum() for i in range(D)])
    return h, s, float(f @ P), float(fdev @ Pdev)


def loss64(c, idx):
    h, s, eb, db = forward64(c, idx)
    return float((c["dh"].astype(np.float64) * h).sum() + c["a1"] * eb + c["a2"] * db)


def oracle_all(c):
    r = O.route(c["x"], c["E"], c["K"], c["b"], want_probs=True)
    st = O.balance_stats(c["T"], c["K"], c["D"], r["counts"], r["prob_sum"])
    tok = np.arange(c["T"], dtype=np.int32)
    bt = O.backward_tokens(tok, c["x"], c["E"], r["idx"], r["gate"], r["probs"], st["f"], st["f_dev"],
                           c["a1"], c["a2"], c["dh"], c["w1_s"], c["w3_s"], c["w2_s"], c["w1_r"], c["w3_r"],
                           c["w2_r"])
    dE, db = O.backward_router(c["x"], bt["dz"])
    return r, st, bt, dE, db


def fd(c, key, pos, idx):
    """Central difference of loss64 w.r.t. c[key][pos], checking the selection stays fixed."""
    orig = c[key][pos]
    vals = []
    for sgn in (1.0, -1.0):
        c[key][pos] = np.float32(orig + sgn * EPS)
        assert c[key][pos] == orig + sgn * EPS        # exact in fp32
        r = O.route(c["x"], c["E"], c["K"], c["b"])
        assert np.array_equal(r["idx"], idx), "selection changed under the perturbation"
        vals.append(loss64(c, idx))
    c[key][pos] = orig
    return (vals[0] - vals[1]) / (2 * EPS)


@pytest.mark.parametrize("seed", [0, 1])
def test_fp64_forward_matches_oracle_forward(seed):
    c = make_case(seed)
    r = O.route(c["x"], c["E"], c["K"], c["b"], want_probs=True)
    h, s, _, _ = forward64(c, r["idx"])
    np.testing.assert_allclose(s, r["probs"], rtol=2e-6, atol=1e-7)
    o = O.layer_tokens(np.arange(c["T"], dtype=np.int32), c["x"], r["idx"], r["gate"], c["w1_s"], c["w3_s"],
                       c["w2_s"], c["w1_r"], c["w3_r"], c["w2_r"])
    # the oracle uses the fp32-rounded gates, the fp64 forward the exact softmax
    np.testing.assert_allclose(h, o["h"], rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("seed", [0, 1])
def test_dx_dE_dbias_match_finite_differences(seed):
    c = make_case(seed)
    r, st, bt, dE, db = oracle_all(c)
    idx = r["idx"]
    rng = np.random.default_rng(100 + seed)
    for _ in range(6):
        pos = (int(rng.integers(c["T"])), int(rng.integers(c["d"])))
        assert abs(fd(c, "x", pos, idx) - bt["dx"][pos]) < 2e-4 * (1 + abs(bt["dx"][pos]))
    for _ in range(6):
        pos = (int(rng.integers(c["Nr"])), int(rng.integers(c["d"])))
        assert abs(fd(c, "E", pos, idx) - dE[pos]) < 2e-4 * (1 + abs(dE[pos]))
    for rr in range(c["Nr"]):
        assert abs(fd(c, "b", (rr,), idx) - db[rr]) < 2e-4 * (1 + abs(db[rr]))


@pytest.mark.parametrize("seed", [0, 1])
def test_weight_rows_match_finite_differences_of_oracle_forward(seed):
    """dW of a shared and a routed expert against the oracle's own fp64 layer output (gates fixed)."""
    c = make_case(seed)
    r, st, bt, dE, db = oracle_all(c)
    tok = np.arange(c["T"], dtype=np.int32)
    dh = c["dh"].astype(np.float64)

    def L():
        o = O.layer_tokens(tok, c["x"], r["idx"], r["gate"], c["w1_s"], c["w3_s"], c["w2_s"], c["w1_r"],
                           c["w3_r"], c["w2_r"])
        return float((dh * o["h"]).sum())

    def fdw(key, pos):
        orig = c[key][pos]
        c[key][pos] = np.float32(orig + EPS)
        lp = L()
        c[key][pos] = np.float32(orig - EPS)
        lm = L()
        c[key][pos] = orig
        return (lp - lm) / (2 * EPS)

    used = sorted(set(r["idx"].ravel().tolist()))
    for e_glob, key_pref, ei in [(0, "s", 0), (c["Ks"] + used[0], "r", used[0]), (c["Ks"] + used[-1], "r", used[-1])]:
        rows_up = np.arange(c["w"], dtype=np.int32)
        rows_dn = np.arange(c["d"], dtype=np.int32)
        dW1, dW3, dW2 = O.backward_weight_rows(e_glob, c["x"], r["idx"], r["gate"], c["dh"], c["w1_s"],
                                               c["w3_s"], c["w2_s"], c["w1_r"], c["w3_r"], c["w2_r"],
                                               rows_up, rows_dn)
        for (key, ref, shape) in [("w1_", dW1, (c["w"], c["d"])), ("w3_", dW3, (c["w"], c["d"])),
                                  ("w2_", dW2, (c["d"], c["w"]))]:
            for j in range(shape[0]):
                k = (j * 3 + 1) % shape[1]
                got = fdw(key + key_pref, (ei, j, k))
                assert abs(got - ref[j, k]) < 1e-5 * (1 + abs(ref[j, k])), (key, e_glob, j, k)


def test_dgate_matches_finite_differences_of_gates():
    c = make_case(3)
    r, st, bt, dE, db = oracle_all(c)
    tok = np.arange(c["T"], dtype=np.int32)
    dh = c["dh"].astype(np.float64)
    gate = r["gate"].copy()
    for t in range(c["T"]):
        for k in range(c["K"]):
            vals = []
            for sgn in (1.0, -1.0):
                g2 = gate.copy()
                g2[t, k] = np.float32(gate[t, k] + sgn * EPS)
                o = O.layer_tokens(tok, c["x"], r["idx"], g2, c["w1_s"], c["w3_s"], c["w2_s"], c["w1_r"],
                                   c["w3_r"], c["w2_r"])
                vals.append(float((dh * o["h"]).sum()))
            got = (vals[0] - vals[1]) / (2 * (np.float32(gate[t, k] + EPS) - gate[t, k]))
            assert abs(got - bt["dgate"][t, k]) < 1e-5 * (1 + abs(bt["dgate"][t, k]))


def test_invariants():
    c = make_case(5, T=9, d=16, Ks=2, Nr=8, K=3, w=8, D=4)
    r, st, bt, dE, db = oracle_all(c)
    # rows of dz sum to zero up to sum_r s_r - 1 (the affinities are the forward's fp32 values)
    scale = np.abs(bt["dz"]).max()
    np.testing.assert_allclose(bt["dz"].sum(axis=1), 0.0, atol=1e-6 * scale)
    np.testing.assert_allclose(db, bt["dz"].sum(axis=0), atol=1e-12)
    np.testing.assert_allclose(dE.sum(axis=0), 0.0, atol=1e-5 * scale)
    c0 = dict(c)
    c0["dh"] = np.zeros_like(c["dh"])
    c0["a1"] = c0["a2"] = 0.0
    r0, st0, bt0, dE0, db0 = oracle_all(c0)
    assert not bt0["dx"].any() and not dE0.any() and not db0.any() and not bt0["dgate"].any()


def test_balance_only_gradient_closed_form():
    """dh = 0: only alpha terms act; ds_{t,r} = (a1 f_r + a2 f'_g(r)) / T, softmax-backward of that."""
    c = make_case(7, T=5, d=8, Ks=0, Nr=4, K=2, w=4, D=2)
    c["dh"] = np.zeros_like(c["dh"])
    r, st, bt, dE, db = oracle_all(c)
    f = st["f"].astype(np.float64)
    fd_ = st["f_dev"].astype(np.float64)
    ds = (c["a1"] * f + c["a2"] * np.repeat(fd_, c["Nr"] // c["D"])) / c["T"]
    s = r["probs"].astype(np.float64)
    dz = s * (ds[None, :] - (s * ds[None, :]).sum(axis=1, keepdims=True))
    np.testing.assert_allclose(bt["dz"], dz, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(bt["dx"], dz @ c["E"].astype(np.float64), rtol=1e-10, atol=1e-14)
