"""Pins of the oracle's routing variants (CPU only): the top-r disabling
ablation against a brute-force sort and against plain routing at r = 0; the
fixed hash routing against hand-computed values and its distribution."""
import numpy as np
import pytest

from oracle import oracle as O


def case(seed, T=60, d=16, Nr=12):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    E = (rng.standard_normal((Nr, d)) / np.sqrt(d)).astype(np.float32)
    b = (0.3 * rng.standard_normal(Nr)).astype(np.float32)
    return x, E, b


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_ablate_with_nothing_disabled_is_plain_routing(seed):
    x, E, b = case(seed)
    a = O.route_ablate(x, E, 3, 0, b, want_probs=True)
    r = O.route(x, E, 3, b, want_probs=True)
    for k in ("idx", "gate", "probs", "counts", "prob_sum"):
        assert np.array_equal(a[k], r[k]), k


@pytest.mark.parametrize("skip,K", [(1, 2), (2, 3), (4, 1), (9, 3)])
def test_ablate_against_brute_force_sort(skip, K):
    x, E, b = case(10 + skip)
    T, Nr = x.shape[0], E.shape[0]
    a = O.route_ablate(x, E, K, skip, b, want_probs=True)
    z = O.logits(x, E, b)
    for t in range(T):
        order = sorted(range(Nr), key=lambda r: (-float(z[t, r]), r))   # -0.0 == 0.0 in the key
        assert list(a["idx"][t]) == order[skip:skip + K]
        s = np.exp(z[t].astype(np.float64) - z[t].max())
        s /= s.sum()
        np.testing.assert_allclose(a["gate"][t], s[order[skip:skip + K]], rtol=1e-6)
    assert np.array_equal(a["counts"], np.bincount(a["idx"].ravel(), minlength=Nr))
    # the disabled experts are exactly each token's top `skip`
    full = O.route(x, E, skip + K, b)
    assert np.array_equal(full["idx"][:, skip:], a["idx"])


def test_hash_routing_hand_values():
    # h = id * 2654435761 mod 2^32, expert = floor(h * N' / 2^32), worked by hand for N' = 64:
    #   id 1: h = 2654435761 -> 39.55 -> 39;  id 2: h = 1013904226 -> 15.1 -> 15;
    #   id 3: h = 3668339987 -> 54.66 -> 54;  id 0 -> 0
    r = O.route_hash(np.array([0, 1, 2, 3], np.int32), 64)
    assert r["idx"].ravel().tolist() == [0, 39, 15, 54]
    assert (r["gate"] == 1.0).all()


def test_hash_routing_is_uniform_and_in_range():
    ids = np.arange(64000, dtype=np.int32)
    for Nr in (16, 63, 64, 256):
        r = O.route_hash(ids, Nr)
        assert r["idx"].min() >= 0 and r["idx"].max() < Nr
        c = r["counts"]
        assert c.sum() == ids.size
        assert np.abs(c - ids.size / Nr).max() <= 0.1 * ids.size / Nr
