"""GPU parity of the routing variants through the C ABI against the CPU oracle.

Top-r disabling (the redundancy ablation of the DeepSeekMoE paper, section
"Expert specialization analysis", Fig. 4) and fixed hash routing (the Hash
Layer baseline of section "Experiment design"): indices and counts bit-exact,
gates, probabilities and probability sums within 1e-5, and a whole layer pass
on variant routing (grouping, expert FFNs, combine, balance statistics)
against the oracle at the bf16/fp32 output bars.
"""
import numpy as np
import pytest

from fine_grained_mixture_moe_amd import workloads as W
from fine_grained_mixture_moe_amd.layer import DeviceLayer, to_device
import parity as PT
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def check_layer_on(dl: DeviceLayer, inp: W.LayerInputs, o_route: dict, tag: str, stats: bool = True):
    """After a variant route call on `dl`: run the rest of the layer, compare everything with the oracle."""
    wl = inp.wl
    dl.permute()
    dl.expert_ffn()
    dl.combine()
    if stats:
        dl.balance_stats()
    dl.expert_sum()
    g = dl.results()
    assert np.array_equal(g["idx"], o_route["idx"]), "expert indices differ"
    assert np.array_equal(g["counts"], o_route["counts"]), "per-expert counts differ"
    assert PT.rel_err(g["gate"], o_route["gate"]) < PT.REL_ROUTE
    o = dict(o_route)
    o.update(O.permute(o_route["idx"], wl.n_routed))
    PT.check_grouping(g, o)
    if stats:
        s = O.balance_stats(wl.T, wl.top_k, wl.groups, o_route["counts"], o_route["prob_sum"])
        PT.check_stats(g, s)
    tokens = W.sample_tokens(wl.T, 512) if wl.T > 512 else np.arange(wl.T, dtype=np.int32)
    ref = PT.oracle_outputs(inp, o_route["idx"], o_route["gate"], tokens)
    PT.check_outputs(g, inp, tokens, ref, tag)
    return g


ABLATE = [
    # (T, d, Ks, Nr, K, w, dtype, seed, zipf, groups, disabled_top)
    (300, 128, 1, 16, 4, 64, "f32", 31, None, 4, 1),
    (513, 256, 2, 64, 6, 128, "bf16", 32, 1.1, 4, 3),
    (2500, 192, 1, 40, 5, 128, "bf16", 33, 1.1, 4, 6),    # 8 waves, last 64-k chunk
    (5000, 64, 0, 256, 8, 64, "bf16", 34, 1.1, 8, 8),     # disabled + K' = 16, N' = 256
    (16400, 192, 0, 32, 4, 64, "f32", 35, None, 4, 2),    # 4 tokens per wave, ragged T
    (200, 128, 0, 12, 2, 64, "f32", 36, None, 3, 10),     # disabled + K' = N': the two lowest-ranked experts
    (96, 1024, 1, 128, 6, 64, "bf16", 37, None, 4, 4),    # decode routing kernel (two waves per token)
]


@pytest.mark.parametrize("case", ABLATE,
                         ids=[f"T{c[0]}_d{c[1]}_r{c[3]}_k{c[4]}_skip{c[10]}_{c[6]}" for c in ABLATE])
def test_route_ablate_layer(case):
    T, d, Ks, Nr, K, w, dt, seed, zipf, groups, skip = case
    PT.say(f"[case] ablate T={T} d={d} Nr={Nr} K={K} skip={skip} {dt}")
    inp = W.make_random_case(T, d, Ks, Nr, K, w, dtype=dt, seed=seed, zipf_s=zipf, groups=groups, w_std=0.05)
    dl = DeviceLayer(inp, want_probs=True)
    dl.route_ablate(skip)
    o = O.route_ablate(inp.x.f32, inp.centroids, K, skip, inp.bias, want_probs=True)
    g = check_layer_on(dl, inp, o, f"ablate{skip}")
    assert PT.rel_err(g["probs"], o["probs"]) < PT.REL_ROUTE
    assert PT.rel_err(g["prob_sum"], o["prob_sum"]) < PT.REL_ROUTE


def test_route_ablate_zero_is_plain_routing():
    inp = W.make_random_case(1000, 256, 1, 64, 6, 64, dtype="bf16", seed=37, zipf_s=1.1, groups=4)
    a = DeviceLayer(inp)
    a.route_ablate(0)
    b = DeviceLayer(inp)
    b.route()
    ga, gb = a.results(), b.results()
    for k in ("idx", "gate", "counts", "prob_sum"):
        assert np.array_equal(ga[k], gb[k]), k


def test_route_ablate_shifts_the_ranking():
    """The experts taken with r disabled are ranks r.. of the plain routing with r + K' experts."""
    T, Nr, K, skip = 700, 64, 4, 5
    inp = W.make_random_case(T, 128, 0, Nr, K, 64, dtype="f32", seed=38)
    a = DeviceLayer(inp)
    a.route_ablate(skip)
    wide = W.make_random_case(T, 128, 0, Nr, skip + K, 64, dtype="f32", seed=38)
    b = DeviceLayer(wide)
    b.route()
    ga, gb = a.results(), b.results()
    assert np.array_equal(ga["idx"], gb["idx"][:, skip:])
    assert np.array_equal(ga["gate"], gb["gate"][:, skip:])


HASH = [
    # (T, d, Ks, Nr, w, dtype, seed, vocab)
    (300, 128, 1, 16, 64, "f32", 41, 8192),
    (4096, 256, 1, 63, 128, "bf16", 42, 8192),      # 2B-like: 1 shared + 63 routed
    (5000, 128, 0, 256, 64, "bf16", 43, 100000),
    (1, 64, 0, 8, 64, "f32", 44, 100),
]


@pytest.mark.parametrize("case", HASH, ids=[f"T{c[0]}_r{c[3]}_{c[5]}" for c in HASH])
def test_route_hash_layer(case):
    T, d, Ks, Nr, w, dt, seed, vocab = case
    PT.say(f"[case] hash T={T} d={d} Nr={Nr} {dt} vocab={vocab}")
    inp = W.make_random_case(T, d, Ks, Nr, 1, w, dtype=dt, seed=seed, groups=1)
    ids = W.token_ids(T, vocab, seed)
    dl = DeviceLayer(inp)
    dids = to_device(ids, "i32", dl.device)
    dl.route_hash(dids)
    o = O.route_hash(ids, Nr)
    o["prob_sum"] = np.zeros(Nr)      # no router: statistics not checked here
    check_layer_on(dl, inp, o, "hash", stats=False)


def test_route_hash_empty_batch_and_extreme_ids():
    inp = W.make_random_case(0, 64, 0, 8, 1, 64, dtype="f32", seed=45)
    dl = DeviceLayer(inp)
    dl.route_hash(to_device(np.zeros(1, np.int32), "i32", dl.device))
    assert np.array_equal(dl.results()["counts"], np.zeros(8, np.int32))
    ids = np.array([0, 1, -1, 2**31 - 1, -2**31, 12345, 7, 7], np.int32)
    inp = W.make_random_case(len(ids), 64, 0, 37, 1, 64, dtype="f32", seed=46)
    dl = DeviceLayer(inp)
    dl.route_hash(to_device(ids, "i32", dl.device))
    g = dl.results()
    o = O.route_hash(ids, 37)
    assert np.array_equal(g["idx"], o["idx"])
    assert np.array_equal(g["counts"], o["counts"])
    assert np.all(g["gate"] == 1.0)


# Inference-time ablations of a trained layer keep its weights and change only which experts run:
# the shared expert switched off, only 4 routed experts activated, Switch-style top-1 on the coarse
# 16-expert layer.  They are shapes of the same calls; the oracle checks them as any other layer.
ABLATIONS = [
    # (config, drop_shared, top_k, sample)
    ("c3", True, None, 128),      # shared expert disabled
    ("c3", False, 4, 128),        # 1 shared + 4 of 63 routed experts
    ("c3", False, 3, 128),        # half-activated 1 + 3
    ("c2a", False, 1, 128),       # Switch-style top-1 of 16 coarse experts
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", ABLATIONS, ids=[f"{c[0]}_noshared{int(c[1])}_k{c[2]}" for c in ABLATIONS])
def test_layer_ablations_at_full_size(case):
    from test_gpu_parity import run_case
    name, drop_shared, top_k, sample = case
    base = W.make_inputs(W.WORKLOADS[name])
    inp = W.ablated_inputs(base, drop_shared=drop_shared, top_k=top_k)
    dl, g, o = run_case(inp, sample=sample, tag="ablation")
    if drop_shared:
        # h of the full layer minus h of the ablated one is the shared experts' output alone
        full = DeviceLayer(base)
        full.forward()
        gf = full.results()
        tokens = W.sample_tokens(inp.wl.T, sample)
        assert np.array_equal(gf["idx"], g["idx"])
        hf = gf["h"][tokens].astype(np.float64)
        ha = g["h"][tokens].astype(np.float64)
        ys = gf["y_shared"][tokens].astype(np.float64)
        # each bf16 h is rounded to nearest (relative error <= 2^-8 per element), and the expert
        # outputs carry the bf16 GEMM bar on top of that
        err = np.linalg.norm(hf - ha - ys, axis=1)
        bound = 2.0 ** -8 * (np.linalg.norm(hf, axis=1) + np.linalg.norm(ha, axis=1)) \
            + PT.TOL["bf16"] * np.linalg.norm(ys, axis=1)
        assert np.all(err <= bound), float((err / bound).max())
