"""moe_layer_forward, the whole layer in one call, against the five calls and the oracle.

Its outputs must be bitwise those of moe_route -> moe_permute -> moe_expert_ffn ->
moe_combine -> moe_balance_stats on the same inputs: on decode batches (one routing
workgroup per token, at most 256 tokens) it runs its own single-workgroup tail kernel
(grouping, routing sums, statistics, FFN control words), elsewhere the five calls' kernels.
"""
import numpy as np
import pytest

from fine_grained_mixture_moe_amd import workloads as W
from fine_grained_mixture_moe_amd.layer import DeviceLayer
import parity as PT

pytestmark = pytest.mark.gpu

KEYS = ("idx", "gate", "probs", "counts", "prob_sum", "offsets", "sorted_token", "slot_of", "y_routed", "y_shared",
        "h", "f", "P", "f_dev", "P_dev", "exp_bal", "dev_bal")


def poison(dl):
    """Every output buffer overwritten, so nothing left by the five-call pass can pass for a result."""
    for t in (dl.idx, dl.slot_of, dl.sorted_token, dl.offsets, dl.counts):
        t.fill_(-7)
    for t in (dl.gate, dl.prob_sum, dl.f, dl.P, dl.f_dev, dl.P_dev, dl.exp_bal, dl.dev_bal, dl.h, dl.y_routed,
              dl.y_acc, dl.probs):
        if t is not None:
            t.fill_(float("nan"))


def same_as_five_calls(inp: W.LayerInputs, tag: str, passes: int = 2):
    wl = inp.wl
    PT.say(f"[case] layer_forward {tag} T={wl.T} d={wl.d} Ks={wl.n_shared} Nr={wl.n_routed} K={wl.top_k} "
           f"w={wl.inter} {wl.dtype} groups={wl.groups}")
    dl = DeviceLayer(inp, want_probs=True)
    dl.forward()
    ref = dl.results()
    for _ in range(passes):   # the tail leaves the control words clear for the next pass
        poison(dl)
        dl.layer_forward()
        got = dl.results()
        for k in KEYS:
            a, b = ref.get(k), got.get(k)
            if a is None:
                assert b is None, k
                continue
            assert np.array_equal(np.asarray(a), np.asarray(b)), f"{tag}: {k} differs from the five calls"
    return dl, got


DECODE = [
    # (T, d, Ks, Nr, K, w, dtype, seed, zipf, groups)
    (64, 2048, 2, 64, 6, 128, "bf16", 41, 1.1, 4),    # 16B-style decode shape (narrow experts)
    (128, 4096, 4, 128, 12, 64, "bf16", 42, None, 4),  # 145B-style decode shape: two routing waves
    (100, 256, 1, 63, 7, 128, "f32", 43, None, 7),     # fp32 layer: the two-launch expert FFN
    (256, 192, 0, 256, 16, 64, "bf16", 44, 1.1, 8),    # the largest batch and expert count of the tail
    (1, 64, 0, 8, 1, 64, "bf16", 45, None, 1),         # one token
    (33, 64, 1, 130, 5, 64, "bf16", 46, None, 5),      # three routing waves, one partial group of rows
    (200, 320, 0, 16, 2, 64, "f32", 47, None, 2),      # no shared experts
]


@pytest.mark.parametrize("case", DECODE, ids=[f"T{c[0]}_d{c[1]}_s{c[2]}_r{c[3]}_k{c[4]}_{c[6]}" for c in DECODE])
def test_decode_tail_equals_five_calls(case):
    T, d, Ks, Nr, K, w, dtype, seed, zipf, groups = case
    inp = W.make_random_case(T, d, Ks, Nr, K, w, dtype=dtype, seed=seed, zipf_s=zipf, groups=groups)
    same_as_five_calls(inp, "decode")


PREFILL = [
    (300, 128, 1, 16, 4, 64, "bf16", 48, None, 4),     # two grouping blocks
    (3000, 256, 1, 64, 6, 128, "bf16", 49, 1.1, 4),    # 12 grouping blocks
    (2500, 192, 1, 100, 5, 64, "f32", 52, None, 5),    # fp32 layer, 10 grouping blocks
    (20000, 64, 0, 256, 8, 64, "bf16", 53, 1.1, 8),    # a histogram large enough for the grouping's scan kernel
    (9000, 2048, 1, 64, 6, 64, "bf16", 54, None, 4),   # several routing workgroups per reduction thread
]


@pytest.mark.parametrize("case", PREFILL, ids=[f"T{c[0]}_d{c[1]}_s{c[2]}_r{c[3]}_k{c[4]}_{c[6]}" for c in PREFILL])
def test_prefill_batches_equal_five_calls(case):
    """Batches of several grouping blocks (the five calls' kernels inside one call)."""
    T, d, Ks, Nr, K, w, dtype, seed, zipf, groups = case
    inp = W.make_random_case(T, d, Ks, Nr, K, w, dtype=dtype, seed=seed, zipf_s=zipf, groups=groups)
    same_as_five_calls(inp, "prefill")


@pytest.mark.parametrize("case", [
    (300, 128, 1, 64, 4, 64, "bf16", 48, None, 4),   # 64 experts over two grouping blocks
    (0, 128, 1, 16, 4, 64, "bf16", 50, None, 4),     # empty batch
])
def test_other_batches_equal_five_calls(case):
    T, d, Ks, Nr, K, w, dtype, seed, zipf, groups = case
    inp = W.make_random_case(T, d, Ks, Nr, K, w, dtype=dtype, seed=seed, zipf_s=zipf, groups=groups)
    same_as_five_calls(inp, "fallback", passes=1)


def test_decode_tail_against_the_oracle():
    """The same bars as the five calls: indices, counts, grouping and f bit-exact, the rest within tolerance."""
    inp = W.make_random_case(96, 512, 2, 64, 6, 128, dtype="bf16", seed=51, zipf_s=1.1, groups=4)
    dl, g = same_as_five_calls(inp, "oracle", passes=1)
    o = PT.oracle_routing(inp)
    PT.check_routing(g, o, inp.wl)
    PT.check_grouping(g, o)
    PT.check_stats(g, o["stats"])
    dl.expert_sum()
    g = dl.results()
    tokens = np.arange(inp.wl.T, dtype=np.int32)
    ref = PT.oracle_outputs(inp, o["idx"], o["gate"], tokens)
    PT.check_outputs(g, inp, tokens, ref, "layer_forward")


@pytest.mark.parametrize("name", ["c5a", "c5c", "c2b", "c5b"])
def test_configs_full_size(name):
    """Decode and prefill workloads at full size: moe_layer_forward bitwise equal to the five calls."""
    if name == "c2b":
        inp = W.make_c2_fine(independent_centroids=True, coarse=W.make_c2_coarse())
    else:
        inp = W.make_inputs(W.WORKLOADS[name])
    same_as_five_calls(inp, name, passes=1)
