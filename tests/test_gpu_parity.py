"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small seeded cases span several tiles with ragged tails (expert row counts
that are not multiples of the 128-row tile, T not a multiple of the 64/256
token blocks) and the method's degenerate cases; the workload shapes of the
five configurations run at full size, with routing, grouping and statistics
compared on every token and expert outputs on a seeded token sample.
"""
import numpy as np
import pytest

from fine_grained_mixture_moe_amd import workloads as W
from fine_grained_mixture_moe_amd.layer import DeviceLayer, to_device
import parity as PT

pytestmark = pytest.mark.gpu


def run_case(inp: W.LayerInputs, sample: int = 0, tag: str = "", accumulate: bool = False):
    wl = inp.wl
    PT.say(f"[case] {tag} {wl.name} T={wl.T} d={wl.d} Ks={wl.n_shared} Nr={wl.n_routed} K={wl.top_k} "
           f"w={wl.inter} {wl.dtype} groups={wl.groups}" + (" accumulating" if accumulate else ""))
    dl = DeviceLayer(inp, want_probs=wl.T * wl.n_routed <= (1 << 24), accumulate=accumulate)
    dl.forward()
    dl.expert_sum()
    g = dl.results()
    o = PT.oracle_routing(inp)
    PT.check_routing(g, o, wl)
    PT.check_grouping(g, o)
    PT.check_stats(g, o["stats"])
    tokens = W.sample_tokens(wl.T, sample) if sample else np.arange(wl.T, dtype=np.int32)
    ref = PT.oracle_outputs(inp, o["idx"], o["gate"], tokens)
    PT.check_outputs(g, inp, tokens, ref, tag)
    return dl, g, o


SMALL = [
    # (T, d, Ks, Nr, K, w, dtype, seed, zipf, groups)
    (300, 128, 1, 16, 4, 64, "f32", 1, None, 4),
    (300, 128, 1, 16, 4, 64, "bf16", 2, None, 2),
    (513, 256, 2, 64, 6, 128, "bf16", 3, 1.1, 4),
    (1, 64, 0, 8, 1, 64, "f32", 4, None, 1),
    (200, 192, 0, 200, 16, 64, "bf16", 5, None, 8),
    (257, 128, 1, 100, 3, 128, "f32", 6, None, 5),
    (700, 128, 3, 2, 2, 192, "bf16", 7, None, 2),
    (130, 64, 0, 1, 1, 64, "f32", 8, None, 1),
    (2500, 192, 1, 40, 5, 128, "bf16", 15, 1.1, 4),    # routing: 8 waves, 128-k chunks + a 64-k last chunk
    (6100, 128, 0, 70, 4, 64, "f32", 16, None, 7),     # routing: 2 tokens per wave, 2 expert lanes, ragged T
    (8200, 256, 0, 64, 6, 64, "bf16", 22, 1.1, 4),    # routing: 4 tokens per wave from 8192 tokens, ragged T
    (300, 128, 0, 100, 4, 64, "bf16", 23, None, 4),   # routing, bf16 readlane form: 1 token x 2 expert lanes
    (600, 256, 0, 64, 4, 64, "bf16", 24, None, 4),    # routing, bf16 readlane form: 1 token x 1 expert lane
    (4500, 128, 0, 128, 8, 64, "bf16", 25, 1.1, 4),   # routing, bf16 DPP form: 2 tokens x 2 expert lanes
    (4100, 128, 0, 64, 8, 64, "bf16", 26, None, 4),   # routing, bf16 DPP form: 2 tokens x 1 lane (2 chains), ragged
    (16500, 64, 0, 130, 3, 64, "bf16", 17, None, 5),   # routing: 4 tokens per wave, 3 of 4 expert lanes
    (5000, 64, 0, 256, 16, 64, "bf16", 18, 1.1, 8),    # routing: N'=256, K'=16, skewed
    (9000, 2048, 1, 64, 6, 64, "bf16", 19, 1.1, 4),    # routing: large d, 16 chunks
    (16400, 192, 0, 32, 4, 64, "f32", 20, None, 4),    # routing: fp32 tokens, 2 pieces per lane, last chunk
    (16400, 64, 0, 48, 2, 64, "f32", 21, None, 4),     # routing: d below one chunk (no full chunk)
    (1000, 448, 0, 64, 6, 64, "bf16", 27, None, 4),    # routing, 4-set load ring: 7 chunks (a partial group)
    (900, 320, 0, 128, 8, 64, "f32", 28, None, 4),     # routing, 4-set load ring, readlane form: 10 chunks
    (64, 2048, 2, 64, 6, 64, "bf16", 29, None, 4),     # decode routing: one wave per token, 8 stages, 64 chunks
    (128, 4096, 4, 128, 12, 64, "bf16", 30, None, 4),  # decode routing: two waves per token, 8 stages each
    (256, 320, 0, 256, 16, 64, "f32", 31, 1.1, 8),     # decode routing: four waves, 4 stages, 10 chunks + 2 past the end
    (33, 64, 1, 130, 5, 64, "bf16", 32, None, 5),      # decode routing: three waves, 6 stages, 2 chunks (< prefetch depth)
    (3, 8192, 0, 64, 4, 64, "bf16", 33, None, 4),      # decode routing: token row beyond one staging batch
    (64, 2112, 1, 64, 6, 64, "bf16", 37, 1.1, 4),      # decode routing: 66 chunks, a partial round of 8 stages
    (5, 8192, 0, 100, 4, 64, "bf16", 38, None, 4),     # decode routing: two waves, 6 stages (d past 8-stage LDS)
    (2, 16384, 0, 128, 8, 64, "f32", 39, None, 4),     # decode routing: two waves, 4 stages, the largest d
    (1000, 192, 0, 100, 6, 64, "bf16", 35, 1.1, 4),    # matrix-core logits: ragged T, 100 experts (partial 4th block)
    (777, 128, 1, 96, 5, 64, "f32", 36, None, 4),      # matrix-core logits, fp32 tokens: 96 experts, empty 4th block
]


@pytest.mark.parametrize("case", SMALL, ids=[f"T{c[0]}_d{c[1]}_s{c[2]}_r{c[3]}_k{c[4]}_w{c[5]}_{c[6]}" for c in SMALL])
def test_small_cases(case):
    T, d, Ks, Nr, K, w, dt, seed, zipf, groups = case
    inp = W.make_random_case(T, d, Ks, Nr, K, w, dtype=dt, seed=seed, zipf_s=zipf, groups=groups,
                             w_std=0.05)
    run_case(inp, tag="small")


def test_c1_full_fp32():
    run_case(W.make_inputs(W.WORKLOADS["c1"]), tag="c1")


def test_zero_tokens_tie_to_lowest_experts():
    inp = W.make_random_case(100, 128, 1, 16, 5, 64, dtype="bf16", seed=9)
    inp.x.f32[:] = 0
    inp.x.bf16[:] = 0
    dl, g, o = run_case(inp, tag="x=0")
    assert np.all(g["idx"] == np.arange(5))


def test_duplicated_centroids_tie_to_lower_index():
    inp = W.make_random_case(256, 128, 0, 32, 4, 64, dtype="f32", seed=10)
    inp.centroids[7] = inp.centroids[3]
    inp.centroids[20] = inp.centroids[3]
    inp.x.f32[:64] = inp.centroids[3] * 5.0
    dl, g, o = run_case(inp, tag="ties")
    assert np.all(g["idx"][:64, :3] == np.array([3, 7, 20]))


def test_shared_only_dense_layer():
    inp = W.make_random_case(300, 128, 2, 0, 0, 128, dtype="bf16", seed=11)
    PT.say("[case] shared-only")
    dl = DeviceLayer(inp)
    dl.forward()
    dl.expert_sum()
    g = dl.results()
    tokens = np.arange(300, dtype=np.int32)
    ref = PT.oracle_outputs(inp, np.zeros((300, 0), np.int32), np.zeros((300, 0), np.float32), tokens)
    PT.check_outputs(g, inp, tokens, ref, "shared-only")


def test_empty_batch():
    inp = W.make_random_case(0, 128, 1, 8, 2, 64, dtype="bf16", seed=12)
    PT.say("[case] T=0")
    dl = DeviceLayer(inp)
    dl.forward()
    g = dl.results()
    assert np.all(g["counts"] == 0) and np.all(g["offsets"] == 0)
    assert np.all(g["f"] == 0) and np.all(g["P"] == 0)


def test_permute_every_expert_active():
    """K' = N' (every token picks every expert), supplied routing; gate 1."""
    inp = W.make_random_case(190, 128, 0, 64, 64, 64, dtype="bf16", seed=13)
    PT.say("[case] K'=N'=64 supplied routing")
    T = 190
    idx = np.tile(np.arange(64, dtype=np.int32), (T, 1))
    gate = np.ones((T, 64), np.float32)
    dl = DeviceLayer(inp)
    dl.forward_with_routing(idx, gate)
    dl.expert_sum()
    g = dl.results()
    from oracle import oracle as O
    p = O.permute(idx, 64)
    PT.check_grouping(g, p)
    tokens = W.sample_tokens(T, 40)
    ref = PT.oracle_outputs(inp, idx, gate, tokens)
    PT.check_outputs(g, inp, tokens, ref, "dense-routing")


def test_two_runs_are_bitwise_identical():
    inp = W.make_random_case(2000, 256, 1, 63, 7, 128, dtype="bf16", seed=14)
    PT.say("[case] determinism")
    dl = DeviceLayer(inp, want_probs=True)
    dl.forward()
    a = dl.results()
    dl.forward()
    b = dl.results()
    for k in ("idx", "gate", "probs", "counts", "prob_sum", "offsets", "sorted_token", "slot_of", "y_routed",
              "y_shared", "h", "f", "P", "f_dev", "P_dev", "exp_bal", "dev_bal"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("case", [
    (4096, 256, 0, 64, 8, 256, 31),    # 256-row token tiles, many groups
    (700, 384, 2, 16, 4, 128, 32),     # shared experts, 128-row token tiles, ragged
    (64, 512, 1, 64, 6, 128, 33),      # decode-sized: most experts hold a few rows
])
def test_fused_ffn_equals_two_launches(case):
    """moe_expert_ffn (one fused launch in bf16) and moe_expert_up + moe_expert_down (two
    launches) run the same tile code: their outputs agree bit for bit."""
    T, d, Ks, Nr, K, w, seed = case
    inp = W.make_random_case(T, d, Ks, Nr, K, w, dtype="bf16", seed=seed, zipf_s=1.1, groups=1)
    PT.say(f"[case] fused vs two launches T={T} d={d} Ks={Ks} Nr={Nr} K={K} w={w}")
    dl = DeviceLayer(inp)
    dl.route()
    dl.permute()
    dl.expert_ffn()
    a = dl.results()
    dl.y_routed.zero_()
    if dl.y_acc is not None:
        dl.y_acc.zero_()
    dl.expert_up()
    dl.expert_down()
    b = dl.results()
    assert np.array_equal(a["y_routed"], b["y_routed"])
    if Ks:
        assert np.array_equal(a["y_shared"], b["y_shared"])


@pytest.mark.parametrize("accumulate", [False, True], ids=["gather", "accumulating"])
def test_second_input_over_the_same_workspace(accumulate):
    """The fused launch hands the SwiGLU activations between workgroups through the workspace and
    reads them back as cached loads; a second call with other tokens (other routing, other
    activations in the same rows of the workspace) must see its own activations, not lines left
    in some XCD's L2 by the first call."""
    import dataclasses
    first = W.make_random_case(3000, 256, 1, 32, 6, 256, dtype="bf16", seed=34, zipf_s=1.1, groups=4)
    other = W.make_random_case(3000, 256, 1, 32, 6, 256, dtype="bf16", seed=35, zipf_s=1.1, groups=4)
    second = dataclasses.replace(first, x=other.x)
    PT.say(f"[case] second input over the same workspace, accumulate={accumulate}")
    dl = DeviceLayer(first, accumulate=accumulate)
    dl.forward()
    dl.check_status()
    dl.x.copy_(to_device(second.x.device_bits("bf16"), "bf16", dl.x.device))
    dl.inp = second
    dl.forward()
    dl.expert_sum()
    g = dl.results()
    o = PT.oracle_routing(second)
    PT.check_routing(g, o, second.wl)
    tokens = np.arange(second.wl.T, dtype=np.int32)
    ref = PT.oracle_outputs(second, o["idx"], o["gate"], tokens)
    PT.check_outputs(g, second, tokens, ref, "second input")
