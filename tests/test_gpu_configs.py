"""GPU parity at the full workload shapes (the five configurations).

Routing, grouping and statistics are compared on every token; expert
outputs, y and h on a seeded token sample (the oracle evaluates those tokens
one by one).  The c2 pair also checks the fine-grained segmentation
identities of "[ACL 2024] DeepSeekMoE: 混合专家语言模型中的极致专家特化",
section "Two core strategies", on the GPU path itself.
"""
import numpy as np
import pytest

from fine_grained_mixture_moe_amd import workloads as W
from fine_grained_mixture_moe_amd.layer import DeviceLayer
import parity as PT
from test_gpu_parity import run_case

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,sample", [("c2a", 192), ("c2b", 192), ("c3", 160), ("c4", 96),
                                         ("c5a", 64), ("c5c", 128), ("c5b", 48)])
def test_config_full_size(name, sample):
    inp = W.make_inputs(W.WORKLOADS[name])
    dl, g, o = run_case(inp, sample=sample, tag="full")
    if name == "c4":
        # Zipf-skewed routing: heavy imbalance is present and visible in the balance terms
        c = g["counts"].astype(np.float64)
        PT.say(f"  c4 load max/mean={c.max() / c.mean():.2f} min/mean={c.min() / c.mean():.3f} "
               f"ExpBal={g['exp_bal']:.4f} DevBal={g['dev_bal']:.4f} f'={g['f_dev']}")
        assert c.max() / c.mean() > 3.0
        assert g["exp_bal"] > 1.5


def _y(g: dict, tokens: np.ndarray, K: int, d: int) -> np.ndarray:
    """The GPU's expert sum (moe_combine with a zero residual) on the tokens."""
    return g["y"][tokens].astype(np.float64)


@pytest.mark.timeout(900)
def test_c2_replicated_centroids_fine_equals_coarse_over_m():
    """Fine experts inheriting the coarse centroid: y_fine = y_coarse / m on the GPU path."""
    coarse = W.make_c2_coarse()
    fine = W.make_c2_fine(independent_centroids=False, coarse=coarse)
    PT.say("[case] c2 replicated-centroid identity")
    dc = DeviceLayer(coarse)
    dc.forward()
    dc.expert_sum()
    gc = dc.results()
    df = DeviceLayer(fine)
    df.forward()
    df.expert_sum()
    gf = df.results()
    m = fine.wl.n_routed // coarse.wl.n_routed
    assert np.array_equal(np.sort(gf["idx"] // m, axis=1), np.sort(np.repeat(gc["idx"], m, axis=1), axis=1))
    tokens = np.arange(coarse.wl.T, dtype=np.int32)
    yc = _y(gc, tokens, coarse.wl.top_k, coarse.wl.d)
    yf = _y(gf, tokens, fine.wl.top_k, fine.wl.d)
    err = PT.row_rel_err(yf, yc / m)
    PT.say(f"  y_fine vs y_coarse/m: {err:.3e}")
    assert err < PT.TOL["bf16"]


@pytest.mark.timeout(900)
def test_c2_dense_check_all_fine_experts_equal_one_wide_ffn():
    """All 64 fine experts at gate 1 (supplied routing) = one FFN of width 32768."""
    coarse = W.make_c2_coarse()
    fine = W.make_c2_fine(independent_centroids=True, coarse=coarse)
    dense = W.make_c2_dense(coarse)
    T, Nr = fine.wl.T, fine.wl.n_routed
    PT.say("[case] c2 dense check")
    allx = W.LayerInputs(fine.wl.replace(top_k=Nr), fine.x, fine.centroids, None, fine.w1, fine.w3, fine.w2)
    da = DeviceLayer(allx)
    da.forward_with_routing(np.tile(np.arange(Nr, dtype=np.int32), (T, 1)), np.ones((T, Nr), np.float32))
    da.expert_sum()
    ga = da.results()
    dd = DeviceLayer(dense)
    dd.forward()
    dd.expert_sum()
    gd = dd.results()
    tokens = np.arange(T, dtype=np.int32)
    ya = _y(ga, tokens, Nr, fine.wl.d)
    yd = gd["y_shared"].astype(np.float64)
    err = PT.row_rel_err(ya, yd)
    PT.say(f"  64 experts @ gate 1 vs width-32768 FFN: {err:.3e}")
    assert err < PT.TOL["bf16"]
    # and the dense path against the oracle on a sample
    sample = W.sample_tokens(T, 24)
    ref = PT.oracle_outputs(dense, np.zeros((T, 0), np.int32), np.zeros((T, 0), np.float32), sample)
    PT.check_outputs(gd, dense, sample, ref, "dense-32768")
