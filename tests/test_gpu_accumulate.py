"""GPU parity of the accumulating expert FFN and the fused launch's error path.

The accumulating mode of moe_expert_ffn (y_routed = NULL) adds the
gate-weighted expert outputs into y_acc inside the down projection, so the
layer output is "[ACL 2024] DeepSeekMoE: 混合专家语言模型中的极致专家特化", section
"Method details" (output formula), with the sum formed by fp32 atomics.  It is
checked against the oracle at the same bars as the gather mode: y (the GPU's
own expert sum, moe_combine with a zero residual) and h per token row.

The error path: a host-side test hook makes every wait of the fused launch
unmeetable with a short spin limit, so each down tile gives up, writes NaN
over its outputs and the launch still ends normally; moe_expert_ffn_status
must report it, and the next call must be clean again.
"""
import numpy as np
import pytest

from fine_grained_mixture_moe_amd import moe as M
from fine_grained_mixture_moe_amd import workloads as W
from fine_grained_mixture_moe_amd.layer import DeviceLayer
import parity as PT
from test_gpu_parity import run_case

pytestmark = pytest.mark.gpu

CASES = [
    # (T, d, Ks, Nr, K, w, dtype, seed, zipf, groups)
    (300, 128, 1, 16, 4, 64, "f32", 61, None, 4),      # fp32 path: atomics from the MFMA registers
    (513, 256, 2, 64, 6, 128, "bf16", 62, 1.1, 4),     # 128-row tiles, shared group, skewed routing
    (4096, 256, 0, 64, 8, 256, "bf16", 63, None, 4),   # 256-row tiles (4 LDS passes per tile), no shared
    (2100, 320, 1, 16, 2, 192, "bf16", 64, None, 2),   # 256-row tiles, shared group, ragged columns (d % 256)
    (64, 512, 1, 64, 6, 128, "bf16", 65, None, 4),     # decode-sized: non-temporal weight loads
    (700, 128, 3, 2, 2, 192, "bf16", 66, None, 2),     # few experts, many rows each
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}_d{c[1]}_s{c[2]}_r{c[3]}_k{c[4]}_{c[6]}" for c in CASES])
def test_accumulating_small_cases(case):
    T, d, Ks, Nr, K, w, dt, seed, zipf, groups = case
    inp = W.make_random_case(T, d, Ks, Nr, K, w, dtype=dt, seed=seed, zipf_s=zipf, groups=groups, w_std=0.05)
    dl, g, o = run_case(inp, tag="accumulating", accumulate=True)
    assert g["y_routed"] is None


def test_accumulating_c1_fp32():
    run_case(W.make_inputs(W.WORKLOADS["c1"]), tag="c1 accumulating", accumulate=True)


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,sample", [("c4", 96), ("c5b", 48), ("c5a", 64)])
def test_accumulating_full_size(name, sample):
    run_case(W.make_inputs(W.WORKLOADS[name]), sample=sample, tag="full accumulating", accumulate=True)


def test_accumulating_matches_gather_mode():
    """Both modes compute the same layer: h within the bf16 bar of each other on every token."""
    inp = W.make_random_case(1500, 256, 1, 32, 4, 128, dtype="bf16", seed=67, zipf_s=1.1, groups=4)
    PT.say("[case] accumulating vs gather")
    a = DeviceLayer(inp, accumulate=True)
    a.forward()
    a.expert_sum()
    ga = a.results()
    b = DeviceLayer(inp)
    b.forward()
    b.expert_sum()
    gb = b.results()
    assert np.array_equal(ga["idx"], gb["idx"])
    e_y = PT.row_rel_err(ga["y"], gb["y"])
    e_acc = PT.row_rel_err(ga["y_acc"], gb["y"])
    PT.say(f"  y {e_y:.3e}, y_acc vs gather y {e_acc:.3e}")
    assert e_y < PT.TOL["bf16"] and e_acc < PT.TOL["bf16"]


@pytest.mark.parametrize("accumulate", [False, True], ids=["gather", "accumulating"])
def test_stalled_wait_is_reported_and_poisons_outputs(monkeypatch, accumulate):
    inp = W.make_random_case(700, 256, 1, 16, 4, 128, dtype="bf16", seed=68, groups=4)
    PT.say(f"[case] forced stall, accumulate={accumulate}")
    dl = DeviceLayer(inp, accumulate=accumulate)
    monkeypatch.setenv("MOE_DEBUG_FFN_STALL", "64")
    dl.forward()
    assert dl.ffn_status() == M.MOE_ERR_STALLED
    with pytest.raises(M.MoEError) as e:
        dl.results()
    assert e.value.status == M.MOE_ERR_STALLED
    g = dl.results(check=False)
    # every down tile gave up: no output was computed from the activations
    if accumulate:
        assert np.all(np.isnan(g["y_acc"]))
    else:
        assert np.all(np.isnan(g["y_routed"]))
        assert np.all(np.isnan(g["y_shared"]))
    assert np.all(np.isnan(g["h"]))
    monkeypatch.delenv("MOE_DEBUG_FFN_STALL")
    dl.forward()
    assert dl.ffn_status() == M.MOE_OK
    dl.expert_sum()
    g = dl.results()
    o = PT.oracle_routing(inp)
    tokens = np.arange(inp.wl.T, dtype=np.int32)
    ref = PT.oracle_outputs(inp, o["idx"], o["gate"], tokens)
    PT.check_outputs(g, inp, tokens, ref, "after stall")
