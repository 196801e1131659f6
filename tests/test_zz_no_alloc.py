"""moe_route_noalloc -- the allocation-free variant of moe_route -- against moe_route.

Both run the same routing kernels; only the home of the per-workgroup partial
statistics differs (the library's static device array instead of the
caller's workspace), so every output must agree bit for bit.  Two calls in a
row, the second on a smaller batch, check that the shared array carries
nothing from one call into the next.
"""
import numpy as np
import pytest

from fine_grained_mixture_moe_amd import moe as M
from fine_grained_mixture_moe_amd import workloads as W
from fine_grained_mixture_moe_amd.layer import DeviceLayer
import parity as PT

pytestmark = pytest.mark.gpu

KEYS = ("idx", "gate", "probs", "counts", "prob_sum")


def _route_both(inp):
    import torch
    dl = DeviceLayer(inp, want_probs=True)
    dl.route()
    torch.cuda.synchronize()
    ref = {k: getattr(dl, k).cpu().numpy().copy() for k in KEYS}
    for k in KEYS:
        getattr(dl, k).fill_(-7)
    M.moe_route_noalloc(dl.prob, dl.x, dl.centroids, dl.bias, dl.idx, dl.gate, dl.probs, dl.counts, dl.prob_sum)
    torch.cuda.synchronize()
    got = {k: getattr(dl, k).cpu().numpy().copy() for k in KEYS}
    return ref, got


@pytest.mark.parametrize("first,second", [
    ((16384, 1280, 1, 63, 7, 512, "bf16", 81, None), (300, 1280, 1, 63, 7, 512, "bf16", 82, None)),
    ((8200, 256, 0, 64, 6, 64, "bf16", 83, 1.1), (1000, 448, 0, 64, 6, 64, "bf16", 84, None)),
    ((4500, 128, 0, 256, 16, 64, "f32", 85, 1.1), (64, 128, 0, 256, 16, 64, "f32", 86, None)),
])
def test_noalloc_route_equals_route_on_two_calls(first, second):
    for case in (first, second):
        T, d, Ks, Nr, K, w, dt, seed, zipf = case
        PT.say(f"[case] moe_route_noalloc T={T} d={d} Nr={Nr} K={K} {dt}")
        inp = W.make_random_case(T, d, Ks, Nr, K, w, dtype=dt, seed=seed, zipf_s=zipf)
        ref, got = _route_both(inp)
        for k in KEYS:
            assert np.array_equal(ref[k], got[k]), k
        assert int(got["counts"].sum()) == T * K


def test_noalloc_route_rejects_problems_beyond_its_scratch():
    p = M.moe_problem.make(60000, 256, 0, 256, 8, 64, "bf16")   # partials above 4 MiB
    with pytest.raises(M.MoEError) as e:
        M.moe_route_noalloc(p, 1 << 20, 1 << 20, None, 1 << 20, 1 << 20, None, 1 << 20, 1 << 20)
    assert e.value.status == M.MOE_ERR_UNSUPPORTED
