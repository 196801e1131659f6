"""Seeded synthetic workloads for the DeepSeekMoE layer forward.

This module only *draws* inputs: token activations u_t, expert centroids
e_i, an optional per-expert logit bias, and the SwiGLU expert weights.  It
holds none of the layer's arithmetic (no routing, no FFN, no statistics), so
both the CPU oracle and the HIP path can consume its arrays without sharing
any of the method.

Shapes follow the model scales of "DeepSeekMoE: Towards Ultimate Expert
Specialization ..." (blog summary, section "Experiment design", model scales:
hidden 1280 / 2048 / 4096; section "Two core strategies": 1 shared + 63
routed with 7 active for the 2B model, 2 shared + 64 routed with 6 active for
the 16B model).  Expert intermediate widths, token counts and the 145B expert
counts are not on the pages; they are chosen values of the workload set.

Generator: NumPy PCG64 seeded with SeedSequence([1000 + config_no, variant,
tensor_id]); tensor ids: 0 x, 1 centroids, 2 bias permutation, 3 W1, 4 W3,
5 W2.  Shared and routed experts are drawn as one stack in global expert
order (shared first).  bf16 configurations round the fp32 draws to bf16 with
round-to-nearest-even on the bit pattern; the fp32 view handed to the oracle
is the exact upcast of those bf16 bits, so both sides see identical values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

T_X, T_E, T_BIAS, T_W1, T_W3, T_W2 = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens
    d: int            # hidden size
    n_shared: int     # K_s
    n_routed: int     # N'
    top_k: int        # K'
    inter: int        # w, expert intermediate width
    dtype: str        # "f32" or "bf16"
    config_no: int
    variant: int = 0
    x_std: float = 1.0
    w_std: float = 0.02
    zipf_s: Optional[float] = None   # per-expert logit bias -s*ln(rank+1)
    groups: int = 1                  # D, device groups for the balance terms
    description: str = ""

    @property
    def n_experts(self) -> int:
        return self.n_shared + self.n_routed

    def flops(self) -> float:
        """Active FLOPs of one layer pass: gating GEMM plus 3 GEMMs per active expert."""
        return float(self.T) * 2.0 * self.d * (self.n_routed + 3.0 * self.inter * (self.n_shared + self.top_k))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "c1": Workload("c1", 512, 256, 1, 63, 7, 128, "f32", 1, x_std=0.02, w_std=0.02,
                   description="tiny fine-grained layer, fp32: T=512 d=256 1+63 experts top-7 w=128"),
    "c2a": Workload("c2a", 4096, 1280, 0, 16, 2, 2048, "bf16", 2, variant=0,
                    description="GShard-style 16 experts of width 2048, top-2, T=4096 d=1280"),
    "c2b": Workload("c2b", 4096, 1280, 0, 64, 8, 512, "bf16", 2, variant=1,
                    description="fine-grained split: 64 experts of width 512, top-8, T=4096 d=1280"),
    "c3": Workload("c3", 16384, 1280, 1, 63, 7, 512, "bf16", 3,
                   description="2B-style layer: T=16384 d=1280 1+63 experts top-7 w=512"),
    "c4": Workload("c4", 16384, 2048, 2, 64, 6, 1408, "bf16", 4, zipf_s=1.1, groups=4,
                   description="16B-style layer, Zipf(1.1)-skewed routing: T=16384 d=2048 2+64 top-6 w=1408, D=4"),
    "c5a": Workload("c5a", 64, 2048, 2, 64, 6, 1408, "bf16", 5, variant=0,
                    description="16B-style decode: T=64 d=2048 2+64 top-6 w=1408"),
    "c5b": Workload("c5b", 8192, 4096, 4, 128, 12, 1024, "bf16", 5, variant=1,
                    description="145B-style prefill: T=8192 d=4096 4+128 top-12 w=1024"),
    "c5c": Workload("c5c", 128, 4096, 4, 128, 12, 1024, "bf16", 5, variant=2,
                    description="145B-style decode: T=128 d=4096 4+128 top-12 w=1024"),
}


def rng_for(wl: Workload, tensor_id: int) -> np.random.Generator:
    ss = np.random.SeedSequence([1000 + wl.config_no, wl.variant, tensor_id])
    return np.random.Generator(np.random.PCG64(ss))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact fp32 upcast of bf16 bit patterns."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Tensor:
    """One input tensor: exact fp32 values plus, for bf16 workloads, the bf16 bits."""
    f32: np.ndarray
    bf16: Optional[np.ndarray] = None

    def device_bits(self, dtype: str) -> np.ndarray:
        return self.bf16 if dtype == "bf16" else self.f32


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def _as_dtype(a: np.ndarray, dtype: str) -> Tensor:
    if dtype == "bf16":
        bits = bf16_bits_from_f32(a)
        return Tensor(f32_from_bf16_bits(bits), bits)
    return Tensor(np.ascontiguousarray(a, dtype=np.float32))


@dataclasses.dataclass
class LayerInputs:
    wl: Workload
    x: Tensor                 # [T, d]
    centroids: np.ndarray     # [N', d] fp32
    bias: Optional[np.ndarray]  # [N'] fp32 or None
    w1: Tensor                # [K_s+N', w, d]   gate projection (out x in)
    w3: Tensor                # [K_s+N', w, d]   up projection
    w2: Tensor                # [K_s+N', d, w]   down projection

    def shared(self, t: Tensor) -> Tensor:
        ks = self.wl.n_shared
        return Tensor(t.f32[:ks], None if t.bf16 is None else t.bf16[:ks])

    def routed(self, t: Tensor) -> Tensor:
        ks = self.wl.n_shared
        return Tensor(t.f32[ks:], None if t.bf16 is None else t.bf16[ks:])


def make_x(wl: Workload) -> Tensor:
    return _as_dtype(_normal(rng_for(wl, T_X), (wl.T, wl.d), wl.x_std), wl.dtype)


def make_centroids(wl: Workload) -> np.ndarray:
    e = _normal(rng_for(wl, T_E), (wl.n_routed, wl.d), 1.0)
    return (e / np.float32(math.sqrt(wl.d))).astype(np.float32)


def make_bias(wl: Workload) -> Optional[np.ndarray]:
    """Zipf(s) logit bias -s*ln(pi(r)+1) with pi a seeded permutation of the routed experts.

    exp(bias) is proportional to (rank+1)^(-s); the permutation keeps the hot
    experts away from the low-index tie-break.
    """
    if wl.zipf_s is None:
        return None
    perm = rng_for(wl, T_BIAS).permutation(wl.n_routed)
    return (-wl.zipf_s * np.log(perm.astype(np.float64) + 1.0)).astype(np.float32)


def make_weights(wl: Workload):
    E, w, d = wl.n_experts, wl.inter, wl.d
    w1 = _as_dtype(_normal(rng_for(wl, T_W1), (E, w, d), wl.w_std), wl.dtype)
    w3 = _as_dtype(_normal(rng_for(wl, T_W3), (E, w, d), wl.w_std), wl.dtype)
    w2 = _as_dtype(_normal(rng_for(wl, T_W2), (E, d, w), wl.w_std), wl.dtype)
    return w1, w3, w2


def make_inputs(wl: Workload) -> LayerInputs:
    if wl.name == "c2b":
        return make_c2_fine(independent_centroids=True)
    w1, w3, w2 = make_weights(wl)
    return LayerInputs(wl, make_x(wl), make_centroids(wl), make_bias(wl), w1, w3, w2)


# ---------------------------------------------------------------------------
# Granularity-equivalence construction (fine-grained expert segmentation,
# blog summary section "Two core strategies": each expert FFN is split into m
# smaller experts whose intermediate width is 1/m of the original).
# ---------------------------------------------------------------------------

def split_experts(w1: Tensor, w3: Tensor, w2: Tensor, m: int):
    """Column-split coarse experts [N, W, d]/[N, d, W] into m*N experts of width W/m.

    Fine expert m*c + j takes intermediate units j*W/m .. (j+1)*W/m of coarse
    expert c: rows of W1/W3 and columns of W2.  Pure re-indexing.
    """
    def split_up(t: np.ndarray) -> np.ndarray:
        n, W, d = t.shape
        return np.ascontiguousarray(t.reshape(n * m, W // m, d))

    def split_down(t: np.ndarray) -> np.ndarray:
        n, d, W = t.shape
        return np.ascontiguousarray(t.reshape(n, d, m, W // m).transpose(0, 2, 1, 3).reshape(n * m, d, W // m))

    def both(t: Tensor, fn) -> Tensor:
        return Tensor(fn(t.f32), None if t.bf16 is None else fn(t.bf16))

    return both(w1, split_up), both(w3, split_up), both(w2, split_down)


def concat_experts(w1: Tensor, w3: Tensor, w2: Tensor):
    """Concatenate N experts [N, W, d]/[N, d, W] into one dense FFN [1, N*W, d]/[1, d, N*W]."""
    def cat_up(t: np.ndarray) -> np.ndarray:
        n, W, d = t.shape
        return np.ascontiguousarray(t.reshape(1, n * W, d))

    def cat_down(t: np.ndarray) -> np.ndarray:
        n, d, W = t.shape
        return np.ascontiguousarray(t.transpose(1, 0, 2).reshape(1, d, n * W))

    def both(t: Tensor, fn) -> Tensor:
        return Tensor(fn(t.f32), None if t.bf16 is None else fn(t.bf16))

    return both(w1, cat_up), both(w3, cat_up), both(w2, cat_down)


def make_c2_coarse() -> LayerInputs:
    return make_inputs(WORKLOADS["c2a"])


def make_c2_fine(independent_centroids: bool = True, coarse: Optional[LayerInputs] = None) -> LayerInputs:
    """c2b: the c2a weights split 4-way; independent centroids, or the coarse ones replicated."""
    coarse = coarse if coarse is not None else make_c2_coarse()
    wl = WORKLOADS["c2b"]
    m = wl.n_routed // coarse.wl.n_routed
    w1, w3, w2 = split_experts(coarse.w1, coarse.w3, coarse.w2, m)
    if independent_centroids:
        cent = make_centroids(wl)
    else:
        cent = np.ascontiguousarray(np.repeat(coarse.centroids, m, axis=0))
    return LayerInputs(wl, coarse.x, cent, None, w1, w3, w2)


def make_c2_dense(coarse: Optional[LayerInputs] = None) -> LayerInputs:
    """One shared expert of width 32768 made of all coarse intermediate units."""
    coarse = coarse if coarse is not None else make_c2_coarse()
    c = coarse.wl
    wl = Workload("c2dense", c.T, c.d, 1, 0, 0, c.n_routed * c.inter, c.dtype, 2, variant=2,
                  description="dense check: one FFN of width 32768 (all c2 units)")
    w1, w3, w2 = concat_experts(coarse.w1, coarse.w3, coarse.w2)
    return LayerInputs(wl, coarse.x, np.zeros((0, c.d), np.float32), None, w1, w3, w2)


def make_random_case(T: int, d: int, n_shared: int, n_routed: int, top_k: int, inter: int,
                     dtype: str = "f32", seed: int = 0, x_std: float = 1.0, w_std: float = 0.05,
                     zipf_s: Optional[float] = None, groups: int = 1) -> LayerInputs:
    """Small seeded case of arbitrary shape (tests: ragged tails, edge cases)."""
    wl = Workload(f"rand{seed}", T, d, n_shared, n_routed, top_k, inter, dtype, 90 + seed % 100,
                  variant=seed, x_std=x_std, w_std=w_std, zipf_s=zipf_s, groups=groups)
    w1, w3, w2 = make_weights(wl)
    return LayerInputs(wl, make_x(wl), make_centroids(wl), make_bias(wl), w1, w3, w2)


def ablated_inputs(inp: LayerInputs, drop_shared: bool = False, top_k: Optional[int] = None) -> LayerInputs:
    """The same layer (same tokens, router and expert weights) run with fewer experts:
    the shared experts removed and/or a different number K' of activated routed experts.
    These are the inference-time ablations of the paper's expert-specialization analysis
    (shared expert disabled; only 4 routed experts activated; Switch-style top-1)."""
    wl = inp.wl
    ks = wl.n_shared
    k = wl.top_k if top_k is None else top_k
    name = wl.name + ("-noshared" if drop_shared else "") + (f"-top{k}" if top_k is not None else "")
    nwl = wl.replace(name=name, n_shared=0 if drop_shared else ks, top_k=k,
                     description=f"{wl.description} [ablation: shared {'off' if drop_shared else 'on'}, top-{k}]")
    cut = ks if drop_shared else 0

    def keep(t: Tensor) -> Tensor:
        return Tensor(t.f32[cut:], None if t.bf16 is None else t.bf16[cut:])

    return LayerInputs(nwl, inp.x, inp.centroids, inp.bias, keep(inp.w1), keep(inp.w3), keep(inp.w2))


def balanced_routing(T: int, n_routed: int, top_k: int) -> np.ndarray:
    """idx[t, k] = (t*K' + k) mod N': every expert gets exactly K'T/N' tokens when N' | K'T."""
    t = np.arange(T, dtype=np.int64)[:, None]
    k = np.arange(top_k, dtype=np.int64)[None, :]
    return ((t * top_k + k) % n_routed).astype(np.int32)


def token_ids(T: int, vocab: int, seed: int = 0, zipf_s: float = 1.0) -> np.ndarray:
    """Seeded token ids in [0, vocab) with a Zipf(s) frequency law over a shuffled vocabulary
    (text-like repetition: frequent ids recur, so hash routing sees realistic collisions).
    The 2B validation model uses an 8K vocabulary, the 16B model a 100K one."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([515151, T, vocab, seed])))
    p = 1.0 / np.arange(1, vocab + 1, dtype=np.float64) ** zipf_s
    ranks = rng.choice(vocab, size=T, p=p / p.sum())
    return rng.permutation(vocab)[ranks].astype(np.int32)


def sample_tokens(T: int, n: int, seed: int = 7) -> np.ndarray:
    """Sorted seeded sample of token ids (always includes the first and last token)."""
    if n >= T:
        return np.arange(T, dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([424242, T, n, seed])))
    pick = rng.choice(T, size=n, replace=False)
    pick[0], pick[-1] = 0, T - 1
    return np.unique(pick).astype(np.int32)
