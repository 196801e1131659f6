"""Device buffers for one DeepSeekMoE layer pass and the five-call sequence.

torch is used only to allocate device memory, upload inputs and read results
back; every step of the layer runs in libmoe's HIP kernels through the C ABI
(moe_route -> moe_permute -> moe_expert_ffn -> moe_combine ->
moe_balance_stats).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import moe as M
from .workloads import LayerInputs


def _torch():
    import torch
    return torch


def to_device(a: np.ndarray, dtype: str, device):
    """Upload an fp32 array (dtype "f32") or bf16 bit patterns (dtype "bf16")."""
    torch = _torch()
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        assert a.dtype == np.uint16
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.int32:
        return torch.from_numpy(a).to(device)
    return torch.from_numpy(a.astype(np.float32, copy=False)).to(device)


def to_numpy_f32(t) -> np.ndarray:
    """Device tensor (bf16 or fp32) -> fp32 NumPy array (exact upcast for bf16)."""
    torch = _torch()
    return t.detach().to(torch.float32).cpu().numpy()


class DeviceLayer:
    """Inputs resident in HBM plus every output buffer of one layer pass."""

    def __init__(self, inp: LayerInputs, device="cuda", want_probs: bool = False, groups: Optional[int] = None,
                 top_k: Optional[int] = None, accumulate: bool = False):
        """accumulate: run moe_expert_ffn in its accumulating mode (no y_routed; the gate-weighted
        expert outputs are added into y_acc inside the down projection, not bitwise reproducible)."""
        torch = _torch()
        wl = inp.wl
        self.inp = inp
        self.device = torch.device(device)
        self.dtype = wl.dtype
        self.groups = groups if groups is not None else wl.groups
        T, d, Ks, Nr, w = wl.T, wl.d, wl.n_shared, wl.n_routed, wl.inter
        K = wl.top_k if top_k is None else top_k
        self.prob = M.moe_problem.make(T, d, Ks, Nr, K, w, wl.dtype)
        dev = self.device
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

        self.x = to_device(inp.x.device_bits(wl.dtype), wl.dtype, dev)
        self.centroids = to_device(inp.centroids, "f32", dev) if Nr else None
        self.bias = None if inp.bias is None else to_device(inp.bias, "f32", dev)
        sh, ro = inp.shared, inp.routed
        self.w1_s = to_device(sh(inp.w1).device_bits(wl.dtype), wl.dtype, dev) if Ks else None
        self.w3_s = to_device(sh(inp.w3).device_bits(wl.dtype), wl.dtype, dev) if Ks else None
        self.w2_s = to_device(sh(inp.w2).device_bits(wl.dtype), wl.dtype, dev) if Ks else None
        self.w1_r = to_device(ro(inp.w1).device_bits(wl.dtype), wl.dtype, dev) if Nr else None
        self.w3_r = to_device(ro(inp.w3).device_bits(wl.dtype), wl.dtype, dev) if Nr else None
        self.w2_r = to_device(ro(inp.w2).device_bits(wl.dtype), wl.dtype, dev) if Nr else None

        i32, f32 = torch.int32, torch.float32
        TK = T * K
        self.idx = torch.empty((T, K), dtype=i32, device=dev)
        self.gate = torch.empty((T, K), dtype=f32, device=dev)
        self.probs = torch.empty((T, Nr), dtype=f32, device=dev) if want_probs else None
        self.counts = torch.empty(max(Nr, 1), dtype=i32, device=dev)
        self.prob_sum = torch.empty(max(Nr, 1), dtype=f32, device=dev)
        self.offsets = torch.empty(Nr + 1, dtype=i32, device=dev)
        self.sorted_token = torch.empty(max(TK, 1), dtype=i32, device=dev)
        self.slot_of = torch.empty((T, K), dtype=i32, device=dev)
        self.accumulate = bool(accumulate) and TK > 0
        self.y_routed = None if self.accumulate else torch.empty((max(TK, 1), d), dtype=tdt, device=dev)
        # y_acc: the shared experts' sum (gather mode) or the whole expert sum (accumulating mode)
        self.y_acc = torch.empty((T, d), dtype=f32, device=dev) if (Ks or self.accumulate) else None
        self.h = torch.empty((T, d), dtype=tdt, device=dev)
        self.x_zero = None     # zero residual and output of expert_sum()
        self.y_sum = None
        D = max(self.groups, 1)
        self.f = torch.empty(max(Nr, 1), dtype=f32, device=dev)
        self.P = torch.empty(max(Nr, 1), dtype=f32, device=dev)
        self.f_dev = torch.empty(D, dtype=f32, device=dev)
        self.P_dev = torch.empty(D, dtype=f32, device=dev)
        self.exp_bal = torch.empty(1, dtype=f32, device=dev)
        self.dev_bal = torch.empty(1, dtype=f32, device=dev)
        self.ws_bytes = M.moe_workspace_size(self.prob)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.ffn_called = False   # the workspace's status word is defined only after moe_expert_ffn

    # -- the five calls ----------------------------------------------------
    def route(self, stream=None):
        M.moe_route(self.prob, self.x, self.centroids, self.bias, self.idx, self.gate, self.probs, self.counts,
                    self.prob_sum, self.ws, self.ws_bytes, stream)

    def route_ablate(self, disabled_top: int, stream=None):
        M.moe_route_ablate(self.prob, disabled_top, self.x, self.centroids, self.bias, self.idx, self.gate,
                           self.probs, self.counts, self.prob_sum, self.ws, self.ws_bytes, stream)

    def route_hash(self, token_ids, stream=None):
        M.moe_route_hash(self.prob, token_ids, self.idx, self.gate, self.counts, stream)

    def permute(self, stream=None):
        M.moe_permute(self.prob, self.idx, self.offsets, self.sorted_token, self.slot_of, self.ws, self.ws_bytes,
                      stream)

    def expert_ffn(self, stream=None):
        M.moe_expert_ffn(self.prob, self.x, self.offsets, self.sorted_token, self.w1_r, self.w3_r, self.w2_r,
                         self.w1_s, self.w3_s, self.w2_s, self.y_routed, self.y_acc, self.gate, self.slot_of,
                         self.ws, self.ws_bytes, stream)
        self.ffn_called = True

    def ffn_status(self, stream=None) -> int:
        """Status of the last moe_expert_ffn (synchronises the stream)."""
        return M.moe_expert_ffn_status(self.prob, self.ws, self.ws_bytes, stream)

    def expert_up(self, stream=None):
        M.moe_expert_up(self.prob, self.x, self.offsets, self.sorted_token, self.w1_r, self.w3_r, self.w1_s,
                        self.w3_s, self.ws, self.ws_bytes, stream)

    def expert_down(self, stream=None):
        M.moe_expert_down(self.prob, self.offsets, self.w2_r, self.w2_s, self.y_routed, self.y_acc, self.ws,
                          self.ws_bytes, stream)

    def combine(self, stream=None):
        M.moe_combine(self.prob, self.x, self.y_routed, self.y_acc, self.gate, self.slot_of, self.h, stream)

    def expert_sum(self, stream=None):
        """y = sum of the shared and gate-weighted routed expert outputs, as the GPU combine forms it:
        moe_combine with an all-zero residual, into a separate buffer (h stays as it is)."""
        torch = _torch()
        if self.x_zero is None:
            self.x_zero = torch.zeros_like(self.x)
            self.y_sum = torch.empty_like(self.h)
        M.moe_combine(self.prob, self.x_zero, self.y_routed, self.y_acc, self.gate, self.slot_of, self.y_sum,
                      stream)

    def balance_stats(self, stream=None):
        M.moe_balance_stats(self.prob, self.groups, self.counts, self.prob_sum, self.f, self.P, self.f_dev,
                            self.P_dev, self.exp_bal, self.dev_bal, stream)

    def forward(self, stream=None, stats: bool = True):
        """One whole layer pass on the stream."""
        if self.prob.n_routed:
            self.route(stream)
        self.permute(stream)
        self.expert_ffn(stream)
        self.combine(stream)
        if stats and self.prob.n_routed:
            self.balance_stats(stream)

    def layer_io(self) -> dict:
        """The buffers of this layer as the fields of moe_layer_io."""
        return dict(x=self.x, centroids=self.centroids, bias=self.bias, w1_routed=self.w1_r, w3_routed=self.w3_r,
                    w2_routed=self.w2_r, w1_shared=self.w1_s, w3_shared=self.w3_s, w2_shared=self.w2_s,
                    idx=self.idx, gate=self.gate, probs=self.probs, counts=self.counts, prob_sum=self.prob_sum,
                    offsets=self.offsets, sorted_token=self.sorted_token, slot_of=self.slot_of,
                    y_routed=self.y_routed, y_shared=self.y_acc, h=self.h, f=self.f, P=self.P, f_dev=self.f_dev,
                    P_dev=self.P_dev, exp_bal=self.exp_bal, dev_bal=self.dev_bal)

    def layer_forward(self, stream=None):
        """The whole layer pass as one moe_layer_forward call (gather mode; needs N' >= 1)."""
        assert not self.accumulate, "moe_layer_forward runs the gather form of the expert FFN"
        M.moe_layer_forward(self.prob, self.groups, self.layer_io(), self.ws, self.ws_bytes, stream)
        self.ffn_called = True

    def forward_with_routing(self, idx: np.ndarray, gate: np.ndarray, stream=None):
        """Layer pass with an externally supplied routing (e.g. every expert at gate 1)."""
        torch = _torch()
        self.idx.copy_(torch.from_numpy(np.ascontiguousarray(idx, np.int32)))
        self.gate.copy_(torch.from_numpy(np.ascontiguousarray(gate, np.float32)))
        self.permute(stream)
        self.expert_ffn(stream)
        self.combine(stream)

    def check_status(self) -> None:
        """Raise if the last moe_expert_ffn reported a stalled wait (its outputs hold NaN)."""
        if not self.ffn_called:
            return
        st = self.ffn_status()
        if st != M.MOE_OK:
            raise M.MoEError("moe_expert_ffn", st)

    # -- backward pass -----------------------------------------------------
    def backward(self, dh: np.ndarray, alpha1: float, alpha2: float, stream=None):
        """Backward pass through the three backward calls, for upstream gradient dh [T, d].

        dh is fp32 values (bf16 bits for a bf16 layer: pass the exact upcast of
        bf16 values).  Needs a forward with want_probs=True and the statistics.
        Leaves dx, dcentroids, dbias, dgate and the weight gradients (fp32) on
        the device.
        """
        torch = _torch()
        p = self.prob
        T, d, Ks, Nr, w = p.T, p.d, p.n_shared, p.n_routed, p.inter
        K = p.top_k
        dev = self.device
        f32 = torch.float32
        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        if not hasattr(self, "bws"):
            self.bws_bytes = M.moe_backward_workspace_size(p)
            self.bws = torch.empty(max(self.bws_bytes, 256), dtype=torch.uint8, device=dev)
            self.dy_routed = torch.empty((max(T * K, 1), d), dtype=tdt, device=dev)
            self.dgate = torch.empty((T, K), dtype=f32, device=dev)
            self.dx_ffn = torch.empty((T, d), dtype=f32, device=dev)
            self.dx = torch.empty((T, d), dtype=f32, device=dev)
            self.dw1_r = torch.empty((Nr, w, d), dtype=f32, device=dev) if Nr else None
            self.dw3_r = torch.empty((Nr, w, d), dtype=f32, device=dev) if Nr else None
            self.dw2_r = torch.empty((Nr, d, w), dtype=f32, device=dev) if Nr else None
            self.dw1_s = torch.empty((Ks, w, d), dtype=f32, device=dev) if Ks else None
            self.dw3_s = torch.empty((Ks, w, d), dtype=f32, device=dev) if Ks else None
            self.dw2_s = torch.empty((Ks, d, w), dtype=f32, device=dev) if Ks else None
            self.dcent = torch.empty((max(Nr, 1), d), dtype=f32, device=dev)
            self.dbias = torch.empty(max(Nr, 1), dtype=f32, device=dev)
        if self.dtype == "bf16":
            from .workloads import bf16_bits_from_f32
            self.dh = to_device(bf16_bits_from_f32(np.ascontiguousarray(dh, np.float32)), "bf16", dev)
        else:
            self.dh = to_device(np.ascontiguousarray(dh, np.float32), "f32", dev)
        if self.accumulate:
            raise ValueError("the backward pass needs y_routed: build the layer in gather mode")
        if Nr:
            M.moe_combine_backward(p, self.dh, self.y_routed, self.gate, self.slot_of, self.dy_routed, self.dgate,
                                   stream)
        M.moe_expert_ffn_backward(p, self.x, self.offsets, self.sorted_token, self.slot_of, self.w1_r, self.w3_r,
                                  self.w2_r, self.w1_s, self.w3_s, self.w2_s, self.dh, self.dy_routed, self.dx_ffn,
                                  self.dw1_r, self.dw3_r, self.dw2_r, self.dw1_s, self.dw3_s, self.dw2_s,
                                  self.bws, self.bws_bytes, stream)
        if Nr:
            M.moe_route_backward(p, max(self.groups, 1), alpha1, alpha2, self.x, self.centroids, self.probs,
                                 self.idx, self.dgate, self.f, self.f_dev, self.dh, self.dx_ffn, self.dx,
                                 self.dcent, self.dbias, self.bws, self.bws_bytes, stream)

    def backward_results(self) -> dict:
        torch = _torch()
        torch.cuda.synchronize(self.device)
        g = lambda t: None if t is None else t.cpu().numpy()
        Nr = self.prob.n_routed
        return dict(dgate=g(self.dgate), dx=g(self.dx), dx_ffn=g(self.dx_ffn), dw1_r=g(self.dw1_r),
                    dw3_r=g(self.dw3_r), dw2_r=g(self.dw2_r), dw1_s=g(self.dw1_s), dw3_s=g(self.dw3_s),
                    dw2_s=g(self.dw2_s), dcent=g(self.dcent)[:Nr], dbias=g(self.dbias)[:Nr])

    # -- readback ----------------------------------------------------------
    def results(self, check: bool = True) -> dict:
        """Read every output back (after checking the expert FFN's status word unless check=False)."""
        torch = _torch()
        torch.cuda.synchronize(self.device)
        if check:
            self.check_status()
        Nr = self.prob.n_routed
        TK = self.prob.T * self.prob.top_k
        y_acc = None if self.y_acc is None else self.y_acc.cpu().numpy()
        out = dict(
            idx=self.idx.cpu().numpy(), gate=self.gate.cpu().numpy(),
            counts=self.counts.cpu().numpy()[:Nr], prob_sum=self.prob_sum.cpu().numpy()[:Nr],
            offsets=self.offsets.cpu().numpy(), sorted_token=self.sorted_token.cpu().numpy()[:TK],
            slot_of=self.slot_of.cpu().numpy(),
            y_routed=None if self.y_routed is None else to_numpy_f32(self.y_routed)[:TK],
            y_shared=None if self.accumulate else y_acc,
            y_acc=y_acc,
            h=to_numpy_f32(self.h),
            f=self.f.cpu().numpy()[:Nr], P=self.P.cpu().numpy()[:Nr],
            f_dev=self.f_dev.cpu().numpy(), P_dev=self.P_dev.cpu().numpy(),
            exp_bal=float(self.exp_bal.cpu()[0]), dev_bal=float(self.dev_bal.cpu()[0]),
        )
        if self.probs is not None:
            out["probs"] = self.probs.cpu().numpy()
        if self.y_sum is not None:
            out["y"] = to_numpy_f32(self.y_sum)
        return out
