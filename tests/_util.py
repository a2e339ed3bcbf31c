"""Helpers shared by the GPU parity tests: move seeded inputs to the device, run
the C ABI through the binding, compare with the oracle at the stated tolerance.

Tolerance (per tensor, max abs error against the unrounded fp64 oracle):
  bf16 path: <= 2e-2 * max |ref|;  fp32 checking mode: <= 1e-4 * max |ref|;
  a reference that is exactly zero must be matched exactly.
"""
from __future__ import annotations

import numpy as np

import synth

TOL = {"bf16": 2e-2, "fp32": 1e-4}


def gateup_to_concat(w: np.ndarray) -> np.ndarray:
    """W_up columns (last axis) from interleaved (gate_j, up_j at 2j, 2j+1) to
    concatenated [gates | ups] order."""
    return np.concatenate([w[..., 0::2], w[..., 1::2]], axis=-1)


def gateup_to_interleaved(w: np.ndarray) -> np.ndarray:
    """Inverse of gateup_to_concat."""
    I = w.shape[-1] // 2
    out = np.empty_like(w)
    out[..., 0::2] = w[..., :I]
    out[..., 1::2] = w[..., I:]
    return out


def f64(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def assert_close(got, ref, tol, name=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if scale == 0.0:
        assert err == 0.0, f"{name}: reference is exactly 0, max |got| = {err}"
    else:
        assert err <= tol * scale, f"{name}: max err {err:.3e} > {tol} * {scale:.3e}"
    return err / scale if scale else 0.0


class Gpu:
    """One case's inputs on the device, in bf16 or fp32 storage."""

    def __init__(self, d: dict, dtype: str = "bf16", capacity=None, device="cuda", layout=0):
        import torch
        from token_routing_grouped_amd import Metadata

        self.torch = torch
        self.d = d
        self.dtype = dtype
        N, H, I, E, K = d["N"], d["H"], d["I"], d["E"], d["K"]
        self.N, self.H, self.I, self.E, self.K = N, H, I, E, K
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

        def dev(bits):
            t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
            return t.to(device).to(tdt).contiguous()

        self.layout = layout  # 1: W_up (and dW_up) in concatenated [gates | ups] order
        self.x = dev(d["x"])
        self.w_up = dev(gateup_to_concat(d["w_up"]) if layout == 1 else d["w_up"])
        self.w_down = dev(d["w_down"])
        self.dout = dev(d["dout"]) if "dout" in d else None
        self.topk_idx = torch.from_numpy(d["topk_idx"]).to(device)
        self.topk_weights = torch.from_numpy(d["topk_weights"]).to(device)
        P = int(((d["topk_idx"] >= 0) & (d["topk_idx"] < E)).sum())
        self.P = P
        cap = P if capacity is None else capacity
        self.meta = Metadata(N, K, E, cap, device=device)
        self.tdt = tdt

    def build(self):
        from token_routing_grouped_amd import moe_build_metadata
        moe_build_metadata(self.topk_idx, self.topk_weights, self.meta)

    def forward(self, save_h=True):
        from token_routing_grouped_amd import moe_expert_forward
        torch = self.torch
        self.out = torch.empty(self.N, self.H, dtype=self.tdt, device=self.x.device)
        self.h = (torch.empty(max(self.meta.capacity, 0), 2 * self.I, dtype=self.tdt,
                              device=self.x.device) if save_h else None)
        moe_expert_forward(self.meta, self.x, self.w_up, self.w_down, self.out, h_save=self.h,
                           layout=self.layout)
        return self.out

    def backward(self):
        from token_routing_grouped_amd import moe_expert_backward
        torch = self.torch
        dev = self.x.device
        self.dx = torch.empty(self.N, self.H, dtype=self.tdt, device=dev)
        self.dw_up = torch.empty(self.E, self.H, 2 * self.I, dtype=self.tdt, device=dev)
        self.dw_down = torch.empty(self.E, self.I, self.H, dtype=self.tdt, device=dev)
        self.dtw = torch.empty(self.N, self.K, dtype=torch.float32, device=dev)
        moe_expert_backward(self.meta, self.topk_idx, self.x, self.w_up, self.w_down, self.h,
                            self.dout, self.dx, self.dw_up, self.dw_down, self.dtw,
                            layout=self.layout)

    def meta_numpy(self) -> dict:
        m = self.meta
        P = int(m.expert_frequency_offset[-1].item())
        cap = m.capacity
        n = min(P, cap)
        c = lambda t: t.cpu().numpy()
        return dict(
            P=P,
            expert_frequency=c(m.expert_frequency),
            expert_frequency_offset=c(m.expert_frequency_offset),
            x_gather_idx=c(m.x_gather_idx)[:n],
            s_scatter_idx=c(m.s_scatter_idx)[:n],
            s_reverse_scatter_idx=c(m.s_reverse_scatter_idx)[:n],
            num_activated_expert_per_token_offset=c(m.num_activated_expert_per_token_offset),
            router_scores=c(m.router_scores)[:n],
            status=int(c(m.status)[0]) & 0xffffffff,
        )


def np64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)
