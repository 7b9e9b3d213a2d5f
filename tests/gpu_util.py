"""Helpers for the GPU parity tests: move synth layers to the device and run
the HIP path through the C ABI; nothing here computes any part of the layer."""
from __future__ import annotations

import numpy as np
import torch

import synth
from sparse_moe_expert_gemv_amd import binding as B
from sparse_moe_expert_gemv_amd.layer import MoELayer

DEV = "cuda"


def x_tensor(L: synth.Layer, x=None) -> torch.Tensor:
    x = L.x if x is None else x
    if L.cfg.x_dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def act_mode(L: synth.Layer) -> int:
    return B.MOE_ACT_Q8 if L.cfg.act_mode == "q8" else B.MOE_ACT_FLOAT


def gpu_layer(L: synth.Layer, mode=None, max_T=None, y_dtype=None) -> MoELayer:
    c = L.cfg
    return MoELayer(L.Wr, L.bias, L.experts, L.shared, d=c.d, f=c.f, k=c.k, wfmt=c.wfmt,
                    act_mode=act_mode(L) if mode is None else mode, max_T=max_T or c.T, y_dtype=y_dtype)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def routing_state(G: MoELayer, T: int):
    n = T * G.k
    return dict(ids=host(G.ids[:T]), gates=host(G.gates[:T]), counts=host(G.counts), offsets=host(G.offsets),
                sorted_idx=host(G.sorted_idx[:n]), dest=host(G.dest[:n]), active=host(G.active))
