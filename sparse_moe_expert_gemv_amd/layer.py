"""One sparse-MoE FFN layer on the GPU, driven through the C ABI.

``MoELayer`` holds a layer's device-resident weights (router, packed expert
blobs, device pointer table, shared expert) plus reusable buffers, and runs

    moe_route_permute -> [moe_quantize_act] -> moe_expert_ffn_combine

(or, with ``fuse_combine=False``, moe_expert_ffn then moe_combine; with
``by_slot=True`` and a decode batch, moe_route_ffn_combine_slots, or with
``select_in_ffn=False`` moe_route -> moe_expert_ffn_combine_slots) on the
current stream.  Device memory comes from PyTorch; all computation is in
libmoe.so.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


def _dev_u8(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


def pack_blobs(canonical: torch.Tensor, wfmt: int, d: int, f: int) -> torch.Tensor:
    """[n, expert_bytes] canonical uint8 device tensor -> packed copy."""
    packed = torch.empty_like(canonical)
    n = canonical.shape[0]
    for i in range(0, n, 65535):
        j = min(n, i + 65535)
        B.moe_pack_experts(canonical[i:j], packed[i:j], j - i, wfmt, d, f)
    return packed


def pointer_table(packed: torch.Tensor) -> torch.Tensor:
    """Device int64 tensor [n] of the addresses of the rows of a packed [n, bytes] tensor."""
    base = packed.data_ptr()
    stride = packed.stride(0) * packed.element_size()
    addrs = base + stride * torch.arange(packed.shape[0], dtype=torch.int64)
    return addrs.to(packed.device)


class MoELayer:
    def __init__(self, Wr, bias, experts, shared, *, d, f, k, wfmt, act_mode, max_T, device="cuda",
                 y_dtype=None, experts_are_packed=False, expert_ptrs=None, fuse_combine=True, by_slot=False,
                 select_in_ffn=True):
        self.device = torch.device(device)
        # forward through moe_expert_ffn_combine (down projection and weighted
        # sum in one kernel where one exists); False: moe_expert_ffn then
        # moe_combine, which leave y_perm / y_shared filled
        self.fuse_combine = fuse_combine
        # decode batches (float mode, int4, T <= 8): no grouping of the slots
        # (counts, offsets, sorted_idx, dest and active are then not written);
        # the gate/up launch selects the experts itself (moe_route_ffn_combine_slots),
        # or with select_in_ffn=False moe_route then moe_expert_ffn_combine_slots
        self.by_slot = by_slot
        self.select_in_ffn = select_in_ffn
        self.d, self.f, self.k, self.wfmt, self.act_mode = d, f, k, wfmt, act_mode
        self.Wr = torch.as_tensor(np.ascontiguousarray(Wr, dtype=np.float32)).to(self.device)
        self.E = self.Wr.shape[0]
        self.bias = None if bias is None else torch.as_tensor(np.ascontiguousarray(bias, np.float32)).to(self.device)
        if expert_ptrs is not None:
            self.experts = experts  # caller-owned packed storage
            self.expert_ptrs = expert_ptrs
        else:
            ex = experts if isinstance(experts, torch.Tensor) else _dev_u8(experts, self.device)
            self.experts = ex if experts_are_packed else pack_blobs(ex, wfmt, d, f)
            self.expert_ptrs = pointer_table(self.experts)
        self.shared = None
        if shared is not None:
            sh = shared if isinstance(shared, torch.Tensor) else _dev_u8(shared, self.device)
            sh = sh.reshape(1, -1)
            self.shared = (sh if experts_are_packed else pack_blobs(sh, wfmt, d, f))[0]
        if y_dtype is None:
            y_dtype = torch.float16 if act_mode == B.MOE_ACT_Q8 else torch.float32
        self.y_dtype = y_dtype
        self._alloc(max_T)

    def _alloc(self, T):
        dev, d, f, E, k = self.device, self.d, self.f, self.E, self.k
        self.max_T = T
        i32 = dict(dtype=torch.int32, device=dev)
        self.ids = torch.empty((T, k), **i32)
        self.gates = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.sorted_idx = torch.empty(max(T * k, 1), **i32)
        self.dest = torch.empty(max(T * k, 1), **i32)
        self.active = torch.empty(E + 1, **i32)
        self.xq = torch.empty((T, d), dtype=torch.int8, device=dev)
        self.sx = torch.empty((T, d // 32), dtype=torch.float32, device=dev)
        self.y_perm = torch.empty((max(T * k, 1), d), dtype=self.y_dtype, device=dev)
        self.y_shared = torch.empty((T, d), dtype=torch.float32, device=dev)
        self.out = torch.empty((T, d), dtype=torch.float32, device=dev)
        ws = B.moe_workspace_size(T, d, f, E, k, self.act_mode)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)

    def _ws_for(self, T):
        need = B.moe_workspace_size(T, self.d, self.f, self.E, self.k, self.act_mode)
        return self.ws[:max(need, 256)]

    def forward(self, x: torch.Tensor, residual: torch.Tensor | None = None, out: torch.Tensor | None = None,
                stream=None, expert_ptrs: torch.Tensor | None = None) -> torch.Tensor:
        T = x.shape[0]
        if T > self.max_T:
            self._alloc(T)
        k, E = self.k, self.E
        ws = self._ws_for(T)
        ids, gates = self.ids[:T], self.gates[:T]
        n = T * k
        if self.by_slot and self.act_mode == B.MOE_ACT_FLOAT and self.wfmt == 4 and T <= 8:
            o = self.out[:T] if out is None else out
            common = dict(T=T, d=self.d, f=self.f, E=E, k=k, wfmt=self.wfmt, act_mode=self.act_mode,
                          expert_ptrs=self.expert_ptrs if expert_ptrs is None else expert_ptrs, ws=ws, ids=ids,
                          gates=gates, out=o, x=x, residual=residual, shared_blob=self.shared, stream=stream)
            if self.select_in_ffn:
                B.moe_route_ffn_combine_slots(Wr=self.Wr, bias=self.bias, **common)
            else:
                B.moe_route(x, self.Wr, self.bias, k, ids, gates, ws, stream)
                B.moe_expert_ffn_combine_slots(**common)
            return o
        B.moe_route_permute(x, self.Wr, self.bias, k, ids, gates, self.counts, self.offsets, self.sorted_idx[:n],
                            self.dest[:n], self.active, ws, stream)
        common = dict(T=T, d=self.d, f=self.f, E=E, k=k, wfmt=self.wfmt, act_mode=self.act_mode,
                      expert_ptrs=self.expert_ptrs if expert_ptrs is None else expert_ptrs,
                      counts=self.counts, offsets=self.offsets, sorted_idx=self.sorted_idx[:n],
                      active=self.active, y_perm=self.y_perm[:n], ws=ws, shared_blob=self.shared,
                      y_shared=self.y_shared[:T] if self.shared is not None else None, stream=stream)
        o = self.out[:T] if out is None else out
        if self.act_mode == B.MOE_ACT_Q8:
            B.moe_quantize_act(x, self.xq[:T], self.sx[:T], stream)
            common.update(xq=self.xq[:T], sx=self.sx[:T])
        else:
            common.update(x=x)
        if self.fuse_combine:
            B.moe_expert_ffn_combine(ids=ids, dest=self.dest[:n], gates=gates, residual=residual, out=o, **common)
        else:
            B.moe_expert_ffn(**common)
            B.moe_combine(self.y_perm[:n], self.dest[:n], gates,
                          self.y_shared[:T] if self.shared is not None else None, residual, o, stream)
        return o
