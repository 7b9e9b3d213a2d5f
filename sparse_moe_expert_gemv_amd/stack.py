"""Multi-layer MoE stack with an HBM expert slot pool and per-layer miss staging.

The Strata pages keep the most-used ~4,500 experts resident in GPU memory,
chosen by a prebuilt usage ranking ("How Strata works", adaptive expert cache
section), and stream the next layer's experts over PCIe while the current
layer computes ("Strata benchmarks", prefill optimisation table).  Here:

* a caller-chosen set of global expert ids (layer * E + e) occupies the slots
  of a device pool (``moe_cache_set_resident``);
* every other expert of a layer is copied from pinned host memory into one of
  two device staging buffers on a side stream (``moe_cache_stage``), which also
  rewrites that layer's device pointer table; layer l + 2 is staged into the
  buffer of layer l as soon as layer l has finished;
* or (decode, ``miss_mode="host"``) every layer's pointer table sends the
  misses to the pinned host blobs themselves (``moe_cache_map_host``): the
  FFN reads a missed expert over the host link only when the routing selects
  it, so a decode pass needs no staging, no side stream and no host round trip
  (the pages' "single RTX 5090 runs a 125B model" report: only the experts the
  gating network picks are computed);
* or (decode, ``pcie_frac < 1``) the misses of each layer are split: a share
  ``pcie_frac`` of the missed experts is read over the host link by the GPU
  as above, the rest is computed by host cores from the canonical blobs in
  system memory (``moe_host_expert_ffn``) while the GPU computes the rest of
  the layer, and the host results are added to the layer output on the GPU
  (``moe_combine``).  This is the pages' split of cached experts on the GPU
  and missed ones on the CPU ("How Strata works", three-tier division;
  "Strata benchmarks", calibration: the share of misses copied to the GPU
  and the number of CPU expert threads);
* the residency can adapt (``AdaptiveResidency``): per-layer selection
  counters on the device, aged into scores on the host, and swaps of the
  weakest resident experts for the strongest missing ones;
* the compute stream waits for layer l's staging event, then runs
  rmsnorm -> route -> permute -> quantise -> expert FFN (through the pointer
  table) -> combine with the residual: h_{l+1} = h_l + MoE_l(norm(h_l)).  The
  pages leave the block around the MoE layer open; without the pre-norm a
  stack of random-weight layers joined by a residual add diverges within a
  few layers.

All device memory comes from PyTorch; all computation is in libmoe.so.
"""
from __future__ import annotations

import os
import time

import numpy as np
import torch

from . import binding as B
from .layer import pack_blobs


class ExpertStack:
    def __init__(self, routers, shared_blobs, host_store: torch.Tensor, host_index: np.ndarray, resident_ids,
                 *, d, f, k, wfmt, act_mode, max_T, staging_slots=None, device="cuda", eps=1e-6,
                 biases=None, miss_mode="stage", by_slot=False, cpu_blobs=None, pcie_frac=1.0, cpu_threads=None,
                 stage_mode="kernel", stage_workgroups=32):
        """
        routers      list of L fp32 arrays [E, d]
        shared_blobs [L, bytes] canonical uint8 (numpy) or None
        host_store   pinned host uint8 tensor [n_blobs, bytes] of PACKED expert blobs
        host_index   int array [L, E]: row of host_store holding expert (l, e)
        resident_ids global ids (l * E + e) kept in the slot pool
        biases       list of L fp32 arrays [E] (router biases) or None
        miss_mode    "stage": misses copied per layer into staging buffers;
                     "host": misses read in place from the pinned host store
        by_slot      decode batches (float mode, int4, T <= 8) without usage
                     counters: moe_route_ffn_combine_slots, no grouping of the
                     slots (same outputs, bit for bit)
        cpu_blobs    canonical host blobs [n_blobs, bytes] (numpy, rows as in
                     host_store) for the host-core share of the misses
        pcie_frac    decode with miss_mode "host" and by_slot: the share of a
                     layer's missed experts the GPU reads over the host link;
                     the others are computed on host cores (1.0: all on the GPU)
        cpu_threads  host threads for that share (default: up to 16)
        stage_mode   "kernel": one copy kernel per staged layer reading the
                     pinned host blobs (stage_workgroups workgroups);
                     "memcpy": one hipMemcpyAsync per missed expert
        """
        self.by_slot = by_slot
        assert miss_mode in ("stage", "host")
        self.miss_mode = miss_mode
        self.device = torch.device(device)
        self.d, self.f, self.k, self.wfmt, self.act_mode = d, f, k, wfmt, act_mode
        self.eps = eps
        self.L = len(routers)
        self.E = routers[0].shape[0]
        self.eb = B.moe_expert_bytes(wfmt, d, f)
        assert host_store.is_pinned() and host_store.shape[1] == self.eb
        self.host_store = host_store
        self.host_index = np.asarray(host_index, dtype=np.int64)
        base = host_store.data_ptr()
        self.host_ptrs = [[base + int(self.host_index[l, e]) * self.eb for e in range(self.E)] for l in range(self.L)]
        self.Wr = [torch.as_tensor(np.ascontiguousarray(w, np.float32)).to(self.device) for w in routers]
        self.bias = None if biases is None else \
            [torch.as_tensor(np.ascontiguousarray(b, np.float32)).to(self.device) for b in biases]
        self.shared = None
        if shared_blobs is not None:
            sh = torch.from_numpy(np.ascontiguousarray(shared_blobs, dtype=np.uint8)).to(self.device)
            self.shared = pack_blobs(sh, wfmt, d, f)
        resident_ids = [int(g) for g in resident_ids]
        self.n_slots = len(resident_ids)
        self.pool = torch.empty((max(self.n_slots, 1), self.eb), dtype=torch.uint8, device=self.device)
        res_per_layer = np.bincount(np.asarray(resident_ids, dtype=np.int64) // self.E, minlength=self.L)
        need = int(self.E - res_per_layer.min()) if self.n_slots else self.E
        if miss_mode == "host":
            need = 0
        self.staging_slots = need if staging_slots is None else staging_slots
        self.staging = torch.empty((2, max(self.staging_slots, 1), self.eb), dtype=torch.uint8, device=self.device)
        self.tables = torch.zeros((self.L, self.E), dtype=torch.int64, device=self.device)
        self.cache = B.SlotCache(self.L, self.E, self.n_slots, self.eb, self.pool, self.staging, 2,
                                 self.staging_slots)
        self.cache.set_resident(resident_ids, [self.host_ptrs[g // self.E][g % self.E] for g in resident_ids])
        assert stage_mode in ("kernel", "memcpy")
        self.stage_mode = stage_mode
        if stage_mode == "kernel":
            self.cache.set_stage_mode(B.MOE_STAGE_KERNEL, stage_workgroups)
        if miss_mode == "host":
            for l in range(self.L):
                self.cache.map_host(l, self.host_ptrs[l], self.tables[l])
        torch.cuda.synchronize()
        self.usage = None  # [L, E] int32 selection counters once enable_usage() is called
        self.resident_mask = np.zeros((self.L, self.E), dtype=bool)
        if resident_ids:
            g = np.asarray(resident_ids, dtype=np.int64)
            self.resident_mask[g // self.E, g % self.E] = True
        self.cpu_blobs = None if cpu_blobs is None else np.ascontiguousarray(cpu_blobs, dtype=np.uint8)
        self.cpu_pool = None
        self.pcie_frac = 1.0
        self.cpu_items = 0        # host-computed (token, slot) items since the last reset
        self.cpu_experts = 0      # host-computed distinct experts since the last reset
        self.set_pcie_frac(pcie_frac, cpu_threads)
        self.side = torch.cuda.Stream(device=self.device)
        self.staged = [torch.cuda.Event() for _ in range(self.L)]
        self.done = [torch.cuda.Event() for _ in range(self.L)]
        self._alloc(max_T)

    def set_pcie_frac(self, frac, cpu_threads=None):
        """Share of each decode layer's missed experts read by the GPU (the rest on host cores)."""
        frac = float(frac)
        assert 0.0 <= frac <= 1.0
        if frac < 1.0:
            assert self.miss_mode == "host" and self.by_slot and self.cpu_blobs is not None
            assert self.cpu_blobs.shape[1] == self.eb
            if self.cpu_pool is None:
                self.cpu_pool = B.HostPool(cpu_threads or max(1, min(16, os.cpu_count() or 1)))
        self.pcie_frac = frac

    def _alloc(self, T):
        dev, d, f, E, k = self.device, self.d, self.f, self.E, self.k
        self.max_T = T
        i32 = dict(dtype=torch.int32, device=dev)
        self.ids = torch.empty((T, k), **i32)
        self.gates = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.sorted_idx = torch.empty(T * k, **i32)
        self.dest = torch.empty(T * k, **i32)
        self.active = torch.empty(E + 1, **i32)
        self.xq = torch.empty((T, d), dtype=torch.int8, device=dev)
        self.sx = torch.empty((T, d // 32), dtype=torch.float32, device=dev)
        ydt = torch.float16 if self.act_mode == B.MOE_ACT_Q8 else torch.float32
        self.y_perm = torch.empty((T * k, d), dtype=ydt, device=dev)
        self.y_shared = torch.empty((T, d), dtype=torch.float32, device=dev)
        self.hbuf = [torch.empty((T, d), dtype=torch.float32, device=dev) for _ in range(2)]
        self.xn = torch.empty((T, d), dtype=torch.float32, device=dev)
        self.ws = torch.empty(B.moe_workspace_size(T, d, f, E, k, self.act_mode), dtype=torch.uint8, device=dev)
        # host share of the misses: pinned staging of ids, gates and inputs, the host
        # results, and the one-row combine that adds them
        self.h_ids = torch.empty((T, k), dtype=torch.int32, pin_memory=True)
        self.h_gates = torch.empty((T, k), dtype=torch.float32, pin_memory=True)
        self.h_x = torch.empty((T, d), dtype=torch.float32, pin_memory=True)
        self.h_gpu_ids = torch.empty((T, k), dtype=torch.int32, pin_memory=True)
        self.h_cpu_out = torch.empty((T, d), dtype=torch.float32, pin_memory=True)
        self.gpu_ids = torch.empty((T, k), **i32)
        self.cpu_out = torch.empty((T, d), dtype=torch.float32, device=dev)
        self.row_dest = torch.arange(T, dtype=torch.int32, device=dev)
        self.row_gate = torch.ones((T, 1), dtype=torch.float32, device=dev)
        self.routed_ev = torch.cuda.Event()

    def enable_usage(self):
        """Count, per layer and expert, how often the routing selects it (device int32)."""
        self.usage = torch.zeros((self.L, self.E), dtype=torch.int32, device=self.device)
        return self.usage

    def misses(self, layer):
        return self.cache.lookup(layer)[1]

    def stage(self, layer):
        """Enqueue the staging of one layer on the side stream (records staged[layer])."""
        self.cache.stage(layer, layer % 2, self.host_ptrs[layer], self.tables[layer], stream=self.side,
                         done_event=self.staged[layer])

    def layer(self, l, h, out, stream=None, table=None):
        """out = h + MoE_l(rmsnorm(h)); the normalised input stays in self.xn."""
        T = h.shape[0]
        k, E, n = self.k, self.E, h.shape[0] * self.k
        xn = self.xn[:T]
        B.moe_rmsnorm(h, xn, self.eps, stream)
        bias = None if self.bias is None else self.bias[l]
        decode = self.by_slot and self.usage is None and self.act_mode == B.MOE_ACT_FLOAT and self.wfmt == 4 and T <= 8
        if decode and self.pcie_frac < 1.0 and table is None:
            return self._layer_split(l, h, out, xn, bias, stream)
        if decode:
            B.moe_route_ffn_combine_slots(T=T, d=self.d, f=self.f, E=E, k=k, wfmt=self.wfmt, act_mode=self.act_mode,
                                          expert_ptrs=self.tables[l] if table is None else table, ws=self.ws,
                                          Wr=self.Wr[l], bias=bias, ids=self.ids[:T], gates=self.gates[:T], out=out,
                                          x=xn, residual=h,
                                          shared_blob=None if self.shared is None else self.shared[l], stream=stream)
            return
        B.moe_route_permute(xn, self.Wr[l], bias, k, self.ids[:T], self.gates[:T], self.counts, self.offsets,
                            self.sorted_idx[:n], self.dest[:n], self.active, self.ws, stream)
        if self.usage is not None:
            B.moe_usage_accumulate(self.usage[l], self.counts, stream)
        common = dict(T=T, d=self.d, f=self.f, E=E, k=k, wfmt=self.wfmt, act_mode=self.act_mode,
                      expert_ptrs=self.tables[l] if table is None else table, counts=self.counts,
                      offsets=self.offsets, sorted_idx=self.sorted_idx[:n], active=self.active,
                      y_perm=self.y_perm[:n], ws=self.ws,
                      shared_blob=None if self.shared is None else self.shared[l],
                      y_shared=None if self.shared is None else self.y_shared[:T], stream=stream)
        if self.act_mode == B.MOE_ACT_Q8:
            B.moe_quantize_act(xn, self.xq[:T], self.sx[:T], stream)
            common.update(xq=self.xq[:T], sx=self.sx[:T])
        else:
            common.update(x=xn)
        B.moe_expert_ffn_combine(ids=self.ids[:T], dest=self.dest[:n], gates=self.gates[:T], residual=h, out=out,
                                 **common)

    def _layer_split(self, l, h, out, xn, bias, stream):
        """Decode layer with the host-core share of the misses (see set_pcie_frac)."""
        T, k, E, d = h.shape[0], self.k, self.E, self.d
        B.moe_route(xn, self.Wr[l], bias, k, self.ids[:T], self.gates[:T], self.ws, stream)
        st = torch.cuda.current_stream(self.device) if stream is None else stream
        with torch.cuda.stream(st):
            self.h_ids[:T].copy_(self.ids[:T], non_blocking=True)
            self.h_gates[:T].copy_(self.gates[:T], non_blocking=True)
            self.h_x[:T].copy_(xn, non_blocking=True)
            self.routed_ev.record(st)
        self.routed_ev.synchronize()
        ids = self.h_ids[:T].numpy()
        miss = ~self.resident_mask[l][ids]
        if miss.any():
            me, cnt = np.unique(ids[miss], return_counts=True)
            order = np.lexsort((me, -cnt))  # GPU share: experts picked by most tokens first, then lower id
            n_gpu = int(round(self.pcie_frac * len(me)))
            cpu_set = np.zeros(E, dtype=bool)
            cpu_set[me[order[n_gpu:]]] = True
        else:
            cpu_set = np.zeros(E, dtype=bool)
        on_cpu = cpu_set[ids]
        gid = self.h_gpu_ids[:T].numpy()
        gid[...] = np.where(on_cpu, -1, ids)  # ids outside [0, E) are skipped by the FFN
        common = dict(T=T, d=d, f=self.f, E=E, k=k, wfmt=self.wfmt, act_mode=self.act_mode,
                      expert_ptrs=self.tables[l], ws=self.ws,
                      shared_blob=None if self.shared is None else self.shared[l], x=xn, stream=stream)
        with torch.cuda.stream(st):
            self.gpu_ids[:T].copy_(self.h_gpu_ids[:T], non_blocking=True)
        B.moe_expert_ffn_combine_slots(ids=self.gpu_ids[:T], gates=self.gates[:T], residual=h, out=out, **common)
        if not on_cpu.any():
            return
        tt, jj = np.nonzero(on_cpu)
        ptrs = self.cpu_blobs.ctypes.data + self.eb * self.host_index[l, ids[tt, jj]]
        hout = self.h_cpu_out[:T].numpy()
        hout[...] = 0.0
        self.cpu_pool.expert_ffn(tt, self.h_gates[:T].numpy()[tt, jj], ptrs, self.wfmt, self.h_x[:T].numpy(), hout,
                                 d, self.f)
        self.cpu_items += len(tt)
        self.cpu_experts += int(cpu_set.sum())
        with torch.cuda.stream(st):
            self.cpu_out[:T].copy_(self.h_cpu_out[:T], non_blocking=True)
        B.moe_combine(self.cpu_out[:T], self.row_dest[:T], self.row_gate[:T], None, out, out, stream)

    def forward(self, x: torch.Tensor, keep=(), copy_only=False, compute_only_tables=None, ids_out=None):
        """Run all layers on x ([T, d] fp32).  Returns (h_L, {l: (h_l, norm(h_l)) for l in keep}).

        copy_only: only the staging (timing aid); compute_only_tables: run the
        compute with these pointer tables [L, E] instead of staging (timing aid);
        ids_out: a list that receives a copy of every layer's routed ids [T, k].
        In "host" miss mode nothing is staged: the tables already point at the
        pool and at the host blobs.
        """
        T = x.shape[0]
        if T > self.max_T:
            self._alloc(T)
        comp = torch.cuda.current_stream(self.device)
        kept = {}
        h = x
        outs = self.hbuf
        if self.miss_mode == "host" and compute_only_tables is None:
            for l in range(self.L):
                out = outs[l % 2]
                self.layer(l, h, out)
                if l in keep:
                    kept[l] = (h.clone(), self.xn[:T].clone())
                if ids_out is not None:
                    ids_out.append(self.ids[:T].clone())
                h = out
            return h, kept
        if compute_only_tables is None:
            self.side.wait_stream(comp)
            for l in range(min(2, self.L)):
                self.stage(l)
        for l in range(self.L):
            if compute_only_tables is None:
                comp.wait_event(self.staged[l])
            out = outs[l % 2]
            if not copy_only:
                self.layer(l, h, out, table=None if compute_only_tables is None else compute_only_tables[l])
                if l in keep:
                    kept[l] = (h.clone(), self.xn[:T].clone())
                if ids_out is not None:
                    ids_out.append(self.ids[:T].clone())
                h = out
            self.done[l].record(comp)
            if compute_only_tables is None and l + 2 < self.L:
                self.side.wait_event(self.done[l])
                self.stage(l + 2)
        return h, kept

    def close(self):
        self.cache.close()
        if self.cpu_pool is not None:
            self.cpu_pool.close()
            self.cpu_pool = None


class AdaptiveResidency:
    """Host side of the adaptive expert cache ("How Strata works", adaptive
    expert cache section: the cache keeps learning the session's hot experts).

    Every update reads the device selection counters, ages them into scores
    (score = decay * score + selections since the last update, in fp32), asks
    moe_cache_plan for up to max_swaps (evict, admit) pairs and carries them
    out with moe_cache_replace on the compute stream.  Work enqueued before an
    update reads the old pool contents, work enqueued after it the new ones.
    """

    def __init__(self, stack: ExpertStack, decay=0.5, max_swaps=128, margin=0.0):
        self.S = stack
        self.decay, self.max_swaps, self.margin = np.float32(decay), int(max_swaps), float(margin)
        n = stack.L * stack.E
        self.usage = stack.usage if stack.usage is not None else stack.enable_usage()
        self.prev = np.zeros(n, dtype=np.int64)
        self.score = np.zeros(n, dtype=np.float32)
        self.resident = np.zeros(n, dtype=np.uint8)
        for l in range(stack.L):
            for e in stack.cache.lookup(l)[0]:
                self.resident[l * stack.E + e] = 1
        self.host_all = [p for row in stack.host_ptrs for p in row]
        self.swaps = 0
        self.policy_s = 0.0  # host time in scoring, planning and enqueueing (after the counters arrive)

    def update(self, stream=None):
        """One policy step; returns the number of swaps enqueued."""
        now = self.usage.reshape(-1).cpu().numpy().astype(np.int64)
        t0 = time.perf_counter()
        delta = (now - self.prev) & 0xFFFFFFFF  # counters wrap modulo 2^32
        self.prev = now
        self.score = self.score * self.decay + delta.astype(np.float32)
        ev, ad = B.moe_cache_plan(self.resident, self.score, self.max_swaps, self.margin)
        if len(ev):
            self.S.cache.replace(ev, ad, self.host_all, self.S.tables, stream)
            self.resident[ev] = 0
            self.resident[ad] = 1
            self.swaps += len(ev)
        self.policy_s += time.perf_counter() - t0
        return len(ev)


def build_host_store(pool_canonical: np.ndarray, wfmt: int, d: int, f: int, device="cuda") -> torch.Tensor:
    """Pack canonical blobs on the device and return them in pinned host memory."""
    n, nb = pool_canonical.shape
    store = torch.empty((n, nb), dtype=torch.uint8, pin_memory=True)
    step = 256
    for i in range(0, n, step):
        j = min(n, i + step)
        dev = torch.from_numpy(np.ascontiguousarray(pool_canonical[i:j])).to(device)
        store[i:j].copy_(pack_blobs(dev, wfmt, d, f).cpu())
    torch.cuda.synchronize()
    return store


def time_pass(fn, reps=1):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / reps
