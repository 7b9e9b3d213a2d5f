"""Benchmark of the sparse-MoE FFN layer hot path on one MI355X.

One step = one pass of the whole layer over one batch of seeded synthetic
input already resident in HBM.  The default run measures both halves of the
metric: the decode layer at T=4 (the line's value) and, nested under
"prefill", the 8,192-token prefill chunk (its own seeded layer).  Steps: moe_route_permute (routing and grouping) ->
[moe_quantize_act] -> moe_expert_ffn_combine (expert FFN and the gate-weighted
combine); for decode batches (T <= 8, int4 weights) moe_route ->
moe_expert_ffn_combine_slots, where every routed slot is its own work item and
the down projection and the combine are one kernel.  Default workload: the decode layer
(d=2048, 512 int4 experts + shared, top-10, f=768) at T=4 tokens, the MTP
verify batch; ``--workload`` selects another layer (decode_t1, prefill, skew,
tiny) or a 48-layer stack over the 4,500-slot expert pool (``stack``: the
8,192-token prefill chunk with per-layer staging; ``decode_stack`` and
``decode_stack_t1``: decode passes with profile-biased routing, misses read in
place from pinned host memory).

Layer weights are replicated into ``--rotate`` device copies and consecutive
steps use consecutive copies with their own inputs, so each step streams its
expert weights from HBM rather than from the 256 MB Infinity Cache.  Each
copy's step is captured in a HIP graph; one graph holds one step on every copy
in turn, so that host launch overhead is paid once per ``--rotate`` steps.
Two timed regions, both bracketed by a device synchronisation: (A) ``--steps``
whole-layer steps, which give ``value`` and ``ms_per_step``; (B) at least 25
whole rotations of back-to-back launches of the dominant kernel alone (the
expert gate/up projection, rotating over the weight copies, also replayed from
graphs) between two HIP events on its launch stream, whose mean launch time
gives the roofline figure.

Prints one JSON line (rank 0).  ``--gpus`` above 1 is not supported: the
benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0          # dense int8 MFMA, TOPS
WORKLOADS = ("decode_t4", "decode_t1", "prefill", "skew", "tiny", "stack", "decode_stack", "decode_stack_t1",
             "decode_stack_drift", "copy", "peak")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="decode_t4", choices=WORKLOADS)
    p.add_argument("--rotate", type=int, default=None, help="device copies of the layer weights")
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU-baseline leg")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true", help="decode_t4 only: skip the nested prefill measurement")
    p.add_argument("--no-split", action="store_true", help="decode stacks: skip the host-core miss split sweep")
    p.add_argument("--seed", type=int, default=0)
    return p.parse_args()


def kernel_source_sha256(workload: str) -> str:
    """SHA-256 over the source of a workload's dominant kernel and the shared
    device headers it includes (common.hpp, topk.hpp, wave.hpp), in that order."""
    import hashlib
    csrc = os.path.join(ROOT, "sparse_moe_expert_gemv_amd", "csrc")
    h = hashlib.sha256()
    for f in ("ffn_q8.hip" if workload == "prefill" else "ffn_float.hip", "common.hpp", "topk.hpp", "wave.hpp"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary, if one exists for this workload and the
    kernel source has not changed since the counters were taken; else None."""
    path = os.path.join(ROOT, "profiles", "gateup_%s_hbm_counters.md" % workload)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "kernel_source_sha256"):
            key, val = line.split(":", 1)
            fields[key] = val.strip()
    if fields.get("kernel_source_sha256") != kernel_source_sha256(workload):
        return None
    return int(fields["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in fields else None


def gateup_algorithmic(cfg, n_active: int, T: int):
    """Algorithmic bytes and ops of one gate/up launch (the dominant kernel).

    Bytes: the gate and up matrices (quants + fp16 block scales) of every
    expert that has tokens, plus the shared expert, plus the activations read
    and the SwiGLU intermediate written.  Ops: 2 per multiply-add over the
    gate and up projections of every routed and shared row.
    """
    import synth
    eb = synth.expert_bytes(cfg.wfmt, cfg.d, cfg.f)
    n_exp = n_active + (1 if cfg.has_shared else 0)
    weight_bytes = n_exp * eb * 2 // 3
    rows = T * cfg.k + (T if cfg.has_shared else 0)
    if cfg.act_mode == "q8":
        xbytes = T * cfg.d + T * (cfg.d // 32) * 4
        hbytes = rows * cfg.f + rows * (cfg.f // 32) * 4
    else:
        xbytes = T * cfg.d * (2 if cfg.x_dtype == "bf16" else 4)
        hbytes = rows * cfg.f * 2
    ops = 2.0 * 2 * cfg.d * cfg.f * rows
    return weight_bytes + xbytes + hbytes, ops


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py runs on one GPU only (the library has no multi-GPU path); got --gpus %d" % a.gpus)
        sys.exit(2)
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    name = a.workload
    if name == "stack":
        return bench_stack(a)
    if name == "decode_stack_drift":
        return bench_decode_stack_drift(a)
    if name.startswith("decode_stack"):
        return bench_decode_stack(a)
    if name == "copy":
        return bench_copy(a)
    if name == "peak":
        return bench_peak(a)
    line = bench_layer(a, name, a.steps, a.warmup, a.rotate, with_cpu=not a.no_cpu_baseline)
    if name == "decode_t4" and not a.no_prefill:
        # the metric's other half: the 8,192-token prefill chunk of the same
        # model, timed in the same run (its own seeded layer)
        torch.cuda.empty_cache()
        pf = bench_layer(a, "prefill", None, None, None, with_cpu=False)
        line["prefill"] = {k: pf[k] for k in ("value", "unit", "ms_per_step", "steps", "warmup", "dtype", "config",
                                              "roofline")}
    print(json.dumps(line), flush=True)


def bench_layer(a, name, steps, warmup, rotate, with_cpu):
    """One layer workload (decode_t4, decode_t1, prefill, skew, tiny): the
    bench line's fields as a dict."""
    import torch

    import synth
    from sparse_moe_expert_gemv_amd import binding as B
    from sparse_moe_expert_gemv_amd.layer import MoELayer, pack_blobs, pointer_table

    dev = torch.device("cuda:0")
    big = name == "prefill"
    steps = steps if steps is not None else (20 if big else 200)
    warmup = warmup if warmup is not None else (3 if big else 20)
    rotate = rotate if rotate is not None else (2 if big else 8)
    t_gen = time.time()
    L = synth.make_layer(name, seed=a.seed)
    cfg = L.cfg
    T = cfg.T
    mode = B.MOE_ACT_Q8 if cfg.act_mode == "q8" else B.MOE_ACT_FLOAT
    print("[bench] workload %s T=%d d=%d E=%d k=%d f=%d wfmt=%d mode=%s rotate=%d (generated in %.1fs)"
          % (name, T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.wfmt, cfg.act_mode, rotate, time.time() - t_gen),
          file=sys.stderr, flush=True)

    # one packed copy, replicated
    canon = torch.from_numpy(L.experts).to(dev)
    packed0 = pack_blobs(canon, cfg.wfmt, cfg.d, cfg.f)
    del canon
    layers, xs = [], []
    for r in range(rotate):
        packed = packed0 if r == 0 else packed0.clone()
        G = MoELayer(L.Wr, L.bias, packed, None, d=cfg.d, f=cfg.f, k=cfg.k, wfmt=cfg.wfmt, act_mode=mode,
                     max_T=T, device=dev, expert_ptrs=pointer_table(packed))
        if L.shared is not None:
            sh = torch.from_numpy(L.shared).to(dev).reshape(1, -1)
            G.shared = pack_blobs(sh, cfg.wfmt, cfg.d, cfg.f)[0]
        layers.append(G)
        xb = synth.gen_x(a.seed, cfg, layer=0, draw=r)
        if cfg.x_dtype == "bf16":
            xs.append(torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16))
        else:
            xs.append(torch.from_numpy(xb).to(dev))
    torch.cuda.synchronize()

    # decode batches with int4 weights need no grouping of the slots: routing
    # gives ids and gates, and every routed slot is its own FFN work item
    by_slot = mode == B.MOE_ACT_FLOAT and cfg.wfmt == 4 and T <= 8

    def run_route(G, x):
        ws = G._ws_for(T)
        n = T * cfg.k
        if by_slot:
            B.moe_route(x, G.Wr, G.bias, cfg.k, G.ids[:T], G.gates[:T], ws)
            return
        B.moe_route_permute(x, G.Wr, G.bias, cfg.k, G.ids[:T], G.gates[:T], G.counts, G.offsets,
                            G.sorted_idx[:n], G.dest[:n], G.active, ws)
        if mode == B.MOE_ACT_Q8:
            B.moe_quantize_act(x, G.xq[:T], G.sx[:T])

    def run_slots(G, x, phase=0):
        B.moe_expert_ffn_combine_slots(T=T, d=cfg.d, f=cfg.f, E=cfg.E, k=cfg.k, wfmt=cfg.wfmt, act_mode=mode,
                                       expert_ptrs=G.expert_ptrs, ws=G._ws_for(T), ids=G.ids[:T], gates=G.gates[:T],
                                       out=G.out[:T], x=x, shared_blob=G.shared, phase=phase)

    def run_route_slots(G, x, phase=0):
        # the whole decode layer: router logits, gate/up selecting its slots' experts, down + combine
        B.moe_route_ffn_combine_slots(T=T, d=cfg.d, f=cfg.f, E=cfg.E, k=cfg.k, wfmt=cfg.wfmt, act_mode=mode,
                                      expert_ptrs=G.expert_ptrs, ws=G._ws_for(T), Wr=G.Wr, bias=G.bias,
                                      ids=G.ids[:T], gates=G.gates[:T], out=G.out[:T], x=x, shared_blob=G.shared,
                                      phase=phase)

    def run_ffn(G, x, phase=0):
        if by_slot:
            return run_route_slots(G, x, phase)
        n = T * cfg.k
        common = dict(T=T, d=cfg.d, f=cfg.f, E=cfg.E, k=cfg.k, wfmt=cfg.wfmt, act_mode=mode,
                      expert_ptrs=G.expert_ptrs, counts=G.counts, offsets=G.offsets, sorted_idx=G.sorted_idx[:n],
                      active=G.active, y_perm=G.y_perm[:n], ws=G._ws_for(T), shared_blob=G.shared,
                      y_shared=G.y_shared[:T] if G.shared is not None else None, phase=phase)
        if mode == B.MOE_ACT_Q8:
            B.moe_expert_ffn(xq=G.xq[:T], sx=G.sx[:T], **common)
        else:
            B.moe_expert_ffn(x=x, **common)

    def run_ffn_combine(G, x):
        # expert FFN and the weighted combine (one kernel for the down projection
        # and the sum where the library has it)
        if by_slot:
            return run_slots(G, x)
        n = T * cfg.k
        common = dict(T=T, d=cfg.d, f=cfg.f, E=cfg.E, k=cfg.k, wfmt=cfg.wfmt, act_mode=mode,
                      expert_ptrs=G.expert_ptrs, counts=G.counts, offsets=G.offsets, sorted_idx=G.sorted_idx[:n],
                      active=G.active, y_perm=G.y_perm[:n], ws=G._ws_for(T), shared_blob=G.shared,
                      y_shared=G.y_shared[:T] if G.shared is not None else None, ids=G.ids[:T], dest=G.dest[:n],
                      gates=G.gates[:T], out=G.out[:T])
        if mode == B.MOE_ACT_Q8:
            B.moe_expert_ffn_combine(xq=G.xq[:T], sx=G.sx[:T], **common)
        else:
            B.moe_expert_ffn_combine(x=x, **common)

    def run_step(G, x):
        if by_slot:
            return run_route_slots(G, x)
        run_route(G, x)
        run_ffn_combine(G, x)

    # warm up eagerly on every copy
    for i in range(max(warmup, rotate)):
        r = i % rotate
        run_step(layers[r], xs[r])
    torch.cuda.synchronize()

    use_graph = not a.no_graph
    stream = torch.cuda.Stream()

    def capture(fn_r, rs):
        """One graph running fn_r(r) for every r in rs, in order."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for r in rs:
                    fn_r(r)
        return g

    def timed(fn, n):
        with torch.cuda.stream(stream):
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record(stream)
            for i in range(n):
                fn(i)
            end.record(stream)
            torch.cuda.synchronize()
        return start.elapsed_time(end)

    def run_all(fn_r, graphs, n):
        """n launches of fn_r over the copies in order: whole rotations from the
        all-copies graph, the remainder from single-copy graphs (eager without graphs)."""
        if graphs is None:
            for i in range(n):
                fn_r(i % rotate)
            return
        chain, singles = graphs
        for _ in range(n // rotate):
            chain.replay()
        for i in range(n % rotate):
            singles[i].replay()

    step_r = lambda r: run_step(layers[r], xs[r])
    gu_r = lambda r: run_ffn(layers[r], xs[r], phase=1)
    # by slot, the step's gate/up also selects the experts; its expert-FFN work
    # alone (the same kernel reading the ids) is timed as well
    alone_r = lambda r: run_slots(layers[r], xs[r], phase=1)
    step_graphs = gu_graphs = alone_graphs = None
    if use_graph:
        step_graphs = (capture(step_r, range(rotate)), [capture(step_r, [r]) for r in range(rotate)])
        gu_graphs = (capture(gu_r, range(rotate)), [capture(gu_r, [r]) for r in range(rotate)])
        if by_slot:
            alone_graphs = (capture(alone_r, range(rotate)), [capture(alone_r, [r]) for r in range(rotate)])
        torch.cuda.synchronize()

    # region A: whole steps
    timed(lambda i: run_all(step_r, step_graphs, rotate), 1)  # one more pass over the copies
    total_ms = timed(lambda i: run_all(step_r, step_graphs, steps), 1)
    ms_step = total_ms / steps

    # region B: the dominant kernel (gate/up) alone: back-to-back launches on the
    # stream, rotating over the weight copies, between two HIP events; always a
    # fixed number of whole rotations (at least 25 chain replays, whatever
    # --steps is), so that host submission gaps between graph replays do not
    # enter the per-launch time
    n_kernel = max(25, -(-steps // rotate)) * rotate
    timed(lambda i: run_all(gu_r, gu_graphs, rotate), 1)
    gu_ms = timed(lambda i: run_all(gu_r, gu_graphs, n_kernel), 1) / n_kernel
    alone_ms = None
    if by_slot:
        timed(lambda i: run_all(alone_r, alone_graphs, rotate), 1)
        alone_ms = timed(lambda i: run_all(alone_r, alone_graphs, n_kernel), 1) / n_kernel

    # algorithmic work per gate/up launch, from each copy's routing (fixed input per copy):
    # the distinct experts picked (the by-slot launch reads an expert once per slot)
    n_act = [int(np.unique(G.ids[:T].cpu().numpy()).size) for G in layers]
    per = [gateup_algorithmic(cfg, n, T) for n in n_act]
    alg_bytes = float(np.mean([p[0] for p in per]))
    alg_ops = float(np.mean([p[1] for p in per]))
    ffn_bytes = alg_bytes
    if by_slot:
        alg_bytes += T * cfg.E * 8  # the fused launch also reads the token's fp64 router logits
    if mode == B.MOE_ACT_Q8:
        achieved = alg_ops / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                "frac": round(achieved / INT8_PEAK_TOPS, 4), "traffic": measured_traffic(name)}
    else:
        achieved = alg_bytes / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(name)}
    if mode == B.MOE_ACT_Q8:
        roof["kernel"] = "ffn_i4_gateup (moe_expert_ffn phase 1)" if cfg.wfmt == 4 else "ffn_q8_gateup (moe_expert_ffn phase 1)"
    else:
        roof["kernel"] = ("ffn_gateup_tok16 by slot, selecting its experts (moe_route_ffn_combine_slots phase 1)"
                          if by_slot
                          else "ffn_gateup_tok16 (moe_expert_ffn phase 1)" if cfg.wfmt == 4 and T <= 16
                          else "ffn_gateup_tok64 (moe_expert_ffn phase 1)" if T <= 64
                          else "ffn_float_gateup (moe_expert_ffn phase 1)")
    roof["kernel_ms"] = round(gu_ms, 5)
    roof["kernel_launches_timed"] = n_kernel
    roof["algorithmic_bytes_per_launch"] = int(alg_bytes)
    roof["algorithmic_ops_per_launch"] = int(alg_ops)
    if alone_ms is not None:
        a_gbs = ffn_bytes / (alone_ms * 1e-3) / 1e9
        roof["expert_ffn_alone"] = {"kernel": "ffn_gateup_tok16 by slot, ids given (moe_expert_ffn_combine_slots phase 1)",
                                    "kernel_ms": round(alone_ms, 5), "achieved": round(a_gbs, 1),
                                    "frac": round(a_gbs / HBM_PEAK_GBS, 4)}

    del layers, xs, step_graphs, gu_graphs, alone_graphs, packed0
    cpu = None
    if with_cpu:
        cpu = cpu_baseline(L, a.cpu_seconds)

    value = T / (ms_step * 1e-3)
    line = {
        "metric": "MoE-layer tokens/s (8192-tok prefill; 1-4 tok decode); % HBM BW / MFMA peak",
        "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8" if mode == B.MOE_ACT_Q8 else "fp16",
        "data": "synthetic (seeded N(0,1) hidden states, N(0,0.02) router and block-32-quantised experts)",
        "config": {"workload": name, "T": T, "d": cfg.d, "E": cfg.E, "k": cfg.k, "f": cfg.f,
                   "weights": "int4-b32" if cfg.wfmt == 4 else "int8-b32", "shared_expert": cfg.has_shared,
                   "act_mode": cfg.act_mode, "x_dtype": cfg.x_dtype, "weight_copies_rotated": rotate,
                   "graph": use_graph, "active_experts_per_step": float(np.mean(n_act))},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    return line


def bench_decode_stack(a):
    """48-layer decode stack: one step = one decode pass of all layers over T = 4
    (or 1) tokens.  Routers are biased toward the residency profile; the
    4,500-slot pool serves the hits and the FFN reads every selected miss in
    place from the pinned host store.  The whole pass is one captured graph."""
    import torch

    import synth
    from sparse_moe_expert_gemv_amd import binding as B
    from sparse_moe_expert_gemv_amd.stack import ExpertStack, build_host_store

    steps = a.steps if a.steps is not None else 20
    warmup = a.warmup if a.warmup is not None else 3
    t0 = time.time()
    S = synth.make_stack(seed=a.seed, name=a.workload)
    c = S.cfg
    store = build_host_store(S.pool, c.wfmt, c.d, c.f)
    G = ExpertStack(S.routers, S.shared_blobs(), store, S.index, S.resident, d=c.d, f=c.f, k=c.k, wfmt=c.wfmt,
                    act_mode=B.MOE_ACT_FLOAT, max_T=c.T, biases=S.biases, miss_mode="host", by_slot=True,
                    cpu_blobs=S.pool)
    x = torch.from_numpy(synth.bf16_bits_to_f32(S.x)).cuda()
    print("[bench] %s: %d layers x %d experts, %d resident, %d-blob host pool, T=%d (ready in %.1fs)"
          % (a.workload, c.n_layers, c.E, len(S.resident), c.n_pool_blobs, c.T, time.time() - t0),
          file=sys.stderr, flush=True)
    # routing statistics of one pass (untimed): selections served by the pool
    ids_l = []
    G.forward(x, ids_out=ids_l)
    torch.cuda.synchronize()
    res = np.zeros(c.n_layers * c.E, dtype=bool)
    res[np.asarray(S.resident, dtype=np.int64)] = True
    res = res.reshape(c.n_layers, c.E)
    sel_hit = np.concatenate([res[l][ids_l[l].cpu().numpy().ravel()] for l in range(c.n_layers)])
    uniq_miss = [int((~res[l][np.unique(ids_l[l].cpu().numpy())]).sum()) for l in range(c.n_layers)]
    miss_bytes = sum(uniq_miss) * G.eb

    def graph_of(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()  # warm the allocator on the capture stream
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    g_step = graph_of(lambda: G.forward(x))
    slot_tables = G.pool.data_ptr() + G.eb * (torch.arange(c.n_layers * c.E, dtype=torch.int64) % G.n_slots)
    slot_tables = slot_tables.reshape(c.n_layers, c.E).cuda()
    g_comp = graph_of(lambda: G.forward(x, compute_only_tables=slot_tables))

    def timed(g, n):
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(n):
            g.replay()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / n

    ms_step = timed(g_step, steps)
    ms_comp = timed(g_comp, steps)
    value = c.T / (ms_step * 1e-3)
    extra = ms_step - ms_comp
    # the pages' split of the misses: a share pcie_frac read by the GPU over the
    # host link, the rest computed on host cores while the GPU computes the
    # layer (eager: every layer waits for its routing on the host)
    split = None
    if a.workload in ("decode_stack", "decode_stack_t1") and not a.no_split:
        G.set_pcie_frac(1.0)
        threads = max(1, min(16, os.cpu_count() or 1))
        fracs, ms_split, items = [1.0, 0.75, 0.5, 0.25, 0.0], [], []
        for fr in fracs:
            G.set_pcie_frac(fr, threads)
            for _ in range(2):
                G.forward(x)
            torch.cuda.synchronize()
            G.cpu_items = 0
            n = max(3, steps // 4)
            t0 = time.perf_counter()
            for _ in range(n):
                G.forward(x)
            torch.cuda.synchronize()
            ms_split.append(round(1e3 * (time.perf_counter() - t0) / n, 3))
            items.append(round(G.cpu_items / n, 2))
            print("[bench] %s split pcie_frac=%.2f: %.3f ms/step, %.1f host items/step"
                  % (a.workload, fr, ms_split[-1], items[-1]), file=sys.stderr, flush=True)
        G.set_pcie_frac(1.0)
        best = int(np.argmin(ms_split))
        split = {"pcie_frac": fracs, "ms_per_step_eager": ms_split, "host_items_per_step": items,
                 "host_threads": threads, "best_pcie_frac": fracs[best],
                 "best_tokens_per_s": round(c.T / (ms_split[best] * 1e-3), 2)}
    line = {
        "metric": "MoE-layer tokens/s (8192-tok prefill; 1-4 tok decode); % HBM BW / MFMA peak",
        "value": round(value, 2), "unit": "tokens/s (48-layer decode stack)", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic (seeded N(0,1) hidden states, N(0,0.02) routers with a profile bias, block-32 int4 "
                "experts)",
        "config": {"workload": a.workload, "T": c.T, "layers": c.n_layers, "experts_total": c.n_layers * c.E,
                   "resident_slots": len(S.resident), "host_pool_blobs": c.n_pool_blobs, "k": c.k,
                   "profile_bias": c.profile_bias, "graph": True},
        "decode_stack": {"hit_rate": round(float(sel_hit.mean()), 4),
                         "missed_experts_per_layer_mean": round(float(np.mean(uniq_miss)), 3),
                         "host_bytes_per_step": int(miss_bytes),
                         "all_resident_ms": round(ms_comp, 4),
                         "host_read_ms": round(extra, 4),
                         "host_read_GBps": round(miss_bytes / (extra * 1e-3) / 1e9, 2) if extra > 0 else None,
                         "split_misses_with_host_cores": split},
        "roofline": None,
        "cpu_baseline": None,
    }
    G.close()
    print(json.dumps(line), flush=True)


def bench_decode_stack_drift(a):
    """Adaptive expert cache on the 48-layer decode stack (T = 4).  The pool is
    filled from one usage profile while the session routes by another (every
    router biased by a second seeded profile), so the static pool serves few
    selections.  A timed adaptation run replays the decode pass (one graph) on
    changing inputs and every 4 steps lets the policy read the device usage
    counters and swap up to 128 experts into the pool; then the adapted pool is
    timed as it stands.  value = tokens/s of the adapted pool."""
    import torch

    import synth
    from sparse_moe_expert_gemv_amd import binding as B
    from sparse_moe_expert_gemv_amd.stack import AdaptiveResidency, ExpertStack, build_host_store

    steps = a.steps if a.steps is not None else 20
    warmup = a.warmup if a.warmup is not None else 3
    n_adapt, every, max_swaps, n_draws = 128, 4, 128, 32
    t0 = time.time()
    S = synth.make_stack(seed=a.seed, name="decode_stack")
    c = S.cfg
    store = build_host_store(S.pool, c.wfmt, c.d, c.f)
    rank_b = synth.stack_profile(a.seed + 1, c.n_layers, c.E)
    biases = [synth.profile_router_bias(rank_b, l, c.E, c.profile_bias) for l in range(c.n_layers)]
    G = ExpertStack(S.routers, S.shared_blobs(), store, S.index, S.resident, d=c.d, f=c.f, k=c.k, wfmt=c.wfmt,
                    act_mode=B.MOE_ACT_FLOAT, max_T=c.T, biases=biases, miss_mode="host")
    A = AdaptiveResidency(G, decay=0.5, max_swaps=max_swaps)
    xs = [torch.from_numpy(synth.bf16_bits_to_f32(synth.gen_x(a.seed, c, draw=j))).cuda() for j in range(n_draws)]
    x_buf = xs[0].clone()
    print("[bench] decode_stack_drift: %d layers, %d resident, T=%d (ready in %.1fs)"
          % (c.n_layers, len(S.resident), c.T, time.time() - t0), file=sys.stderr, flush=True)

    def hit_rate(draws=16):
        hits = []
        for j in range(draws):
            ids_l = []
            G.forward(xs[j], ids_out=ids_l)
            for l in range(c.n_layers):
                hits.append(A.resident[ids_l[l].cpu().numpy().ravel() + l * c.E])
        return float(np.concatenate(hits).mean())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        G.forward(x_buf)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        G.forward(x_buf)

    def timed(n):
        for j in range(warmup):
            x_buf.copy_(xs[j % n_draws])
            g.replay()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for j in range(n):
            x_buf.copy_(xs[j % n_draws])
            g.replay()
        torch.cuda.synchronize()
        return 1e3 * (time.perf_counter() - t) / n

    hit_static = hit_rate()
    ms_static = timed(steps)
    torch.cuda.synchronize()
    t = time.perf_counter()
    upd = 0.0
    for j in range(n_adapt):
        x_buf.copy_(xs[j % n_draws])
        g.replay()
        if j % every == every - 1:
            tu = time.perf_counter()
            A.update()
            upd += time.perf_counter() - tu
    torch.cuda.synchronize()
    ms_adapt_run = 1e3 * (time.perf_counter() - t) / n_adapt
    hit_adapted = hit_rate()
    ms_adapted = timed(steps)
    value = c.T / (ms_adapted * 1e-3)
    line = {
        "metric": "MoE-layer tokens/s (8192-tok prefill; 1-4 tok decode); % HBM BW / MFMA peak",
        "value": round(value, 2), "unit": "tokens/s (48-layer decode stack, adapted pool)", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_adapted, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic (seeded N(0,1) hidden states, N(0,0.02) routers biased by a second profile, block-32 "
                "int4 experts)",
        "config": {"workload": "decode_stack_drift", "T": c.T, "layers": c.n_layers,
                   "experts_total": c.n_layers * c.E, "resident_slots": len(S.resident), "k": c.k,
                   "profile_bias": c.profile_bias, "graph": True},
        "adaptive": {"hit_rate_static": round(hit_static, 4), "hit_rate_adapted": round(hit_adapted, 4),
                     "ms_per_step_static": round(ms_static, 4), "ms_per_step_adapted": round(ms_adapted, 4),
                     "adaptation_steps": n_adapt, "update_every": every, "max_swaps_per_update": max_swaps,
                     "swaps": A.swaps, "ms_per_step_during_adaptation": round(ms_adapt_run, 4),
                     "ms_per_update_incl_counter_readback": round(1e3 * upd / (n_adapt // every), 3),
                     "host_policy_ms_per_update": round(1e3 * A.policy_s / (n_adapt // every), 3)},
        "roofline": None,
        "cpu_baseline": None,
    }
    G.close()
    print(json.dumps(line), flush=True)


def bench_stack(a):
    """48-layer stack: one step = one pass of all layers over the 8,192-token chunk,
    with the non-resident experts of every layer staged from pinned host memory
    on a side stream while the previous layer computes."""
    import torch

    import synth
    from sparse_moe_expert_gemv_amd import binding as B
    from sparse_moe_expert_gemv_amd.stack import ExpertStack, build_host_store

    steps = a.steps if a.steps is not None else 3
    warmup = a.warmup if a.warmup is not None else 1
    t0 = time.time()
    S = synth.make_stack(seed=a.seed)
    c = S.cfg
    store = build_host_store(S.pool, c.wfmt, c.d, c.f)
    G = ExpertStack(S.routers, S.shared_blobs(), store, S.index, S.resident, d=c.d, f=c.f, k=c.k, wfmt=c.wfmt,
                    act_mode=B.MOE_ACT_Q8, max_T=c.T)
    x = torch.from_numpy(synth.bf16_bits_to_f32(S.x)).cuda()
    print("[bench] stack: %d layers x %d experts, %d resident, %d-blob host pool, T=%d (ready in %.1fs)"
          % (c.n_layers, c.E, len(S.resident), c.n_pool_blobs, c.T, time.time() - t0), file=sys.stderr, flush=True)
    n_miss = [len(G.misses(l)) for l in range(c.n_layers)]
    h2d_bytes = sum(n_miss) * G.eb
    for _ in range(warmup):
        G.forward(x)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        G.forward(x)
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / steps
    # components: staging alone, compute alone (every expert read from a resident slot)
    t_copy = 1e3 * time_it(lambda: G.forward(x, copy_only=True))
    slot_tables = G.pool.data_ptr() + G.eb * (torch.arange(c.n_layers * c.E, dtype=torch.int64) % G.n_slots)
    slot_tables = slot_tables.reshape(c.n_layers, c.E).cuda()
    t_comp = 1e3 * time_it(lambda: G.forward(x, compute_only_tables=slot_tables))
    overlap = (t_copy + t_comp - ms_step) / min(t_copy, t_comp)
    # the same staging with one hipMemcpyAsync per missed expert
    G.cache.set_stage_mode(B.MOE_STAGE_MEMCPY)
    t_copy_memcpy = 1e3 * time_it(lambda: G.forward(x, copy_only=True))
    G.forward(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    G.forward(x)
    torch.cuda.synchronize()
    ms_step_memcpy = 1e3 * (time.perf_counter() - t0)
    G.cache.set_stage_mode(B.MOE_STAGE_KERNEL, 32)
    value = c.T / (ms_step * 1e-3)
    line = {
        "metric": "MoE-layer tokens/s (8192-tok prefill; 1-4 tok decode); % HBM BW / MFMA peak",
        "value": round(value, 2), "unit": "tokens/s (48-layer stack)", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8",
        "data": "synthetic (seeded N(0,1) hidden states, N(0,0.02) routers and block-32 int4 experts)",
        "config": {"workload": "stack", "T": c.T, "layers": c.n_layers, "experts_total": c.n_layers * c.E,
                   "resident_slots": len(S.resident), "host_pool_blobs": c.n_pool_blobs, "k": c.k,
                   "misses_per_layer_mean": float(np.mean(n_miss))},
        "stack": {"h2d_bytes_per_pass": int(h2d_bytes), "h2d_GBps": round(h2d_bytes / (t_copy * 1e-3) / 1e9, 2),
                  "copy_only_ms": round(t_copy, 3), "compute_only_ms": round(t_comp, 3),
                  "overlap_efficiency": round(overlap, 3),
                  "staging": "one copy kernel per layer (32 workgroups) reading pinned host memory",
                  "per_expert_memcpy": {"copy_only_ms": round(t_copy_memcpy, 3),
                                        "h2d_GBps": round(h2d_bytes / (t_copy_memcpy * 1e-3) / 1e9, 2),
                                        "ms_per_step": round(ms_step_memcpy, 3)},
                  "layer_tokens_per_s": round(c.T * c.n_layers / (ms_step * 1e-3), 1)},
        "roofline": None,
        "cpu_baseline": None,
    }
    G.close()
    print(json.dumps(line), flush=True)


def bench_copy(a):
    """Calibration aid for HBM byte counters: a plain device-to-device copy of
    exactly 1 GiB (reads 1 GiB, writes 1 GiB), repeated --steps times."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    steps = a.steps if a.steps is not None else 5
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"workload": "copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n,
                      "ms_per_copy": round(dt * 1e3, 3), "GBps_read_plus_write": round(2 * n / dt / 1e9, 1)}),
          flush=True)


def bench_peak(a):
    """Measured ceilings (calibration kernels of libmoe_probe.so): the issue
    rate of each matrix-core instruction the FFN kernels use, the plain fp32
    FMA rate of the vector unit, the rate of one int8 32x32x32 MFMA per block
    followed by the exact two-operation block-scale epilogue (and by a
    one-operation one), a non-temporal HBM read stream over 4 GiB, and single
    launches that read 10-70 MiB (the per-launch reads of the decode kernels).
    Workgroups of 256 threads; ``waves/SIMD`` = grid / 256 (one wavefront of
    each workgroup per SIMD).  Best rate over the grid sizes tried."""
    import ctypes
    import torch
    from sparse_moe_expert_gemv_amd import build as _b
    if not os.path.exists(_b.PROBE_LIB):
        raise RuntimeError("libmoe_probe.so is not built (python -m sparse_moe_expert_gemv_amd.build)")
    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.moe_probe_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    out = torch.empty(n_cu * 16 * 256, dtype=torch.float32, device="cuda")

    def run(kind, grid, iters, inp=None, nbytes=0, reps=5):
        def launch():
            rc = lib.moe_probe_run(kind, grid, iters, 1, out.data_ptr(), inp, nbytes, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError("moe_probe_run(kind=%d) returned %d" % (kind, rc))
        launch()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    res = {}
    # (kind, name, ops per instruction per wavefront, instructions per iteration, unit)
    mfma = [(0, "mfma_i8_32x32x32", 32 * 32 * 32 * 2, 4, "TOPS"), (1, "mfma_i8_16x16x64", 16 * 16 * 64 * 2, 4, "TOPS"),
            (2, "mfma_f16_32x32x16", 32 * 32 * 16 * 2, 4, "TFLOPS"),
            (3, "mfma_f16_16x16x32", 16 * 16 * 32 * 2, 4, "TFLOPS"),
            (5, "i8_32x32x32_plus_two_fp32_fma_per_output", 32 * 32 * 32 * 2, 2, "TOPS (int8 MFMA ops)"),
            (7, "i8_32x32x32_plus_one_fp32_fma_per_output", 32 * 32 * 32 * 2, 2, "TOPS (int8 MFMA ops)")]
    for kind, nm, ops, per_it, unit in mfma:
        best, by_w = None, {}
        for w in (1, 2, 3, 4):
            grid, iters = n_cu * w, 4000 // w
            t = run(kind, grid, iters)
            rate = grid * 4 * iters * per_it * ops / t / 1e12
            by_w[w] = round(rate, 1)
            if best is None or rate > best[0]:
                best = (rate, w, t)
        res[nm] = {"rate": round(best[0], 1), "unit": unit, "waves_per_simd": best[1], "ms": round(best[2] * 1e3, 3),
                   "rate_by_waves_per_simd": by_w}
    best, by_w = None, {}
    for w in (1, 2, 3, 4):
        grid, iters = n_cu * w, 40000 // w
        t = run(4, grid, iters)
        rate = grid * 256 * iters * 16 * 2 / t / 1e12
        by_w[w] = round(rate, 1)
        if best is None or rate > best[0]:
            best = (rate, w, t)
    res["valu_fma_f32"] = {"rate": round(best[0], 1), "unit": "TFLOPS (v_fma_f32, not packed)",
                           "waves_per_simd": best[1], "ms": round(best[2] * 1e3, 3), "rate_by_waves_per_simd": by_w}
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    best = None
    for w in (2, 4, 8, 16):
        grid = n_cu * w
        t = run(6, grid, 0, buf.data_ptr(), nbytes, reps=3)
        gbs = nbytes / t / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, w, t)
    res["hbm_stream_read"] = {"rate": round(best[0], 1), "unit": "GB/s", "workgroups_per_cu": best[1],
                              "bytes": nbytes, "ms": round(best[2] * 1e3, 3)}
    # short reads: one launch reads `size` bytes, the sizes the decode kernels
    # read per launch; consecutive launches take consecutive windows of the
    # 4 GiB buffer, so every launch reads cold data (not held in the 256 MB
    # last-level cache); best over kernel shape and grid
    short = {}
    for size in (10 << 20, 20 << 20, 35 << 20, 70 << 20):
        n_win = nbytes // size
        best = None
        for kind in (6, 8):
            for w in (1, 2, 4, 8):
                grid = n_cu * w
                reps = 40

                def launch(r):
                    rc = lib.moe_probe_run(kind, grid, 0, 1, out.data_ptr(), buf.data_ptr() + (r % n_win) * size,
                                           size, stream.cuda_stream)
                    if rc != 0:
                        raise RuntimeError("moe_probe_run(kind=%d) returned %d" % (kind, rc))
                for r in range(reps):
                    launch(r)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for r in range(reps):
                    launch(reps + r)
                e1.record(stream)
                torch.cuda.synchronize()
                t = e0.elapsed_time(e1) / reps * 1e-3
                if best is None or size / t > best[0]:
                    best = (size / t / 1e9, "burst" if kind == 8 else "single", w, t)
        short["%d_MiB" % (size >> 20)] = {"rate": round(best[0], 1), "unit": "GB/s", "us_per_launch":
                                          round(best[3] * 1e6, 2), "kernel": best[1], "workgroups_per_cu": best[2]}
    res["short_read_one_launch"] = short
    del buf
    # the vendor library's fp16 rate at the prefill expert shapes: torch.bmm
    # (hipBLASLt) over 512 experts of 176 token rows with dense fp16 weights
    # (four times the weight bytes of int4), gate/up (2,048 k, 1,536 outputs)
    # and down (768 k, 2,048 outputs); operands contiguous, fp16 outputs
    vendor = {}
    for nm, (G, M, K, N) in (("gateup_512x176x2048x1536", (512, 176, 2048, 1536)),
                             ("down_512x176x768x2048", (512, 176, 768, 2048))):
        A = torch.randn(G, M, K, device="cuda", dtype=torch.float16)
        Bm = torch.randn(G, K, N, device="cuda", dtype=torch.float16).contiguous()
        Cm = torch.empty(G, M, N, device="cuda", dtype=torch.float16)
        time_it(lambda: torch.bmm(A, Bm, out=Cm), reps=2)  # warm-up (the library's kernel selection)
        t = time_it(lambda: torch.bmm(A, Bm, out=Cm), reps=10)
        fl = 2.0 * G * M * K * N
        vendor[nm] = {"ms": round(t * 1e3, 3), "rate": round(fl / t / 1e12, 1), "unit": "TFLOPS",
                      "frac_of_f16_peak": round(fl / t / 1e12 / 2500.0, 4)}
        del A, Bm, Cm
    res["vendor_fp16_bmm"] = vendor
    print(json.dumps({"workload": "peak", "compute_units": n_cu, "datasheet": {
        "int8_mfma_TOPS": INT8_PEAK_TOPS, "f16_mfma_TFLOPS": 2500.0, "fp32_vector_TFLOPS": 157.3,
        "hbm_GBps": HBM_PEAK_GBS}, "measured": res}), flush=True)


def time_it(fn, reps=1):
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / reps


def cpu_baseline(L, budget_s: float):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import oracle
    cfg = L.cfg
    om = oracle.ACT_Q8 if cfg.act_mode == "q8" else oracle.ACT_FLOAT
    x = L.x_f32()
    if cfg.T <= 64:
        toks, sample = None, "full layer (all %d tokens), repeated" % cfg.T
        per_call = cfg.T
    else:
        toks = np.arange(0, cfg.T, cfg.T // 16, dtype=np.int32)[:16]
        sample = ("routing of all %d tokens + expert FFN and combine of 16 evenly spaced tokens; "
                  "tokens/s counts the 16 tokens" % cfg.T)
        per_call = len(toks)
    t0 = time.time()
    n = 0
    while True:
        oracle.moe_layer(x, L.Wr, L.bias, L.experts, L.shared, cfg.wfmt, cfg.f, cfg.k, act_mode=om, tokens=toks)
        n += 1
        el = time.time() - t0
        if el >= budget_s or (n >= 1 and el * (n + 1) / n > 3 * budget_s):
            break
    return {"value": round(per_call * n / el, 3), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": sample + "; %d call(s) in %.1fs" % (n, el)}


if __name__ == "__main__":
    main()
