"""GPU parity of the layer stack with the expert slot pool and miss staging.

Each layer computes h_{l+1} = h_l + MoE_l(rmsnorm(h_l)).  It is checked
teacher-forced: the oracle receives the GPU's fp32 residual h_l and normalised
input rmsnorm(h_l) of that layer, computes the MoE layer on the canonical blobs
of that layer's experts, and its ids/permutation must match bit for bit and its
output within the float tolerance; the GPU norm itself is checked against the
oracle's to fp32 rounding.  Staged (missed) experts and pool
(resident) experts must give bit-identical results to a plain device copy of
the same weights.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import refmath as R

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from sparse_moe_expert_gemv_amd import binding as B  # noqa: E402
from sparse_moe_expert_gemv_amd.layer import pack_blobs, pointer_table  # noqa: E402
from sparse_moe_expert_gemv_amd.stack import ExpertStack, build_host_store  # noqa: E402

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    oracle.build(force=False)


def _stack_gpu(S):
    c = S.cfg
    store = build_host_store(S.pool, c.wfmt, c.d, c.f)
    mode = B.MOE_ACT_Q8 if c.act_mode == "q8" else B.MOE_ACT_FLOAT
    return ExpertStack(S.routers, S.shared_blobs() if c.has_shared else None, store, S.index, S.resident,
                       d=c.d, f=c.f, k=c.k, wfmt=c.wfmt, act_mode=mode, max_T=c.T)


def _x0(S):
    return torch.from_numpy(synth.bf16_bits_to_f32(S.x)).to(DEV)


def _check_layer(S, l, h_in, xn_in, tokens=None):
    c = S.cfg
    om = oracle.ACT_Q8 if c.act_mode == "q8" else oracle.ACT_FLOAT
    ref_norm = oracle.rmsnorm(h_in, 1e-6)
    assert np.max(np.abs(xn_in - ref_norm)) <= 1e-6 * (1 + np.max(np.abs(ref_norm)))
    o = oracle.moe_layer(xn_in, S.routers[l], None, S.layer_experts(l),
                         S.shared_blobs()[l] if c.has_shared else None, c.wfmt, c.f, c.k, act_mode=om,
                         residual=h_in, tokens=tokens)
    return o


SMALL = dict(T=300, d=256, E=64, k=4, f=128, wfmt=synth.WFMT_I8B32, has_shared=True, act_mode="q8", n_layers=4,
             n_resident=100, n_pool_blobs=40)


def test_small_stack_teacher_forced_and_pool_vs_staging_bitexact():
    S = synth.make_stack(overrides=SMALL)
    G = _stack_gpu(S)
    x = _x0(S)
    hL, kept = G.forward(x, keep=range(S.cfg.n_layers))
    torch.cuda.synchronize()
    hs = [kept[l][0].cpu().numpy() for l in range(S.cfg.n_layers)] + [hL.cpu().numpy()]
    xns = [kept[l][1].cpu().numpy() for l in range(S.cfg.n_layers)]
    for l in range(S.cfg.n_layers):
        hit, miss = G.cache.lookup(l)
        assert sorted(hit + miss) == list(range(S.cfg.E))
        resident_l = sorted(int(g) % S.cfg.E for g in S.resident if int(g) // S.cfg.E == l)
        assert hit == resident_l
        o = _check_layer(S, l, hs[l], xns[l])
        # routing of this layer as the GPU computed it, from the layer's own run
        ok, rel, mx = R.within_tolerance(hs[l + 1], o["out"])
        assert ok, "layer %d: rel %.3e max %.3e" % (l, rel, mx)
    # the last layer through a plain contiguous copy of its experts: bit-identical
    l = S.cfg.n_layers - 1
    c = S.cfg
    plain = pack_blobs(torch.from_numpy(S.layer_experts(l)).to(DEV), c.wfmt, c.d, c.f)
    table = pointer_table(plain)
    out_a = torch.empty_like(x)
    out_b = torch.empty_like(x)
    h_in = torch.from_numpy(hs[l]).to(DEV)
    G.layer(l, h_in, out_a)  # through the cache's table (last staged state of layer l)
    G.layer(l, h_in, out_b, table=table)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    assert np.array_equal(out_a.cpu().numpy(), hs[l + 1])
    G.close()


def test_small_stack_ids_and_permutation_bitexact_per_layer():
    S = synth.make_stack(overrides=SMALL)
    G = _stack_gpu(S)
    x = _x0(S)
    h = x
    out = torch.empty_like(x)
    for l in range(S.cfg.n_layers):
        G.stage(l)
        torch.cuda.current_stream().wait_event(G.staged[l])
        G.layer(l, h, out)
        torch.cuda.synchronize()
        T = S.cfg.T
        h_np = h.cpu().numpy()
        o = _check_layer(S, l, h_np, G.xn[:T].cpu().numpy())
        assert np.array_equal(G.ids[:T].cpu().numpy(), o["ids"])
        assert np.array_equal(G.counts.cpu().numpy(), o["counts"])
        assert np.array_equal(G.sorted_idx[:T * S.cfg.k].cpu().numpy(), o["sorted_idx"])
        assert np.array_equal(G.dest[:T * S.cfg.k].cpu().numpy(), o["dest"])
        h, out = out, h
    G.close()


def test_cache_capacity_error_when_staging_too_small():
    S = synth.make_stack(overrides=SMALL)
    c = S.cfg
    store = build_host_store(S.pool, c.wfmt, c.d, c.f)
    G = ExpertStack(S.routers, None, store, S.index, S.resident, d=c.d, f=c.f, k=c.k, wfmt=c.wfmt,
                    act_mode=B.MOE_ACT_Q8, max_T=c.T, staging_slots=8)
    with pytest.raises(B.MoeError) as ei:
        G.stage(0)
    assert ei.value.status == B.MOE_ERR_CACHE_CAPACITY
    G.close()


@pytest.mark.parametrize("stage_mode", ["memcpy", "kernel"])
def test_injected_staging_failure_then_retry_bitexact(stage_mode):
    """A staging copy forced to fail from the host (the cache's fault hook)
    makes moe_cache_stage report MOE_ERR_HIP with the injected code; residency
    and the other buffer's layer stay intact, and staging the layer again gives
    the same output, bit for bit, as a run that never failed."""
    S = synth.make_stack(overrides=SMALL)
    c = S.cfg
    store = build_host_store(S.pool, c.wfmt, c.d, c.f)
    G = ExpertStack(S.routers, S.shared_blobs(), store, S.index, S.resident, d=c.d, f=c.f, k=c.k, wfmt=c.wfmt,
                    act_mode=B.MOE_ACT_Q8, max_T=c.T, stage_mode=stage_mode)
    x = _x0(S)
    ref = [torch.empty_like(x) for _ in range(2)]
    for l in range(2):
        G.stage(l)
        torch.cuda.current_stream().wait_event(G.staged[l])
        G.layer(l, x, ref[l])
    torch.cuda.synchronize()
    hits_before = [G.cache.lookup(l)[0] for l in range(c.n_layers)]
    miss1 = G.misses(1)
    assert len(miss1) > 6
    fail_at, injected = 5, 2  # hipErrorOutOfMemory
    calls = []

    def hook(layer, index, expert):
        calls.append((layer, index, expert))
        return injected if (layer == 1 and index == fail_at) else 0

    G.cache.set_stage_fault_hook(hook)
    with pytest.raises(B.MoeError) as ei:
        G.stage(1)
    assert ei.value.status == B.MOE_ERR_HIP and ei.value.hip_error == injected
    assert calls == [(1, i, miss1[i]) for i in range(fail_at + 1)]
    G.cache.set_stage_fault_hook(None)
    torch.cuda.synchronize()
    assert [G.cache.lookup(l)[0] for l in range(c.n_layers)] == hits_before
    out = torch.empty_like(x)
    # layer 0 lives in the other staging buffer: untouched by the failed call
    G.layer(0, x, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref[0])
    G.stage(1)
    torch.cuda.current_stream().wait_event(G.staged[1])
    G.layer(1, x, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref[1])
    G.close()


def test_full_stack_48_layers_sampled():
    """The 48-layer, 24,576-expert stack at T=8192 with 4,500 resident slots:
    on every layer, teacher-forced, the routing of all tokens (ids, counts,
    offsets, sorted_idx, dest) bit-exact against the oracle; outputs on 128
    sampled tokens for seven layers spread over the stack."""
    S = synth.make_stack()
    c = S.cfg
    assert c.n_layers * c.E == 24576 and len(S.resident) == 4500
    G = _stack_gpu(S)
    x = _x0(S)
    ids_l = []
    hL, kept = G.forward(x, keep=range(c.n_layers), ids_out=ids_l)
    torch.cuda.synchronize()
    T, k, E = c.T, c.k, c.E
    n = T * k
    for l in range(c.n_layers):
        xn_t = kept[l][1]
        # the routing of the pass's own normalised input, through the library
        B.moe_route_permute(xn_t, G.Wr[l], None, k, G.ids[:T], G.gates[:T], G.counts, G.offsets, G.sorted_idx[:n],
                            G.dest[:n], G.active, G.ws)
        torch.cuda.synchronize()
        ids_gpu = G.ids[:T].cpu().numpy()
        assert np.array_equal(ids_gpu, ids_l[l].cpu().numpy()), "layer %d: ids differ from the pass" % l
        o_ids, _ = oracle.route(xn_t.cpu().numpy(), S.routers[l], None, k)
        assert np.array_equal(ids_gpu, o_ids), "layer %d ids" % l
        oc, oo, os_, od = oracle.permute(o_ids, E)
        assert np.array_equal(G.counts.cpu().numpy(), oc), "layer %d counts" % l
        assert np.array_equal(G.offsets.cpu().numpy(), oo), "layer %d offsets" % l
        assert np.array_equal(G.sorted_idx[:n].cpu().numpy(), os_), "layer %d sorted_idx" % l
        assert np.array_equal(G.dest[:n].cpu().numpy(), od), "layer %d dest" % l
    rng = np.random.Generator(np.random.PCG64(21))
    tokens = np.sort(rng.choice(c.T, 128, replace=False)).astype(np.int32)
    for l in (0, 8, 16, 24, 32, 40, 47):
        h_in = kept[l][0].cpu().numpy()
        # recompute layer l from its recorded input; its staging buffer has been
        # reused by later layers, so stage it again first
        G.stage(l)
        torch.cuda.current_stream().wait_event(G.staged[l])
        out = torch.empty_like(x)
        G.layer(l, kept[l][0], out)
        torch.cuda.synchronize()
        h_out = out.cpu().numpy()
        xn = G.xn[:c.T].cpu().numpy()
        assert np.array_equal(xn, kept[l][1].cpu().numpy())
        assert np.all(np.isfinite(h_out))
        assert np.array_equal(h_out, (kept[l + 1][0] if l + 1 < c.n_layers else hL).cpu().numpy())
        o = _check_layer(S, l, h_in, xn, tokens=tokens)
        ok, rel, mx = R.within_tolerance(h_out[tokens], o["out"])
        print("[stack] layer %d: rel-L2 %.3e max-abs/RMS %.3e" % (l, rel, mx), flush=True)
        assert ok, "layer %d: rel %.3e max %.3e" % (l, rel, mx)
    hit, miss = G.cache.lookup(0)
    assert len(hit) + len(miss) == c.E
    G.close()


# ---------------------------------------------------------------------------
# Decode stack: profile-biased routers, misses read in place from pinned host
# memory through the layer's pointer table (moe_cache_map_host).
# ---------------------------------------------------------------------------

DSMALL = dict(T=4, d=512, E=64, k=4, f=256, n_layers=4, n_resident=100, n_pool_blobs=40)


def _decode_stack_gpu(S, by_slot=False):
    c = S.cfg
    store = build_host_store(S.pool, c.wfmt, c.d, c.f)
    return ExpertStack(S.routers, S.shared_blobs() if c.has_shared else None, store, S.index, S.resident,
                       d=c.d, f=c.f, k=c.k, wfmt=c.wfmt, act_mode=B.MOE_ACT_FLOAT, max_T=c.T, biases=S.biases,
                       miss_mode="host", by_slot=by_slot)


def _check_decode_layer(S, l, h_in, xn_in):
    c = S.cfg
    ref_norm = oracle.rmsnorm(h_in, 1e-6)
    assert np.max(np.abs(xn_in - ref_norm)) <= 1e-6 * (1 + np.max(np.abs(ref_norm)))
    return oracle.moe_layer(xn_in, S.routers[l], S.biases[l], S.layer_experts(l),
                            S.shared_blobs()[l] if c.has_shared else None, c.wfmt, c.f, c.k,
                            act_mode=oracle.ACT_FLOAT, residual=h_in)


def _resident_mask(S):
    c = S.cfg
    m = np.zeros(c.n_layers * c.E, dtype=bool)
    m[np.asarray(S.resident, dtype=np.int64)] = True
    return m.reshape(c.n_layers, c.E)


@pytest.mark.parametrize("T,by_slot", [(1, False), (4, False), (1, True), (4, True)])
def test_small_decode_stack_host_misses_teacher_forced(T, by_slot):
    """Every layer teacher-forced against the oracle (ids bit-exact, outputs
    within the float tolerance), grouped or by slot; across the layers the
    routing selects both resident experts and misses, so both kinds of table
    entry are read."""
    S = synth.make_stack(name="decode_stack", overrides=DSMALL, T=T)
    c = S.cfg
    G = _decode_stack_gpu(S, by_slot)
    x = _x0(S)
    ids_l = []
    hL, kept = G.forward(x, keep=range(c.n_layers), ids_out=ids_l)
    torch.cuda.synchronize()
    hs = [kept[l][0].cpu().numpy() for l in range(c.n_layers)] + [hL.cpu().numpy()]
    res = _resident_mask(S)
    n_hit = n_miss = 0
    for l in range(c.n_layers):
        o = _check_decode_layer(S, l, hs[l], kept[l][1].cpu().numpy())
        ids = ids_l[l].cpu().numpy()
        assert np.array_equal(ids, o["ids"]), "layer %d ids" % l
        ok, rel, mx = R.within_tolerance(hs[l + 1], o["out"])
        assert ok, "layer %d: rel %.3e max %.3e" % (l, rel, mx)
        used = np.unique(ids)
        n_hit += int(res[l][used].sum())
        n_miss += int((~res[l][used]).sum())
    assert n_hit > 0 and n_miss > 0, (n_hit, n_miss)
    G.close()


@pytest.mark.parametrize("T,frac", [(4, 0.0), (4, 0.5), (1, 0.0)])
def test_small_decode_stack_host_core_misses_teacher_forced(T, frac):
    """Decode with a share (1 - pcie_frac) of each layer's missed experts
    computed on host cores (moe_host_expert_ffn) and added on the GPU: every
    layer teacher-forced against the oracle (ids bit-exact, outputs within the
    float tolerance), and host items were computed."""
    S = synth.make_stack(name="decode_stack", overrides=DSMALL, T=T)
    c = S.cfg
    store = build_host_store(S.pool, c.wfmt, c.d, c.f)
    G = ExpertStack(S.routers, S.shared_blobs() if c.has_shared else None, store, S.index, S.resident,
                    d=c.d, f=c.f, k=c.k, wfmt=c.wfmt, act_mode=B.MOE_ACT_FLOAT, max_T=c.T, biases=S.biases,
                    miss_mode="host", by_slot=True, cpu_blobs=S.pool, pcie_frac=frac, cpu_threads=4)
    x = _x0(S)
    ids_l = []
    hL, kept = G.forward(x, keep=range(c.n_layers), ids_out=ids_l)
    torch.cuda.synchronize()
    hs = [kept[l][0].cpu().numpy() for l in range(c.n_layers)] + [hL.cpu().numpy()]
    for l in range(c.n_layers):
        o = _check_decode_layer(S, l, hs[l], kept[l][1].cpu().numpy())
        assert np.array_equal(ids_l[l].cpu().numpy(), o["ids"]), "layer %d ids" % l
        ok, rel, mx = R.within_tolerance(hs[l + 1], o["out"])
        print("[split] T=%d frac=%.2f layer %d: rel-L2 %.3e max-abs/RMS %.3e" % (T, frac, l, rel, mx), flush=True)
        assert ok, "layer %d: rel %.3e max %.3e" % (l, rel, mx)
    assert G.cpu_items > 0
    G.close()


def test_small_decode_stack_by_slot_equals_grouped_bitexact():
    """The 4-layer decode stack by slot (no grouping) gives every layer's output
    bit for bit as the grouped path."""
    S = synth.make_stack(name="decode_stack", overrides=DSMALL)
    outs = []
    for by_slot in (False, True):
        G = _decode_stack_gpu(S, by_slot)
        hL, kept = G.forward(_x0(S), keep=range(S.cfg.n_layers))
        torch.cuda.synchronize()
        outs.append([kept[l][0].cpu().numpy() for l in range(S.cfg.n_layers)] + [hL.cpu().numpy()])
        G.close()
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_small_decode_stack_host_reads_match_device_copy_bitexact():
    """A layer computed through the host-mapped table equals, bit for bit, the
    same layer computed from a plain device copy of its experts."""
    S = synth.make_stack(name="decode_stack", overrides=DSMALL)
    c = S.cfg
    G = _decode_stack_gpu(S)
    x = _x0(S)
    res = _resident_mask(S)
    for l in range(c.n_layers):
        plain = pack_blobs(torch.from_numpy(S.layer_experts(l)).to(DEV), c.wfmt, c.d, c.f)
        out_a = torch.empty_like(x)
        out_b = torch.empty_like(x)
        G.layer(l, x, out_a)
        ids = G.ids[:c.T].cpu().numpy()
        G.layer(l, x, out_b, table=pointer_table(plain))
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), "layer %d" % l
        assert np.array_equal(G.ids[:c.T].cpu().numpy(), ids)
    # the tables hold host addresses for exactly the non-resident experts
    tables = G.tables.cpu().numpy()
    pool_lo = G.pool.data_ptr()
    pool_hi = pool_lo + G.pool.numel()
    in_pool = (tables >= pool_lo) & (tables < pool_hi)
    assert np.array_equal(in_pool, res)
    G.close()


def test_full_decode_stack_48_layers():
    """The 48-layer decode stack at T=4 over the 4,500-slot pool, misses read
    from the 24,576-expert pinned host store: first, middle and last layer
    teacher-forced against the oracle; the hit rate near the intended 72%."""
    S = synth.make_stack(name="decode_stack")
    c = S.cfg
    assert c.n_layers * c.E == 24576 and len(S.resident) == 4500 and c.T == 4
    G = _decode_stack_gpu(S)
    x = _x0(S)
    check = [0, 23, 47]
    ids_l = []
    hL, kept = G.forward(x, keep=check, ids_out=ids_l)
    torch.cuda.synchronize()
    for l in check:
        h_in = kept[l][0].cpu().numpy()
        o = _check_decode_layer(S, l, h_in, kept[l][1].cpu().numpy())
        assert np.array_equal(ids_l[l].cpu().numpy(), o["ids"]), "layer %d ids" % l
        out = torch.empty_like(x)
        G.layer(l, kept[l][0], out)
        torch.cuda.synchronize()
        ok, rel, mx = R.within_tolerance(out.cpu().numpy(), o["out"])
        assert ok, "layer %d: rel %.3e max %.3e" % (l, rel, mx)
        if l == c.n_layers - 1:
            assert np.array_equal(out.cpu().numpy(), hL.cpu().numpy())
    res = _resident_mask(S)
    sel = np.concatenate([res[l][ids_l[l].cpu().numpy().ravel()] for l in range(c.n_layers)])
    assert 0.55 < sel.mean() < 0.9, sel.mean()
    G.close()


def test_small_decode_stack_adaptive_residency():
    """The session routes by another profile than the one the pool was filled
    from.  Usage counters match the routing exactly; periodic swaps keep the
    cache's bookkeeping, the pointer tables and the pool contents consistent
    (every layer bit-identical to a plain device copy of its experts), and the
    adapted pool serves clearly more selections than the static one."""
    from sparse_moe_expert_gemv_amd.stack import AdaptiveResidency
    S = synth.make_stack(name="decode_stack", overrides=DSMALL)
    c = S.cfg
    G = _decode_stack_gpu(S)
    rank_b = synth.stack_profile(1, c.n_layers, c.E)
    for l in range(c.n_layers):
        G.bias[l].copy_(torch.from_numpy(synth.profile_router_bias(rank_b, l, c.E, c.profile_bias)))
    A = AdaptiveResidency(G, decay=0.5, max_swaps=16)
    res0 = A.resident.copy()
    static_hits, adaptive_hits = [], []
    for step in range(24):
        x = torch.from_numpy(synth.bf16_bits_to_f32(synth.gen_x(0, c, layer=0, draw=step))).to(DEV)
        before = G.usage.cpu().numpy().copy()
        ids_l = []
        G.forward(x, ids_out=ids_l)
        torch.cuda.synchronize()
        after = G.usage.cpu().numpy()
        cur = A.resident.copy()
        for l in range(c.n_layers):
            ids = ids_l[l].cpu().numpy().ravel()
            assert np.array_equal(after[l] - before[l], np.bincount(ids, minlength=c.E)), (step, l)
            static_hits.append(res0[ids + l * c.E])
            adaptive_hits.append(cur[ids + l * c.E])
        if step % 2 == 1:
            A.update()
    torch.cuda.synchronize()
    assert A.swaps > 0
    for l in range(c.n_layers):
        hit, _ = G.cache.lookup(l)
        assert hit == [e for e in range(c.E) if A.resident[l * c.E + e]]
    tail = c.n_layers * 8
    s_rate = np.concatenate(static_hits[-tail:]).mean()
    a_rate = np.concatenate(adaptive_hits[-tail:]).mean()
    assert a_rate > s_rate + 0.1, (a_rate, s_rate)
    x = _x0(S)
    for l in range(c.n_layers):
        plain = pack_blobs(torch.from_numpy(S.layer_experts(l)).to(DEV), c.wfmt, c.d, c.f)
        out_a = torch.empty_like(x)
        out_b = torch.empty_like(x)
        G.layer(l, x, out_a)
        G.layer(l, x, out_b, table=pointer_table(plain))
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), "layer %d" % l
    tables = G.tables.cpu().numpy()
    pool_lo = G.pool.data_ptr()
    in_pool = (tables >= pool_lo) & (tables < pool_lo + G.pool.numel())
    assert np.array_equal(in_pool.ravel(), A.resident.astype(bool))
    G.close()
