"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Integer outputs (ids, counts, offsets, permutation,
active list, int8 activations) must match bit for bit; float outputs must meet
rel-L2 <= 2e-3 and max-abs <= 1e-2 * RMS(oracle) (exactly zero where the oracle
is exactly zero).
"""
import numpy as np
import pytest

import oracle
import synth
from tests import refmath as R

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_util import DEV, act_mode, gpu_layer, host, routing_state, x_tensor  # noqa: E402
from sparse_moe_expert_gemv_amd import binding as B  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    oracle.build(force=False)


def _oracle_mode(L):
    return oracle.ACT_Q8 if L.cfg.act_mode == "q8" else oracle.ACT_FLOAT


def check_routing(st, o, E):
    assert np.array_equal(st["ids"], o["ids"]), "expert ids differ"
    assert np.max(np.abs(st["gates"] - o["gates"])) <= 1e-6
    assert np.array_equal(st["counts"], o["counts"])
    assert np.array_equal(st["offsets"], o["offsets"])
    assert np.array_equal(st["sorted_idx"], o["sorted_idx"])
    assert np.array_equal(st["dest"], o["dest"])
    act = np.nonzero(o["counts"])[0]
    assert st["active"][0] == len(act)
    assert np.array_equal(st["active"][1:1 + len(act)], act)


def check_float(got, ref, what):
    ok, rel, mx = R.within_tolerance(got, ref)
    print("[parity] %s: rel-L2 %.3e, max-abs/RMS %.3e" % (what, rel, mx), flush=True)
    assert ok, "%s: rel-L2 %.3e, max-abs/RMS %.3e" % (what, rel, mx)


def run_layer(L, mode=None, x=None, residual=None, tokens=None, y_dtype=None):
    G = gpu_layer(L, mode=mode, y_dtype=y_dtype)
    xt = x_tensor(L, x)
    res_t = None if residual is None else torch.from_numpy(residual).to(DEV)
    out = host(G.forward(xt, residual=res_t))
    torch.cuda.synchronize()
    st = routing_state(G, xt.shape[0])
    xf = L.x_f32() if x is None else (synth.bf16_bits_to_f32(x) if L.cfg.x_dtype == "bf16" else x)
    om = _oracle_mode(L) if mode is None else (oracle.ACT_Q8 if mode == B.MOE_ACT_Q8 else oracle.ACT_FLOAT)
    o = oracle.moe_layer(xf, L.Wr, L.bias, L.experts, L.shared, L.cfg.wfmt, L.cfg.f, L.cfg.k, act_mode=om,
                         residual=residual, tokens=tokens)
    return G, out, st, o


# ------------------------------------------------------------- building blocks

@pytest.mark.parametrize("name", ["tiny", "decode_t1", "skew"])
def test_pack_unpack_roundtrip_bitexact(name):
    L = synth.make_layer(name, overrides={"E": 8} if name != "tiny" else None)
    c = L.cfg
    src = torch.from_numpy(L.experts).to(DEV)
    packed = torch.empty_like(src)
    back = torch.empty_like(src)
    B.moe_pack_experts(src, packed, src.shape[0], c.wfmt, c.d, c.f)
    B.moe_unpack_experts(packed, back, src.shape[0], c.wfmt, c.d, c.f)
    torch.cuda.synchronize()
    assert torch.equal(back, src)
    assert not torch.equal(packed, src)


@pytest.mark.parametrize("name,T", [("tiny", 32), ("decode_t4", 4), ("prefill", 8192), ("tiny", 37)])
def test_quantize_act_bitexact(name, T):
    L = synth.make_layer(name, overrides={"E": 16})
    x = synth.gen_x(0, L.cfg, T=T, draw=3)
    xt = x_tensor(L, x)
    xq = torch.empty((T, L.cfg.d), dtype=torch.int8, device=DEV)
    sx = torch.empty((T, L.cfg.d // 32), dtype=torch.float32, device=DEV)
    B.moe_quantize_act(xt, xq, sx)
    q_ref, s_ref = oracle.quant8(synth.bf16_bits_to_f32(x) if L.cfg.x_dtype == "bf16" else x)
    assert np.array_equal(host(xq), q_ref)
    assert np.array_equal(host(sx).view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("name", ["tiny", "decode_t1", "decode_t4", "skew"])
def test_route_and_permute_bitexact(name):
    L = _layer(name)
    G = gpu_layer(L)
    xt = x_tensor(L)
    T, k, E = L.cfg.T, L.cfg.k, L.cfg.E
    ws = G._ws_for(T)
    B.moe_route(xt, G.Wr, G.bias, k, G.ids[:T], G.gates[:T], ws)
    B.moe_permute(G.ids[:T], E, G.counts, G.offsets, G.sorted_idx[:T * k], G.dest[:T * k], G.active, ws)
    torch.cuda.synchronize()
    ids, gates = oracle.route(L.x_f32(), L.Wr, L.bias, k)
    counts, offsets, sorted_idx, dest = oracle.permute(ids, E)
    check_routing(routing_state(G, T), dict(ids=ids, gates=gates, counts=counts, offsets=offsets,
                                            sorted_idx=sorted_idx, dest=dest), E)


def _route_filter_scratch_overflow(ws, T, E):
    """Overflow count of the large-batch router, read from the library's
    internal scratch layout (256-byte aligned: T E fp32 filter logits, E
    doubles, then the count) to show which pass handled the tokens."""
    up = lambda v: (v + 255) // 256 * 256
    off = up(T * E * 4) + up(E * 8)
    return int(ws[off:off + 4].cpu().numpy().view(np.int32)[0])


@pytest.mark.parametrize("case", ["near_ties", "overflow"])
def test_route_filter_near_ties_and_overflow(case):
    """Large bf16 batches route through the certified bf16 filter and the exact
    refine of the candidates.  Router rows built to defeat the filter: a row
    scaled by (1 + 2^-18) (logits ~1e-6 apart, far inside the filter's error
    bound), an exact duplicate (an exact tie: the lower index wins), a nudged
    copy; and, for the overflow case, 100 identical dominant rows (more than
    64 candidates: the exact full-row pass).  Ids bit-exact, gates within 1e-6."""
    rng = np.random.Generator(np.random.PCG64(5))
    T, d, E, k = 600, 256, 128 if case == "near_ties" else 256, 8
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    Wr = (0.02 * rng.standard_normal((E, d))).astype(np.float32)
    bias = (0.01 * rng.standard_normal(E)).astype(np.float32)
    if case == "near_ties":
        Wr[2] *= 3.0
        Wr[5] = Wr[2] * np.float32(1 + 2.0 ** -18)
        Wr[9] = Wr[2]
        Wr[40] = Wr[2]
        Wr[40, 7] = np.nextafter(Wr[2, 7], np.float32(1.0))
        bias[[5, 9, 40]] = bias[2]
    else:
        Wr[:100] = 4.0 * Wr[0]
        bias[:100] = bias[0]
    xt = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    Wt = torch.from_numpy(Wr).to(DEV)
    bt = torch.from_numpy(bias).to(DEV)
    ws = torch.zeros(B.moe_workspace_size(T, d, 128, E, k, B.MOE_ACT_FLOAT), dtype=torch.uint8, device=DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    gates = torch.empty((T, k), dtype=torch.float32, device=DEV)
    B.moe_route(xt, Wt, bt, k, ids, gates, ws)
    torch.cuda.synchronize()
    n_ovf = _route_filter_scratch_overflow(ws, T, E)
    ref_ids, ref_gates = oracle.route(synth.bf16_bits_to_f32(x), Wr, bias, k)
    got = host(ids)
    assert np.array_equal(got, ref_ids), "ids differ in %d tokens" % int((got != ref_ids).any(axis=1).sum())
    assert np.max(np.abs(host(gates) - ref_gates)) <= 1e-6
    if case == "near_ties":
        tie = np.isin(ref_ids, [2, 5, 9, 40]).sum(axis=1)
        assert (tie == 4).sum() > 50  # the tied group is selected whole, in order, for many tokens
        assert n_ovf == 0
    else:
        # the tied rows lead for about a third of the tokens; every such token
        # has all 100 of them as candidates and takes the full-row pass
        assert (ref_ids[:, 0] == 0).sum() > 100
        assert n_ovf >= (ref_ids[:, 0] == 0).sum()


@pytest.mark.parametrize("T,d,E,k", [(300, 4096, 200, 32), (257, 128, 1024, 1), (1000, 384, 96, 7),
                                     (513, 2048, 1024, 10), (300, 256, 64, 32)])
def test_route_filter_shapes(T, d, E, k):
    """The large-batch router (bf16 filter + exact refine) at shapes that
    exercise its other instances and edges: router rows not a multiple of the
    128-row filter tile, E = 1024 (16 logits per lane), d = 4096 (the wider token
    layout of the refine), k = 32 (the filter's limit) and k = 1, d = 128, a
    token count not a multiple of the 64-token tile.  Ids bit-exact against the
    oracle, gates within 1e-6."""
    rng = np.random.Generator(np.random.PCG64(1000 + T + d + E + k))
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    Wr = (0.02 * rng.standard_normal((E, d))).astype(np.float32)
    bias = (0.01 * rng.standard_normal(E)).astype(np.float32)
    xt = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    ws = torch.empty(B.moe_workspace_size(T, d, 128, E, k, B.MOE_ACT_FLOAT), dtype=torch.uint8, device=DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    gates = torch.empty((T, k), dtype=torch.float32, device=DEV)
    B.moe_route(xt, torch.from_numpy(Wr).to(DEV), torch.from_numpy(bias).to(DEV), k, ids, gates, ws)
    torch.cuda.synchronize()
    ref_ids, ref_gates = oracle.route(synth.bf16_bits_to_f32(x), Wr, bias, k)
    got = host(ids)
    assert np.array_equal(got, ref_ids), "ids differ in %d tokens" % int((got != ref_ids).any(axis=1).sum())
    assert np.max(np.abs(host(gates) - ref_gates)) <= 1e-6


_LAYERS = {}


def _layer(name):
    if name not in _LAYERS:
        _LAYERS[name] = synth.make_layer(name)
    return _LAYERS[name]


# ---------------------------------------------------------------- full layers

@pytest.mark.parametrize("mode", [B.MOE_ACT_FLOAT, B.MOE_ACT_Q8])
def test_layer_tiny(mode):
    """Tiny layer (T=32, d=256, E=64, top-4, f=128, int8 weights), both modes."""
    L = _layer("tiny")
    G, out, st, o = run_layer(L, mode=mode)
    check_routing(st, o, L.cfg.E)
    check_float(out, o["out"], "tiny layer")


@pytest.mark.parametrize("name", ["decode_t1", "decode_t4"])
def test_layer_decode(name):
    """Decode layer: T=1 and the T=4 MTP-verify batch, int4 experts + shared."""
    L = _layer(name)
    G, out, st, o = run_layer(L)
    check_routing(st, o, L.cfg.E)
    check_float(out, o["out"], name)


def test_layer_skew():
    """T=64 with a Zipf(1.1) router bias: a few experts take most tokens."""
    L = _layer("skew")
    G, out, st, o = run_layer(L)
    check_routing(st, o, L.cfg.E)
    assert o["counts"].max() >= 48 and (o["counts"] == 0).sum() > 400  # the skew is real
    check_float(out, o["out"], "skew")


def test_layer_prefill_sampled():
    """8,192-token prefill chunk in int8-activation mode: routing compared in
    full, outputs on a seeded sample of 48 tokens (plus the first and last)."""
    L = _layer("prefill")
    rng = np.random.Generator(np.random.PCG64(11))
    tokens = np.r_[0, np.sort(rng.choice(np.arange(1, L.cfg.T - 1), 48, replace=False)), L.cfg.T - 1]
    G, out, st, o = run_layer(L, tokens=tokens)
    check_routing(st, o, L.cfg.E)
    assert o["counts"].min() > 0  # every expert sees tokens (~160 each)
    check_float(out[tokens], o["out"], "prefill sample")


# ------------------------------------------------------------------ edge cases

def test_ragged_token_counts_and_float_mode_large_batch():
    """T=77 (not a multiple of any tile) on the decode-shaped layer with fewer
    experts, float mode: experts receive >64 tokens, exercising multi-pass
    m-tiles and ragged tails in both projections."""
    L = synth.make_layer("decode_t4", T=77, overrides={"E": 16, "k": 14})
    G, out, st, o = run_layer(L)
    check_routing(st, o, L.cfg.E)
    assert o["counts"].max() > 64
    check_float(out, o["out"], "T=77 float")


@pytest.mark.parametrize("T", [8, 9, 16, 17, 64, 65, 256, 257, 409, 410])
def test_dispatch_boundaries_decode_layer(T):
    """The decode-shaped layer (int4 + shared, float mode) at token counts on
    both sides of every kernel switch: router logits (T <= 8 one wavefront per
    row, <= 256 split-k fp64 MFMA, then tiled fp64 MFMA), single-workgroup
    selection (T <= 64, T*k <= 512), one-workgroup permutation (T*k <= 4096),
    and the FFN families (T <= 16 token-dense int4, <= 64 token-dense, then
    gathered rows).  Routing bit-exact, outputs within tolerance."""
    L = synth.make_layer("decode_t4", T=T)
    G, out, st, o = run_layer(L)
    check_routing(st, o, L.cfg.E)
    check_float(out, o["out"], "decode layer T=%d" % T)


@pytest.mark.parametrize("T", [5, 300])
def test_q8_mode_small_and_mid_batches(T):
    """int8-activation mode on the decode-shaped layer with few tokens per
    expert: tiles of one or two rows, and the shared expert's tile of all T."""
    L = synth.make_layer("decode_t4", T=T, overrides={"act_mode": "q8"})
    G, out, st, o = run_layer(L)
    check_routing(st, o, L.cfg.E)
    check_float(out, o["out"], "q8 T=%d" % T)


@pytest.mark.parametrize("T", [4, 40])
def test_wide_model_dimension(T):
    """d = 4096 (twice the decode layer's width), f = 512, 64 experts, top-8:
    the token-dense kernels with 32 k-tiles per row, the router's split-k and
    four-wavefront row kernels at another width."""
    L = synth.make_layer("decode_t4", T=T, overrides={"d": 4096, "f": 512, "E": 64, "k": 8})
    G, out, st, o = run_layer(L)
    check_routing(st, o, L.cfg.E)
    check_float(out, o["out"], "d=4096 T=%d" % T)


@pytest.mark.parametrize("T,mode", [(3, "float"), (30, "float"), (30, "q8")])
def test_many_experts_large_k(T, mode):
    """E = 1024 experts (sixteen logits per lane in the top-k) with k = 32 (past
    the sixteen group maxima of the threshold search, so the lane-maximum path
    runs) on a narrow layer, both activation modes."""
    L = synth.make_layer("tiny", T=T, overrides={"E": 1024, "k": 32, "act_mode": mode})
    G, out, st, o = run_layer(L)
    check_routing(st, o, L.cfg.E)
    check_float(out, o["out"], "E=1024 k=32 T=%d %s" % (T, mode))


def test_one_expert_takes_every_token_q8():
    """Router bias forces one expert into every token's top-k (count = T = 300
    > one 128-token tile) in int8 mode; ties elsewhere still resolve to the
    lower index."""
    L = synth.make_layer("tiny", T=300, overrides={"act_mode": "q8"})
    L.bias = np.zeros(L.cfg.E, np.float32)
    L.bias[37] = 50.0
    G, out, st, o = run_layer(L, mode=B.MOE_ACT_Q8)
    check_routing(st, o, L.cfg.E)
    assert o["counts"][37] == 300
    check_float(out, o["out"], "one expert q8")


def test_zero_input_gives_exact_zero_both_modes():
    L = _layer("tiny")
    z = np.zeros_like(L.x)
    for mode in (B.MOE_ACT_FLOAT, B.MOE_ACT_Q8):
        G, out, st, o = run_layer(L, mode=mode, x=z)
        check_routing(st, o, L.cfg.E)
        assert np.all(out == 0.0)


def test_residual_and_shared_expert_tiny():
    L = synth.make_layer("tiny", overrides={"has_shared": True})
    res = np.random.Generator(np.random.PCG64(12)).standard_normal((L.cfg.T, L.cfg.d)).astype(np.float32)
    G, out, st, o = run_layer(L, residual=res)
    check_float(out, o["out"], "tiny + shared + residual")


def test_identical_experts_equal_dense_ffn_on_gpu():
    """All routed experts identical: GPU layer output equals the oracle's
    single dense FFN plus shared expert (the layer-level invariant)."""
    L = synth.make_layer("decode_t4", overrides={"E": 32})
    L.experts = np.tile(L.experts[3], (L.cfg.E, 1))
    G = gpu_layer(L)
    out = host(G.forward(x_tensor(L)))
    ref = (oracle.expert_ffn(L.x_f32(), L.experts[3], L.cfg.wfmt, L.cfg.f)
           + oracle.expert_ffn(L.x_f32(), L.shared, L.cfg.wfmt, L.cfg.f))
    check_float(out, ref, "identical experts")


def test_deterministic_two_runs_bit_identical():
    L = _layer("skew")
    G = gpu_layer(L)
    xt = x_tensor(L)
    a = host(G.forward(xt)).copy()
    b = host(G.forward(xt)).copy()
    assert np.array_equal(a, b)


def test_zero_tokens_is_noop():
    L = _layer("tiny")
    G = gpu_layer(L)
    xt = x_tensor(L)[:0]
    out = G.forward(xt)
    torch.cuda.synchronize()
    assert out.shape == (0, L.cfg.d)


@pytest.mark.parametrize("name", ["decode_t4", "tiny"])
def test_graph_replays_match_eager(name):
    """The whole layer captured in a HIP graph: several replays, with eager
    work and synchronisation between them, each bit-identical to the eager
    result."""
    L = _layer(name)
    G = gpu_layer(L)
    xt = x_tensor(L)
    eager = host(G.forward(xt)).copy()
    ids_eager = host(G.ids[:L.cfg.T]).copy()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            G.forward(xt)
    torch.cuda.synchronize()
    for _ in range(3):
        G.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(G.out[:L.cfg.T]), eager)
        assert np.array_equal(host(G.ids[:L.cfg.T]), ids_eager)
        junk = torch.randn(1024, device=DEV).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        del junk


@pytest.mark.parametrize("name,T", [("decode_t4", 4), ("decode_t4", 16), ("tiny", 32), ("skew", 17),
                                    ("skew", 64), ("skew", 256)])
def test_route_permute_fused_equals_separate_calls(name, T):
    """moe_route_permute (selection and grouping in one workgroup for T <= 16)
    equals moe_route followed by moe_permute, also when the workspace starts
    with arbitrary bytes (no state may carry over in it)."""
    L = synth.make_layer(name, T=T)
    G = gpu_layer(L)
    xt = x_tensor(L)
    T, k, E = L.cfg.T, L.cfg.k, L.cfg.E
    ws = G._ws_for(T)
    ws.fill_(0x5A)
    B.moe_route_permute(xt, G.Wr, G.bias, k, G.ids[:T], G.gates[:T], G.counts, G.offsets, G.sorted_idx[:T * k],
                        G.dest[:T * k], G.active, ws)
    torch.cuda.synchronize()
    a = routing_state(G, T)
    a = {kk: v.copy() for kk, v in a.items()}
    B.moe_route(xt, G.Wr, G.bias, k, G.ids[:T], G.gates[:T], ws)
    B.moe_permute(G.ids[:T], E, G.counts, G.offsets, G.sorted_idx[:T * k], G.dest[:T * k], G.active, ws)
    torch.cuda.synchronize()
    b = routing_state(G, T)
    for kk in a:
        if kk == "active":
            n = a[kk][0]
            assert np.array_equal(a[kk][:n + 1], b[kk][:n + 1])
        else:
            assert np.array_equal(a[kk], b[kk]), kk


@pytest.mark.parametrize("T,f", [(1, 768), (2, 768), (4, 768), (8, 768), (4, 256), (3, 512), (5, 1024), (9, 768)])
def test_ffn_combine_entry_matches_separate_calls_and_oracle(T, f):
    """moe_expert_ffn_combine (T <= 8, int4: the down projection and the
    gate-weighted sum in one kernel; T = 9: moe_expert_ffn then moe_combine)
    against moe_expert_ffn with fp32 rows + moe_combine on the same routing,
    with a residual, and against the oracle.  The fused kernel takes exact
    block sums h . (q - 8) and applies the block scale in fp32; the separate
    down kernel rounds each (q - 8) * s to fp16 first (relative 2^-11 per
    weight), so the two agree to that rounding, not bit for bit."""
    L = synth.make_layer("decode_t4", T=T, overrides={"f": f})
    res = np.random.Generator(np.random.PCG64(21)).standard_normal((T, L.cfg.d)).astype(np.float32)
    G, out, st, o = run_layer(L, residual=res, y_dtype=torch.float32)
    check_routing(st, o, L.cfg.E)
    check_float(out, o["out"], "ffn + combine entry, T=%d f=%d" % (T, f))
    G.fuse_combine = False
    ref = host(G.forward(x_tensor(L), residual=torch.from_numpy(res).to(DEV)))
    torch.cuda.synchronize()
    ok, rel, mx = R.within_tolerance(out, ref, rel=2e-4, maxabs_frac=1e-3)
    assert ok, "fused vs separate: rel-L2 %.3e, max-abs/RMS %.3e" % (rel, mx)


@pytest.mark.parametrize("T,f,select_in_ffn", [(1, 768, True), (2, 768, True), (4, 768, True), (8, 768, True),
                                                (3, 512, True), (4, 768, False), (1, 256, False), (8, 1024, True)])
def test_ffn_combine_slots_equals_grouped_path_and_oracle(T, f, select_in_ffn):
    """The by-slot decode paths (no grouping: every routed slot its own work
    item), moe_route_ffn_combine_slots (the gate/up launch selects its experts)
    and moe_route + moe_expert_ffn_combine_slots, give the same ids, gates and
    layer output, bit for bit, as moe_route_permute + moe_expert_ffn_combine,
    and meet the float bar against the oracle."""
    L = synth.make_layer("decode_t4", T=T, overrides={"f": f})
    c = L.cfg
    res = np.random.Generator(np.random.PCG64(23)).standard_normal((T, c.d)).astype(np.float32)
    G, out, st, o = run_layer(L, residual=res)
    G2 = gpu_layer(L)
    G2.by_slot = True
    G2.select_in_ffn = select_in_ffn
    G2.ids.fill_(-5)
    G2.gates.fill_(-1.0)
    out2 = host(G2.forward(x_tensor(L), residual=torch.from_numpy(res).to(DEV)))
    torch.cuda.synchronize()
    assert np.array_equal(host(G2.ids[:T]), st["ids"])
    assert np.array_equal(host(G2.gates[:T]).view(np.uint32), st["gates"].view(np.uint32))
    assert np.array_equal(out2, out)
    check_float(out2, o["out"], "by-slot decode layer, T=%d f=%d" % (T, f))


@pytest.mark.parametrize("select_in_ffn", [True, False])
def test_ffn_combine_slots_many_experts_large_k(select_in_ffn):
    """By slot with E = 1024 and k = 32 (two tokens): the selection inside the
    gate/up launch takes its 16-values-per-lane instance and the top-k path
    for k > 16; ids, gates and output bit for bit as the grouped path."""
    L = synth.make_layer("decode_t4", T=2, overrides={"E": 1024, "k": 32})
    c = L.cfg
    G, out, st, o = run_layer(L)
    check_routing(st, o, c.E)
    G2 = gpu_layer(L)
    G2.by_slot = True
    G2.select_in_ffn = select_in_ffn
    out2 = host(G2.forward(x_tensor(L)))
    torch.cuda.synchronize()
    assert np.array_equal(host(G2.ids[:c.T]), st["ids"])
    assert np.array_equal(host(G2.gates[:c.T]).view(np.uint32), st["gates"].view(np.uint32))
    assert np.array_equal(out2, out)
    check_float(out2, o["out"], "by-slot decode layer, E=1024 k=32")


def test_ffn_combine_slots_phase1_then_whole_call():
    """Phase 1 of the by-slot entry (gate/up alone) followed by the whole call
    on the same workspace gives the whole call's output (the phase leaves the
    workspace in a state the whole call does not depend on)."""
    L = synth.make_layer("decode_t4", T=4)
    c = L.cfg
    G = gpu_layer(L)
    G.by_slot = True
    xt = x_tensor(L)
    ref = host(G.forward(xt)).copy()
    common = dict(T=c.T, d=c.d, f=c.f, E=c.E, k=c.k, wfmt=c.wfmt, act_mode=G.act_mode, expert_ptrs=G.expert_ptrs,
                  ws=G._ws_for(c.T), ids=G.ids[:c.T], gates=G.gates[:c.T], out=G.out[:c.T], x=xt,
                  shared_blob=G.shared)
    G.out.zero_()
    B.moe_expert_ffn_combine_slots(phase=1, **common)
    torch.cuda.synchronize()
    assert not np.any(host(G.out[:c.T]))  # phase 1 writes no output
    B.moe_expert_ffn_combine_slots(**common)
    torch.cuda.synchronize()
    assert np.array_equal(host(G.out[:c.T]), ref)
    # moe_route_ffn_combine_slots: phase 1 (gate/up alone, logits left in the
    # workspace by the whole call) selects the same ids and gates again
    ids0, gates0 = host(G.ids[:c.T]).copy(), host(G.gates[:c.T]).copy()
    G.ids.fill_(-3)
    G.gates.fill_(0.0)
    G.out.zero_()
    B.moe_route_ffn_combine_slots(phase=1, Wr=G.Wr, bias=G.bias, **common)
    torch.cuda.synchronize()
    assert np.array_equal(host(G.ids[:c.T]), ids0)
    assert np.array_equal(host(G.gates[:c.T]).view(np.uint32), gates0.view(np.uint32))
    assert not np.any(host(G.out[:c.T]))


def test_ffn_combine_entry_skips_ids_outside_range():
    """An id outside [0, E) contributes nothing: the output equals the one with
    that slot's gate set to zero (bit for bit: gate 0 adds an exact zero)."""
    L = synth.make_layer("decode_t4", T=4)
    c = L.cfg
    G = gpu_layer(L, y_dtype=torch.float32)
    xt = x_tensor(L)
    T, k, E, n = c.T, c.k, c.E, c.T * c.k
    G.forward(xt)
    torch.cuda.synchronize()
    ids0, gates0 = G.ids[:T].clone(), G.gates[:T].clone()

    def run(ids, gates):
        ws = G._ws_for(T)
        B.moe_permute(ids, E, G.counts, G.offsets, G.sorted_idx[:n], G.dest[:n], G.active, ws)
        out = torch.empty((T, c.d), dtype=torch.float32, device=DEV)
        B.moe_expert_ffn_combine(T=T, d=c.d, f=c.f, E=E, k=k, wfmt=c.wfmt, act_mode=G.act_mode,
                                 expert_ptrs=G.expert_ptrs, counts=G.counts, offsets=G.offsets,
                                 sorted_idx=G.sorted_idx[:n], active=G.active, y_perm=G.y_perm[:n], ws=ws,
                                 shared_blob=G.shared, y_shared=G.y_shared[:T], x=xt, ids=ids, dest=G.dest[:n],
                                 gates=gates, out=out)
        torch.cuda.synchronize()
        return host(out)

    bad = ids0.clone()
    bad[1, 3] = -1
    bad[2, 0] = E
    zg = gates0.clone()
    zg[1, 3] = 0.0
    zg[2, 0] = 0.0
    assert np.array_equal(run(bad, gates0), run(ids0, zg))


@pytest.mark.parametrize("name", ["decode_t4", "tiny"])
def test_ffn_phases_equal_whole_call(name):
    """moe_expert_ffn with phase 1 (gate/up) then phase 2 (down) on the same
    workspace gives bit-identical outputs to phase 0."""
    L = _layer(name)
    G = gpu_layer(L)
    G.fuse_combine = False  # the separate calls leave y_perm filled
    xt = x_tensor(L)
    T, k = L.cfg.T, L.cfg.k
    G.forward(xt)
    torch.cuda.synchronize()
    y0 = host(G.y_perm[:T * k]).copy()
    ys0 = host(G.y_shared[:T]).copy() if G.shared is not None else None
    G.y_perm.zero_()
    G.y_shared.zero_()
    common = dict(T=T, d=L.cfg.d, f=L.cfg.f, E=L.cfg.E, k=k, wfmt=L.cfg.wfmt, act_mode=G.act_mode,
                  expert_ptrs=G.expert_ptrs, counts=G.counts, offsets=G.offsets, sorted_idx=G.sorted_idx[:T * k],
                  active=G.active, y_perm=G.y_perm[:T * k], ws=G._ws_for(T), shared_blob=G.shared,
                  y_shared=G.y_shared[:T] if G.shared is not None else None, x=xt)
    B.moe_expert_ffn(phase=1, **common)
    B.moe_expert_ffn(phase=2, **common)
    torch.cuda.synchronize()
    assert np.array_equal(host(G.y_perm[:T * k]), y0)
    if ys0 is not None:
        assert np.array_equal(host(G.y_shared[:T]), ys0)


@pytest.mark.parametrize("name,T", [("decode_t4", 4), ("tiny", 48), ("skew", 40)])
def test_duplicate_expert_ids_through_permute_ffn_combine(name, T):
    """Ids handed to moe_permute directly, every token listing expert 3 twice
    (each time with its own gate): the permutation keeps both slots (stable,
    bit-exact against the oracle) and the float-mode FFN writes the expert's
    output to both rows.  Expert 3 then holds 2T rows, more than 64 for T >= 33,
    which takes the moderate-batch kernels through their multi-pass paths."""
    L = synth.make_layer(name, T=T)
    c = L.cfg
    G = gpu_layer(L, mode=B.MOE_ACT_FLOAT)
    xt = x_tensor(L)
    k, E = c.k, c.E
    rng = np.random.Generator(np.random.PCG64(77))
    ids = np.empty((T, k), np.int32)
    others = np.setdiff1d(np.arange(E), [3])
    for t in range(T):
        row = np.concatenate([[3, 3], rng.choice(others, size=k - 2, replace=False)]).astype(np.int32)
        rng.shuffle(row)
        ids[t] = row
    gates = rng.random((T, k)).astype(np.float32) + 0.1
    gates /= gates.sum(axis=1, keepdims=True)
    n = T * k
    G.ids[:T].copy_(torch.from_numpy(ids).to(DEV))
    G.gates[:T].copy_(torch.from_numpy(gates).to(DEV))
    ws = G._ws_for(T)
    B.moe_permute(G.ids[:T], E, G.counts, G.offsets, G.sorted_idx[:n], G.dest[:n], G.active, ws)
    B.moe_expert_ffn(x=xt, T=T, d=c.d, f=c.f, E=E, k=k, wfmt=c.wfmt, act_mode=B.MOE_ACT_FLOAT,
                     expert_ptrs=G.expert_ptrs, counts=G.counts, offsets=G.offsets, sorted_idx=G.sorted_idx[:n],
                     active=G.active, y_perm=G.y_perm[:n], ws=ws, shared_blob=G.shared,
                     y_shared=G.y_shared[:T] if G.shared is not None else None)
    B.moe_combine(G.y_perm[:n], G.dest[:n], G.gates[:T], G.y_shared[:T] if G.shared is not None else None, None,
                  G.out[:T])
    torch.cuda.synchronize()
    st = routing_state(G, T)
    counts, offsets, sorted_idx, dest = oracle.permute(ids, E)
    assert counts[3] == 2 * T
    assert np.array_equal(st["counts"], counts)
    assert np.array_equal(st["offsets"], offsets)
    assert np.array_equal(st["sorted_idx"], sorted_idx)
    assert np.array_equal(st["dest"], dest)
    xf = synth.bf16_bits_to_f32(L.x) if c.x_dtype == "bf16" else L.x
    ref = np.zeros((T, c.d))
    for e in np.unique(ids):
        tt, jj = np.nonzero(ids == e)
        ye = oracle.expert_ffn(xf[tt], L.experts[e], c.wfmt, c.f, oracle.ACT_FLOAT)
        np.add.at(ref, tt, gates[tt, jj][:, None].astype(np.float64) * ye)  # a token may list e twice
    if L.shared is not None:
        ref += oracle.expert_ffn(xf, L.shared, c.wfmt, c.f, oracle.ACT_FLOAT)
    check_float(host(G.out[:T]), ref, "%s duplicate ids" % name)


@pytest.mark.parametrize("d", [132, 136, 2048])
def test_combine_fp16_rows_equal_fp32_rows(d):
    """moe_combine on fp16 expert rows (eight outputs per thread when d % 8 == 0,
    four otherwise) equals, bit for bit, moe_combine on the same rows widened
    to fp32: the same products summed in the same order."""
    rng = np.random.default_rng(d)
    T, k = 37, 5
    n = T * k
    y16 = torch.from_numpy(rng.standard_normal((n, d)).astype(np.float16)).cuda()
    y32 = y16.float()
    dest = torch.from_numpy(rng.permutation(n).astype(np.int32)).cuda()
    gates = torch.from_numpy(rng.random((T, k)).astype(np.float32)).cuda()
    ysh = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).cuda()
    res = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).cuda()
    for sh, r in ((None, None), (ysh, res)):
        a = torch.empty((T, d), dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        B.moe_combine(y16, dest, gates, sh, r, a)
        B.moe_combine(y32, dest, gates, sh, r, b)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
