"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what it pins and which plausible mistake would make it fail.
All run on the CPU (not marked gpu).
"""
import math

import numpy as np
import pytest

import oracle
import synth
from tests import refmath as R


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


# ---------------------------------------------------------------- formats ----

def test_half_decoder_matches_ieee_binary16_for_all_patterns():
    """binary16 decode vs numpy's IEEE float16 for all 65,536 bit patterns
    (catches a wrong exponent bias, a lost subnormal path or sign)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("wfmt", [synth.WFMT_I4B32, synth.WFMT_I8B32])
def test_dequant_closed_form_blob(wfmt):
    """Hand-built blob with q = known pattern and power-of-two scales: the
    oracle's Wg/Wu/Wd must equal q * s exactly, in the right matrix and
    orientation (catches nibble order, offset, scale indexing, matrix order)."""
    d, f = 64, 32
    qmin, qmax = (-8, 7) if wfmt == synth.WFMT_I4B32 else (-127, 127)
    span = qmax - qmin + 1

    def pattern(R_, K, salt):
        r = np.arange(R_)[:, None]
        c = np.arange(K)[None, :]
        return ((r * 7 + c * 3 + salt) % span + qmin).astype(np.int8)

    def pscale(R_, K, salt):
        r = np.arange(R_)[:, None]
        b = np.arange(K // 32)[None, :]
        return (2.0 ** -((r + 2 * b + salt) % 5)).astype(np.float16)

    qg, qu, qd = pattern(f, d, 0), pattern(f, d, 5), pattern(d, f, 11)
    sg, su, sd = pscale(f, d, 0), pscale(f, d, 1), pscale(d, f, 2)
    blob = synth.build_blob(qg, sg, qu, su, qd, sd, wfmt)
    assert blob.size == oracle.expert_bytes(wfmt, d, f) == synth.expert_bytes(wfmt, d, f)
    wg, wu, wd = oracle.dequant_expert(blob, wfmt, d, f)
    for w, q, s in ((wg, qg, sg), (wu, qu, su), (wd, qd, sd)):
        ref = q.astype(np.float64) * np.repeat(s.astype(np.float64), 32, axis=1)
        assert np.array_equal(w, ref)


@pytest.mark.parametrize("wfmt", [synth.WFMT_I4B32, synth.WFMT_I8B32])
def test_dequant_generator_roundtrip_error_bound(wfmt):
    """Generated N(0,0.02) weights: the oracle's dequantised value is within
    half a quantisation step of the drawn weight (catches a wrong scale or a
    sign/offset error in the decoder)."""
    d, f = 256, 128
    rng = np.random.Generator(np.random.PCG64(7))
    wg = rng.standard_normal((f, d), dtype=np.float32) * np.float32(0.02)
    wu = rng.standard_normal((f, d), dtype=np.float32) * np.float32(0.02)
    wd = rng.standard_normal((d, f), dtype=np.float32) * np.float32(0.02)
    parts = [synth.quantize_rows_b32(w, wfmt) for w in (wg, wu, wd)]
    blob = synth.build_blob(parts[0][0], parts[0][1], parts[1][0], parts[1][1], parts[2][0], parts[2][1], wfmt)
    for w, (q, s), got in zip((wg, wu, wd), parts, oracle.dequant_expert(blob, wfmt, d, f)):
        step = np.repeat(s.astype(np.float64), 32, axis=1)
        assert np.all(np.abs(got - w.astype(np.float64)) <= 0.5 * step * (1 + 1e-3) + 1e-12)
        # the block maximum is reproduced to within the fp16 rounding of its scale
        assert np.allclose(np.abs(got).reshape(w.shape[0], -1, 32).max(axis=2),
                           np.abs(w).reshape(w.shape[0], -1, 32).max(axis=2), rtol=2e-3, atol=0)


# ----------------------------------------------------------------- router ----

def test_router_ids_match_exact_rational_ranking_tiny():
    """Tiny layer (T=32, d=256, E=64, k=4): ids equal the ranking of the exact
    logits (integer arithmetic on the dyadic inputs), including order within
    the top-k (catches a sign error, wrong operand, tie-break or slot order)."""
    L = synth.make_layer("tiny")
    ids, gates, logits = oracle.route(L.x_f32(), L.Wr, L.bias, L.cfg.k, return_logits=True)
    z = R.exact_logits(L.x_f32(), L.Wr, L.bias)
    for t in range(L.cfg.T):
        assert list(ids[t]) == R.exact_topk(z[t], L.cfg.k)
        # the oracle's double logits agree with the exact ones to double rounding
        zf = R.logits_to_float(z[t])
        assert np.max(np.abs(logits[t] - zf)) <= 1e-13 * (1 + np.max(np.abs(zf)))


def test_router_ids_exact_ranking_decode_shape_with_bias():
    """Decode-shaped router (d=2048, E=512, k=10) with the Zipf bias of the
    skewed workload on 3 tokens: exact ranking again (catches a bias added
    after selection or with the wrong sign)."""
    L = synth.make_layer("skew", overrides={"E": 512})
    x = L.x_f32()[:3]
    ids, _ = oracle.route(x, L.Wr, L.bias, 10)
    z = R.exact_logits(x, L.Wr, L.bias)
    for t in range(3):
        assert list(ids[t]) == R.exact_topk(z[t], 10)


def test_router_zero_input_all_ties_lower_index_and_uniform_gates():
    """Zero hidden state: every logit ties at 0, so ids are 0..k-1 and the
    gates are exactly 1/k."""
    E, d, k = 16, 64, 5
    Wr = np.random.Generator(np.random.PCG64(1)).standard_normal((E, d), dtype=np.float32)
    ids, gates = oracle.route(np.zeros((2, d), np.float32), Wr, None, k)
    assert np.array_equal(ids, np.tile(np.arange(k, dtype=np.int32), (2, 1)))
    assert np.all(gates == np.float32(1.0 / k))


def test_router_duplicate_rows_tie_goes_to_lower_index():
    """Two identical router rows that both win: the lower expert index takes
    slot 0, the higher slot 1, with equal gates."""
    E, d = 8, 32
    rng = np.random.Generator(np.random.PCG64(2))
    Wr = rng.standard_normal((E, d), dtype=np.float32) * np.float32(0.01)
    x = np.ones((1, d), np.float32)
    Wr[6] = 1.0
    Wr[3] = 1.0
    ids, gates = oracle.route(x, Wr, None, 3)
    assert list(ids[0][:2]) == [3, 6]
    assert gates[0][0] == gates[0][1]


def test_gates_closed_forms():
    """k=1 gives gate 1; k=2 gives the logistic of the logit gap; k=E gives
    the full softmax; gates always sum to 1 (catches a missing max-shift,
    wrong normalisation or softmax over the wrong set)."""
    L = synth.make_layer("tiny")
    x = L.x_f32()[:6]
    z = R.exact_logits(x, L.Wr, None)
    ids1, g1 = oracle.route(x, L.Wr, None, 1)
    assert np.all(g1 == 1.0)
    ids2, g2 = oracle.route(x, L.Wr, None, 2)
    idsE, gE = oracle.route(x, L.Wr, None, L.cfg.E)
    for t in range(6):
        zf = R.logits_to_float(z[t])
        a, b = ids2[t]
        assert abs(g2[t][0] - 1.0 / (1.0 + math.exp(zf[b] - zf[a]))) <= 1e-7
        full = np.exp(zf - zf.max())
        full /= full.sum()
        assert np.allclose(gE[t], full[idsE[t]], rtol=1e-6, atol=1e-9)
        assert abs(float(np.sum(g2[t], dtype=np.float64)) - 1.0) <= 1e-6
        # renormalised top-k of the full softmax equals the top-k softmax
        ids4, g4 = oracle.route(x[t:t + 1], L.Wr, None, 4)
        sel = full[ids4[0]]
        assert np.allclose(g4[0], sel / sel.sum(), rtol=1e-6, atol=1e-9)


# ---------------------------------------------------------------- permute ----

@pytest.mark.parametrize("case", ["random", "one_expert", "sparse", "empty"])
def test_permutation_equals_stable_sort(case):
    """counts/offsets/sorted_idx/dest vs Python's stable sort of the routing
    slots by (expert, slot) (catches instability, off-by-one offsets, a
    transposed dest)."""
    rng = np.random.Generator(np.random.PCG64(3))
    E, T, k = 40, 37, 6
    if case == "random":
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    elif case == "one_expert":
        ids = np.stack([np.r_[7, rng.choice(np.r_[0:7, 8:E], k - 1, replace=False)] for _ in range(T)]).astype(np.int32)
    elif case == "sparse":
        ids = np.stack([rng.choice(np.array([1, 5, 9, 13, 17, 33]), k, replace=False) for _ in range(T)]).astype(np.int32)
    else:
        T = 0
        ids = np.zeros((0, k), np.int32)
    counts, offsets, sorted_idx, dest = oracle.permute(ids, E)
    flat = ids.reshape(-1)
    ref = sorted(range(T * k), key=lambda f: (flat[f], f))
    assert list(sorted_idx) == ref
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts) and offsets[-1] == T * k
    assert np.array_equal(dest[sorted_idx], np.arange(T * k))


# ---------------------------------------------------------------- quant8 -----

def test_quant8_rounding_ties_to_even_and_bounds():
    """Block with amax 127 has scale exactly 1: x = n + 1/2 rounds to even;
    |x - s q| <= s/2; the amax element maps to +-127; a zero block gives
    scale 0 and q = 0 (catches round-half-away, wrong scale, no clamp)."""
    x = np.zeros((1, 64), np.float32)
    x[0, :8] = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5]
    q, s = oracle.quant8(x)
    assert s[0, 0] == np.float32(1.0) and s[0, 1] == 0.0
    assert list(q[0, :8]) == [127, 2, 4, -2, -4, 0, 2, 0]
    assert np.all(q[0, 32:] == 0)
    rng = np.random.Generator(np.random.PCG64(4))
    y = (rng.standard_normal((8, 256)) * 3).astype(np.float32)
    q, s = oracle.quant8(y)
    sr = np.repeat(s, 32, axis=1).astype(np.float64)
    assert np.all(np.abs(y - sr * q) <= sr / 2 + 1e-12)
    blk = np.abs(y).reshape(8, -1, 32)
    am = blk.argmax(axis=2)
    qb = q.reshape(8, -1, 32)
    assert np.all(np.abs(np.take_along_axis(qb, am[:, :, None], 2)) == 127)
    assert np.all(s == (blk.max(axis=2) / np.float32(127.0)).astype(np.float32))


# -------------------------------------------------------------------- FFN ----

def _identity_expert(d, f, wfmt, perm_g, perm_d, up_scale):
    """Expert with Wg = permutation rows, Wu = up_scale * I, Wd = permutation."""
    qg = np.zeros((f, d), np.int8)
    qu = np.zeros((f, d), np.int8)
    qd = np.zeros((d, f), np.int8)
    for n in range(f):
        qg[n, perm_g[n]] = 1
        qu[n, n] = 1
    for o in range(f):
        qd[o, perm_d[o]] = 1
    one = np.ones((f, d // 32), np.float16)
    sd = np.ones((d, f // 32), np.float16)
    su = (one.astype(np.float32) * up_scale).astype(np.float16)
    return synth.build_blob(qg, one, qu, su, qd, sd, wfmt)


@pytest.mark.parametrize("wfmt", [synth.WFMT_I4B32, synth.WFMT_I8B32])
def test_ffn_closed_form_permutation_expert(wfmt):
    """y[o] = silu(x[pg[pd[o]]]) * 2 x[pd[o]] for o < f, 0 beyond -- a
    transposed matrix, swapped gate/up or a wrong activation fails."""
    d, f = 64, 32
    rng = np.random.Generator(np.random.PCG64(5))
    pg = rng.permutation(f)
    pd = rng.permutation(f)
    blob = _identity_expert(d, f, wfmt, pg, pd, 2.0)
    x = rng.standard_normal((3, d)).astype(np.float32)
    y = oracle.expert_ffn(x, blob, wfmt, f)
    for m in range(3):
        for o in range(d):
            if o < f:
                n = pd[o]
                gval = float(x[m, pg[n]])
                ref = gval / (1.0 + math.exp(-gval)) * 2.0 * float(x[m, n])
            else:
                ref = 0.0
            assert abs(y[m, o] - ref) <= 1e-14 * (1 + abs(ref))


def test_ffn_q8_lossless_case_matches_float_gate_up():
    """x_i = q_i / 16 with a +-127 in every block gives scale 1/16 exactly, so
    Q8 quantisation is lossless and the gate/up projections equal the float
    mode's (links the two modes; catches a wrong activation scale)."""
    L = synth.make_layer("tiny")
    d, f = L.cfg.d, L.cfg.f
    rng = np.random.Generator(np.random.PCG64(6))
    q = rng.integers(-127, 128, size=(4, d))
    q[:, ::32] = 127
    x = (q / 16.0).astype(np.float32)
    for e in (0, 17):
        _, g0, u0 = oracle.expert_ffn(x, L.experts[e], L.cfg.wfmt, f, oracle.ACT_FLOAT, return_gu=True)
        _, g1, u1 = oracle.expert_ffn(x, L.experts[e], L.cfg.wfmt, f, oracle.ACT_Q8, return_gu=True)
        assert np.allclose(g1, g0, rtol=1e-12, atol=1e-12)
        assert np.allclose(u1, u0, rtol=1e-12, atol=1e-12)


def test_ffn_q8_error_bound_vs_float():
    """Q8 output stays within the quantisation error expected from int8
    activations (a few 1e-2 relative) of the float output, and is not equal
    to it (catches Q8 silently falling back to float, or a garbage path)."""
    L = synth.make_layer("tiny")
    x = L.x_f32()[:8]
    y0 = oracle.expert_ffn(x, L.experts[3], L.cfg.wfmt, L.cfg.f, oracle.ACT_FLOAT)
    y1 = oracle.expert_ffn(x, L.experts[3], L.cfg.wfmt, L.cfg.f, oracle.ACT_Q8)
    r = R.rel_l2(y1, y0)
    assert 1e-4 < r < 3e-2


@pytest.mark.parametrize("wfmt", [synth.WFMT_I4B32, synth.WFMT_I8B32])
def test_ffn_q8_matches_independent_int8_brute_force(wfmt):
    """Int8-activation expert vs the numpy brute force of tests/refmath.py
    (its own quantiser of x and of h, exact int64 block sums times both block
    scales, h rounded to fp32 before requantisation): gate, up and output
    agree to 1e-12 relative.  Catches an error in the h block scale or codes,
    g/u rounded to fp32 before SwiGLU, a wrong scale or block in the int8 down
    projection, and a dropped block element."""
    d, f = 256, 128
    rng = np.random.Generator(np.random.PCG64(11))
    x = rng.standard_normal((24, d)).astype(np.float32)
    x[3] = 0.0                      # an all-zero row: every scale 0, output exactly 0
    x[5, 64:96] = 0.0               # one all-zero block inside a row
    for e in range(3):
        blob = synth.gen_expert_blob(np.random.Generator(np.random.PCG64(100 + e)), d, f, wfmt)
        y, g, u = oracle.expert_ffn(x, blob, wfmt, f, oracle.ACT_Q8, return_gu=True)
        yr, gr, ur = R.q8_ffn(x, blob, wfmt, d, f)
        for got, ref in ((g, gr), (u, ur), (y, yr)):
            assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
        assert np.all(y[3] == 0.0)


@pytest.mark.parametrize("shared", [False, True])
def test_layer_q8_matches_dense_masked_brute_force(shared):
    """Whole tiny layer in int8-activation mode vs the dense masked brute
    force with the int8 expert of tests/refmath.py (ids exact, output to the
    fp32 rounding of the stored result)."""
    L = synth.make_layer("tiny", overrides={"has_shared": shared})
    x = L.x_f32()
    res = np.random.Generator(np.random.PCG64(9)).standard_normal(x.shape).astype(np.float32) if shared else None
    o = oracle.moe_layer(x, L.Wr, L.bias, L.experts, L.shared, L.cfg.wfmt, L.cfg.f, L.cfg.k,
                         act_mode=oracle.ACT_Q8, residual=res)
    ids, ref = R.brute_force_layer_q8(x, L.Wr, L.bias, L.experts, L.shared, L.cfg.wfmt, L.cfg.d, L.cfg.f,
                                      L.cfg.k, residual=res)
    assert np.array_equal(o["ids"], ids)
    assert np.max(np.abs(o["out"] - ref)) <= 1e-6 * np.max(np.abs(ref))


def test_int8_brute_force_quantiser_pins():
    """The brute force's own quantiser against hand values (so the two int8
    implementations cannot share a mistake): scale 1 for a block whose amax
    is 127, ties to even, zero block, clamp never exceeded."""
    x = np.zeros((1, 64), np.float32)
    x[0, :8] = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5]
    q, s = R.quant8_blocks(x)
    assert s[0, 0] == np.float32(1.0) and s[0, 1] == 0.0
    assert list(q[0, :8]) == [127, 2, 4, -2, -4, 0, 2, 0] and np.all(q[0, 32:] == 0)
    # block sums times scales: one block of ones against a row of twos, scales 0.5 and 0.25
    qa = np.ones((1, 32), np.int64)
    qw = np.full((1, 32), 2, np.int64)
    assert R.block_scaled_products(qa, np.array([[0.5]]), qw, np.array([[0.25]]))[0, 0] == 0.5 * 0.25 * 64


# ------------------------------------------------------------------ layer ----

@pytest.mark.parametrize("shared", [False, True])
def test_layer_matches_dense_masked_brute_force(shared):
    """Whole tiny layer vs dense masked float64 brute force (all 64 experts on
    all tokens, masked by the exact top-4 and its gates), with and without a
    shared expert and a residual (catches a wrong gather/scatter, gate
    applied to the wrong slot, missing shared or residual term)."""
    L = synth.make_layer("tiny", overrides={"has_shared": shared})
    x = L.x_f32()
    res = np.random.Generator(np.random.PCG64(8)).standard_normal(x.shape).astype(np.float32) if shared else None
    o = oracle.moe_layer(x, L.Wr, L.bias, L.experts, L.shared, L.cfg.wfmt, L.cfg.f, L.cfg.k, residual=res)
    ids, ref = R.brute_force_layer(x, L.Wr, L.bias, L.experts, L.shared, L.cfg.wfmt, L.cfg.d, L.cfg.f,
                                   L.cfg.k, residual=res)
    assert np.array_equal(o["ids"], ids)
    assert np.allclose(o["out"], ref, rtol=1e-6, atol=1e-6 * np.sqrt(np.mean(ref ** 2)))


def test_layer_identical_experts_reduce_to_dense_ffn():
    """All routed experts identical: gates sum to 1, so the layer equals one
    dense FFN plus the shared expert."""
    L = synth.make_layer("tiny", overrides={"has_shared": True})
    x = L.x_f32()
    same = np.tile(L.experts[5], (L.cfg.E, 1))
    o = oracle.moe_layer(x, L.Wr, None, same, L.shared, L.cfg.wfmt, L.cfg.f, L.cfg.k)
    ref = (oracle.expert_ffn(x, L.experts[5], L.cfg.wfmt, L.cfg.f)
           + oracle.expert_ffn(x, L.shared, L.cfg.wfmt, L.cfg.f))
    assert R.rel_l2(o["out"], ref) < 1e-6


def test_layer_zero_input_gives_exact_zero_and_residual_passthrough():
    L = synth.make_layer("tiny", overrides={"has_shared": True})
    x = np.zeros_like(L.x_f32())
    for mode in (oracle.ACT_FLOAT, oracle.ACT_Q8):
        o = oracle.moe_layer(x, L.Wr, None, L.experts, L.shared, L.cfg.wfmt, L.cfg.f, L.cfg.k, act_mode=mode)
        assert np.all(o["out"] == 0.0)
        assert np.array_equal(o["ids"][0], np.arange(L.cfg.k))
    res = np.arange(x.size, dtype=np.float32).reshape(x.shape)
    o = oracle.moe_layer(x, L.Wr, None, L.experts, L.shared, L.cfg.wfmt, L.cfg.f, L.cfg.k, residual=res)
    assert np.array_equal(o["out"], res)


def test_layer_single_expert_top1_is_dense_ffn():
    """E=1, k=1: the layer is one dense FFN with gate 1."""
    L = synth.make_layer("tiny")
    x = L.x_f32()
    o = oracle.moe_layer(x, L.Wr[:1], None, L.experts[:1], None, L.cfg.wfmt, L.cfg.f, 1)
    ref = R.dense_ffn(x, R.decode_blob(L.experts[0], L.cfg.wfmt, L.cfg.d, L.cfg.f))
    assert np.allclose(o["out"], ref, rtol=1e-6, atol=1e-7)


def test_layer_linear_in_down_projection_scale():
    """Doubling every routed expert's down-projection scales (exact in fp16)
    doubles the routed contribution and leaves ids unchanged."""
    L = synth.make_layer("tiny")
    d, f, wfmt = L.cfg.d, L.cfg.f, L.cfg.wfmt
    n = d * f
    sd_off = 3 * n + 2 * (n // 32) * 2
    doubled = L.experts.copy()
    s = doubled[:, sd_off:].view(np.float16)
    doubled[:, sd_off:] = (s.astype(np.float32) * 2).astype(np.float16).view(np.uint8)
    x = L.x_f32()
    a = oracle.moe_layer(x, L.Wr, None, L.experts, None, wfmt, f, L.cfg.k)
    b = oracle.moe_layer(x, L.Wr, None, doubled, None, wfmt, f, L.cfg.k)
    assert np.array_equal(a["ids"], b["ids"])
    assert np.allclose(b["out"], 2 * a["out"], rtol=1e-6, atol=1e-7)


def test_layer_token_subset_matches_full():
    """Outputs for a token subset equal the same rows of the full output."""
    L = synth.make_layer("tiny", overrides={"has_shared": True})
    x = L.x_f32()
    full = oracle.moe_layer(x, L.Wr, None, L.experts, L.shared, L.cfg.wfmt, L.cfg.f, L.cfg.k)
    sub = [31, 0, 7]
    part = oracle.moe_layer(x, L.Wr, None, L.experts, L.shared, L.cfg.wfmt, L.cfg.f, L.cfg.k, tokens=sub)
    assert np.array_equal(part["out"], full["out"][sub])


def test_rmsnorm_closed_forms():
    """Constant row c: output is c / sqrt(c^2 + eps); output rows have mean
    square 1 up to eps; scale invariance; zero row stays zero (catches a
    missing square root, mean over the wrong axis, eps outside the root)."""
    d = 64
    x = np.zeros((4, d), np.float32)
    x[0] = 3.0
    x[1] = np.arange(d, dtype=np.float32) - 20
    x[2] = 1e3 * x[1]
    out = oracle.rmsnorm(x, eps=1e-6)
    assert abs(out[0, 0] - 3.0 / math.sqrt(9.0 + 1e-6)) < 1e-7
    ms = (x[1].astype(np.float64) ** 2).mean()
    assert np.allclose(out[1], x[1] / math.sqrt(ms + 1e-6), rtol=1e-7)
    assert abs((out[1].astype(np.float64) ** 2).mean() - ms / (ms + 1e-6)) < 1e-6
    assert np.allclose(out[2], out[1], rtol=1e-6)
    assert np.all(out[3] == 0.0)
