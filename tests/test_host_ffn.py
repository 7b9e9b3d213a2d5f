"""The host-core expert FFN (moe_host_expert_ffn, the CPU share of missed
experts) against the oracle's float-mode expert on the CPU: decode-shaped int4
and tiny int8 experts, several items per token, accumulation into an existing
output, and results independent of the pool size."""
import ctypes as C

import numpy as np
import pytest

import oracle
import synth
from sparse_moe_expert_gemv_amd import binding as B
from tests import refmath as R


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)
    B.lib()


@pytest.mark.parametrize("wfmt,d,f", [(synth.WFMT_I4B32, 2048, 768), (synth.WFMT_I8B32, 256, 128)])
def test_host_ffn_matches_oracle(wfmt, d, f):
    rng = np.random.Generator(np.random.PCG64(41))
    blobs = [synth.gen_expert_blob(np.random.Generator(np.random.PCG64(200 + e)), d, f, wfmt) for e in range(3)]
    T = 3
    x = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32)))
    # items: token 0 twice (experts 0, 2), token 2 once (expert 1); token 1 none
    tok = [0, 2, 0]
    which = [0, 1, 2]
    gates = np.array([0.7, 0.25, 0.3], np.float32)
    base = rng.standard_normal((T, d)).astype(np.float32)
    ref = base.astype(np.float64).copy()
    for t, e, g in zip(tok, which, gates):
        ref[t] += float(g) * oracle.expert_ffn(x[t:t + 1], blobs[e], wfmt, f, oracle.ACT_FLOAT)[0]
    outs = []
    for n_threads in (1, 5):
        pool = B.HostPool(n_threads)
        out = base.copy()
        pool.expert_ffn(tok, gates, [blobs[e].ctypes.data for e in which], wfmt, x, out, d, f)
        pool.close()
        outs.append(out)
    assert np.array_equal(outs[0], outs[1])  # the pool size does not change a bit
    assert np.array_equal(outs[0][1], base[1])  # a token without items is untouched
    delta = outs[0].astype(np.float64) - base
    assert R.rel_l2(delta, ref - base) < 1e-5


def test_host_ffn_argument_errors():
    L = B.lib()
    h = C.c_void_p()
    assert L.moe_host_pool_create(0, C.byref(h)) == B.MOE_ERR_INVALID_ARG
    assert L.moe_host_pool_create(2, C.byref(h)) == B.MOE_OK
    dummy = C.c_void_p(0x1000)
    tok = (C.c_int32 * 1)(5)
    assert L.moe_host_expert_ffn(h, 1, tok, dummy, dummy, 4, 2, 64, 64, dummy, dummy) == B.MOE_ERR_INVALID_ARG
    assert L.moe_host_expert_ffn(h, 1, dummy, dummy, dummy, 4, 2, 60, 64, dummy, dummy) == B.MOE_ERR_INVALID_ARG
    assert L.moe_host_expert_ffn(h, 0, None, None, None, 4, 2, 64, 64, None, None) == B.MOE_OK
    assert L.moe_host_pool_destroy(h) == B.MOE_OK
