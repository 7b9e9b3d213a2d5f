"""GPU: the no-allocation decode entry (moe_route_ffn_combine_slots_noalloc,
scratch kept by the library) against moe_route_ffn_combine_slots with a
caller workspace: ids, gates and output bit for bit, on two calls in a row,
the second with fewer tokens (the scratch then holds the first call's bytes),
and against the oracle at the float bar."""
import numpy as np
import pytest

import oracle
import synth
from tests import refmath as R

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_util import DEV, gpu_layer, host, x_tensor  # noqa: E402
from sparse_moe_expert_gemv_amd import binding as B  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    oracle.build(force=False)


def _run(G, L, T, x, res, noalloc):
    c = L.cfg
    ids = torch.full((T, c.k), -7, dtype=torch.int32, device=DEV)
    gates = torch.full((T, c.k), -1.0, dtype=torch.float32, device=DEV)
    out = torch.full((T, c.d), float("nan"), dtype=torch.float32, device=DEV)
    common = dict(T=T, d=c.d, f=c.f, E=c.E, k=c.k, wfmt=c.wfmt, act_mode=B.MOE_ACT_FLOAT,
                  expert_ptrs=G.expert_ptrs, Wr=G.Wr, bias=G.bias, ids=ids, gates=gates, out=out, x=x,
                  residual=res, shared_blob=G.shared)
    if noalloc:
        B.moe_route_ffn_combine_slots_noalloc(**common)
    else:
        B.moe_route_ffn_combine_slots(ws=G._ws_for(T), **common)
    torch.cuda.synchronize()
    return host(ids), host(gates), host(out)


@pytest.mark.parametrize("Ts", [(4, 2), (8, 1)])
def test_noalloc_decode_layer_equals_workspace_entry(Ts):
    L = synth.make_layer("decode_t4", T=max(Ts))
    c = L.cfg
    G = gpu_layer(L)
    xt_all = x_tensor(L)
    rng = np.random.Generator(np.random.PCG64(31))
    for T in Ts:
        print("[noalloc] T=%d" % T, flush=True)
        res_np = rng.standard_normal((T, c.d)).astype(np.float32)
        res = torch.from_numpy(res_np).to(DEV)
        x = xt_all[:T].contiguous()
        ref = _run(G, L, T, x, res, noalloc=False)
        got = _run(G, L, T, x, res, noalloc=True)
        assert np.array_equal(got[0], ref[0])
        assert np.array_equal(got[1].view(np.uint32), ref[1].view(np.uint32))
        assert np.array_equal(got[2].view(np.uint32), ref[2].view(np.uint32))
        o = oracle.moe_layer(L.x_f32()[:T], L.Wr, L.bias, L.experts, L.shared, c.wfmt, c.f, c.k,
                             act_mode=oracle.ACT_FLOAT, residual=res_np)
        assert np.array_equal(got[0], o["ids"])
        ok, rel, mx = R.within_tolerance(got[2], o["out"])
        print("[noalloc] T=%d rel-L2 %.3e max-abs/RMS %.3e" % (T, rel, mx), flush=True)
        assert ok
