"""Host-side checks of the C-ABI library that need no GPU: it loads, exports
every entry point declared in include/moe.h, sizes agree with the format
definition, and invalid arguments are rejected before any HIP call."""
import ctypes as C
import os
import re

import pytest

import oracle
import synth
from sparse_moe_expert_gemv_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_entry_points():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    names = declared_entry_points()
    assert len(names) >= 17
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTED) == names


def test_version_and_status_strings():
    assert B.moe_version() == 10100
    assert B.lib().moe_status_string(B.MOE_ERR_CACHE_CAPACITY) == b"MOE_ERR_CACHE_CAPACITY"


@pytest.mark.parametrize("wfmt", [4, 8])
@pytest.mark.parametrize("d,f", [(2048, 768), (256, 128), (64, 32)])
def test_expert_bytes_agree_with_format(wfmt, d, f):
    n = B.moe_expert_bytes(wfmt, d, f)
    assert n == synth.expert_bytes(wfmt, d, f) == oracle.expert_bytes(wfmt, d, f)
    assert B.moe_expert_bytes(3, d, f) == 0


def test_workspace_size_grows_with_tokens_and_rejects_bad_shapes():
    a = B.moe_workspace_size(1, 2048, 768, 512, 10, B.MOE_ACT_FLOAT)
    b = B.moe_workspace_size(8192, 2048, 768, 512, 10, B.MOE_ACT_Q8)
    assert 0 < a < b
    with pytest.raises(B.MoeError):
        B.moe_workspace_size(4, 2000, 768, 512, 10, B.MOE_ACT_FLOAT)  # d % 128 != 0
    with pytest.raises(B.MoeError):
        B.moe_workspace_size(4, 2048, 768, 8, 10, B.MOE_ACT_FLOAT)  # k > E
    with pytest.raises(B.MoeError):
        B.moe_workspace_size(4, 2048, 768, 2048, 10, B.MOE_ACT_FLOAT)  # E > 1024


def test_workspace_for_a_batch_serves_every_smaller_batch():
    # callers size one workspace for their largest batch (the layer objects and
    # the decode stack do); the split-k router planes must not break that
    for d, f, E, k in ((2048, 768, 512, 10), (4096, 1024, 1024, 32), (256, 128, 64, 4)):
        for mode in (B.MOE_ACT_FLOAT, B.MOE_ACT_Q8):
            sizes = [B.moe_workspace_size(T, d, f, E, k, mode) for T in range(1, 601)]
            assert all(a <= b for a, b in zip(sizes, sizes[1:])), (d, f, E, k, mode)


def test_invalid_arguments_rejected_before_any_hip_call():
    L = B.lib()
    null = None
    assert L.moe_route(null, B.MOE_DT_F32, 4, 2048, null, null, 512, 10, null, null, null, 0, null) == \
        B.MOE_ERR_INVALID_ARG
    assert L.moe_route(null, 7, 4, 2048, null, null, 512, 10, null, null, null, 0, null) == B.MOE_ERR_INVALID_ARG
    assert L.moe_route(null, B.MOE_DT_F32, -1, 2048, null, null, 512, 10, null, null, null, 0, null) == \
        B.MOE_ERR_INVALID_ARG
    # T == 0 is a no-op even with null pointers
    assert L.moe_route(null, B.MOE_DT_F32, 0, 2048, null, null, 512, 10, null, null, null, 0, null) == B.MOE_OK
    assert L.moe_permute(null, 4, 11, 10, null, null, null, null, null, null, 0, null) == B.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_act(null, B.MOE_DT_BF16, 4, 100, null, null, null) == B.MOE_ERR_INVALID_ARG
    assert L.moe_combine(null, B.MOE_DT_F32, null, null, null, null, 2, 10, 2048, null, null) == \
        B.MOE_ERR_INVALID_ARG
    assert L.moe_combine(null, 5, null, null, null, null, 2, 10, 2048, null, null) == B.MOE_ERR_INVALID_ARG
    assert L.moe_pack_experts(null, null, 3, 5, 2048, 768, null) == B.MOE_ERR_INVALID_ARG
    assert L.moe_pack_experts(null, null, 3, 4, 2048, 760, null) == B.MOE_ERR_INVALID_ARG
    assert L.moe_expert_ffn(None, None) == B.MOE_ERR_INVALID_ARG
    a = B.FfnArgs()
    a.T, a.d, a.f, a.E, a.k, a.wfmt, a.act_mode, a.y_dtype = 4, 2048, 768, 512, 10, 4, 0, 0
    assert L.moe_expert_ffn(C.byref(a), None) == B.MOE_ERR_INVALID_ARG  # null pointers
    a.act_mode = 9
    assert L.moe_expert_ffn(C.byref(a), None) == B.MOE_ERR_INVALID_ARG
    a.act_mode, a.T = 0, 0
    assert L.moe_expert_ffn(C.byref(a), None) == B.MOE_OK
    # the FFN + combine entry: its own arguments first, then those of moe_expert_ffn
    dummy = C.c_void_p(0x1000)
    assert L.moe_expert_ffn_combine(None, dummy, dummy, dummy, None, dummy, None) == B.MOE_ERR_INVALID_ARG
    a.T = 4
    assert L.moe_expert_ffn_combine(C.byref(a), None, dummy, dummy, None, dummy, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_expert_ffn_combine(C.byref(a), dummy, dummy, dummy, None, None, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_expert_ffn_combine(C.byref(a), dummy, dummy, dummy, None, dummy, None) == B.MOE_ERR_INVALID_ARG
    a.phase = 1
    assert L.moe_expert_ffn_combine(C.byref(a), dummy, dummy, dummy, None, dummy, None) == B.MOE_ERR_INVALID_ARG
    a.phase, a.T = 0, 0
    assert L.moe_expert_ffn_combine(C.byref(a), None, None, None, None, None, None) == B.MOE_OK
    # the by-slot decode entry: argument checks, then the supported shapes, all before any HIP call
    a.T, a.x_dtype = 4, B.MOE_DT_BF16
    assert L.moe_expert_ffn_combine_slots(None, dummy, dummy, None, dummy, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_expert_ffn_combine_slots(C.byref(a), dummy, dummy, None, dummy, None) == B.MOE_ERR_INVALID_ARG
    a.x, a.expert_ptrs, a.ws = 0x1000, 0x1000, 0x1000
    assert L.moe_expert_ffn_combine_slots(C.byref(a), None, dummy, None, dummy, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_expert_ffn_combine_slots(C.byref(a), dummy, dummy, None, dummy, None) == B.MOE_ERR_NO_MEMORY
    a.ws_bytes = 1 << 40
    a.phase = 2
    assert L.moe_expert_ffn_combine_slots(C.byref(a), dummy, dummy, None, dummy, None) == B.MOE_ERR_INVALID_ARG
    a.phase = 0
    for field, value in (("T", 9), ("act_mode", B.MOE_ACT_Q8), ("wfmt", 8), ("f", 640), ("d", 1536)):
        old = getattr(a, field)
        setattr(a, field, value)
        assert L.moe_expert_ffn_combine_slots(C.byref(a), dummy, dummy, None, dummy, None) == B.MOE_ERR_UNSUPPORTED, field
        setattr(a, field, old)
    a.T = 0
    assert L.moe_expert_ffn_combine_slots(C.byref(a), None, None, None, None, None) == B.MOE_OK
    # routing + by-slot FFN + combine: null router weights or outputs, then the shapes
    a.T = 4
    assert L.moe_route_ffn_combine_slots(C.byref(a), None, None, dummy, dummy, None, dummy, None) == \
        B.MOE_ERR_INVALID_ARG
    assert L.moe_route_ffn_combine_slots(C.byref(a), dummy, None, None, dummy, None, dummy, None) == \
        B.MOE_ERR_INVALID_ARG
    a.T = 9
    assert L.moe_route_ffn_combine_slots(C.byref(a), dummy, None, dummy, dummy, None, dummy, None) == \
        B.MOE_ERR_UNSUPPORTED
    a.T = 0
    assert L.moe_route_ffn_combine_slots(C.byref(a), None, None, None, None, None, None, None) == B.MOE_OK


def test_noalloc_decode_entry_rejects_before_any_hip_call():
    """The no-allocation decode entry validates everything, including the
    scratch limit, before it touches the device (no GPU here)."""
    L = B.lib()
    dummy = C.c_void_p(0x1000)
    a = B.FfnArgs()
    a.T, a.d, a.f, a.E, a.k, a.wfmt, a.act_mode, a.y_dtype = 4, 2048, 768, 512, 10, 4, 0, 0
    a.x_dtype = B.MOE_DT_BF16
    fn = L.moe_route_ffn_combine_slots_noalloc
    assert fn(None, dummy, None, dummy, dummy, None, dummy, None) == B.MOE_ERR_INVALID_ARG
    assert fn(C.byref(a), dummy, None, dummy, dummy, None, dummy, None) == B.MOE_ERR_INVALID_ARG  # null x
    a.x, a.expert_ptrs = 0x1000, 0x1000  # ws stays null: it is not used
    assert fn(C.byref(a), None, None, dummy, dummy, None, dummy, None) == B.MOE_ERR_INVALID_ARG  # null Wr
    a.phase = 1
    assert fn(C.byref(a), dummy, None, dummy, dummy, None, dummy, None) == B.MOE_ERR_INVALID_ARG
    a.phase = 0
    # a shape whose workspace exceeds the scratch: 8 tokens, 64 slots each, f = 2048
    a.T, a.k, a.f, a.E = 8, 64, 2048, 1024
    assert fn(C.byref(a), dummy, None, dummy, dummy, None, dummy, None) == B.MOE_ERR_NO_MEMORY
    a.T, a.k, a.f, a.E = 9, 10, 768, 512  # no by-slot kernel beyond 8 tokens
    assert fn(C.byref(a), dummy, None, dummy, dummy, None, dummy, None) == B.MOE_ERR_UNSUPPORTED
    a.T = 0
    assert fn(C.byref(a), None, None, None, None, None, None, None) == B.MOE_OK
    assert B.MOE_NOALLOC_SCRATCH_BYTES == 2 << 20


def test_workspace_too_small_is_reported():
    """A too-small workspace is rejected with MOE_ERR_NO_MEMORY (pointers are
    never dereferenced on the host, so fake non-null values are safe)."""
    L = B.lib()
    fake = C.c_void_p(0x1000)
    st = L.moe_route(fake, B.MOE_DT_F32, 4, 2048, fake, None, 512, 10, fake, fake, fake, 16, None)
    assert st == B.MOE_ERR_NO_MEMORY
    st = L.moe_permute(fake, 4, 10, 512, fake, fake, fake, fake, fake, fake, 16, None)
    assert st == B.MOE_ERR_NO_MEMORY


def test_cache_argument_validation():
    L = B.lib()
    h = C.c_void_p()
    assert L.moe_cache_create(None, 48, 512, 10, 100, None, None, 2, 10) == B.MOE_ERR_INVALID_ARG
    assert L.moe_cache_create(C.byref(h), 0, 512, 10, 100, C.c_void_p(1), C.c_void_p(1), 2, 10) == \
        B.MOE_ERR_INVALID_ARG
    assert L.moe_cache_create(C.byref(h), 48, 512, 10, 0, C.c_void_p(1), C.c_void_p(1), 2, 10) == \
        B.MOE_ERR_INVALID_ARG
    assert L.moe_cache_destroy(None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_cache_lookup(None, 0, None, None, None, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_cache_map_host(None, 0, C.c_void_p(1), C.c_void_p(1), None, None) == B.MOE_ERR_INVALID_ARG


def test_decode_stack_inputs_follow_the_profile():
    """The decode stack's router biases are alpha * ln w(rank) of the residency
    profile: within a layer, a better-ranked expert has a larger bias, and the
    resident set is the profile's top ranks."""
    import numpy as np
    import synth
    S = synth.make_stack(name="decode_stack", overrides=dict(d=256, E=64, f=128, n_layers=3, n_resident=40,
                                                              n_pool_blobs=8))
    c = S.cfg
    rank = synth.stack_profile(0, c.n_layers, c.E)
    assert sorted(S.resident.tolist()) == sorted(np.argsort(rank)[:40].tolist())
    for l in range(c.n_layers):
        r = rank[l * c.E:(l + 1) * c.E]
        b = S.biases[l]
        assert b.dtype == np.float32 and b.shape == (c.E,)
        order = np.argsort(r)
        assert np.all(np.diff(b[order]) < 0)
        assert abs(float(b[order[0]]) - (-0.38 * 1.1 * np.log(r[order[0]] + 1.0))) < 1e-5


def test_stage_fault_hook_rejects_null_cache():
    """The staging fault hook is host bookkeeping only: a NULL cache is an
    argument error, with or without a hook."""
    L = B.lib()
    assert L.moe_cache_set_stage_fault_hook(None, B.STAGE_FAULT_FN(lambda *a: 0), None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_cache_set_stage_fault_hook(None, B.STAGE_FAULT_FN(), None) == B.MOE_ERR_INVALID_ARG
