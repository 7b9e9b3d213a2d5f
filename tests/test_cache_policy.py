"""Host logic of the adaptive expert cache: moe_cache_plan through the C ABI
(no GPU needed) against a direct statement of the rule, plus argument checks.

The rule ("How Strata works", adaptive expert cache section: the cache keeps
learning which experts the session uses and adjusts its contents; the pages
give no policy, so the plainest one is taken): the missing experts with the
highest aged usage replace the resident experts with the lowest, pair by pair,
while the newcomer's score beats the incumbent's by the margin.
"""
import numpy as np
import pytest

from sparse_moe_expert_gemv_amd import binding as B


def rule(resident, score, max_swaps, margin):
    n = len(score)
    f32 = np.float32
    ins = sorted((g for g in range(n) if resident[g]), key=lambda g: (float(score[g]), g))
    outs = sorted((g for g in range(n) if not resident[g]), key=lambda g: (-float(score[g]), g))
    ev, ad = [], []
    for v, a in zip(ins, outs):
        if len(ev) == max_swaps:
            break
        if not f32(score[a]) > (f32(1.0) + f32(margin)) * f32(score[v]):
            break
        ev.append(v)
        ad.append(a)
    return ev, ad


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("margin", [0.0, 0.25])
def test_plan_matches_rule(seed, margin):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 400))
    res = (rng.random(n) < rng.random()).astype(np.uint8)
    # small integer scores: many ties, so the id tie-break is exercised
    score = rng.integers(0, 6, n).astype(np.float32) * np.float32(rng.choice([0.5, 1.0, 3.0]))
    for max_swaps in (0, 1, 7, n):
        ev, ad = B.moe_cache_plan(res, score, max_swaps, margin)
        rev, rad = rule(res, score, max_swaps, margin)
        assert ev.tolist() == rev and ad.tolist() == rad
        assert len(set(ev.tolist()) | set(ad.tolist())) == 2 * len(ev)
        assert all(res[g] == 1 for g in ev) and all(res[g] == 0 for g in ad)


def test_plan_special_cases():
    score = np.array([5, 0, 3, 3, 1], dtype=np.float32)
    # nothing resident / everything resident: no pairs
    assert B.moe_cache_plan(np.zeros(5, np.uint8), score, 5)[0].size == 0
    assert B.moe_cache_plan(np.ones(5, np.uint8), score, 5)[0].size == 0
    # resident {0, 1}: the unused expert 1 (score 0) goes first, for expert 2
    # (score 3, the lower id of the tie with 3); expert 0 (5) stays
    ev, ad = B.moe_cache_plan(np.array([1, 1, 0, 0, 0], np.uint8), score, 5)
    assert ev.tolist() == [1] and ad.tolist() == [2]
    # a zero-score candidate never displaces a zero-score resident
    ev, _ = B.moe_cache_plan(np.array([1, 0], np.uint8), np.zeros(2, np.float32), 1)
    assert ev.size == 0
    # the margin blocks a swap that is not clearly better
    ev, _ = B.moe_cache_plan(np.array([1, 0], np.uint8), np.array([4, 4.5], np.float32), 1, margin=0.25)
    assert ev.size == 0
    ev, _ = B.moe_cache_plan(np.array([1, 0], np.uint8), np.array([4, 5.5], np.float32), 1, margin=0.25)
    assert ev.tolist() == [0]


def test_plan_and_cache_argument_validation():
    import ctypes as C
    L = B.lib()
    res = np.zeros(4, np.uint8)
    sc = np.zeros(4, np.float32)
    n = C.c_int()
    buf = np.zeros(4, np.int32)
    ok = (4, res.ctypes.data, sc.ctypes.data, 4, C.c_float(0.0), buf.ctypes.data, buf.ctypes.data, C.byref(n))
    assert L.moe_cache_plan(*ok) == B.MOE_OK
    bad = [(0,) + ok[1:], ok[:1] + (None,) + ok[2:], ok[:3] + (-1,) + ok[4:], ok[:4] + (C.c_float(-0.5),) + ok[5:],
           ok[:4] + (C.c_float(float("nan")),) + ok[5:], ok[:5] + (None,) + ok[6:], ok[:7] + (None,)]
    for args in bad:
        assert L.moe_cache_plan(*args) == B.MOE_ERR_INVALID_ARG
    sc[2] = -1.0
    assert L.moe_cache_plan(*ok) == B.MOE_ERR_INVALID_ARG
    sc[2] = np.inf
    assert L.moe_cache_plan(*ok) == B.MOE_ERR_INVALID_ARG
    sc[2] = 0.0
    res[1] = 2
    assert L.moe_cache_plan(*ok) == B.MOE_ERR_INVALID_ARG
    assert L.moe_cache_replace(None, 1, None, None, None, None, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_usage_accumulate(None, None, 4, None) == B.MOE_ERR_INVALID_ARG
