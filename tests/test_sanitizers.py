"""Host code under sanitizers (CPU only): the oracle, built with
AddressSanitizer + UndefinedBehaviorSanitizer, runs every entry point on a
small layer and must give the normal build's outputs bit for bit; the
library's host-only code (adaptive-cache replacement plan, host-core expert
FFN and its thread pool) runs under ASan + UBSan and under ThreadSanitizer."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "sparse_moe_expert_gemv_amd", "csrc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           TSAN_OPTIONS="halt_on_error=1")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="no gcc")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, env=ENV, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-6000:])
    return r


@pytest.mark.parametrize("wfmt", [synth.WFMT_I4B32, synth.WFMT_I8B32])
def test_oracle_under_asan_ubsan_equals_normal_build(tmp_path, wfmt):
    oracle.build(force=False)
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-fast-math", "-ffp-contract=off", "-Wno-unknown-pragmas",
          os.path.join(ROOT, "oracle", "moe_oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"])
    T, d, f, E, k = 8, 256, 128, 16, 4
    rng = np.random.Generator(np.random.PCG64(71))
    x = rng.standard_normal((T, d)).astype(np.float32)
    x[2, 32:64] = 0.0  # an all-zero quantisation block
    wr = (rng.standard_normal((E, d)) * 0.02).astype(np.float32)
    experts = synth.gen_expert_blobs(0, 99, 0, 0, E, d, f, wfmt)
    shared = synth.gen_expert_blobs(0, 99, 0, 1, 1, d, f, wfmt)[0]
    res = rng.standard_normal((T, d)).astype(np.float32)
    for name, a in (("x", x), ("wr", wr), ("experts", experts), ("shared", shared), ("residual", res)):
        np.ascontiguousarray(a).tofile(str(tmp_path / (name + ".bin")))
    _run([exe, str(tmp_path), str(T), str(d), str(f), str(E), str(k), str(wfmt)])

    def out(name, dt, shape):
        return np.fromfile(str(tmp_path / ("out_%s.bin" % name)), dtype=dt).reshape(shape)

    ids, gates, logits = oracle.route(x, wr, None, k, return_logits=True)
    assert np.array_equal(out("ids", np.int32, ids.shape), ids)
    assert np.array_equal(out("gates", np.float32, gates.shape), gates)
    assert np.array_equal(out("logits", np.float64, logits.shape), logits)
    assert np.array_equal(out("sorted", np.int32, (T * k,)), oracle.permute(ids, E)[2])
    assert np.array_equal(out("xq", np.int8, (T, d)), oracle.quant8(x)[0])
    assert np.array_equal(out("rmsnorm", np.float32, (T, d)), oracle.rmsnorm(x))
    wg, wu, wd = oracle.dequant_expert(experts[0], wfmt, d, f)
    assert np.array_equal(out("dequant", np.float64, (3 * d * f,)), np.concatenate([wg.ravel(), wu.ravel(), wd.ravel()]))
    for mode, nm in ((oracle.ACT_FLOAT, "float"), (oracle.ACT_Q8, "q8")):
        assert np.array_equal(out("ffn_" + nm, np.float64, (T, d)), oracle.expert_ffn(x, experts[1], wfmt, f, mode))
        o = oracle.moe_layer(x, wr, None, experts, shared, wfmt, f, k, act_mode=mode, residual=res)
        assert np.array_equal(out("layer_" + nm, np.float32, (T, d)), o["out"])
        o = oracle.moe_layer(x, wr, None, experts, None, wfmt, f, k, act_mode=mode, tokens=[T - 1, 0, T // 2])
        assert np.array_equal(out("subset_" + nm, np.float32, (3, d)), o["out"])


def _host_driver(tmp_path, sanitize):
    exe = str(tmp_path / ("host_driver_" + sanitize.replace(",", "_")))
    _run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=" + sanitize,
          "-fno-sanitize-recover=all", "-pthread", "-I", os.path.join(ROOT, "include"),
          os.path.join(SAN, "host_driver.cpp"), os.path.join(CSRC, "host_ffn.cpp"),
          os.path.join(CSRC, "cache_plan.cpp"), "-o", exe])
    return exe


def test_host_code_under_asan_ubsan(tmp_path):
    r = _run([_host_driver(tmp_path, "address,undefined"), "40"])
    assert "host driver ok" in r.stdout


def test_host_thread_pool_under_tsan(tmp_path):
    r = _run([_host_driver(tmp_path, "thread"), "30"])
    assert "host driver ok" in r.stdout
