"""Host-side logic of bench.py (no GPU): the algorithmic byte count the
roofline divides by, the staleness check of the committed traffic counters,
and the single-GPU guard."""
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_prefill_gateup_bytes_from_first_principles():
    # 8,192 tokens, d = 2048, f = 768, 512 experts all active, top-10, one shared
    # expert; int4 block-32 weights with one fp16 scale per 32; int8 activations
    # with one fp32 scale per 32, and h written the same way.
    import synth
    b = _bench()
    T, d, f, k, active = 8192, 2048, 768, 10, 512
    per_matrix = f * d // 2 + (f * d // 32) * 2          # quants + scales of one f x d matrix
    weights = (active + 1) * 2 * per_matrix               # gate and up of every active expert + the shared one
    x = T * d + T * (d // 32) * 4
    rows = T * k + T
    h = rows * f + rows * (f // 32) * 4
    nbytes, ops = b.gateup_algorithmic(synth.CONFIGS["prefill"], active, T)
    assert nbytes == weights + x + h == 1004470272
    assert ops == 2.0 * 2 * d * f * rows


def test_traffic_reported_only_while_the_sources_are_unchanged(tmp_path, monkeypatch):
    b = _bench()
    root = tmp_path / "repo"
    shutil.copytree(os.path.join(ROOT, "sparse_moe_expert_gemv_amd", "csrc"),
                    root / "sparse_moe_expert_gemv_amd" / "csrc")
    (root / "profiles").mkdir()
    monkeypatch.setattr(b, "ROOT", str(root))
    sha = b.kernel_source_sha256("prefill")
    (root / "profiles" / "gateup_prefill_hbm_counters.md").write_text(
        "traffic_bytes_per_launch: 1234\nkernel_source_sha256: %s\n" % sha)
    assert b.measured_traffic("prefill") == 1234
    assert b.measured_traffic("skew") is None  # no summary for this workload in the copy
    # a change to an included header invalidates the figure as well as one to the kernel source
    hdr = root / "sparse_moe_expert_gemv_amd" / "csrc" / "topk.hpp"
    hdr.write_text(hdr.read_text() + "\n")
    assert b.kernel_source_sha256("prefill") != sha
    assert b.measured_traffic("prefill") is None


@pytest.mark.parametrize("n", [0, 2, 8])
def test_bench_refuses_anything_but_one_gpu(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout
