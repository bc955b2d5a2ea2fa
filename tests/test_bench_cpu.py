"""Host-side checks of bench.py (no GPU): the one-GPU guard and the CPU
baseline leg on the two small workloads."""
from __future__ import annotations

import importlib.util
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    """--gpus 2 stops before touching a device, with exit status 2 and a
    message naming the single-GPU scope."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("idx", [1, 2])
def test_cpu_baseline_leg(idx):
    """The oracle leg runs on the host for the small workloads and reports
    positive times, its core count and a dense-equivalent rate."""
    b = _bench_module()
    import workloads as wl
    w = wl.get(idx)
    q, k, v = wl.make_qkv(w, 0)
    cb = b._cpu_baseline(w, q, k, v, blocks_per_head=2)
    assert cb["nb"] * w.B >= w.N  # every token has a slot
    assert cb["blocks_per_head"] == min(2, cb["nb"])
    for key in ("layer_s", "plan_gather_s", "score_select_s", "attn_sample_s"):
        assert cb[key] > 0.0 and math.isfinite(cb[key])
    assert cb["cores"] >= 1
    rec = b._cpu_record(cb, flop_dense=4.0 * w.N * w.N * w.D * w.heads)
    assert rec["kind"] == "oracle" and rec["unit"].startswith("TFLOP/s")
    assert rec["value"] > 0.0 and rec["cores"] == cb["cores"]
