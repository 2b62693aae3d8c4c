"""bench.py end to end: the JSON line it prints (GPU), and the one-GPU guard
(host only).

The GPU test runs the small shape for a few steps in a subprocess, as the
driver runs the default workload, and checks the line's keys and the
relations between its numbers: value = unique bytes per step / step time,
tokens/s = verified positions per step / step time, the roofline's fraction
= achieved / peak and achieved = the algorithmic flops or bytes of a call /
the call time, the host-inclusive (eager) step figures, and a CPU baseline
from the oracle.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=timeout, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    res = _bench("--gpus", "2", timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and not res.stdout.strip()


@pytest.mark.gpu
def test_bench_line_of_the_small_shape():
    res = _bench("--workload", "tiny", "--steps", "4", "--warmup", "2", "--no-compare")
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    r = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "tokens_per_s", "hbm_frac"):
        assert key in r, key
    assert r["n_gpus"] == 1 and r["steps"] == 4 and r["warmup"] == 2
    assert r["config"]["workload"] == "tiny" and r["unit"] == "GB/s"
    # (the line rounds ms_per_step to 1e-5 ms and value to 0.01 GB/s)
    t = r["ms_per_step"] / 1e3
    assert r["value"] == pytest.approx(r["unique_kv_bytes_per_step"] / t / 1e9, rel=2e-3, abs=0.01)
    # the small shape: one sequence, a 4-token block
    assert r["tokens_per_s"] == pytest.approx(4 / t, rel=2e-3)
    roof = r["roofline"]
    assert roof["bound"] in ("hbm", "mfma")
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4)
    call_s = roof["launch_us"] * 1e-6
    work = roof["algorithmic_bytes"] / 1e9 if roof["bound"] == "hbm" else roof["algorithmic_flops"] / 1e12
    assert roof["achieved"] == pytest.approx(work / call_s, rel=2e-3)
    cpu = r["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    # the same steps issued eagerly: host work included, never faster than
    # the work itself by more than timing noise
    hi = r["host_inclusive"]
    te = hi["ms_per_step"] / 1e3
    assert te > 0
    assert hi["GB/s"] == pytest.approx(r["unique_kv_bytes_per_step"] / te / 1e9, rel=2e-3, abs=0.01)
    assert hi["tokens_per_s"] == pytest.approx(4 / te, rel=2e-3)
