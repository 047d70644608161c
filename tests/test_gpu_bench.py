"""bench.py end to end on the GPU (small workloads): the one JSON line carries
the fields its readers rely on."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [line for line in r.stdout.strip().splitlines() if line.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def check_common(d, steps):
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "stages"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["higher_is_better"] is True
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert "workload" in d["config"]
    rl = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rl, k
    assert rl["bound"] in ("hbm", "mfma") and 0 < rl["frac"] < 1
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-9
    for st in d["stages"].values():
        assert st["us_p10"] <= st["us_median"] <= st["us_p90"]


def test_tiny_workload_with_cpu_baseline():
    d = bench("--workload", "c1", "--steps", "20", "--warmup", "5")
    check_common(d, 20)
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert set(d["stages"]) == {"act_quant_block", "gemm_blockscaled"}


def test_decode_fused_and_per_tensor_lines():
    d = bench("--workload", "c3", "--M", "1", "--fused", "--steps", "20", "--warmup", "5", "--no-cpu-baseline")
    check_common(d, 20)
    assert d["roofline"]["bound"] == "hbm" and d["roofline"]["kernel"] == "act_quant_gemm_blockscaled"
    d = bench("--workload", "c2", "--M", "64", "--steps", "20", "--warmup", "5", "--no-cpu-baseline")
    check_common(d, 20)
    assert d["unit"] == "GB/s"


def test_default_line_carries_every_workload():
    # the default (large-M) line with the other workloads' figures under
    # "configs", as the full test run records it
    d = bench("--steps", "5", "--warmup", "2", "--no-cpu-baseline")
    check_common(d, 5)
    c = d["configs"]
    assert set(c) == {"c1", "c2", "c3", "c4"}
    assert set(c["c2"]) == {f"M={m}" for m in (1, 64, 256, 1024, 65536)}
    for r in c["c2"].values():
        assert {"amax_quant_tensor", "amax_tensor"} <= set(r["stages"]) and r["b200_amax_us_context"] > 0
    assert set(c["c3"]) == {f"M={m}" for m in (1, 8, 32, 64)}
    for r in c["c3"].values():
        assert r["two_calls"]["roofline"]["bound"] == "hbm" and "fused_call" in r
    assert c["c4"]["roofline"]["bound"] == "mfma" and 0 < c["c4"]["roofline"]["frac"] < 1
