"""bench.py on the GPU: one short run (2 timed steps) prints exactly one
JSON line with the fields of the measurement contract."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    print("[gpu-bench] bench.py --steps 2 --warmup 1 (short sections, short CPU baseline)",
          flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2",
                        "--warmup", "1", "--cpu-budget", "0.5", "--no-attention",
                        "--no-transfer", "--no-large"],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "kernels"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["unit"] == "GB/s" and d["config"]["workload"] == "qwen32b_16k"
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s" and rl["peak"] == 8000.0
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    # measured HBM bytes (committed counter summary of the same kernel
    # sources) within 5% of the algorithmic bytes, or null when stale
    assert rl["traffic"] is None or (
        abs(rl["traffic"] / rl["algorithmic_bytes_per_launch"] - 1.0) <= 0.05)
    assert set(d["kernels"]) == {"quantize", "dequant_anchor", "dequant_full"}
    assert "split_variants" in d and "verify" in d
    sp = d["single_page"]
    assert sp["blocks"] == 2 and set(sp["us_per_call"]) == set(d["kernels"])
    assert all(v > 0 for v in sp["us_per_call"].values())
    for k in d["kernels"].values():
        assert 0 < k["ms_min"] <= k["ms_median"] and k["ms"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s" and cb["value"] > 0
    assert cb["cores"] >= 1 and cb["elements_per_s"] > 0 and cb["cpu_model"]
    st = cb["single_thread"]
    assert st["value"] > 0 and st["elements"] == 256 * 32768
