"""The committed HBM-traffic summaries (rocprofv3 FETCH_SIZE / WRITE_SIZE
per launch, scaled by a plain copy) hold each codec kernel's measured bytes
within 5% of its algorithmic bytes: read the bf16 KV once and write the
codes (quantize), read the codes once and write the bf16 KV (dequants).
Traffic well above the model would mean re-reads or partial-line writes."""
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNELS = ("quantize", "dequant_anchor", "dequant_full")
# algorithmic bytes per bf16 element: bf16 in / out 2, each 4-bit stream
# 0.5, metadata 0.28125 (2 x 128 + 2 x 8 x 128 binary32 per 32768 elements)
BYTES_PER_ELEM = {"quantize": 2.0 + 0.5 + 0.5 + 0.28125,
                  "dequant_anchor": 0.5 + 0.28125 + 2.0,
                  "dequant_full": 0.5 + 0.5 + 0.28125 + 2.0}


def _summary(name):
    with open(os.path.join(ROOT, "profiles", name)) as f:
        text = f.read()
    return json.loads(text.split("```json", 1)[1].split("```", 1)[0])


@pytest.mark.parametrize("name,elements", [
    ("traffic_qwen32b_16k.md", 64 * 2 * 16384 * 1024),         # 4 GiB set
    ("large_qwen3_235b_128k.md", 94 * 2 * 131072 * 512),       # 23.5 GiB set
])
def test_codec_traffic_within_five_percent(name, elements):
    t = _summary(name)
    assert t["fetch_scale"] > 0 and t["write_scale"] > 0
    for k in KERNELS:
        e = t["kernels"][k]
        algo = BYTES_PER_ELEM[k] * elements
        assert e["algorithmic_bytes_per_launch"] == pytest.approx(algo, rel=1e-9)
        ratio = e["hbm_bytes_per_launch"] / algo
        assert 0.95 <= ratio <= 1.05, (name, k, ratio)
        # reads and writes each match their own share of the model
        assert e["hbm_read_bytes"] + e["hbm_write_bytes"] == pytest.approx(
            e["hbm_bytes_per_launch"], rel=1e-6)
