"""The bench.py output line on a GPU: one JSON object on stdout with the
fields its readers depend on (the metric, the timing, the roofline of the
attention kernel and the CPU oracle baseline), on a small layer so that it
finishes in seconds (with the probe kernels and the zero-operand attention
timings)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_bench_line_fields():
    _cuda()
    print("case bench line llama3-8b-32k-b64", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"),
                        "--workload", "llama3-8b-32k-b64", "--steps", "3", "--warmup", "1",
                        "--no-dense"],
                       capture_output=True, text=True, timeout=280, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    j = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in j, key
    assert j["n_gpus"] == 1 and j["steps"] == 3 and j["warmup"] == 1
    assert j["higher_is_better"] is False and j["unit"] == "ms" and j["dtype"] == "bf16"
    assert j["value"] > 0 and j["value"] == j["ms_per_step"]
    assert j["config"]["workload"] == "llama3-8b-32k-b64"
    rf = j["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert 0 < rf["achieved"] < rf["peak"]
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert "traffic" in rf
    # the attention's event time is a part of the step
    assert 0 < j["stages_ms"]["attn"] < j["value"]
    s = j["step_ms_spread"]
    assert s["min"] <= s["median"] <= s["max"]
    c = j["ceilings"]
    assert c["mfma_bf16_random_tflops"] > 0 and c["hbm_read_gbs"] > 0
    assert set(c["attn_ms_by_operands"]) == {"real", "zero_v", "zero_q", "zero_qkv"}
    assert all(t > 0 for t in c["attn_ms_by_operands"].values())
    cb = j["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "ms" and cb["value"] > 0 and cb["cores"] >= 1
    assert set(cb["stages_ms"]) == {"pool", "score", "budget_select", "attn"}
    assert cb["fp32"]["value"] > 0
