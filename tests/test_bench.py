"""bench.py's command-line contract: more than one GPU is refused with a
message before anything runs, and a short run prints exactly one JSON line
that carries every field the contract names, with `roofline.frac` equal to
`achieved / peak` and the oracle's CPU baseline beside it."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


@pytest.mark.parametrize("mode", [[], ["--backward"], ["--capacity-curve"]])
def test_more_than_one_gpu_is_refused(mode):
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"] + mode,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_short_run_prints_the_contract_line():
    r = subprocess.run([sys.executable, BENCH, "--workload", "tiny_f32", "--steps", "3",
                        "--warmup", "1", "--kernel-steps", "2", "--cpu-seconds", "1"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-3000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "tiny_f32" and d["dtype"] == "f32"
    rf = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rf, key
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])
    assert rf["traffic"] is None  # the counter summary covers another launch
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0
