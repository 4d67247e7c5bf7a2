"""bench.py's output contract on a real device: one JSON line on stdout with
the fields its readers parse, numbers that agree with each other (tokens/s
from the step time, the roofline fraction from achieved over peak), the copy
floors, and the CPU oracle baseline.  Run on the tiny workload with a few
steps, so it takes seconds."""
import json
import math
import os
import subprocess
import sys

import pytest

from gpu_common import require_gpu, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_complete_line():
    require_gpu()
    say("[bench line] tiny, 3 steps")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--also", "none",
                        "--steps", "3", "--warmup", "1", "--cpu-seconds", "0.5"],
                       cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "roofline_dispatch", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "tokens/s" and d["higher_is_better"] is True and d["vs_baseline"] is None
    cfg = d["config"]
    assert cfg["workload"] == "tiny" and cfg["tokens"] == 64
    assert math.isclose(d["value"], cfg["tokens"] / (d["ms_per_step"] * 1e-3), rel_tol=1e-9)
    rf = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rf, key
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert math.isclose(rf["frac"], rf["achieved"] / rf["peak"], rel_tol=1e-9)
    assert rf["achieved"] > 0 and rf["mean_launch_us"] > 0
    fl = cfg["floor"]
    for key in ("pack_shaped_copy", "combine_shaped_copy", "pack_writes_only", "receive_buffer_fill"):
        assert fl[key]["mean_us"] > 0 and fl[key]["gbps"] > 0, key
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["single_thread"]["cores"] == 1 and cb["sample"]
