"""GPU: bench.py end to end on the small workload, checking the JSON line's
contract fields (one line, the metric, the roofline and the oracle baseline)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("extra", [[], ["--graph", "--no-cpu-baseline"], ["--graph", "--host-scaler", "--no-cpu-baseline"],
                                   ["--reduce", "3", "--no-cpu-baseline"],
                                   ["--host-scaler", "--accum", "2", "--no-cpu-baseline"]])
def test_bench_json_line(extra):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "5",
                        "--warmup", "2", *extra], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2 and d["value"] > 0
    assert d["config"]["workload"] == "tiny_4tensors_nd4_rank1"
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-12
    assert d["skipped_step"]["steps"] == 5
    if "--no-cpu-baseline" in extra:
        assert d["cpu_baseline"] is None
    else:
        cb = d["cpu_baseline"]
        assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["unit"] == "params/s"
    if "--reduce" in extra:
        assert d["reduce"]["slices"] == 3 and d["reduce"]["gbps"] > 0
    if "--accum" in extra:
        f = d["accumulate"]["first"]
        assert f["gbps"] > 0 and f["widening_copy_gbps"] > 0 and abs(f["frac_of_widening_copy"] - f["gbps"] / f["widening_copy_gbps"]) < 1e-12
    # the shard's buffers come from the library's contiguous pool; the label
    # says whether any segment fell back to ordinary memory
    assert d["config"]["buffers"].startswith("physically contiguous HBM") and "none fell back" in d["config"]["buffers"]
    if not extra:
        # default path: the 100B model's 250M-parameter rank shard is timed as well
        x = d["extra_workload"]
        assert x["workload"] == "gpt_100b_nd400_rank200" and x["shard_params"] == 250_749_440
        assert x["ms_per_step"] > 0 and 0 < x["update"]["frac"] < 1.1 and x["skipped_step"]["steps"] == 5
        cb = d["cpu_baseline"]
        assert 1 <= cb["cores"] <= cb["host_cores_affinity"] <= cb["host_cpu_count"]
    else:
        assert d["extra_workload"] is None
