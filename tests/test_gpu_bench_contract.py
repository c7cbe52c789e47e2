"""bench.py's one-line JSON report on the GPU: the keys and units the report
promises, run as a child process on the default workload (needs the GPU)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_default_bench_line():
    print("[bench] python bench.py --steps 5 --warmup 2", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "5",
                        "--warmup", "2"],
                       capture_output=True, text=True, timeout=540, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 5 and line["warmup"] == 2
    assert line["value"] > 0 and line["ms_per_step"] > 0 and line["higher_is_better"] is True
    assert line["config"]["workload"] == "ragged_mixed_v262144"
    rf = line["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0 < rf["achieved"] < rf["peak"] and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    cb = line["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["sample"]
    assert cb["variants"] and all(v["value"] > 0 for v in cb["variants"].values())
    par = line["parity"]
    assert par["requests"] == 512 and par["mismatches"] == 0, par
    assert par["c_oracle_agrees"] is True, par        # the two oracles on the full batch
    assert any(k.startswith("c_all_rows") for k in cb["variants"]), cb["variants"]
    cf = line["configs"]
    assert len(cf) == 5 and "ragged_mixed_v262144" in cf
    for name, c in cf.items():
        assert c["step_us"] > 0 and c["positions_per_s"] >= 0, name
        assert c["parity"]["mismatches"] == 0, (name, c["parity"])
