"""bench.py's output contract on a GPU: one JSON line with the metric, the
roofline entry, the CPU baseline, the matrix-core ceiling, the loops and the
cold launches, on the small 256^3 workload (a few seconds)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_one_json_line_with_every_record():
    sys.stderr.write("[gpu-bench] bench.py --workload sq256\n")
    sys.stderr.flush()
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "sq256",
                        "--steps", "3", "--warmup", "1", "--cold-launches", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline", "loops", "mfma_ceiling", "cold"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["config"]["workload"] == "sq256" and d["parity_gate"] == "every output"
    roof = d["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s"
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0
    assert len(d["loops"]["per_launch_ms"]) == 5
    assert d["cold"]["launches"] == 2 and d["cold"]["median_ms"] > 0
    assert d["mfma_ceiling"]["frac_of_ceiling"] > 0
