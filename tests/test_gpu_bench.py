"""bench.py end to end on one GPU, on small sets: the JSON line carries the
fields its contract names (metric, value, unit, n_gpus, steps, warmup,
ms_per_step, higher_is_better, scaling, vs_baseline, dtype, data, config),
the roofline and oracle-baseline objects, and a bit-exact round trip; the
fused decode + GEMM line as well."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CONTRACT = ["metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
            "vs_baseline", "dtype", "data", "config"]


def _run(args):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    print(lines[0][:300], flush=True)
    return json.loads(lines[0])


@pytest.mark.parametrize("workload", ["bf16-768x2304", "fp32-768x2304"])
def test_bench_line(workload):
    d = _run(["--workload", workload, "--steps", "3", "--warmup", "1", "--cpu-seconds", "0.5", "--cold-reps", "1"])
    for k in CONTRACT:
        assert k in d, k
    assert d["metric"].startswith("rANS decode/encode GB/s") and d["unit"] == "GB/s"
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["higher_is_better"] is True
    assert d["config"]["workload"] == workload and d["data"] == "synthetic" and d["dtype"] == "u32"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["round_trip_bit_exact"] is True
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3 and r["alg_bytes"] > 0
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]
    assert 0.6 < d["ratio"] < (0.9 if workload.startswith("fp32") else 0.7)


def test_bench_rejects_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "8"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_fused_gemm_line():
    d = _run(["--fused-gemm", "16", "--workload", "bf16-768x2304", "--steps", "2", "--warmup", "1"])
    for k in CONTRACT:
        assert k in d, k
    assert d["config"]["m"] == 16 and d["value"] > 0
    assert d["max_rel_diff_vs_bf16_gemm"] <= 2.0 ** -6
    assert d["cpu_baseline"]["kind"] == "oracle"
