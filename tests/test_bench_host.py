"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the oracle
baseline leg, the coded-symbol view used by the entropy report, and the
traffic lookup that only accepts counters taken on the current sources."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from lossless_weight_compression_bf16_amd import synthetic as S  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_leg(oracle_lib):
    w = S.workload("bf16-768x2304")
    xs = S.set_bits(w)
    r = bench.cpu_baseline(w, xs, 0.5, "bf16", 0)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s"
    assert r["value"] > 0 and r["cores"] >= 1 and r["seconds"] > 0
    assert "pass" in r["sample"] and w.name in r["sample"]
    assert r["one_thread"]["elements"] % 65536 == 0


@pytest.mark.parametrize("layout", ["bf16", "bf16r", "fp16", "fp16r"])
def test_coded_symbols_match_the_oracle_split_16(oracle_lib, layout):
    v = np.arange(65536, dtype=np.uint16)  # every pattern
    coded, _ = oracle_lib.split_u16(layout, v)
    assert np.array_equal(bench.coded_symbols(layout, v), coded)


@pytest.mark.parametrize("layout", ["fp8e4m3", "fp8e5m2"])
def test_coded_symbols_match_the_oracle_split_fp8(oracle_lib, layout):
    v = np.arange(256, dtype=np.uint8)
    coded, _ = oracle_lib.split_fp8(layout, v)
    assert np.array_equal(bench.coded_symbols(layout, v), coded)


def test_coded_symbols_match_the_oracle_split_fp32(oracle_lib):
    g = np.random.default_rng(4)
    u = g.integers(0, 2 ** 32, 100000, dtype=np.uint64).astype(np.uint32)
    exp, _ = oracle_lib.split_fp32(u)
    assert np.array_equal(bench.coded_symbols("fp32", u), exp)


def test_entropy_report_orders_its_figures(oracle_lib):
    w = S.workload("bf16-768x2304")
    x = S.set_bits(w)[0][: 5 * 65536 + 777]
    e = oracle_lib.encode(x, "bf16", threads=4)
    r = bench.coded_plane_entropy([x], e.tables.reshape(-1, 256), e.seek, "bf16", False)
    # cross-entropy under the 12-bit table is at least the empirical entropy;
    # the payload (states and padding included) is at least the ideal length
    assert r["H_emp"] <= r["H_q"] + 1e-9
    assert r["H_q"] <= r["payload_bits"] + 1e-9
    assert r["chunks_sampled"] == 6


def test_traffic_is_only_taken_for_the_current_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"rans_decode@x": {"traffic_bytes": 123, "source_sha256": bench.source_digest()},
                             "rans_decode@y": {"traffic_bytes": 456, "source_sha256": "0" * 64}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("rans_decode", "x") == 123
    assert bench.measured_traffic("rans_decode", "y") is None
    assert bench.measured_traffic("rans_encode", "x") is None
