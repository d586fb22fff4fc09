"""Host-side pieces of bench.py (CPU only): the flop conventions and peaks it
reports against, and the committed HBM-traffic record of the dominant kernel,
which bench.py reports only while it was taken on the current sources."""
import json
import os

import pytest

import bench
import coda_inputs as ci

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_peaks():
    # 256 CUs x 4096 bf16 flop per CU and clock at 2.4 GHz; fp8 twice that
    assert bench.PEAK_BF16_TFLOPS == pytest.approx(2516.58, abs=0.01)
    assert bench.PEAK_FP8_TFLOPS == pytest.approx(2 * bench.PEAK_BF16_TFLOPS)


def test_flop_conventions():
    # algorithmic GEMM flops only: forward 2MKD + 2MDN2, backward twice that
    wl = ci.WORKLOADS["7b-bf16"]
    assert (wl.M, wl.K, wl.D, wl.N2) == (16384, 4096, 4096, 28672)
    assert wl.fwd_flops == 2 * 16384 * 4096 * 4096 + 2 * 16384 * 4096 * 28672
    assert wl.bwd_flops == 2 * wl.fwd_flops


def test_traffic_record_matches_the_current_sources():
    # the counter profile behind roofline.traffic must be re-taken whenever
    # the second GEMM's sources or flags change (bench.py then reports null)
    with open(os.path.join(ROOT, "profiles", "traffic_gemm_rowscale_7b-bf16.json")) as f:
        rec = json.load(f)
    assert rec["sources_sha256"] == bench.second_gemm_sources_sha256(), \
        "the second GEMM changed since its HBM counters were taken: profile it again"
    assert rec["bytes_per_launch"] > 0
    assert bench.measured_traffic("7b-bf16") == rec["bytes_per_launch"]
