"""bench.py's contract on the host: the one-GPU refusal, the algorithmic
bytes it divides by, the counter summaries it reads and the roofline it
picks for query-tiled calls."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from split_kv_fd_amd import inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


@pytest.mark.parametrize("name,want", [("tiny_f32", 2_097_152), ("mha32k_f16", 536_870_912),
                                       ("gqa128k_bf16", 2_147_483_648), ("gqa_b64_bf16", 8_589_934_592)])
def test_algorithmic_kv_bytes(name, want):
    # every valid K and V row read once: 2 * sum(T_b) * Hkv * D * element bytes
    s = inputs.spec(name)
    assert bench.kv_bytes_of(s, [s.T] * s.B) == want


def test_paged_kv_bytes_follow_the_lengths():
    s = inputs.spec("paged_ragged_bf16")
    lens = inputs.ragged_lengths(s).tolist()
    assert bench.kv_bytes_of(s, lens) == 2 * sum(lens) * s.Hkv * s.D * 2


def test_traffic_summary_lookup():
    # the committed counter summary of the default workload, when it was
    # taken on the current kernel sources; nothing for an unknown workload
    t = bench.read_traffic("mha32k_f16", "fd_split")
    if t is not None:
        assert 0.99 * 536_870_912 <= t <= 1.05 * 536_870_912
    assert bench.read_traffic("no_such_workload", "fd_split") is None


def test_query_tiled_roofline_follows_intensity():
    ridge = bench.MFMA_PEAK_TFLOPS * 1e12 / (bench.HBM_PEAK_GBS * 1e9)
    kv = 8 * 2**30
    low = bench.query_tiled_roofline(int(64 * kv), kv, 1.5)         # 64 flop/B: K/V reads bound it
    assert low["bound"] == "hbm" and low["unit"] == "GB/s"
    assert abs(low["achieved"] - kv / 1.5e-3 / 1e9) < 0.01
    high = bench.query_tiled_roofline(int(2 * ridge * kv), kv, 1.5)  # past the ridge: matrix cores
    assert high["bound"] == "mfma" and high["unit"] == "TFLOP/s"
    assert high["frac"] == round(high["achieved"] / bench.MFMA_PEAK_TFLOPS, 4)
