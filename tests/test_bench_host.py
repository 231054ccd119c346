"""Host-side parts of bench.py, on the CPU: the one-GPU guard, the roofline
arithmetic, the algorithmic byte counts of one expert, and the lookup of the
recorded HBM counters (which are keyed to the text of the kernels' sources,
so a source edit without new counters would silently drop `traffic` from the
bench line)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_roofline_picks_the_binding_roof():
    # below the ridge (2500e12 / 8000e9 = 312.5 flop/B): HBM-bound
    r = bench.roofline_entry("k", nbytes=1e9, flops=100e9, kernel_us=250.0, traffic=None)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(1e9 / 250e-6 / 1e9)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0)
    assert r["mfma_frac"] == pytest.approx(100e9 / 250e-6 / 1e12 / 2500.0)
    # above the ridge: MFMA-bound, the fraction is of the bf16 peak
    r = bench.roofline_entry("k", nbytes=1e8, flops=100e9, kernel_us=100.0, traffic=123.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(1000.0)
    assert r["frac"] == pytest.approx(0.4)
    assert r["traffic"] == 123.0
    # no flops: always HBM
    r = bench.roofline_entry("k", nbytes=8e9, flops=0, kernel_us=1e6, traffic=None)
    assert r["bound"] == "hbm" and r["frac"] == pytest.approx(1e-3)


def test_expert_byte_counts_follow_the_layout():
    # int4 codes (two per byte) and one bf16 scale per 128 of K: gate and up
    # are 512 rows of K = 2048 each, down 2048 rows of K = 512
    gu = 2 * 512 * 2048 // 2 + 2 * 512 * (2048 // 128) * 2
    d = 2048 * 512 // 2 + 2048 * (512 // 128) * 2
    assert bench.EXPERT_GU_BYTES == gu
    assert bench.EXPERT_D_BYTES == d
    assert bench.EXPERT_BYTES == 1_622_016
    assert bench.ROUTER_BYTES == 256 * 2048 * 2
    assert bench.SHARED_BYTES == 3 * 1024 * 2048 * 2
    # NVFP4: the same code bytes, one E4M3 byte per 16 of K, one fp32 tensor scale per Linear
    assert bench.NV_GU_BYTES == 2 * 512 * 2048 // 2 + 2 * 512 * (2048 // 16) + 2 * 4
    assert bench.NV_D_BYTES == 2048 * 512 // 2 + 2048 * (512 // 16) + 4


@pytest.mark.parametrize("workload,T", [("decode_t1", 1), ("decode_t32", 32), ("prefill_t2048", 2048)])
def test_dominant_kernel_counters_match_the_sources(workload, T):
    traffic = bench.recorded_traffic(workload, "routed_gateup", T)
    assert traffic is not None, (f"profiles/hbm_traffic.txt holds no counters for {workload}'s gate/up kernel "
                                 "at the current source text: take FETCH_SIZE / WRITE_SIZE again")
    assert traffic > 0
