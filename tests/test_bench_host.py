"""Host logic of bench.py that sets the roofline's algorithmic work: the
attended (query, key) pairs of causal and sliding-window attention, against
brute-force counting."""
import bench


def brute_pairs(T, window):
    return sum(1 for i in range(T) for j in range(i + 1) if window is None or j > i - window)


def test_attention_pairs_brute_force():
    for T in (1, 2, 7, 64, 130, 700):
        for window in (None, 1, 3, 64, 512, 4096):
            assert bench.attention_pairs(T, window) == brute_pairs(T, window), (T, window)


def test_attention_pairs_beam_shapes():
    # T = 8192: the global layer attends to 8192*8193/2 pairs; a 512-token window to
    # 512*513/2 pairs in the first 512 rows and 512 per row after
    assert bench.attention_pairs(8192, None) == 33_558_528
    assert bench.attention_pairs(8192, 512) == 512 * 513 // 2 + (8192 - 512) * 512


def test_gateup_roofline_accounting():
    # decode: 222 touched experts' gate and up weights, x in, h out; HBM-bound
    r = bench.gateup_roofline("none", 64, 5120, 2560, 8, 222, 2, 1.0)
    assert r["algorithmic_per_launch"]["bytes"] == 222 * 2 * 2560 * 5120 * 2 + 64 * 5120 * 2 + 512 * 2560 * 2
    assert r["algorithmic_per_launch"]["flops"] == 64 * 8 * 4 * 5120 * 2560
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["achieved"] - r["algorithmic_per_launch"]["bytes"] / 1e-3 / 1e9) < 0.1
    # prefill: 256 FLOP per byte is below the 312.5 ridge only by the weights;
    # at T = 16384 the launch is above it and reported against the MFMA peak
    r = bench.gateup_roofline("none", 16384, 5120, 2560, 8, 256, 2, 2.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert abs(r["achieved"] - 16384 * 8 * 4 * 5120 * 2560 / 2e-3 / 1e12) < 0.1


def test_expert_load_stats():
    import numpy as np
    # an exact power law load(r) = 1000 r^-1.1 is fitted back to s = 1.1
    loads = 1000.0 * np.arange(1, 65, dtype=np.float64) ** -1.1
    st = bench.expert_load(np.concatenate([loads, np.zeros(8)]))
    assert abs(st["fitted_zipf_s"] - 1.1) < 1e-9
    assert st["max"] == 1000 and st["top5"][0] == 1000
    st = bench.expert_load([3, 0, 5, 5])
    assert st["max"] == 5 and st["min_active"] == 3 and st["mean"] == 3.25


def test_bench_refuses_several_gpus():
    """One GPU only: `--gpus N` above 1 exits with status 2 and says why, before
    any device work."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert "one GPU only" in r.stderr and r.stdout == ""
