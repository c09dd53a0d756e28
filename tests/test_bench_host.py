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
