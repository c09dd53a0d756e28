"""Pins of the FP8 (E4M3) weight encoding in the oracle against torch's
float8_e4m3fn conversion (a library routine) and the scale rule's definition."""
import numpy as np
import pytest
import torch

import oracle as O


def torch_codes(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_table_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert O.e4m3_decode([0x7E])[0] == O.E4M3_MAX


def test_rounding_matches_torch_on_random_ties_and_edges():
    rng = np.random.default_rng(3)
    grid = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))          # 0 .. 448
    mids = (grid[1:] + grid[:-1]) / 2                               # exact ties
    v = np.concatenate([
        rng.standard_normal(20000) * 30.0,
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 5000),                  # subnormal range
        grid, -grid, mids, -mids,
        np.nextafter(mids, 0), np.nextafter(mids, 1e9),
        [0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11],
    ])
    v = v[np.abs(v) <= 448.0].astype(np.float32).astype(np.float64)  # exactly fp32
    assert np.array_equal(O.e4m3_round(v), torch_codes(v))


def test_rounding_rejects_out_of_range():
    with pytest.raises(ValueError):
        O.e4m3_round([449.0])


def test_scale_exponent_is_minimal():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 10, (64, 1)))).astype(np.float32)
    bits = (torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    e = O.row_scale_exponents(bits)
    amax = np.max(np.abs(O.bf16_bits_to_f64(bits)), axis=1)
    assert np.all(amax <= 448.0 * np.exp2(e))
    assert np.all(amax > 448.0 * np.exp2(e - 1.0))
    # exact boundary: a row whose max is exactly 448 * 2^3 needs e = 3
    row = np.zeros((1, 8), np.float32); row[0, 2] = 448.0 * 8
    rb = torch.from_numpy(row).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert O.row_scale_exponents(rb)[0] == 3
    assert O.row_scale_exponents(np.zeros((1, 8), np.uint16))[0] == 0


def test_quantize_dequantize_error_bound():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((32, 512)) * 0.02).astype(np.float32)
    bits = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes, e = O.quantize_rows(bits)
    deq = O.dequantize_rows(codes, e)
    wf = O.bf16_bits_to_f64(bits)
    # nearest E4M3 value: error <= half a step, a step being 2^-3 of the
    # binade (2^-9 * 2^e in the subnormal range)
    step = np.maximum(np.exp2(np.floor(np.log2(np.maximum(np.abs(wf) * np.exp2(-e)[:, None], 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(deq - wf) <= 0.5 * step * np.exp2(e)[:, None] * (1 + 1e-12))
    # the row maximum keeps its binade: at least 224 after scaling
    assert np.all(np.max(np.abs(deq), axis=1) * np.exp2(-e) >= 224.0)
