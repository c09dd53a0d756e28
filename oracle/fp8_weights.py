"""FP8 (OCP E4M3) expert-weight encoding -- TEST INFRASTRUCTURE ONLY.

The Beam pages say that an FP8 checkpoint of the model exists, meant for
GPUs older than Blackwell (page "Reflection 发布 501B 开放模型 Beam，支持自托管
定制与扩展" (sihot.dev), sections 混合专家（Mixture of Experts） and 硬件要求),
but not its scaling scheme.  The encoding
checked here is this repository's reading, written from the format's
definition:

  * E4M3 ("fn": finite, no infinities): sign bit, 4 exponent bits with bias 7,
    3 mantissa bits.  Exponent field 0 holds subnormals m/8 * 2^-6; fields
    1..15 hold normals (1 + m/8) * 2^(E-7), except field 15 with m = 7, which
    is NaN.  The largest finite value is 448.
  * One power-of-two scale per output row (per expert, per matrix): the
    smallest integer e with max_k |W[r,k]| <= 448 * 2^e (e = 0 for an all-zero
    row).  Scaling a bf16 value by 2^-e is exact, so the code of every weight
    is a deterministic function of the bf16 input.
  * code = E4M3 value nearest to W[r,k] * 2^-e, ties to the even mantissa.
  * dequantised weight = value(code) * 2^e.

Pins (tests/test_oracle_fp8.py): the decode table and the rounding against
torch's float8_e4m3fn conversion, and the scale rule's minimality.  The
choice of scheme itself is not fixed by the pages ("parity unpinned" against
them); a layer computed with these weights is checked against the oracle
block run on the dequantised weights.
"""
from __future__ import annotations

import numpy as np

from .beam_moe_oracle import bf16_bits_to_f64

__all__ = ["E4M3_MAX", "e4m3_decode", "e4m3_round", "row_scale_exponents",
           "quantize_rows", "dequantize_rows"]

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each E4M3 code (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = m / 8.0 * 2.0 ** -6
    nrm = (1.0 + m / 8.0) * np.exp2(ef.astype(np.float64) - 7.0)
    v = sign * np.where(ef == 0, sub, nrm)
    return np.where((ef == 15) & ((c & 0x7) == 7), np.nan, v)


def e4m3_round(v) -> np.ndarray:
    """Code of the E4M3 value nearest to v (|v| <= 448), ties to even."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > E4M3_MAX):
        raise ValueError("value outside the E4M3 range")
    # subnormal range: grid step 2^-9; r = 8 lands exactly on the smallest
    # normal 2^-6, whose code is also 8
    r_sub = np.rint(a / 2.0 ** -9)
    # normal range: exponent of a in [2^E, 2^(E+1)), grid step 2^(E-3)
    _, x = np.frexp(np.where(a > 0, a, 1.0))
    E = x.astype(np.int64) - 1
    r = np.rint(a / np.exp2((E - 3).astype(np.float64)))  # 8 .. 16
    carry = r >= 16
    E = np.where(carry, E + 1, E)
    r = np.where(carry, 8, r)
    code_n = ((E + 7) << 3) | (r.astype(np.int64) - 8)
    code = np.where(a < 2.0 ** -6, r_sub.astype(np.int64), code_n)
    code = np.where(np.signbit(v), code | 0x80, code)
    return code.astype(np.uint8)


def row_scale_exponents(w_bits) -> np.ndarray:
    """Per row: smallest integer e with max|w| <= 448 * 2^e (0 for zero rows)."""
    w = bf16_bits_to_f64(np.asarray(w_bits, dtype=np.uint16))
    amax = np.max(np.abs(w), axis=-1)
    f, x = np.frexp(np.where(amax > 0, amax, 1.0))   # amax = f * 2^x, f in [0.5, 1)
    # 448 = 0.875 * 2^9:  amax <= 0.875 * 2^(9+e)  <=>  e >= x - 9 + [f > 0.875]
    e = x.astype(np.int64) - 9 + (f > 0.875)
    return np.where(amax > 0, e, 0).astype(np.int32)


def quantize_rows(w_bits):
    """(codes uint8 [..., N, K], exponents int32 [..., N]) of bf16 weights."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    e = row_scale_exponents(w_bits)
    w = bf16_bits_to_f64(w_bits)
    v = w * np.exp2(-e.astype(np.float64))[..., None]
    return e4m3_round(v), e


def dequantize_rows(codes, exps) -> np.ndarray:
    """float64 weights value(code) * 2^e."""
    return e4m3_decode(codes) * np.exp2(np.asarray(exps, dtype=np.float64))[..., None]
