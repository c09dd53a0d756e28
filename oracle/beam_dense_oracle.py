"""Plain FP64 CPU oracle for one Beam dense SwiGLU layer -- TEST
INFRASTRUCTURE ONLY.

Used by tests/ and the benchmark's CPU-baseline leg.  It shares no code with
the HIP path and never imports it.

Source: "Willkommen Beam: ein offenes 501B-Modell, das Sie besitzen, anpassen
und skalieren können" (spke.com), section "Mixture of Experts": the first
three layers are dense SwiGLU MLPs instead of expert layers; section
"Residual Stream": the SwiGLU product in FP32.

Reading where the pages are silent: the intermediate size is not given.  The
layer is taken as 20480 = 8 x 2560 wide (the per-token work of the 8 routed
experts); with the pages' total and active parameter counts this leaves
room for a vocabulary near 138k, so the counts agree with it.  Layouts,
rounding points and SiLU follow the expert of the MoE oracle: gate and up
unrounded, the product rounded once to bf16, the down output unrounded.

Pins (tests/test_oracle_dense.py): torch's SiLU and bf16 conversion of the
product; splitting the intermediate dimension into chunks and summing the
chunks' outputs gives the same result; zero input or a zero up projection
gives zero.  "Parity unpinned" applies to the absolute values (no page
prints any).
"""
from __future__ import annotations

import numpy as np

from .beam_moe_oracle import bf16_bits_to_f64, swiglu_expert

__all__ = ["DENSE_INTERMEDIATE", "dense_mlp"]

DENSE_INTERMEDIATE = 8 * 2560


def dense_mlp(x_bits, wg_bits, wu_bits, wd_bits) -> np.ndarray:
    """y = down( bf16( SiLU(gate x) * (up x) ) ) for rows x [T, H] (bf16 bits);
    gate, up [I, H] and down [H, I] as bf16 bits, or float64 values (weights
    already dequantised, e.g. from the FP8 encoding).  Returns y [T, H]
    float64, unrounded."""
    x = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))

    def widen(w):
        w = np.asarray(w)
        return w if w.dtype == np.float64 else bf16_bits_to_f64(w.astype(np.uint16))
    return swiglu_expert(x, widen(wg_bits), widen(wu_bits), widen(wd_bits), round_h=True)
