"""Fit the per-expert logit offsets of the skewed-load workload.

Writes moe_inputs/data/zipf_offsets_h5120_e256.txt.  Uses only the oracle's
router and selection (FP64) and the seeded input generator; run it as
`python -m oracle.calibrate_zipf_offsets` from the repository root.

Target: expert of Zipf rank r is picked by a fraction q_r = min(1, c * r**-1.1)
of tokens, with c chosen so that sum(q) = k = 8 (a token picks an expert at
most once, so the plain Zipf law is capped at 1 and the excess is spread over
the other ranks).  Offsets b are fitted on a seeded 4096-token calibration
batch by the multiplicative update b += 0.5 * (ln(q*Tc + 0.5) - ln(L + 0.5))
on the realised loads L, 200 times, clamped to [-8, 6] so the FP32 sigmoid
never saturates into ties.  b is kept in float32 throughout, because that is
the value both implementations receive.
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import moe_inputs as MI  # noqa: E402
from oracle import beam_moe_oracle as O  # noqa: E402

E, H, G, KG, K = 256, 5120, 8, 4, 8
TC = 4096
ZIPF_S = 1.1
ITERS = 200


def water_filled_targets(ranks: np.ndarray, total: float, s: float) -> np.ndarray:
    base = ranks.astype(np.float64) ** (-s)
    lo, hi = 0.0, 1e6
    for _ in range(200):
        c = 0.5 * (lo + hi)
        if np.minimum(1.0, c * base).sum() > total:
            hi = c
        else:
            lo = c
    return np.minimum(1.0, lo * base)


def main(out_path=MI.ZIPF_OFFSETS_FILE):
    ranks = MI.zipf_rank_permutation(E)
    q = water_filled_targets(ranks, K, ZIPF_S)
    x = MI.bf16_bits(MI.zipf_calibration_x(TC, H))
    wr = MI.bf16_bits(MI.make_router(E, H))
    z0 = O.router_logits(x, wr)
    b = np.zeros(E, dtype=np.float32)
    for it in range(ITERS):
        s = O.sigmoid(z0 + b.astype(np.float64)[None, :])
        ids, _, _, _ = O.group_limited_topk(s, G, KG, K, 2.5)
        load = np.bincount(ids.reshape(-1), minlength=E).astype(np.float64)
        step = 0.5 * (np.log(q * TC + 0.5) - np.log(load + 0.5))
        b = np.clip(b.astype(np.float64) + step, -8.0, 6.0).astype(np.float32)
    s = O.sigmoid(z0 + b.astype(np.float64)[None, :])
    ids, _, m_g, m_e = O.group_limited_topk(s, G, KG, K, 2.5)
    load = np.bincount(ids.reshape(-1), minlength=E)
    order = np.argsort(ranks)
    print("target loads (rank 1..8):", np.round(q[order][:8] * TC, 1).tolist())
    print("realised loads (rank 1..8):", load[order][:8].tolist())
    print("max/mean load: %.2f" % (load.max() / load.mean()))
    print("tokens under 1e-6 margin:", int((np.minimum(m_g, m_e) < 1e-6).sum()))
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        f.write("# per-expert fp32 logit offsets, skewed-load workload (Zipf s=1.1 over 256 experts)\n")
        f.write("# written by oracle/calibrate_zipf_offsets.py; one value per expert, expert 0 first\n")
        for v in b:
            f.write("%.9g\n" % float(v))
    return b


if __name__ == "__main__":
    main()
