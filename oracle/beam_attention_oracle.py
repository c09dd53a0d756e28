"""Plain FP64 CPU oracle for one Beam attention sublayer (prefill of one
sequence) -- TEST INFRASTRUCTURE ONLY.

Used by tests/, the smoke check and the benchmark's CPU-baseline leg.  It
shares no code with the HIP path and never imports it.

Sources (cited by page title and section):
  [ATT]  "Willkommen Beam: ein offenes 501B-Modell, das Sie besitzen, anpassen
         und skalieren können" (spke.com), section "Attention" (and its
         paragraph on the attention block of both layer types); the same
         paragraphs on "Reflection 发布 501B 开放模型 Beam，支持自托管定制与扩展"
         (sihot.dev).
  [LONG] the same page, section "Long Context" (2 x 8 KV heads x 128 dims
         cached per token, which fixes the head size at 128).
  [RES]  the same page, section "Residual Stream" (RoPE and the query scaling
         are computed in FP32; every sublayer is normalised).

What the pages fix, restated:
  * hidden size 5120; grouped-query attention with 48 query heads and 8
    key/value heads of 128 dims; RMSNorm on queries and keys;
  * most layers attend over a sliding window of the previous 512 tokens and
    use RoPE; every sixth and the last layer attend over the whole context,
    use no position encoding, and multiply each query by
    (1 + (pos + 1) / 2048) ** 0.1;
  * a learned sigmoid gate computed from the layer input scales every
    channel of every head before the output projection.

Readings where the pages are silent (each listed in the design notes):
  * projections are bias-free nn.Linear layouts: Wq [48*128, H], Wk and Wv
    [8*128, H], the gate Wg [48*128, H], Wo [H, 48*128];
  * query head h reads key/value head h // 6 (contiguous groups of 6);
  * RMSNorm over the 128 dims of each head, eps 1e-6, unit gain, applied
    before RoPE / the query scaling;
  * RoPE rotates dims (i, i + 64) by pos * theta**(-i/64), theta = 10000,
    all 128 dims (the pages give no base);
  * a window of W tokens admits keys j with i - W < j <= i (the token itself
    is one of the W); scores are scaled by 1/sqrt(128);
  * rounding points mirror what the device computes on: the normalised and
    rotated (or scaled) q and k, v, and the gated head outputs are rounded
    once to bf16 (they are bf16 MFMA operands); projections, norms, softmax
    and gate stay in high precision; the output y is returned unrounded.

Pins (tests/test_oracle_attention.py): RoPE preserves pair norms, is the
identity at position 0 and depends only on relative positions in q.k;
per-head RMSNorm against torch's rms_norm; the query scaling's closed form
at pos + 1 = 2048; attention against a brute-force double loop with the
key/value heads repeated (plain multi-head attention) on small shapes, a
single key (output = v), identical keys (window mean), window 1 (output =
own v) and window >= T (= full causal); a zero gate weight halves the output.
"Parity unpinned" applies to the absolute output values: no page prints any.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from .beam_moe_oracle import bf16_bits_to_f64, f64_to_bf16_bits, round_to_bf16

__all__ = [
    "ATT_Q_HEADS", "ATT_KV_HEADS", "ATT_HEAD_DIM", "ATT_WINDOW",
    "head_rmsnorm", "rope", "query_scale", "attention_core",
    "attention_sublayer",
]

ATT_Q_HEADS = 48
ATT_KV_HEADS = 8
ATT_HEAD_DIM = 128
ATT_WINDOW = 512


def head_rmsnorm(v: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm over the last axis (one head's dims), unit gain, float64."""
    v = np.asarray(v, dtype=np.float64)
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)


def rope(x: np.ndarray, pos: np.ndarray, theta: float = 10000.0) -> np.ndarray:
    """Rotate pairs (i, i + D/2) of the last axis by pos * theta**(-2i/D).

    x: [..., T, heads, D]; pos: [T] token positions.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / D)     # [half]
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]   # [T, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def query_scale(pos) -> np.ndarray:
    """Scalable-softmax query scaling of the global layers: (1 + (pos+1)/2048)^0.1."""
    return (1.0 + (np.asarray(pos, dtype=np.float64) + 1.0) / 2048.0) ** 0.1


def attention_core(q: np.ndarray, k: np.ndarray, v: np.ndarray, window: Optional[int],
                   q_pos: Optional[Sequence[int]] = None) -> np.ndarray:
    """Causal (optionally windowed) grouped-query attention in float64.

    q: [Tq, Hq, D] for the query positions q_pos (default 0..Tq-1);
    k, v: [Tk, Hkv, D] for positions 0..Tk-1.  Query head h reads key/value
    head h // (Hq // Hkv).  Returns o: [Tq, Hq, D].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, Hq, D = q.shape
    Tk, Hkv, _ = k.shape
    rep = Hq // Hkv
    qp = np.arange(Tq) if q_pos is None else np.asarray(q_pos)
    kp = np.arange(Tk)
    allowed = kp[None, :] <= qp[:, None]
    if window is not None:
        allowed &= kp[None, :] > qp[:, None] - window
    o = np.empty((Tq, Hq, D))
    scale = 1.0 / math.sqrt(D)
    for h in range(Hq):
        g = h // rep
        s = (q[:, h, :] @ k[:, g, :].T) * scale                    # [Tq, Tk]
        s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        o[:, h, :] = p @ v[:, g, :]
    return o


def attention_sublayer(u_bits, wq_bits, wk_bits, wv_bits, wg_bits, wo_bits, global_layer: bool,
                       window: int = ATT_WINDOW, theta: float = 10000.0, eps: float = 1e-6,
                       rows: Optional[Sequence[int]] = None) -> dict:
    """One attention sublayer over a sequence of T tokens at positions 0..T-1.

    u: [T, H] bf16 bits (the normalised layer input).  Weights are bf16 bits in
    nn.Linear layout.  `rows` restricts the queries (and the output) to those
    token positions; keys and values are always computed for every token up
    to the last requested row.  Returns {"y": [R, H] float64 (unrounded),
    "rows": the positions}.
    """
    u = bf16_bits_to_f64(np.asarray(u_bits, dtype=np.uint16))
    T = u.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(sorted(set(int(r) for r in rows)))
    last = int(rows.max()) + 1 if rows.size else 0
    wq = bf16_bits_to_f64(wq_bits)
    wk = bf16_bits_to_f64(wk_bits)
    wv = bf16_bits_to_f64(wv_bits)
    wg = bf16_bits_to_f64(wg_bits)
    wo = bf16_bits_to_f64(wo_bits)
    Hq, Hkv, D = wq.shape[0] // ATT_HEAD_DIM, wk.shape[0] // ATT_HEAD_DIM, ATT_HEAD_DIM

    uk = u[:last]
    uq = u[rows]
    q = (uq @ wq.T).reshape(len(rows), Hq, D)
    k = (uk @ wk.T).reshape(last, Hkv, D)
    v = (uk @ wv.T).reshape(last, Hkv, D)
    gate = 1.0 / (1.0 + np.exp(-(uq @ wg.T)))                      # [R, Hq*D]

    qn = head_rmsnorm(q, eps)
    kn = head_rmsnorm(k, eps)
    if global_layer:
        qn = qn * query_scale(rows)[:, None, None]
    else:
        qn = rope(qn, rows, theta)
        kn = rope(kn, np.arange(last), theta)
    qn, kn, vr = round_to_bf16(qn), round_to_bf16(kn), round_to_bf16(v)
    o = attention_core(qn, kn, vr, None if global_layer else window, q_pos=rows)
    og = round_to_bf16(o.reshape(len(rows), Hq * D) * gate)
    return {"y": og @ wo.T, "rows": rows}
