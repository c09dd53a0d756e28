"""Plain FP64 CPU oracle for one Beam Mixture-of-Experts block.

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the benchmark's
CPU-baseline leg.  It shares no code with the HIP path and never imports it.

Sources (cited by page title and section):
  [MoE]  "Willkommen Beam: ein offenes 501B-Modell, das Sie besitzen, anpassen
         und skalieren können" (spke.com), section "Mixture of Experts"; the
         same paragraph on "Reflection 发布 501B 开放模型 Beam，支持自托管定制与扩展"
         (sihot.dev), section 混合专家（Mixture of Experts）.
  [RES]  the same pages, section "Residual Stream" / 残差流（Residual Stream）.

What the pages fix, restated:
  * [MoE] every one of the 256 experts is scored with a sigmoid; the experts
    are split into 8 groups of 32; a group is ranked by the sum of its two
    best scores; the best 4 groups are kept; the 8 best experts inside the
    kept groups are chosen.  Each expert is a SwiGLU MLP with intermediate
    size 2560 (hidden size 5120 from section "Attention").  There is no
    shared expert.  Expert outputs are combined with the router weights after
    normalisation, and the result is multiplied by 2.5.
  * [RES] the router and the SwiGLU product are computed in FP32; every
    sublayer is normalised before and after; the residual stream counts the
    embedding as step 1 and at step k keeps sqrt((k-1)/k) of the stream and
    adds 1/sqrt(k) of the sublayer output.

Readings where the pages are silent:
  groups are contiguous blocks of E/groups experts; exact ties go to the lower
  index; normalisation is over the k selected sigmoid scores with no epsilon,
  and the 2.5 is folded into the returned weights; no router or expert bias;
  nn.Linear layouts Wr [E,H], gate/up [E,I,H], down [E,H,I]; gate and up stay
  unrounded, the SwiGLU product h is rounded once to bf16 (the down
  projection consumes bf16), the down output stays unrounded; RMSNorm uses
  eps = 1e-6 and unit gain.  An optional per-expert fp32 logit offset is added
  to the router logit before the sigmoid (the skewed-load workload).

Pins (tests/test_oracle_*.py): brute-force enumeration of the selection,
sum of weights = scale, single expert => scale * SwiGLU_e(x) against torch's
SiLU, exactly-rounded router sums (math.fsum), bf16 rounding against torch's
conversion, residual closed form, and the parameter counts printed on the
pages.  "Parity unpinned" applies only to the absolute output values, which
no page prints for any input.
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence, Tuple, Union

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "round_to_bf16",
    "router_logits", "sigmoid", "group_scores", "group_limited_topk",
    "expert_major_order", "swiglu_expert", "moe_forward", "moe_block",
    "rmsnorm", "residual_step", "stack_sublayer", "selection_margin",
    "expert_param_count",
]


# --------------------------------------------------------------------------
# bf16 <-> fp64 (exact widening; round-to-nearest-even narrowing)
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even) in one step.

    bf16 keeps 8 significant bits and the fp32 exponent range.  A finite value
    v = m * 2**e (0.5 <= |m| < 1) has quantum 2**(e-8); below the smallest
    normal (2**-126) the quantum is fixed at 2**-133.  np.rint rounds halves to
    even.  Results of magnitude >= 2**128 become infinity.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    finite = np.isfinite(v)
    _, e = np.frexp(np.where(finite, v, 1.0))
    e = np.maximum(e, -125)
    q = np.ldexp(1.0, e - 8)
    r = np.rint(np.where(finite, v, 0.0) / q) * q
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
    r = np.where(finite, r, v)
    bits32 = r.astype(np.float32).view(np.uint32)
    out[...] = (bits32 >> np.uint32(16)).astype(np.uint16)
    out[np.isnan(v)] = np.uint16(0x7FC0)
    return out


def round_to_bf16(v) -> np.ndarray:
    """Nearest bf16 value of each float64, returned as float64."""
    return bf16_bits_to_f64(f64_to_bf16_bits(v))


# --------------------------------------------------------------------------
# Router and group-limited selection  ([MoE]; FP32 rule from [RES])
# --------------------------------------------------------------------------

def router_logits(x_bits, wr_bits, logit_offset=None) -> np.ndarray:
    """z[t, e] = sum_h x[t, h] * Wr[e, h]  (+ offset[e]), in float64.

    Each bf16*bf16 product is exact in float64; the float64 sum of H <= 8192
    such products is within a few ulp of the exact value.
    """
    x = bf16_bits_to_f64(x_bits)
    wr = bf16_bits_to_f64(wr_bits)
    z = x @ wr.T
    if logit_offset is not None:
        off = np.asarray(logit_offset, dtype=np.float32).astype(np.float64)
        z = z + off[None, :]
    return z


def sigmoid(z) -> np.ndarray:
    """Logistic function 1 / (1 + exp(-z)) in float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def group_scores(s: np.ndarray, groups: int) -> np.ndarray:
    """Score of each contiguous expert group: the sum of its two largest scores."""
    T, E = s.shape
    gsz = E // groups
    top2 = np.sort(s.reshape(T, groups, gsz), axis=2)[:, :, gsz - 2:]
    return top2[:, :, 1] + top2[:, :, 0]


def _descending_order(v: np.ndarray) -> np.ndarray:
    """Indices sorting each row by decreasing value; equal values keep index order."""
    return np.argsort(-v, axis=1, kind="stable")


def group_limited_topk(s: np.ndarray, groups: int, topk_groups: int, k: int,
                       scale: float):
    """Group-limited top-k of [MoE] on sigmoid scores s [T, E].

    Returns (ids [T,k] int64 ordered by decreasing score, weights [T,k] float64
    = scale * (s_sel / sum(s_sel)), group_margin [T], expert_margin [T]).
    Margins are the score gaps at the two selection boundaries (inf when the
    boundary does not exist); a token whose smaller margin is tiny has several
    equally valid selections.
    """
    s = np.asarray(s, dtype=np.float64)
    T, E = s.shape
    gsz = E // groups
    gs = group_scores(s, groups)                                  # [T, G]
    gorder = _descending_order(gs)
    kept = gorder[:, :topk_groups]                                # [T, KG]
    gs_sorted = np.take_along_axis(gs, gorder, axis=1)
    if topk_groups < groups:
        m_g = gs_sorted[:, topk_groups - 1] - gs_sorted[:, topk_groups]
    else:
        m_g = np.full(T, np.inf)

    keep = np.zeros((T, groups), dtype=bool)
    np.put_along_axis(keep, kept, True, axis=1)
    eligible = np.repeat(keep, gsz, axis=1)                       # [T, E]
    s_elig = np.where(eligible, s, -np.inf)
    eorder = _descending_order(s_elig)
    ids = eorder[:, :k]
    s_sorted = np.take_along_axis(s_elig, eorder, axis=1)
    n_elig = topk_groups * gsz
    if k < n_elig:
        m_e = s_sorted[:, k - 1] - s_sorted[:, k]
    else:
        m_e = np.full(T, np.inf)

    sel = np.take_along_axis(s, ids, axis=1)
    denom = sel.sum(axis=1, keepdims=True)
    assert np.all(denom > 0.0), "sum of selected sigmoid scores must be positive"
    # normalise first, then scale: the page describes normalised router
    # weights that are afterwards multiplied by the scale
    w = scale * (sel / denom)
    return ids.astype(np.int64), w, m_g, m_e


def selection_margin(m_g: np.ndarray, m_e: np.ndarray) -> np.ndarray:
    return np.minimum(m_g, m_e)


# --------------------------------------------------------------------------
# Token permutation (definition: stable sort of assignments by expert id)
# --------------------------------------------------------------------------

def expert_major_order(ids: np.ndarray, E: int):
    """Expert-major order of the (token, slot) assignments.

    Assignment a = t*k + j goes to expert ids[t, j].  Sorting assignments by
    expert with a stable sort keeps ascending token order inside an expert.
    Returns counts [E], offsets [E+1], sorted_tokens [n] (token of each
    expert-major row) and row_of [T*k] (row of each assignment; -1 for an id
    outside [0, E), which is dropped).
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    a_valid = np.nonzero(valid)[0]
    order = a_valid[np.argsort(flat[a_valid], kind="stable")]
    sorted_tokens = order // k
    row_of = np.full(T * k, -1, dtype=np.int64)
    row_of[order] = np.arange(order.size)
    return counts, offsets, sorted_tokens, row_of


# --------------------------------------------------------------------------
# Experts and combine ([MoE]; SwiGLU product in FP32 per [RES])
# --------------------------------------------------------------------------

def swiglu_expert(x_rows: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
                  round_h: bool = True) -> np.ndarray:
    """One SwiGLU expert on float64 rows: down( SiLU(gate x) * (up x) ).

    gate, up: [I, H]; down: [H, I]; SiLU(g) = g / (1 + exp(-g)).  With
    round_h the product is rounded to bf16 before the down projection.
    """
    g = x_rows @ wg.T
    u = x_rows @ wu.T
    with np.errstate(over="ignore"):
        h = g / (1.0 + np.exp(-g)) * u
    if round_h:
        h = round_to_bf16(h)
    return h @ wd.T


ExpertSource = Union[Tuple[np.ndarray, np.ndarray, np.ndarray],
                     Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]]


def _widen(w):
    """bf16 bit patterns -> float64; float64 weights (already dequantised,
    e.g. FP8-encoded experts) pass through unchanged."""
    w = np.asarray(w)
    return w if w.dtype == np.float64 else bf16_bits_to_f64(w)


def _expert_getter(experts: ExpertSource):
    """Per-expert float64 weights from bf16-bit arrays or a callable (which
    may also return float64 weights)."""
    if callable(experts):
        def get(e):
            wg, wu, wd = experts(e)
            return _widen(wg), _widen(wu), _widen(wd)
        return get
    wg_b, wu_b, wd_b = experts

    def get(e):
        return bf16_bits_to_f64(wg_b[e]), bf16_bits_to_f64(wu_b[e]), bf16_bits_to_f64(wd_b[e])
    return get


def moe_forward(x_bits, ids, weights, experts: ExpertSource, E: int,
                round_h: bool = True) -> np.ndarray:
    """y[t] = sum_j weights[t, j] * expert_{ids[t,j]}(x[t]) in float64.

    `weights` already include the scale.  Ids outside [0, E) add nothing.
    Weights of each expert are fetched once (streaming large models).
    """
    x = bf16_bits_to_f64(x_bits)
    ids = np.asarray(ids, dtype=np.int64)
    w = np.asarray(weights, dtype=np.float64)
    T, k = ids.shape
    H = x.shape[1]
    get = _expert_getter(experts)
    y = np.zeros((T, H), dtype=np.float64)
    contrib = np.zeros((T, k, H), dtype=np.float64)
    for e in np.unique(ids[(ids >= 0) & (ids < E)]):
        tt, jj = np.nonzero(ids == e)
        wg, wu, wd = get(int(e))
        contrib[tt, jj] = swiglu_expert(x[tt], wg, wu, wd, round_h=round_h)
    for j in range(k):
        y += w[:, j:j + 1] * contrib[:, j]
    return y


def moe_block(x_bits, wr_bits, experts: ExpertSource, groups: int, topk_groups: int,
              k: int, scale: float, logit_offset=None, round_h: bool = True) -> dict:
    """Whole block: router -> group-limited top-k -> experts -> combine."""
    wr_e = np.asarray(wr_bits).shape[0]
    z = router_logits(x_bits, wr_bits, logit_offset)
    s = sigmoid(z)
    ids, w, m_g, m_e = group_limited_topk(s, groups, topk_groups, k, scale)
    counts, offsets, sorted_tokens, row_of = expert_major_order(ids, wr_e)
    y = moe_forward(x_bits, ids, w, experts, wr_e, round_h=round_h)
    return dict(z=z, s=s, ids=ids, weights=w, group_margin=m_g, expert_margin=m_e,
                margin=selection_margin(m_g, m_e), counts=counts, offsets=offsets,
                sorted_tokens=sorted_tokens, row_of=row_of, y=y)


# --------------------------------------------------------------------------
# Sandwich norm and scaled residual ([RES])
# --------------------------------------------------------------------------

def rmsnorm(v: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """v / sqrt(mean(v^2) + eps) over the last axis, unit gain, float64."""
    v = np.asarray(v, dtype=np.float64)
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)


def residual_step(stream: np.ndarray, out: np.ndarray, step: int) -> np.ndarray:
    """Residual update at step `step` >= 2 (the embedding is step 1)."""
    if step < 2:
        raise ValueError("residual steps start at 2")
    return math.sqrt((step - 1) / step) * stream + out / math.sqrt(step)


def stack_sublayer(stream: np.ndarray, step: int, wr_bits, experts: ExpertSource,
                   groups: int, topk_groups: int, k: int, scale: float,
                   eps: float = 1e-6, moe_input_bits=None) -> dict:
    """One sandwich-normed MoE sublayer followed by the residual update.

    The MoE input is bf16(RMSNorm(stream)); `moe_input_bits` overrides it
    (teacher forcing with the device's own layer input).  Returns the block
    result plus the normalised output and the new stream.
    """
    if moe_input_bits is None:
        moe_input_bits = f64_to_bf16_bits(rmsnorm(stream, eps))
    blk = moe_block(moe_input_bits, wr_bits, experts, groups, topk_groups, k, scale)
    y_bf16 = round_to_bf16(blk["y"])
    out = rmsnorm(y_bf16, eps)
    blk["moe_input_bits"] = moe_input_bits
    blk["out"] = out
    blk["stream"] = residual_step(stream, out, step)
    return blk


# --------------------------------------------------------------------------
# Parameter arithmetic ([MoE]: about 39M parameters per expert)
# --------------------------------------------------------------------------

def expert_param_count(H: int, I: int) -> int:
    """Parameters of one bias-free SwiGLU expert: gate, up and down matrices."""
    return 3 * H * I
