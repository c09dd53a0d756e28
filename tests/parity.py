"""Parity helpers shared by the GPU tests: compare the HIP path with the oracle.

Acceptance rules:
  * a token whose oracle selection margin (min of the group-boundary and the
    expert-boundary score gap) is below 1e-6 has several valid selections; it
    is excluded and reported;
  * selected ids are compared as sets per token (bit-exact), counts after
    dropping excluded tokens' assignments on both sides (bit-exact); an
    excluded token's selection must still be one of its valid selections
    within the margin;
  * routing weights |w_gpu - w_oracle| <= W_TOL per (token, expert), every
    token, against the oracle's scores at the GPU's own ids;
  * outputs: relative L2 <= 5e-3 and max abs <= 2e-2 * RMS(oracle), over
    non-excluded tokens.
"""
import itertools

import numpy as np
import torch

import oracle as O
from moe_inputs import bf16_bits

MARGIN = 1e-6
REL_L2 = 5e-3
MAX_ABS_RMS = 2e-2
W_TOL = 1e-6


def keep_mask(ref, margin=MARGIN):
    return ref["margin"] >= margin


def selection_valid(sel, s, groups, topk_groups, k, delta=MARGIN):
    """True when the k experts `sel` are a group-limited top-k of the scores
    s [E] under some resolution of near-ties: there is a set G of
    `topk_groups` groups, containing every group of `sel`, whose scores (sum
    of the two best in the group) are all >= every other group's score minus
    delta, and every selected score is >= every other score inside G minus
    delta.  With delta = 0 and distinct scores only the exact selection
    passes; the group-limited rule is the one of page "Willkommen Beam",
    section "Mixture of Experts"."""
    s = np.asarray(s, dtype=np.float64)
    E = s.size
    gsz = E // groups
    sel = [int(e) for e in sel]
    if len(sel) != k or len(set(sel)) != k or min(sel) < 0 or max(sel) >= E:
        return False
    gs = np.sort(s.reshape(groups, gsz), axis=1)[:, -2:].sum(axis=1)
    need = sorted({e // gsz for e in sel})
    if len(need) > topk_groups:
        return False
    others = [g for g in range(groups) if g not in need]
    chosen = np.zeros(E, dtype=bool)
    chosen[sel] = True
    for extra in itertools.combinations(others, topk_groups - len(need)):
        G = set(need) | set(extra)
        dropped = [g for g in range(groups) if g not in G]
        if dropped and min(gs[g] for g in G) < max(gs[g] for g in dropped) - delta:
            continue
        elig = np.repeat(np.isin(np.arange(groups), list(G)), gsz)
        rest = s[elig & ~chosen]
        if rest.size and s[chosen].min() < rest.max() - delta:
            continue
        return True
    return False


def check_routing(ids_gpu, w_gpu, ref, shape, counts_gpu=None):
    """ids/weights of the HIP router vs the oracle (`ref` holds the oracle's
    scores "s", ids, weights and margins); returns a stats dict.

    Tokens at or above the margin: ids equal the oracle's as sets.  Tokens
    below it (several valid selections): the GPU's selection must be one of
    the valid ones within the margin (selection_valid).  Every token's
    weights must equal scale * s / sum(s) of the oracle's scores at the
    GPU's own ids, within W_TOL."""
    E = shape.E
    ids_g = ids_gpu.cpu().numpy().astype(np.int64)
    w_g = w_gpu.cpu().numpy().astype(np.float64)
    s = np.asarray(ref["s"], dtype=np.float64)
    keep = keep_mask(ref)
    T = ids_g.shape[0]
    # ids per token distinct and in range
    assert ids_g.min() >= 0 and ids_g.max() < E
    for t in range(T):
        assert len(set(ids_g[t].tolist())) == ids_g.shape[1]
    for t in np.nonzero(keep)[0]:
        sg, so = set(ids_g[t].tolist()), set(ref["ids"][t].tolist())
        assert sg == so, f"token {t}: gpu ids {sorted(sg)} != oracle {sorted(so)}"
    differ = []
    for t in np.nonzero(~keep)[0]:
        assert selection_valid(ids_g[t], s[t], shape.groups, shape.topk_groups, shape.k, MARGIN), \
            f"excluded token {t}: gpu ids {sorted(ids_g[t].tolist())} are no valid selection"
        if set(ids_g[t].tolist()) != set(ref["ids"][t].tolist()):
            differ.append(int(t))
    sel = np.take_along_axis(s, ids_g, axis=1)
    w_ref = shape.scale * (sel / sel.sum(axis=1, keepdims=True))
    err = np.abs(w_g - w_ref)
    max_w = float(err.max()) if err.size else 0.0
    assert max_w <= W_TOL, f"max weight error {max_w:.3e}"
    stats = dict(excluded=int((~keep).sum()), excluded_tokens=np.nonzero(~keep)[0].tolist(),
                 excluded_with_other_valid_selection=differ, max_weight_err=max_w)
    if counts_gpu is not None:
        cg = counts_gpu.cpu().numpy().astype(np.int64)
        # full counts: histogram of the GPU's own ids (exact)
        assert np.array_equal(cg, np.bincount(ids_g.reshape(-1), minlength=E))
        # against the oracle after dropping excluded tokens on both sides
        kg = np.bincount(ids_g[keep].reshape(-1), minlength=E)
        ko = np.bincount(ref["ids"][keep].reshape(-1), minlength=E)
        assert np.array_equal(kg, ko)
    return stats


def check_output(y_gpu, y_ref, keep=None, out_rounding_slack=False):
    """rel-L2 and max-abs/RMS of the bf16 device output against the unrounded
    oracle output.  With out_rounding_slack each element may also differ by
    half a bf16 ulp of the oracle value: the output is bf16, and for one-expert
    outputs (k = 1) the tails reach ~12 RMS, where half an ulp alone is
    2.3e-2 RMS."""
    yg = O.bf16_bits_to_f64(bf16_bits(y_gpu))
    yo = np.asarray(y_ref, dtype=np.float64)
    if keep is not None:
        yg, yo = yg[keep], yo[keep]
    assert np.all(np.isfinite(yg))
    rms = np.sqrt(np.mean(yo ** 2))
    rel = np.linalg.norm(yg - yo) / max(np.linalg.norm(yo), 1e-300)
    err = np.abs(yg - yo)
    if out_rounding_slack:
        # half a bf16 ulp: |v| = m 2^e with m in [0.5, 1) has an ulp of 2^(e-8)
        _, ex = np.frexp(yo)
        err = np.maximum(err - np.ldexp(1.0, ex - 9), 0.0)
    mx = err.max() / max(rms, 1e-300) if yo.size else 0.0
    assert rel <= REL_L2, f"rel-L2 {rel:.3e}"
    assert mx <= MAX_ABS_RMS, f"max-abs/RMS {mx:.3e}"
    return dict(rel_l2=float(rel), max_abs_over_rms=float(mx))


def expert_fetcher(wg, wu, wd):
    """Oracle expert source that copies one expert's weights from the device."""
    def get(e):
        return bf16_bits(wg[e]), bf16_bits(wu[e]), bf16_bits(wd[e])
    return get


def oracle_route(x, wr, shape, offset=None):
    """Oracle routing of all tokens (cheap: one FP64 GEMM and a sort)."""
    z = O.router_logits(bf16_bits(x), bf16_bits(wr),
                        None if offset is None else offset.cpu().numpy())
    s = O.sigmoid(z)
    ids, w, m_g, m_e = O.group_limited_topk(s, shape.groups, shape.topk_groups, shape.k, shape.scale)
    return dict(s=s, ids=ids, weights=w, margin=np.minimum(m_g, m_e))


def sample_tokens(keep, n, seed=0):
    """n evenly spread non-excluded tokens (deterministic)."""
    idx = np.nonzero(keep)[0]
    if idx.size <= n:
        return idx
    pos = np.linspace(0, idx.size - 1, n).round().astype(np.int64)
    return idx[pos]


def oracle_block_rows(x, tokens, wr, wg, wu, wd, shape, offset=None):
    """Oracle block for a subset of token rows (the block is per-token)."""
    xb = bf16_bits(x)[tokens]
    return O.moe_block(xb, bf16_bits(wr), expert_fetcher(wg, wu, wd), shape.groups,
                       shape.topk_groups, shape.k, shape.scale,
                       None if offset is None else offset.cpu().numpy())


def sync():
    torch.cuda.synchronize()
