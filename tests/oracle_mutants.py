"""Plausible mistakes planted in the oracle, one at a time, to show that its
pins (the oracle tests) catch each of them: a dropped term, a wrong sign,
index or exponent, a transposed operand, a rounding mode.  conftest.py applies
the one named by the environment variable BEAM_ORACLE_MUTANT before any test
module imports the oracle; nothing else imports this module's mutants."""
import math

import numpy as np

import oracle as O
import oracle.beam_attention_oracle as A
import oracle.beam_dense_oracle as D
import oracle.beam_moe_oracle as M
import oracle.fp8_weights as F8

MODULES = (M, A, D, F8, O)
MUTANTS = {}


def _patch(name, fn):
    """Replace `name` in every oracle module that binds it (the oracle's own
    functions call each other through their module globals)."""
    hit = [mod for mod in MODULES if hasattr(mod, name)]
    assert hit, name
    for mod in hit:
        setattr(mod, name, fn)


def mutant(f):
    MUTANTS[f.__name__] = f
    return f


def apply(name):
    MUTANTS[name]()


# ---- router and selection ([MoE])

@mutant
def router_drops_offset():
    orig = M.router_logits
    _patch("router_logits", lambda x_bits, wr_bits, logit_offset=None: orig(x_bits, wr_bits, None))


@mutant
def sigmoid_wrong_sign():
    _patch("sigmoid", lambda z: 1.0 / (1.0 + np.exp(np.asarray(z, dtype=np.float64))))


@mutant
def group_score_best_only():
    def gs(s, groups):
        T, E = s.shape
        return np.max(s.reshape(T, groups, E // groups), axis=2)
    _patch("group_scores", gs)


@mutant
def group_score_sums_all():
    def gs(s, groups):
        T, E = s.shape
        return np.sum(s.reshape(T, groups, E // groups), axis=2)
    _patch("group_scores", gs)


@mutant
def keeps_one_group_too_few():
    orig = M.group_limited_topk
    _patch("group_limited_topk",
           lambda s, groups, topk_groups, k, scale: orig(s, groups, max(topk_groups - 1, 1), k, scale))


@mutant
def weights_not_normalised():
    orig = M.group_limited_topk

    def f(s, groups, topk_groups, k, scale):
        ids, w, m_g, m_e = orig(s, groups, topk_groups, k, scale)
        sel = np.take_along_axis(np.asarray(s, dtype=np.float64), ids, axis=1)
        return ids, scale * sel, m_g, m_e
    _patch("group_limited_topk", f)


@mutant
def weights_scale_dropped():
    orig = M.group_limited_topk

    def f(s, groups, topk_groups, k, scale):
        ids, w, m_g, m_e = orig(s, groups, topk_groups, k, scale)
        return ids, w / scale, m_g, m_e
    _patch("group_limited_topk", f)


@mutant
def ties_resolved_to_last_index():
    _patch("_descending_order", lambda v: v.shape[1] - 1 - np.argsort(-v[:, ::-1], axis=1, kind="stable"))


# ---- permutation

@mutant
def expert_order_not_stable():
    orig = M.expert_major_order

    def f(ids, E):
        counts, offsets, sorted_tokens, row_of = orig(ids, E)
        st = sorted_tokens.copy()
        for e in range(E):   # reverse the token order inside each expert
            st[offsets[e]:offsets[e + 1]] = st[offsets[e]:offsets[e + 1]][::-1].copy()
        return counts, offsets, st, row_of
    _patch("expert_major_order", f)


# ---- experts and combine ([MoE], [RES])

@mutant
def silu_on_up_not_gate():
    def f(x_rows, wg, wu, wd, round_h=True):
        g = x_rows @ wg.T
        u = x_rows @ wu.T
        with np.errstate(over="ignore"):
            h = u / (1.0 + np.exp(-u)) * g
        if round_h:
            h = M.round_to_bf16(h)
        return h @ wd.T
    _patch("swiglu_expert", f)


@mutant
def h_not_rounded():
    orig = M.swiglu_expert
    _patch("swiglu_expert", lambda x_rows, wg, wu, wd, round_h=True: orig(x_rows, wg, wu, wd, round_h=False))


@mutant
def down_transposed():
    def f(x_rows, wg, wu, wd, round_h=True):
        g = x_rows @ wg.T
        u = x_rows @ wu.T
        with np.errstate(over="ignore"):
            h = g / (1.0 + np.exp(-g)) * u
        if round_h:
            h = M.round_to_bf16(h)
        return h @ wd.reshape(wd.shape[1], wd.shape[0])  # the right bytes, read as [I, H]
    _patch("swiglu_expert", f)


@mutant
def combine_ignores_weights():
    orig = M.moe_forward
    _patch("moe_forward", lambda x_bits, ids, weights, experts, E, round_h=True:
           orig(x_bits, ids, np.ones_like(np.asarray(weights, dtype=np.float64)), experts, E, round_h))


@mutant
def rmsnorm_sum_not_mean():
    _patch("rmsnorm", lambda v, eps=1e-6: np.asarray(v, dtype=np.float64) / np.sqrt(
        np.sum(np.asarray(v, dtype=np.float64) ** 2, axis=-1, keepdims=True) + eps))


@mutant
def residual_weights_swapped():
    def f(stream, out, step):
        if step < 2:
            raise ValueError("residual steps start at 2")
        return stream / math.sqrt(step) + math.sqrt((step - 1) / step) * out
    _patch("residual_step", f)


@mutant
def bf16_truncates():
    def f(v):
        v = np.asarray(v, dtype=np.float64)
        bits32 = v.astype(np.float32).view(np.uint32)
        out = (bits32 >> np.uint32(16)).astype(np.uint16)
        out[np.isnan(v)] = np.uint16(0x7FC0)
        return out
    _patch("f64_to_bf16_bits", f)
    _patch("round_to_bf16", lambda v: M.bf16_bits_to_f64(f(v)))


# ---- attention ([ATT], [LONG])

@mutant
def rope_rotates_backwards():
    orig = A.rope
    _patch("rope", lambda x, pos, theta=10000.0: orig(x, -np.asarray(pos, dtype=np.float64), theta))


@mutant
def rope_adjacent_pairs():
    def f(x, pos, theta=10000.0):
        x = np.asarray(x, dtype=np.float64)
        D_ = x.shape[-1]
        half = D_ // 2
        inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / D_)
        ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
        c = np.cos(ang)[:, None, :]
        s = np.sin(ang)[:, None, :]
        x1, x2 = x[..., 0::2], x[..., 1::2]
        out = np.empty_like(x)
        out[..., 0::2] = x1 * c - x2 * s
        out[..., 1::2] = x2 * c + x1 * s
        return out
    _patch("rope", f)


@mutant
def query_scale_without_plus_one():
    _patch("query_scale", lambda pos: (1.0 + np.asarray(pos, dtype=np.float64) / 2048.0) ** 0.1)


@mutant
def query_scale_wrong_exponent():
    _patch("query_scale", lambda pos: (1.0 + (np.asarray(pos, dtype=np.float64) + 1.0) / 2048.0) ** 0.01)


def _attention_core_variant(mask_fn=None, head_fn=None, use_scale=True):
    def f(q, k, v, window, q_pos=None):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        Tq, Hq, D_ = q.shape
        Tk, Hkv, _ = k.shape
        rep = Hq // Hkv
        qp = np.arange(Tq) if q_pos is None else np.asarray(q_pos)
        kp = np.arange(Tk)
        allowed = mask_fn(kp, qp, window)
        o = np.empty((Tq, Hq, D_))
        scale = 1.0 / math.sqrt(D_) if use_scale else 1.0
        for h in range(Hq):
            g = head_fn(h, rep, Hkv)
            s = (q[:, h, :] @ k[:, g, :].T) * scale
            s = np.where(allowed, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            o[:, h, :] = p @ v[:, g, :]
        return o
    return f


def _mask(kp, qp, window):
    m = kp[None, :] <= qp[:, None]
    if window is not None:
        m &= kp[None, :] > qp[:, None] - window
    return m


@mutant
def window_one_key_too_many():
    def mask(kp, qp, window):
        m = kp[None, :] <= qp[:, None]
        if window is not None:
            m &= kp[None, :] >= qp[:, None] - window
        return m
    _patch("attention_core", _attention_core_variant(mask, lambda h, rep, hkv: h // rep))


@mutant
def causal_mask_excludes_self():
    def mask(kp, qp, window):
        m = (kp[None, :] < qp[:, None]) | ((kp[None, :] == 0) & (qp[:, None] == 0))
        if window is not None:
            m &= kp[None, :] > qp[:, None] - window
        return m
    _patch("attention_core", _attention_core_variant(mask, lambda h, rep, hkv: h // rep))


@mutant
def gqa_heads_interleaved():
    _patch("attention_core", _attention_core_variant(_mask, lambda h, rep, hkv: h % hkv))


@mutant
def softmax_scale_missing():
    _patch("attention_core", _attention_core_variant(_mask, lambda h, rep, hkv: h // rep, use_scale=False))


@mutant
def head_norm_without_mean():
    _patch("head_rmsnorm", lambda v, eps=1e-6: np.asarray(v, dtype=np.float64) / np.sqrt(
        np.sum(np.asarray(v, dtype=np.float64) ** 2, axis=-1, keepdims=True) + eps))


# ---- FP8 weights (next row: E4M3 codes, power-of-two row scales)

@mutant
def e4m3_truncates():
    orig = F8.e4m3_round

    def f(v):
        v = np.asarray(v, dtype=np.float64)
        codes = orig(v)
        back = F8.e4m3_decode(codes)
        # step one code toward zero wherever nearest rounding went away from zero
        away = np.abs(back) > np.abs(v)
        return np.where(away & ((codes & 0x7F) > 0), codes - 1, codes).astype(np.uint8)
    _patch("e4m3_round", f)


@mutant
def e4m3_exponent_bias_8():
    orig = F8.e4m3_decode
    _patch("e4m3_decode", lambda codes: orig(codes) / 2.0)


@mutant
def scale_exponent_one_too_large():
    orig = F8.row_scale_exponents
    _patch("row_scale_exponents", lambda w_bits: orig(w_bits) + 1)


# ---- dense layer (next row)

@mutant
def dense_h_not_rounded():
    def f(x_bits, wg_bits, wu_bits, wd_bits):
        x = M.bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))

        def widen(w):
            w = np.asarray(w)
            return w if w.dtype == np.float64 else M.bf16_bits_to_f64(w.astype(np.uint16))
        return M.swiglu_expert(x, widen(wg_bits), widen(wu_bits), widen(wd_bits), round_h=False)
    _patch("dense_mlp", f)
