"""Pins of the attention-sublayer oracle against properties the pages and the
mathematics fix, brute force on small shapes and a library routine."""
import math

import numpy as np
import pytest
import torch

import oracle as O


def test_rope_preserves_pair_norms_and_is_identity_at_zero():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 3, 128))
    pos = np.arange(9) * 37
    y = O.rope(x, pos)
    n_x = np.hypot(x[..., :64], x[..., 64:])
    n_y = np.hypot(y[..., :64], y[..., 64:])
    assert np.allclose(n_x, n_y, rtol=0, atol=1e-12)
    assert np.array_equal(O.rope(x[:1], np.array([0])), x[:1])


def test_rope_scores_depend_only_on_relative_position():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    for m, n, s in [(5, 2, 100), (0, 0, 7), (300, 811, 4093), (17, 17, 1)]:
        a = np.sum(O.rope(q, np.array([m])) * O.rope(k, np.array([n])))
        b = np.sum(O.rope(q, np.array([m + s])) * O.rope(k, np.array([n + s])))
        assert abs(a - b) < 1e-9 * max(1.0, abs(a))
    # rotation by a position the other way round is the inverse
    qq = O.rope(O.rope(q, np.array([123])), np.array([-123]))
    assert np.allclose(qq, q, atol=1e-12)


def test_rope_frequencies_first_and_last_pair():
    # pair 0 turns by pos radians (theta^0 = 1); pair 63 by pos * theta^(-63/64)
    x = np.zeros((1, 1, 128))
    x[0, 0, 0] = 1.0
    x[0, 0, 63] = 1.0
    y = O.rope(x, np.array([3]))
    assert math.isclose(y[0, 0, 0], math.cos(3.0), abs_tol=1e-15)
    assert math.isclose(y[0, 0, 64], math.sin(3.0), abs_tol=1e-15)
    ang = 3.0 * 10000.0 ** (-63 / 64)
    assert math.isclose(y[0, 0, 127], math.sin(ang), abs_tol=1e-15)


def test_head_rmsnorm_matches_torch():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 48, 128)) * 3.0
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), eps=1e-6).numpy()
    assert np.allclose(O.head_rmsnorm(x), ref, rtol=1e-13, atol=1e-13)


def test_query_scale_closed_form():
    assert O.query_scale(0) == (1 + 1 / 2048) ** 0.1
    assert math.isclose(O.query_scale(2047), 2.0 ** 0.1, rel_tol=1e-15)  # pos + 1 = 2048
    s = O.query_scale(np.arange(0, 10 ** 6, 997))
    assert np.all(np.diff(s) > 0) and s[0] > 1.0


def brute_gqa(q, k, v, window):
    """Plain multi-head attention with the 8 kv heads repeated 6 times, by loops."""
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    rep = Hq // Hkv
    o = np.zeros_like(q)
    for h in range(Hq):
        for i in range(Tq):
            js = [j for j in range(i + 1) if window is None or j > i - window]
            s = [sum(q[i, h, d] * k[j, h // rep, d] for d in range(D)) / math.sqrt(D) for j in js]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = sum(w)
            for d in range(D):
                o[i, h, d] = sum(w[t] * v[js[t], h // rep, d] for t in range(len(js))) / z
    return o


@pytest.mark.parametrize("window", [None, 1, 3, 100])
def test_attention_core_brute_force(window):
    rng = np.random.default_rng(4)
    T, D = 7, 8
    q = rng.standard_normal((T, 12, D))
    k = rng.standard_normal((T, 2, D))
    v = rng.standard_normal((T, 2, D))
    got = O.attention_core(q, k, v, window)
    assert np.allclose(got, brute_gqa(q, k, v, window), rtol=1e-12, atol=1e-12)


def test_attention_core_special_cases():
    rng = np.random.default_rng(5)
    T = 40
    q = rng.standard_normal((T, 48, 128))
    v = rng.standard_normal((T, 8, 128))
    k = rng.standard_normal((T, 8, 128))
    # a single key: the output is that key's value
    o1 = O.attention_core(q[:1], k[:1], v[:1], None)
    assert np.allclose(o1[0], np.repeat(v[0], 6, axis=0), atol=1e-14)
    # window 1: every query sees only itself
    ow = O.attention_core(q, k, v, 1)
    assert np.allclose(ow, np.repeat(v, 6, axis=1), atol=1e-14)
    # identical keys: uniform weights, the mean of the values in the window
    kc = np.broadcast_to(k[:1], k.shape)
    oc = O.attention_core(q, kc, v, 5)
    for i in range(T):
        lo = max(0, i - 4)
        assert np.allclose(oc[i], np.repeat(v[lo:i + 1].mean(axis=0), 6, axis=0), atol=1e-12)
    # a window at least T long is plain causal attention
    assert np.array_equal(O.attention_core(q, k, v, T), O.attention_core(q, k, v, None))
    # restricting the queries to a subset of rows changes nothing for those rows
    rows = [0, 9, 31, 39]
    sub = O.attention_core(q[rows], k, v, 16, q_pos=rows)
    assert np.allclose(sub, O.attention_core(q, k, v, 16)[rows], atol=1e-13)


def bits(a):
    return O.f64_to_bf16_bits(a)


def small_layer(seed, T=24, H=64):
    rng = np.random.default_rng(seed)
    u = bits(rng.standard_normal((T, H)))
    w = [bits(rng.standard_normal(s) * 0.1) for s in [(48 * 128, H), (8 * 128, H), (8 * 128, H),
                                                        (48 * 128, H), (H, 48 * 128)]]
    return u, w


@pytest.mark.parametrize("global_layer", [False, True])
def test_gate_scales_every_channel(global_layer):
    rng = np.random.default_rng(6)
    T, H = 24, 64
    u = bits(np.abs(rng.standard_normal((T, H))) + 0.5)   # positive inputs
    wq, wk, wv, wo = [bits(rng.standard_normal(s) * 0.1) for s in
                      [(48 * 128, H), (8 * 128, H), (8 * 128, H), (H, 48 * 128)]]
    closed = np.zeros((48 * 128, H), dtype=np.uint16)           # gate logit 0: sigmoid = 1/2
    opened = bits(np.ones((48 * 128, H)))                       # gate logit > 40: sigmoid = 1
    y_half = O.attention_sublayer(u, wq, wk, wv, closed, wo, global_layer, window=5)["y"]
    y_full = O.attention_sublayer(u, wq, wk, wv, opened, wo, global_layer, window=5)["y"]
    # halving before the bf16 rounding of the head outputs is exact
    assert np.allclose(y_full, 2.0 * y_half, rtol=1e-12, atol=1e-12)
    assert np.abs(y_full).max() > 0


def test_zero_values_give_zero_output_and_rows_subset_agrees():
    u, (wq, wk, wv, wg, wo) = small_layer(7)
    y = O.attention_sublayer(u, wq, wk, np.zeros_like(wv), wg, wo, False)["y"]
    assert np.all(y == 0.0)
    full = O.attention_sublayer(u, wq, wk, wv, wg, wo, True)["y"]
    part = O.attention_sublayer(u, wq, wk, wv, wg, wo, True, rows=[3, 0, 17])
    assert list(part["rows"]) == [0, 3, 17]
    assert np.allclose(part["y"], full[[0, 3, 17]], rtol=1e-12, atol=1e-12)
