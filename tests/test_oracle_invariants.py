"""Pins for the oracle's arithmetic against things other than itself:
library routines (torch's SiLU / RMSNorm / bf16 conversion, scipy's expit,
math.fsum), closed forms (residual stream, sum of weights), special cases
(single expert, linearity) and the figures printed on the pages.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def rand_bf16_bits(rng, shape, sigma):
    v = (rng.standard_normal(shape) * sigma).astype(np.float32)
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- bf16 helpers

def test_bf16_widening_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**16, size=4096, dtype=np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    o = O.bf16_bits_to_f64(bits)
    same = (t == o) | (np.isnan(t) & np.isnan(o))
    assert same.all()


def test_bf16_rounding_matches_torch_for_fp32_inputs():
    """For fp32-representable inputs the one-step fp64->bf16 rounding must equal
    torch's fp32->bf16 round-to-nearest-even."""
    rng = np.random.default_rng(1)
    parts = [
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),      # fp32 subnormals
        (rng.standard_normal(2000) * 1e38).astype(np.float32),       # near overflow
        # exact halfway cases: low 16 bits = 0x8000
        ((rng.integers(0x3F800000, 0x40800000, 2000, dtype=np.uint32) & 0xFFFF0000) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 3.3895313892515355e38, -3.4e38, 1.0, -2.0], dtype=np.float32),
    ]
    v = np.concatenate(parts)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16_bits(v.astype(np.float64))
    assert np.array_equal(ref, got)


def test_bf16_rounding_ties_to_even():
    one = 1.0
    ulp = 2.0 ** -7
    assert O.round_to_bf16(np.array([one + ulp / 2]))[0] == one            # tie -> even (1.0)
    assert O.round_to_bf16(np.array([one + 1.5 * ulp]))[0] == one + 2 * ulp  # tie -> even
    assert O.round_to_bf16(np.array([one + ulp / 2 + 1e-12]))[0] == one + ulp
    assert np.isinf(O.round_to_bf16(np.array([3.4e38]))[0])


# ---------------------------------------------------------------- router

def test_router_logits_exactly_rounded_sums():
    rng = np.random.default_rng(4)
    x = rand_bf16_bits(rng, (6, 5120), 1.0)
    wr = rand_bf16_bits(rng, (16, 5120), 0.02)
    z = O.router_logits(x, wr)
    xf = O.bf16_bits_to_f64(x)
    wf = O.bf16_bits_to_f64(wr)
    for t in range(6):
        for e in range(16):
            exact = math.fsum((xf[t] * wf[e]).tolist())   # products are exact in fp64
            assert abs(z[t, e] - exact) <= 1e-12 * max(1.0, abs(exact))


def test_router_offset_added_before_sigmoid():
    rng = np.random.default_rng(5)
    x = rand_bf16_bits(rng, (4, 64), 1.0)
    wr = rand_bf16_bits(rng, (8, 64), 0.02)
    off = np.linspace(-1, 1, 8).astype(np.float32)
    z0 = O.router_logits(x, wr)
    z1 = O.router_logits(x, wr, off)
    np.testing.assert_array_equal(z1 - z0, np.broadcast_to(off.astype(np.float64), z0.shape))


def test_sigmoid_library_and_closed_forms():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(O.sigmoid(z), scipy.special.expit(z), rtol=1e-15, atol=0)
    assert O.sigmoid(np.array([0.0]))[0] == 0.5
    np.testing.assert_allclose(O.sigmoid(z) + O.sigmoid(-z), 1.0, rtol=0, atol=1e-15)


# ---------------------------------------------------------------- experts

def torch_swiglu(x64, wg64, wu64, wd64):
    """Textbook SwiGLU MLP via torch's SiLU (float64, no rounding)."""
    xt = torch.from_numpy(x64)
    return (F.silu(xt @ torch.from_numpy(wg64).T) * (xt @ torch.from_numpy(wu64).T)) @ torch.from_numpy(wd64).T


def small_block(rng, T=12, H=64, I=32, E=16):
    x = rand_bf16_bits(rng, (T, H), 1.0)
    wr = rand_bf16_bits(rng, (E, H), 0.02)
    wg = rand_bf16_bits(rng, (E, I, H), 0.02 * 8)
    wu = rand_bf16_bits(rng, (E, I, H), 0.02 * 8)
    wd = rand_bf16_bits(rng, (E, H, I), 0.02 * 8)
    return x, wr, wg, wu, wd


def test_swiglu_expert_matches_torch_silu():
    rng = np.random.default_rng(6)
    x, wr, wg, wu, wd = small_block(rng)
    xf = O.bf16_bits_to_f64(x)
    for e in (0, 5, 15):
        got = O.swiglu_expert(xf, O.bf16_bits_to_f64(wg[e]), O.bf16_bits_to_f64(wu[e]),
                              O.bf16_bits_to_f64(wd[e]), round_h=False)
        ref = torch_swiglu(xf, O.bf16_bits_to_f64(wg[e]), O.bf16_bits_to_f64(wu[e]),
                           O.bf16_bits_to_f64(wd[e])).numpy()
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_h_rounding_is_bf16_of_product():
    """With rounding on, the down projection sees bf16(SiLU(g)*u) exactly."""
    rng = np.random.default_rng(7)
    x, wr, wg, wu, wd = small_block(rng)
    xf = O.bf16_bits_to_f64(x)
    g = torch.from_numpy(xf) @ torch.from_numpy(O.bf16_bits_to_f64(wg[3])).T
    u = torch.from_numpy(xf) @ torch.from_numpy(O.bf16_bits_to_f64(wu[3])).T
    h = (F.silu(g) * u).numpy()
    # round through fp32 only where that is a single rounding (h exactly fp32)
    h_bf = O.round_to_bf16(h)
    assert np.all(np.abs(h_bf - h) <= np.abs(h) * 2.0 ** -8 + 1e-300)
    ref = h_bf @ O.bf16_bits_to_f64(wd[3]).T
    got = O.swiglu_expert(xf, O.bf16_bits_to_f64(wg[3]), O.bf16_bits_to_f64(wu[3]),
                          O.bf16_bits_to_f64(wd[3]), round_h=True)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_single_expert_gives_scale_times_expert():
    """k = 1: weight is s/s * 2.5 = 2.5 exactly, so y = 2.5 * SwiGLU_e(x)."""
    rng = np.random.default_rng(8)
    x, wr, wg, wu, wd = small_block(rng)
    res = O.moe_block(x, wr, (wg, wu, wd), groups=4, topk_groups=2, k=1, scale=2.5, round_h=False)
    assert np.all(res["weights"] == 2.5)
    xf = O.bf16_bits_to_f64(x)
    for t in range(x.shape[0]):
        e = int(res["ids"][t, 0])
        ref = 2.5 * torch_swiglu(xf[t:t + 1], O.bf16_bits_to_f64(wg[e]), O.bf16_bits_to_f64(wu[e]),
                                 O.bf16_bits_to_f64(wd[e])).numpy()[0]
        np.testing.assert_allclose(res["y"][t], ref, rtol=1e-12, atol=1e-12)


def test_injected_weights_are_linear():
    """Two experts with injected weights (a, b) give a*E1(x) + b*E2(x)."""
    rng = np.random.default_rng(9)
    x, wr, wg, wu, wd = small_block(rng, T=5)
    xf = O.bf16_bits_to_f64(x)
    ids = np.tile(np.array([[3, 11]]), (5, 1))
    a, b = 0.75, -1.25
    w = np.tile(np.array([[a, b]]), (5, 1))
    y = O.moe_forward(x, ids, w, (wg, wu, wd), E=16, round_h=False)
    e1 = torch_swiglu(xf, *(O.bf16_bits_to_f64(t[3]) for t in (wg, wu, wd))).numpy()
    e2 = torch_swiglu(xf, *(O.bf16_bits_to_f64(t[11]) for t in (wg, wu, wd))).numpy()
    np.testing.assert_allclose(y, a * e1 + b * e2, rtol=1e-12, atol=1e-12)


def test_out_of_range_ids_contribute_nothing():
    rng = np.random.default_rng(10)
    x, wr, wg, wu, wd = small_block(rng, T=3)
    ids = np.array([[2, -1], [16, 2], [2, 99]])
    w = np.ones((3, 2))
    y = O.moe_forward(x, ids, w, (wg, wu, wd), E=16)
    y1 = O.moe_forward(x, ids[:, :1] * 0 + 2, w[:, :1], (wg, wu, wd), E=16)
    np.testing.assert_array_equal(y, y1)


def test_block_invariants():
    rng = np.random.default_rng(11)
    x, wr, wg, wu, wd = small_block(rng, T=40, E=32, H=64, I=32)
    res = O.moe_block(x, wr, (wg, wu, wd), groups=8, topk_groups=4, k=8, scale=2.5)
    np.testing.assert_allclose(res["weights"].sum(axis=1), 2.5, rtol=0, atol=1e-12)
    assert res["counts"].sum() == 40 * 8
    for t in range(40):
        assert len(set(res["ids"][t].tolist())) == 8
        assert len({int(e) // 4 for e in res["ids"][t]}) <= 4
    # permutation equivariance: permuting tokens permutes outputs
    perm = rng.permutation(40)
    res_p = O.moe_block(x[perm], wr, (wg, wu, wd), groups=8, topk_groups=4, k=8, scale=2.5)
    np.testing.assert_allclose(res_p["y"], res["y"][perm], rtol=1e-12, atol=1e-12)


def test_expert_major_order_brute_force():
    rng = np.random.default_rng(12)
    ids = rng.integers(-1, 9, size=(30, 3))
    counts, offsets, toks, row_of = O.expert_major_order(ids, 8)
    exp_rows = []
    for e in range(8):
        for t in range(30):
            for j in range(3):
                if ids[t, j] == e:
                    exp_rows.append((t, j))
    assert toks.tolist() == [t for t, _ in exp_rows]
    for r, (t, j) in enumerate(exp_rows):
        assert row_of[t * 3 + j] == r
    assert np.all(row_of[(ids.reshape(-1) < 0) | (ids.reshape(-1) >= 8)] == -1)
    assert counts.tolist() == [sum(1 for t, j in exp_rows if ids[t, j] == e) for e in range(8)]
    assert offsets[-1] == len(exp_rows)


# ---------------------------------------------------------------- norm / residual

def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(13)
    v = rng.standard_normal((7, 5120)) * 3.0
    ref = F.rms_norm(torch.from_numpy(v), (5120,), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rmsnorm(v, 1e-6), ref, rtol=1e-13, atol=0)


def test_residual_closed_form():
    """Embedding = step 1; after steps 2..K every term carries weight 1/sqrt(K)."""
    rng = np.random.default_rng(14)
    x = rng.standard_normal(64)
    outs = rng.standard_normal((104, 64))
    stream = x.copy()
    for i, step in enumerate(range(2, 106)):
        stream = O.residual_step(stream, outs[i], step)
        K = step
        closed = (x + outs[:i + 1].sum(axis=0)) / math.sqrt(K)
        np.testing.assert_allclose(stream, closed, rtol=1e-12, atol=1e-12)
    # the two weights' squares sum to one at every step
    for k in range(2, 106):
        assert math.isclose((k - 1) / k + 1 / k, 1.0)


# ---------------------------------------------------------------- page figures

def test_page_parameter_figures():
    with open(GOLDEN) as f:
        p = json.load(f)
    per = O.expert_param_count(p["hidden"], p["expert_intermediate"])
    assert per == 39_321_600
    assert round(per / 1e6) == p["params_per_expert_millions_approx"]
    expert_total = p["moe_layers"] * p["experts_per_layer"] * per
    share = 100 * expert_total / (p["total_params_billions"] * 1e9)
    assert abs(share - p["expert_share_percent"]) < 0.06
    non_expert = p["total_params_billions"] * 1e9 - expert_total
    active = p["moe_layers"] * p["routed_per_token"] * per + non_expert
    assert round(active / 1e9) == p["active_params_billions_approx"]
    # expert parallelism: replicated 16 GB + bf16 experts split over devices
    for n, gb in ((16, p["ep_gb_per_gpu_16"]), (8, p["ep_gb_per_gpu_8"])):
        per_gpu = p["replicated_gb_bf16"] + 2 * expert_total / 1e9 / n
        assert abs(per_gpu - gb) < 1.0
    # the figures rule out a 2-matrix MLP or biases of the printed size
    assert round(2 * p["hidden"] * p["expert_intermediate"] / 1e6) != p["params_per_expert_millions_approx"]
