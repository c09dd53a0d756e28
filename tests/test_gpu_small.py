"""GPU parity of the HIP path against the oracle at small shapes that span
several tiles and ragged tails, plus the edge cases: T in {1, 7, 1000},
k = 1, E = 64 / 4 groups, all tokens pushed into one group, injected
routing (one-hot and out-of-range ids), run-to-run bit equality, T = 0, the
permutation, norms and residual update."""
import numpy as np
import pytest
import torch

import moe_inputs as MI
import oracle as O
from moe_inputs import BlockShape, bf16_bits

from layouts import bf16_chunk_swizzle
from parity import (check_output, check_routing, keep_mask, oracle_route, sync)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def bm():
    import sparse_moe_transformer_group_amd as bm
    yield bm
    bm.set_schedule("auto")


def oracle_full(inp, shape):
    return O.moe_block(bf16_bits(inp.x), bf16_bits(inp.wr),
                       (bf16_bits(inp.wg), bf16_bits(inp.wu), bf16_bits(inp.wd)),
                       shape.groups, shape.topk_groups, shape.k, shape.scale,
                       None if inp.offset is None else inp.offset.cpu().numpy())


def run_block(bm, inp, shape):
    out = bm.block(inp.x, inp.wr, *bm.pack_experts(inp.wg, inp.wu, inp.wd), shape.groups,
                   shape.topk_groups, shape.k, shape.scale, logit_offset=inp.offset)
    sync()
    return out


def full_check(bm, shape, case=0, offset=None, out_rounding_slack=False):
    print(f"[case] shape={shape} case={case}", flush=True)
    inp = MI.make_block_inputs(shape, DEV, case=case)
    if offset is not None:
        inp.offset = offset.to(DEV)
    y, ids, w, counts = run_block(bm, inp, shape)
    ref = oracle_full(inp, shape)
    st = check_routing(ids, w, ref, shape, counts)
    st.update(check_output(y, ref["y"], keep_mask(ref), out_rounding_slack))
    print(st)
    return inp, ref, (y, ids, w, counts)


TINY = MI.WORKLOADS["tiny"]


def test_route_tiny(bm):
    inp = MI.make_block_inputs(TINY, DEV)
    ids, w, counts = bm.route(inp.x, inp.wr, TINY.groups, TINY.topk_groups, TINY.k, TINY.scale)
    sync()
    ref = oracle_route(inp.x, inp.wr, TINY)
    st = check_routing(ids, w, ref, TINY, counts)
    np.testing.assert_allclose(w.sum(1).cpu().numpy(), 2.5, rtol=0, atol=8 * 2.5 * 2 ** -23)
    print(st)


@pytest.mark.parametrize("schedule", ["auto", "stream", "tiled"])
def test_block_tiny(bm, schedule):
    bm.set_schedule(schedule)
    try:
        full_check(bm, TINY)
    finally:
        bm.set_schedule("auto")


# 65: two 64-token router tiles, the second holding one token (4-wave router
# workgroups); 257: 4-token selection workgroups, the last with one token
@pytest.mark.parametrize("T", [1, 7, 65, 257, 1000])
@pytest.mark.parametrize("schedule", ["stream", "tiled"])
def test_block_ragged_T(bm, T, schedule):
    bm.set_schedule(schedule)
    try:
        full_check(bm, BlockShape(T=T, H=256, I=128), case=T)
    finally:
        bm.set_schedule("auto")


def test_block_larger_dims_tiled(bm):
    """H=640, I=384: several K steps, a 64-wide K tail in the stream kernel and
    partial feature tiles in the tiled kernel."""
    for schedule in ("stream", "tiled"):
        bm.set_schedule(schedule)
        try:
            full_check(bm, BlockShape(T=300, H=640, I=384), case=11)
        finally:
            bm.set_schedule("auto")


@pytest.mark.parametrize("schedule", ["stream", "tiled"])
def test_block_padded_rows(bm, schedule):
    """H = 320, I = 192: neither is a multiple of the 128-row packed block, so
    both GEMMs read zero-padded rows, and K is 64 past a multiple of 128 (the
    streaming schedule's tail step)."""
    shape = BlockShape(T=300, H=320, I=192)
    inp = MI.make_block_inputs(shape, DEV, case=11)
    bm.set_schedule(schedule)
    try:
        y, ids, w, counts = run_block(bm, inp, shape)
    finally:
        bm.set_schedule("auto")
    ref = oracle_full(inp, shape)
    st = check_routing(ids, w, ref, shape, counts)
    st.update(check_output(y, ref["y"], keep_mask(ref)))


def pack_layout_reference(bits):
    """The packed block layout written out with numpy index arithmetic: rows
    padded to a multiple of 128, blocks of 128 rows x 32 k in (row block,
    k-block) order, 16-byte chunk c of block row j stored at c ^ swz(j)."""
    E, N, K = bits.shape
    NB, KB = -(-N // 128), K // 32
    pad = np.zeros((E, NB * 128, K), np.uint16)
    pad[:, :N] = bits
    blocks = pad.reshape(E, NB, 128, KB, 4, 8).transpose(0, 1, 3, 2, 4, 5)  # e, rb, kb, j, c, 8
    j = np.arange(128)[:, None]
    logical = np.arange(4)[None, :] ^ bf16_chunk_swizzle(j)  # physical slot p holds logical chunk p ^ swz
    out = blocks[:, :, :, np.arange(128)[:, None], logical, :]
    return out.reshape(-1)


@pytest.mark.parametrize("E,N,K", [(3, 192, 128), (2, 256, 320), (1, 64, 64)])
def test_pack_layout_bit_exact(bm, E, N, K):
    g = torch.Generator(device="cpu").manual_seed(E * 1000 + N + K)
    w = torch.randn(E, N, K, generator=g).to(torch.bfloat16).to(DEV)
    packed = bm.pack_weights(w)
    sync()
    assert packed.data.numel() == E * bm.packed_weight_bytes(N, K)
    got = packed.data.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, pack_layout_reference(bf16_bits(w)))


def test_block_k1(bm):
    shape = BlockShape(T=96, H=256, I=128, k=1)
    inp, ref, (y, ids, w, counts) = full_check(bm, shape, case=3, out_rounding_slack=True)
    assert torch.all(w == 2.5)


def test_block_e64_g4(bm):
    full_check(bm, BlockShape(T=200, H=256, I=128, E=64, groups=4, topk_groups=2, k=6), case=4)


def test_block_irregular_groups(bm):
    """E=96 in 12 groups of 8 (group score path without whole-lane groups)."""
    full_check(bm, BlockShape(T=50, H=128, I=64, E=96, groups=12, topk_groups=5, k=7), case=5)


def test_block_all_tokens_one_group(bm):
    shape = BlockShape(T=256, H=256, I=128)
    off = torch.zeros(256, dtype=torch.float32)
    off[:32] = 4.0
    inp, ref, (y, ids, w, counts) = full_check(bm, shape, case=6, offset=off)
    c = counts.cpu().numpy()
    assert c[:32].sum() >= 0.9 * shape.T * shape.k


def test_forward_injected_one_hot_and_dropped_ids(bm):
    shape = BlockShape(T=40, H=256, I=128)
    inp = MI.make_block_inputs(shape, DEV, case=7)
    rng = np.random.default_rng(7)
    ids = np.stack([rng.permutation(256)[:8] for _ in range(40)]).astype(np.int32)
    ids[::5, 3] = -1
    ids[::7, 6] = 300
    w = np.zeros((40, 8), dtype=np.float32)
    w[:, 0] = 1.0
    w[1::2, 1] = 0.5
    ids_t = torch.from_numpy(ids).to(DEV)
    w_t = torch.from_numpy(w).to(DEV)
    packed = bm.pack_experts(inp.wg, inp.wu, inp.wd)
    for schedule in ("stream", "tiled"):
        bm.set_schedule(schedule)
        try:
            y, counts = bm.forward(inp.x, ids_t, w_t, *packed, return_counts=True)
            sync()
        finally:
            bm.set_schedule("auto")
        ref_y = O.moe_forward(bf16_bits(inp.x), ids, w,
                              (bf16_bits(inp.wg), bf16_bits(inp.wu), bf16_bits(inp.wd)), E=256)
        check_output(y, ref_y)
        valid = ids[(ids >= 0) & (ids < 256)]
        assert np.array_equal(counts.cpu().numpy(), np.bincount(valid, minlength=256))


def test_forward_single_expert_is_scale_times_swiglu(bm):
    """Every token routed to expert 17 only, weight 2.5: y = 2.5 * SwiGLU_17(x)."""
    shape = BlockShape(T=64, H=256, I=128)
    inp = MI.make_block_inputs(shape, DEV, case=8)
    ids = torch.full((64, 1), 17, dtype=torch.int32, device=DEV)
    w = torch.full((64, 1), 2.5, dtype=torch.float32, device=DEV)
    y = bm.forward(inp.x, ids, w, *bm.pack_experts(inp.wg, inp.wu, inp.wd))
    sync()
    xf = O.bf16_bits_to_f64(bf16_bits(inp.x))
    ref = 2.5 * O.swiglu_expert(xf, O.bf16_bits_to_f64(bf16_bits(inp.wg[17])),
                                O.bf16_bits_to_f64(bf16_bits(inp.wu[17])),
                                O.bf16_bits_to_f64(bf16_bits(inp.wd[17])))
    check_output(y, ref, out_rounding_slack=True)


def test_block_bitwise_deterministic(bm):
    inp = MI.make_block_inputs(TINY, DEV, case=9)
    a = run_block(bm, inp, TINY)
    b = run_block(bm, inp, TINY)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_block_T0(bm):
    shape = BlockShape(T=0, H=256, I=128)
    inp = MI.make_block_inputs(BlockShape(T=4, H=256, I=128), DEV)
    x0 = inp.x[:0]
    y, ids, w, counts = bm.block(x0, inp.wr, *bm.pack_experts(inp.wg, inp.wu, inp.wd))
    sync()
    assert y.shape == (0, 256) and ids.shape == (0, 8)


@pytest.mark.parametrize("T,k,E", [(1, 8, 256), (1000, 8, 256), (3000, 3, 512), (64, 32, 40)])
def test_permute_matches_stable_sort(bm, T, k, E):
    rng = np.random.default_rng(T + k + E)
    ids = rng.integers(-2, E + 2, size=(T, k)).astype(np.int32)
    ids[: T // 3] = rng.integers(0, 3, size=(T // 3, k))   # heavy experts, repeated ids
    counts, offsets, sorted_tokens, row_of = bm.permute(torch.from_numpy(ids).to(DEV), E)
    sync()
    c, o, s, r = O.expert_major_order(ids, E)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(sorted_tokens.cpu().numpy()[: o[-1]], s)
    assert np.array_equal(row_of.cpu().numpy(), r)


def test_norms_and_residual(bm):
    rng = np.random.default_rng(12)
    T, H = 33, 640
    xb = MI.make_x(T, H).to(DEV)
    s = bm.stream_init(xb)
    sync()
    assert torch.equal(s, xb.float())
    v = torch.from_numpy((rng.standard_normal((T, H)) * 3).astype(np.float32)).to(DEV)
    out = bm.rmsnorm(v, 1e-6)
    sync()
    ref = O.rmsnorm(v.cpu().numpy().astype(np.float64), 1e-6)
    got = O.bf16_bits_to_f64(bf16_bits(out))
    # fp32 vs fp64 may land on opposite sides of a bf16 rounding boundary: <= 1 ulp
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-30)
    y = MI.make_x(T, H, layer=5).to(DEV)
    st = v.clone()
    bm.residual_update(st, y, step=3, eps=1e-6)
    sync()
    ref_s = O.residual_step(v.cpu().numpy().astype(np.float64),
                            O.rmsnorm(O.bf16_bits_to_f64(bf16_bits(y)), 1e-6), 3)
    np.testing.assert_allclose(st.cpu().numpy(), ref_s, rtol=2e-6, atol=2e-6)


def test_sublayer_tiny_teacher_forced(bm):
    """Two stacked sandwich-normed sublayers at tiny shape, checked per layer
    with the device's own layer input (teacher forcing)."""
    shape = TINY
    x = MI.make_x(shape.T, shape.H, case=10).to(DEV)
    stream = bm.stream_init(x)
    for step in (2, 3):
        layer = step - 2
        wr = MI.make_router(shape.E, shape.H, layer=layer, case=10).to(DEV)
        wg, wu, wd = MI.make_expert_weights(shape.E, shape.H, shape.I, DEV, layer=layer, case=10)
        prev = stream.clone()
        xin, yb, ids, w, counts = bm.sublayer(stream, step, wr, *bm.pack_experts(wg, wu, wd))
        sync()
        prev64 = prev.cpu().numpy().astype(np.float64)
        # MoE input = bf16(RMSNorm(stream)), within one bf16 ulp
        ref_in = O.rmsnorm(prev64)
        got_in = O.bf16_bits_to_f64(bf16_bits(xin))
        assert np.all(np.abs(got_in - ref_in) <= np.abs(ref_in) * 2.0 ** -7 + 1e-30)
        blk = O.stack_sublayer(prev64, step, bf16_bits(wr),
                               (bf16_bits(wg), bf16_bits(wu), bf16_bits(wd)), shape.groups,
                               shape.topk_groups, shape.k, shape.scale, moe_input_bits=bf16_bits(xin))
        check_routing(ids, w, blk, shape, counts)
        check_output(yb, blk["y"], keep_mask(blk))
        # residual update from the device's own y
        ref_stream = O.residual_step(prev64, O.rmsnorm(O.bf16_bits_to_f64(bf16_bits(yb))), step)
        np.testing.assert_allclose(stream.cpu().numpy(), ref_stream, rtol=1e-5, atol=1e-5)
