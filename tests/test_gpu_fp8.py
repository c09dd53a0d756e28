"""GPU checks of the FP8 (E4M3) expert-weight path against the oracle: the
packed codes and row scales bit for bit, and blocks computed with FP8
weights against the oracle block run on the oracle's own dequantised
weights."""
import numpy as np
import pytest
import torch

import moe_inputs as MI
import oracle as O
from moe_inputs import BlockShape, bf16_bits

from layouts import fp8_chunk_swizzle
from parity import check_output, check_routing, keep_mask, sync

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def bm():
    import sparse_moe_transformer_group_amd as bm
    yield bm
    bm.set_schedule("auto")


def unpack_fp8(data, E, N, K):
    """Codes [E, N, K] from the packed FP8 layout (numpy index arithmetic:
    blocks of 128 rows x 32 k in (row block, k-block) order, 8-byte chunk c of
    block row j stored at c ^ fp8_chunk_swizzle(j))."""
    NB, KB = -(-N // 128), K // 32
    b = np.asarray(data).reshape(E, NB, KB, 128, 4, 8)
    j = np.arange(128)[:, None]
    phys = np.arange(4)[None, :] ^ fp8_chunk_swizzle(j)  # logical chunk c sits at phys[j, c]
    logical = b[:, :, :, j, phys, :]                    # e, rb, kb, j, c, 8
    return logical.transpose(0, 1, 3, 2, 4, 5).reshape(E, NB * 128, K)[:, :N]


def special_weights(E, N, K, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    w = torch.randn(E, N, K, generator=g) * 0.02
    w[0, 0] = 0.0                                       # all-zero row: scale 1
    w[0, 1] = -0.0
    w[0, 2, :5] = torch.tensor([448.0 * 4, -3.0, 1e-6, -1e-7, 0.5])
    w[-1, -1] *= 1e4                                    # large row
    w[-1, -2] *= 1e-6                                   # tiny row
    return w.to(torch.bfloat16)


@pytest.mark.parametrize("E,N,K", [(3, 192, 128), (2, 256, 320), (1, 64, 64)])
def test_pack_fp8_bit_exact(bm, E, N, K):
    w = special_weights(E, N, K, E * 100 + N + K)
    pk = bm.pack_weights_fp8(w.to(DEV))
    sync()
    assert pk.data.numel() == E * bm.packed_fp8_bytes(N, K)
    codes, ex = O.quantize_rows(bf16_bits(w))
    got = unpack_fp8(pk.data.cpu().numpy(), E, N, K)
    assert np.array_equal(got, codes)
    assert np.array_equal(pk.scales.cpu().numpy().astype(np.float64), np.exp2(ex.astype(np.float64)))
    # padding rows of the last block are zero
    if N % 128:
        NB, KB = -(-N // 128), K // 32
        raw = pk.data.cpu().numpy().reshape(E, NB, KB, 128, 32)
        assert not raw[:, -1, :, N % 128:].any()


def fp8_experts_oracle(wg, wu, wd):
    """Oracle expert source: each expert's weights quantised by the oracle's
    own E4M3 encoder and dequantised to float64."""
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = tuple(O.dequantize_rows(*O.quantize_rows(bf16_bits(w[e]))) for w in (wg, wu, wd))
        return cache[e]
    return get


def oracle_fp8_block(x_bits, wr, wg, wu, wd, shape, offset=None, experts=None):
    experts = experts or fp8_experts_oracle(wg, wu, wd)
    return O.moe_block(x_bits, bf16_bits(wr), experts, shape.groups,
                       shape.topk_groups, shape.k, shape.scale,
                       None if offset is None else offset.cpu().numpy())


def run_fp8_block(bm, inp, shape, packed=None):
    packed = packed or bm.pack_experts_fp8(inp.wg, inp.wu, inp.wd)
    out = bm.block(inp.x, inp.wr, *packed, shape.groups, shape.topk_groups, shape.k, shape.scale,
                   logit_offset=inp.offset)
    sync()
    return out


@pytest.mark.parametrize("schedule", ["stream", "tiled"])
@pytest.mark.parametrize("T,H,I,k", [(128, 256, 128, 8), (7, 256, 128, 8), (1000, 256, 128, 8),
                                     (300, 320, 192, 8), (200, 256, 128, 1)])
def test_block_fp8_small(bm, schedule, T, H, I, k):
    shape = BlockShape(T=T, H=H, I=I, k=k)
    inp = MI.make_block_inputs(shape, DEV, case=20 + T % 17)
    bm.set_schedule(schedule)
    try:
        y, ids, w, counts = run_fp8_block(bm, inp, shape)
    finally:
        bm.set_schedule("auto")
    ref = oracle_fp8_block(bf16_bits(inp.x), inp.wr, inp.wg, inp.wu, inp.wd, shape)
    st = check_routing(ids, w, ref, shape, counts)
    st.update(check_output(y, ref["y"], keep_mask(ref), out_rounding_slack=(k == 1)))


def test_forward_fp8_single_expert(bm):
    """All tokens on one expert with weight 1: y = SwiGLU of the dequantised expert."""
    shape = BlockShape(T=40, H=256, I=128)
    inp = MI.make_block_inputs(shape, DEV, case=31)
    ids = torch.full((40, 8), -1, dtype=torch.int32, device=DEV)
    ids[:, 0] = 17
    w = torch.zeros((40, 8), dtype=torch.float32, device=DEV)
    w[:, 0] = 1.0
    y = bm.forward(inp.x, ids, w, *bm.pack_experts_fp8(inp.wg, inp.wu, inp.wd))
    sync()
    wg, wu, wd = fp8_experts_oracle(inp.wg, inp.wu, inp.wd)(17)
    ref = O.swiglu_expert(O.bf16_bits_to_f64(bf16_bits(inp.x)), wg, wu, wd)
    check_output(y, ref, out_rounding_slack=True)


@pytest.fixture(scope="module")
def beam_fp8(bm):
    s = MI.WORKLOADS["prefill"]
    print("[setup] Beam-shape weights, FP8", flush=True)
    wr = MI.make_router(s.E, s.H).to(DEV)
    wg, wu, wd = MI.make_expert_weights(s.E, s.H, s.I, DEV)
    packed = bm.pack_experts_fp8(wg, wu, wd)
    sync()
    # one cache of oracle-quantised experts shared by the cases (host work)
    yield wr, wg, wu, wd, packed, fp8_experts_oracle(wg, wu, wd)
    del wg, wu, wd, packed
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_beam_fp8_sampled(bm, beam_fp8, name):
    from parity import oracle_route, sample_tokens
    shape = MI.WORKLOADS[name]
    print(f"[case] fp8 {name} T={shape.T}", flush=True)
    wr, wg, wu, wd, packed, experts = beam_fp8
    x = MI.make_x(shape.T, shape.H).to(DEV)
    y, ids, w, counts = bm.block(x, wr, *packed, shape.groups, shape.topk_groups, shape.k,
                                 shape.scale)
    sync()
    ref_r = oracle_route(x, wr, shape)
    check_routing(ids, w, ref_r, shape, counts)
    toks = sample_tokens(keep_mask(ref_r), 3)
    ref = oracle_fp8_block(bf16_bits(x)[toks], wr, wg, wu, wd, shape, experts=experts)
    st = check_output(y[torch.from_numpy(toks).to(DEV)], ref["y"])
    print(st, flush=True)


@pytest.mark.parametrize("schedule", ["stream", "tiled"])
def test_sublayer_fp8_teacher_forced(bm, schedule):
    """Two stacked sublayers with FP8 expert weights, each checked with the
    device's own layer input against the oracle on its dequantised E4M3
    encoding; the residual update from the device's own output."""
    shape = BlockShape(T=128, H=256, I=128)
    print(f"[case] fp8 sublayer schedule={schedule}", flush=True)
    x = MI.make_x(shape.T, shape.H, case=14).to(DEV)
    stream = bm.stream_init(x)
    bm.set_schedule(schedule)
    try:
        for step in (2, 3):
            layer = step - 2
            wr = MI.make_router(shape.E, shape.H, layer=layer, case=14).to(DEV)
            wg, wu, wd = MI.make_expert_weights(shape.E, shape.H, shape.I, DEV, layer=layer, case=14)
            prev = stream.clone()
            xin, yb, ids, w, counts = bm.sublayer(stream, step, wr, *bm.pack_experts_fp8(wg, wu, wd))
            sync()
            prev64 = prev.cpu().numpy().astype(np.float64)
            blk = O.stack_sublayer(prev64, step, bf16_bits(wr), fp8_experts_oracle(wg, wu, wd),
                                   shape.groups, shape.topk_groups, shape.k, shape.scale,
                                   moe_input_bits=bf16_bits(xin))
            check_routing(ids, w, blk, shape, counts)
            print(check_output(yb, blk["y"], keep_mask(blk)))
            ref_stream = O.residual_step(prev64, O.rmsnorm(O.bf16_bits_to_f64(bf16_bits(yb))), step)
            np.testing.assert_allclose(stream.cpu().numpy(), ref_stream, rtol=1e-5, atol=1e-5)
    finally:
        bm.set_schedule("auto")
