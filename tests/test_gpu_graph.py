"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph on the
capturing stream) and replayed: every replay, with eager work and device
synchronisations between replays and the graph's input rewritten in place,
must equal the eager result on the same input bit for bit (every path is
deterministic).  The calls record kernels only -- no memset, copy,
allocation or synchronisation -- so they can sit inside a serving loop's
graph."""
import pytest
import torch

import moe_inputs as MI
from moe_inputs import BlockShape

from parity import sync

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def bm():
    import sparse_moe_transformer_group_amd as bm
    yield bm
    bm.set_schedule("auto")


def replay_matches_eager(fn, x_static, inputs):
    """Capture fn(x_static), then for each input: copy it into x_static,
    replay, run unrelated eager work, synchronise, and compare the graph's
    output with an eager call on that input."""
    out = fn(x_static)            # warm-up: workspace and device checks outside the capture
    sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn(x_static)
    for i, x in enumerate(inputs):
        x_static.copy_(x)
        g.replay()
        junk = torch.randn(1 << 20, device=DEV).mul_(3.0).sum()     # eager work between replays
        sync()
        ref = fn(x.clone())
        sync()
        assert torch.equal(out, ref), f"replay {i} differs from the eager result"
        del junk


@pytest.mark.parametrize("weights", ["bf16", "fp8"])
@pytest.mark.parametrize("schedule", ["stream", "tiled"])
def test_graph_moe_block(bm, schedule, weights):
    shape = BlockShape(T=256, H=320, I=384)
    print(f"[case] graph moe block T={shape.T} schedule={schedule} weights={weights}", flush=True)
    inp = MI.make_block_inputs(shape, DEV, case=11)
    pack = bm.pack_experts_fp8 if weights == "fp8" else bm.pack_experts
    packed = pack(inp.wg, inp.wu, inp.wd)
    bm.set_schedule(schedule)
    try:
        def fn(x):
            return bm.block(x, inp.wr, *packed, shape.groups, shape.topk_groups, shape.k, shape.scale,
                            return_routing=False)
        xs = [MI.make_x(shape.T, shape.H, case=c).to(DEV) for c in (21, 22, 23)]
        replay_matches_eager(fn, inp.x.clone(), xs)
    finally:
        bm.set_schedule("auto")


@pytest.mark.parametrize("global_layer", [False, True])
def test_graph_attention(bm, global_layer):
    T, H = 300, 256
    print(f"[case] graph attention T={T} global={global_layer}", flush=True)
    w_qkvg, w_o = bm.pack_attention_weights(*[w.to(DEV) for w in MI.make_attention_weights(H, case=12)])

    def fn(u):
        return bm.attention(u, w_qkvg, w_o, global_layer, window=64)
    us = [MI.make_attention_input(T, H, case=c).to(DEV) for c in (31, 32, 33)]
    replay_matches_eager(fn, us[0].clone(), us)


@pytest.mark.parametrize("fp8", [False, True])
def test_graph_dense(bm, fp8):
    T, H, I = 200, 256, 512
    print(f"[case] graph dense T={T} fp8={fp8}", flush=True)
    packed = bm.pack_dense(*MI.make_dense_weights(H, I, DEV, case=13), chunks=2, fp8=fp8)

    def fn(x):
        return bm.dense_mlp(x, *packed)
    xs = [MI.make_x(T, H, case=c).to(DEV) for c in (41, 42, 43)]
    replay_matches_eager(fn, xs[0].clone(), xs)


@pytest.mark.parametrize("weights", ["bf16", "fp8"])
def test_graph_sublayer_stack(bm, weights):
    """Two stacked sublayers (norms, block, residual update), in place on the
    FP32 stream, captured as one graph."""
    shape = BlockShape(T=192, H=256, I=128)
    print(f"[case] graph sublayer stack T={shape.T} weights={weights}", flush=True)
    pack = bm.pack_experts_fp8 if weights == "fp8" else bm.pack_experts
    layers = []
    for layer in range(2):
        wr = MI.make_router(shape.E, shape.H, layer=layer, case=15).to(DEV)
        layers.append((wr, pack(*MI.make_expert_weights(shape.E, shape.H, shape.I, DEV, layer=layer,
                                                       case=15))))

    def fn(s):
        for step, (wr, packed) in zip((2, 3), layers):
            bm.sublayer(s, step, wr, *packed, shape.groups, shape.topk_groups, shape.k, shape.scale,
                        keep_io=False)
        return s
    xs = [bm.stream_init(MI.make_x(shape.T, shape.H, case=c).to(DEV)) for c in (51, 52, 53)]
    replay_matches_eager(fn, xs[0].clone(), xs)
