"""beam_moe_block_noalloc (static device scratch, no allocation) against
beam_moe_block (caller's workspace), through the C ABI: two calls in a row,
the second with a smaller batch, must give bit-identical outputs, ids,
weights and counts.  The no-allocation call and its binding allocate
nothing, so torch's allocated-bytes figure does not move across it."""
import numpy as np
import pytest
import torch

import moe_inputs as MI
from moe_inputs import BlockShape

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def bm():
    import sparse_moe_transformer_group_amd as bm
    bm.set_schedule("auto")
    return bm


def run_both(bm, x, wr, packed, shape, off=None):
    T, E, k = x.shape[0], shape.E, shape.k
    y_ref, ids_ref, w_ref, c_ref = bm.block(x, wr, *packed, shape.groups, shape.topk_groups, k,
                                            shape.scale, logit_offset=off)
    y = torch.empty((T, shape.H), dtype=torch.bfloat16, device=DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    c = torch.empty((E,), dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(DEV)
    bm.block_noalloc(x, wr, *packed, y, shape.groups, shape.topk_groups, k, shape.scale,
                     logit_offset=off, topk_ids=ids, topk_weights=w, counts=c)
    assert torch.cuda.memory_allocated(DEV) == before
    torch.cuda.synchronize()
    for name, a, b in (("y", y, y_ref), ("ids", ids, ids_ref), ("weights", w, w_ref),
                       ("counts", c, c_ref)):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b), \
            f"T={T}: {name} differs from beam_moe_block"


@pytest.mark.parametrize("schedule", ["auto", "tiled"])
@pytest.mark.parametrize("H,I,Ts", [(256, 128, (128, 37)), (640, 384, (300, 1))])
def test_noalloc_matches_block_small(bm, H, I, Ts, schedule):
    shape = BlockShape(T=max(Ts), H=H, I=I)
    print(f"[case] noalloc H={H} I={I} T={Ts} schedule={schedule}", flush=True)
    inp = MI.make_block_inputs(shape, DEV, case=50 + H % 11)
    packed = bm.pack_experts(inp.wg, inp.wu, inp.wd)
    bm.set_schedule(schedule)
    try:
        for T in Ts:                       # second call smaller than the first
            run_both(bm, inp.x[:T].contiguous(), inp.wr, packed, shape)
    finally:
        bm.set_schedule("auto")


def test_noalloc_matches_block_beam_decode(bm):
    """Beam shape: the decode batch (T = 64), then 9 tokens, then the largest
    batch the scratch holds (T = 259), then 64 again."""
    shape = MI.WORKLOADS["decode"]
    print("[case] noalloc Beam shape T=64,9,259,64", flush=True)
    wr = MI.make_router(shape.E, shape.H).to(DEV)
    wg, wu, wd = MI.make_expert_weights(shape.E, shape.H, shape.I, DEV, case=3)
    packed = bm.pack_experts(wg, wu, wd)
    del wg, wu, wd
    x = MI.make_x(259, shape.H, case=3).to(DEV)
    for T in (64, 9, 259, 64):
        run_both(bm, x[:T].contiguous(), wr, packed, shape)
    with pytest.raises(ValueError):
        y = torch.empty((260, shape.H), dtype=torch.bfloat16, device=DEV)
        bm.block_noalloc(MI.make_x(260, shape.H).to(DEV), wr, *packed, y)
    del packed
    torch.cuda.empty_cache()


def test_noalloc_captured_graph_replays(bm):
    """The no-allocation block captured in a HIP graph (its callers' use):
    replays on rewritten inputs, with eager work and synchronisations between
    them, equal eager beam_moe_block bit for bit."""
    shape = BlockShape(T=96, H=256, I=128)
    print("[case] noalloc graph replay", flush=True)
    inp = MI.make_block_inputs(shape, DEV, case=57)
    packed = bm.pack_experts(inp.wg, inp.wu, inp.wd)
    xs = [MI.make_x(shape.T, shape.H, case=70 + i).to(DEV) for i in range(3)]
    x_static = xs[0].clone()
    y_static = torch.empty((shape.T, shape.H), dtype=torch.bfloat16, device=DEV)
    ids_static = torch.empty((shape.T, shape.k), dtype=torch.int32, device=DEV)
    bm.block_noalloc(x_static, inp.wr, *packed, y_static, topk_ids=ids_static)   # device checks
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bm.block_noalloc(x_static, inp.wr, *packed, y_static, topk_ids=ids_static)
    for x in xs:
        x_static.copy_(x)
        g.replay()
        junk = torch.randn(1 << 18, device=DEV).mul_(2.0).sum()   # eager work between replays
        torch.cuda.synchronize()
        y_ref, ids_ref, _, _ = bm.block(x, inp.wr, *packed)
        torch.cuda.synchronize()
        assert torch.equal(y_static.view(torch.int16), y_ref.view(torch.int16))
        assert torch.equal(ids_static, ids_ref)
        del junk
    del g
