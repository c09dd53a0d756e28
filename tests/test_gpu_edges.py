"""GPU parity of the MoE block at the edges of its dimension rules, element by
element against the oracle (group-limited selection of page "Willkommen
Beam", section "Mixture of Experts"):

  * the most experts and slots the library takes: E = 512 in 16 groups of
    32, 8 kept groups, k = 32 (8 experts per lane in the selection, 32 slots
    in the combine, the multi-block permutation);
  * an expert count that is not a multiple of 4 and groups that are not a
    power of two (E = 250 in 5 groups of 50): the selection's scalar path;
  * the largest hidden size (H = 32768: long router and gate/up reductions)
    and the largest intermediate size (I = 32768: long down reduction, many
    gate/up feature tiles);
on both expert-GEMM schedules."""
import pytest
import torch

import moe_inputs as MI
import oracle as O
from moe_inputs import BlockShape, bf16_bits

from parity import check_output, check_routing, keep_mask, sync

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def bm():
    import sparse_moe_transformer_group_amd as bm
    yield bm
    bm.set_schedule("auto")


def edge_case(bm, shape, schedule, case):
    print(f"[case] edges {shape} schedule={schedule}", flush=True)
    inp = MI.make_block_inputs(shape, DEV, case=case)
    bm.set_schedule(schedule)
    try:
        y, ids, w, counts = bm.block(inp.x, inp.wr, *bm.pack_experts(inp.wg, inp.wu, inp.wd),
                                     shape.groups, shape.topk_groups, shape.k, shape.scale)
        sync()
    finally:
        bm.set_schedule("auto")
    ref = O.moe_block(bf16_bits(inp.x), bf16_bits(inp.wr),
                      (bf16_bits(inp.wg), bf16_bits(inp.wu), bf16_bits(inp.wd)),
                      shape.groups, shape.topk_groups, shape.k, shape.scale)
    st = check_routing(ids, w, ref, shape, counts)
    st.update(check_output(y, ref["y"], keep_mask(ref)))
    print({k: v for k, v in st.items() if k != "excluded_tokens"}, flush=True)


@pytest.mark.parametrize("schedule", ["stream", "tiled"])
def test_block_512_experts_k32(bm, schedule):
    edge_case(bm, BlockShape(T=100, H=256, I=128, E=512, groups=16, topk_groups=8, k=32),
              schedule, case=61)


@pytest.mark.parametrize("schedule", ["stream", "tiled"])
def test_block_250_experts_5_groups(bm, schedule):
    edge_case(bm, BlockShape(T=64, H=256, I=128, E=250, groups=5, topk_groups=2, k=6),
              schedule, case=62)


@pytest.mark.parametrize("schedule", ["stream", "tiled"])
def test_block_largest_hidden(bm, schedule):
    edge_case(bm, BlockShape(T=5, H=32768, I=64, E=8, groups=2, topk_groups=1, k=2),
              schedule, case=63)


@pytest.mark.parametrize("schedule", ["stream", "tiled"])
def test_block_largest_intermediate(bm, schedule):
    edge_case(bm, BlockShape(T=3, H=64, I=32768, E=4, groups=2, topk_groups=1, k=2),
              schedule, case=64)


def test_block_prefill_router_ragged(bm):
    """The prefill-size router (128-token tiles, T >= 1024) with a ragged last
    tile (T = 1100) and fewer experts than a workgroup covers (E = 96: three
    of its four waves have no experts and only take part in the barriers)."""
    edge_case(bm, BlockShape(T=1100, H=320, I=128, E=96, groups=12, topk_groups=3, k=6),
              "auto", case=65)
