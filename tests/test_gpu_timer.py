"""The library's stage timer on the GPU: with no mask every stage of a block
call records its events; with a mask only the chosen stages do, so a timed
loop can carry the events of the one kernel it reports and no others."""
import pytest
import torch

import moe_inputs as MI
from moe_inputs import BlockShape

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
MOE_STAGES = ["router_logits", "select", "permute", "gateup", "down", "combine"]


def test_stage_timer_all_stages_and_mask():
    import sparse_moe_transformer_group_amd as bm
    shape = BlockShape(T=64, H=256, I=128, E=16, groups=4, topk_groups=2, k=4)
    print(f"[case] stage timer {shape}", flush=True)
    inp = MI.make_block_inputs(shape, DEV, case=71)
    packed = bm.pack_experts(inp.wg, inp.wu, inp.wd)

    def call():
        bm.block(inp.x, inp.wr, *packed, shape.groups, shape.topk_groups, shape.k, shape.scale)

    call()
    torch.cuda.synchronize()
    with bm.StageTimer(3) as t_all:
        for _ in range(3):
            call()
    assert t_all.calls == 3
    for n in MOE_STAGES:
        assert t_all.result[n] > 0, n
    assert all(v == 0 for n, v in t_all.result.items() if n.startswith("attn_"))

    with bm.StageTimer(4, stages=["gateup"]) as t_gu:
        for _ in range(3):
            call()
    assert t_gu.calls == 3
    assert set(t_gu.result) == {"gateup"} and t_gu.result["gateup"] > 0

    with pytest.raises(ValueError):
        bm.StageTimer(1, stages=["no_such_stage"]).__enter__()
    # the rejected mask started nothing: a new timer begins normally
    with bm.StageTimer(1, stages=["down", "combine"]) as t_dc:
        call()
    assert t_dc.calls == 1 and set(t_dc.result) == {"down", "combine"}
    assert t_dc.result["down"] > 0 and t_dc.result["combine"] > 0
