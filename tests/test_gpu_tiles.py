"""GPU parity of the tiled grouped-GEMM schedule over every tile shape it has.

Routing is injected, so each expert's token count is chosen: counts from 1 to
1000 give tiles of every token-block count (1..10 blocks of 32 tokens, up to
320 tokens per tile, blocks 8 and 9 accumulating in VGPRs), partial last
blocks, and experts split over 2, 3 and 4 token tiles.  Hot experts of 2600
to 5000 tokens (9 to 16 token tiles) take the blocked order in which runs of
32 tiles cover 4 feature tiles x 8 token tiles: full and partial chunks of
token tiles, and feature-tile groups of 4 with a remainder (5 feature tiles
at I = 640 and H = 1280).  Outputs are compared element by element with the
oracle's forward pass, for bf16 weights and for FP8 weights (oracle run on
its own dequantised E4M3 weights)."""
import numpy as np
import pytest
import torch

import moe_inputs as MI
import oracle as O
from moe_inputs import BlockShape, bf16_bits

from parity import check_output, sync

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

# tokens per expert: one tile of 1..10 token blocks (full and partial last
# blocks), then experts split into 2 (321, 640), 3 (641) and 4 (1000) tiles
COUNTS = [1, 31, 32, 33, 64, 95, 130, 200, 255, 256, 257, 288, 300, 319, 320, 321, 640, 641, 1000]
# hot experts: 9 token tiles (one chunk of 8 + a chunk of 1), 9 (2880 = 9 x 320,
# full tiles), 13 (8 + 5) and 16 (two full chunks of 8), beside small experts
HOT_COUNTS = [2600, 2880, 4000, 5000, 333, 17]


@pytest.fixture(scope="module")
def bm():
    import sparse_moe_transformer_group_amd as bm
    yield bm
    bm.set_schedule("auto")


def injected_routing(E, seed, counts=COUNTS):
    """ids [T, 2] / weights [T, 2]: slot 0 sends token t to its expert (the
    experts of `counts` spread over [0, E)), slot 1 is a dropped id (-1)."""
    rng = np.random.default_rng(seed)
    experts = (13 * np.arange(len(counts)) + 5) % E
    ids0 = np.concatenate([np.full(c, e) for c, e in zip(counts, experts)])
    ids0 = ids0[rng.permutation(ids0.size)]             # tokens of an expert scattered over x
    T = ids0.size
    ids = np.stack([ids0, np.full(T, -1)], axis=1).astype(np.int32)
    w = np.stack([rng.uniform(0.5, 2.5, T), np.ones(T)], axis=1).astype(np.float32)
    return ids, w


def fp8_oracle_experts(wg, wu, wd):
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = tuple(O.dequantize_rows(*O.quantize_rows(bf16_bits(m[e]))) for m in (wg, wu, wd))
        return cache[e]
    return get


def tiled_case(bm, weights, H, I, counts, what):
    E = 256
    ids, w = injected_routing(E, seed=H + I, counts=counts)
    T = ids.shape[0]
    print(f"[case] tiled {what} weights={weights} T={T} H={H} I={I}", flush=True)
    shape = BlockShape(T=T, H=H, I=I)
    inp = MI.make_block_inputs(shape, DEV, case=40 + H % 7)
    if weights == "fp8":
        packed = bm.pack_experts_fp8(inp.wg, inp.wu, inp.wd)
        experts = fp8_oracle_experts(inp.wg, inp.wu, inp.wd)
    else:
        packed = bm.pack_experts(inp.wg, inp.wu, inp.wd)
        experts = (bf16_bits(inp.wg), bf16_bits(inp.wu), bf16_bits(inp.wd))
    bm.set_schedule("tiled")
    try:
        y, got_counts = bm.forward(inp.x, torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV),
                                   *packed, return_counts=True)
        sync()
    finally:
        bm.set_schedule("auto")
    valid = ids[(ids >= 0) & (ids < E)]
    assert np.array_equal(got_counts.cpu().numpy(), np.bincount(valid, minlength=E))
    ref = O.moe_forward(bf16_bits(inp.x), ids, w, experts, E=E)
    # one expert per token: the bf16 output's own rounding (half an ulp of
    # tails up to ~12 RMS) is allowed on top of the usual bar
    print(check_output(y, ref, out_rounding_slack=True), flush=True)


@pytest.mark.parametrize("weights", ["bf16", "fp8"])
@pytest.mark.parametrize("H,I", [(256, 128), (320, 384)])
def test_tiled_every_tile_shape(bm, weights, H, I):
    tiled_case(bm, weights, H, I, COUNTS, "tile shapes")


@pytest.mark.parametrize("weights", ["bf16", "fp8"])
@pytest.mark.parametrize("H,I", [(256, 128), (1280, 640)])
def test_tiled_hot_expert_blocks(bm, weights, H, I):
    tiled_case(bm, weights, H, I, HOT_COUNTS, "hot-expert blocks")
