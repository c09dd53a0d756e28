"""GPU parity of the attention sublayer (beam_attn_forward) against the FP64
oracle, through the C ABI.

Small hidden size (H = 256) with every output element compared: sequence
lengths from a single token to several 128-query tiles with a ragged tail,
both layer types, windows narrower than a tile, window 1 (each token sees
only itself) and a window wider than the sequence.  At the full shape
(T = 8192, H = 5120) sampled rows are compared: the first tokens, both sides
of the 512-token window edge, tile edges and the last token."""
import numpy as np
import pytest
import torch

import moe_inputs as MI
import oracle as O
from moe_inputs import bf16_bits

from parity import check_output, sync

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def bm():
    import sparse_moe_transformer_group_amd as bm
    return bm


def run_case(bm, T, H, global_layer, window=512, theta=10000.0, case=0, rows=None):
    print(f"[case] attention T={T} H={H} global={global_layer} window={window} "
          f"theta={theta} case={case}", flush=True)
    u = MI.make_attention_input(T, H, case=case)
    ws = MI.make_attention_weights(H, case=case)
    w_qkvg, w_o = bm.pack_attention_weights(*[w.to(DEV) for w in ws])
    y = bm.attention(u.to(DEV), w_qkvg, w_o, global_layer, window=window, theta=theta)
    sync()
    ref = O.attention_sublayer(bf16_bits(u), *[bf16_bits(w) for w in ws], global_layer,
                               window=window, theta=theta, rows=rows)
    yg = y[torch.from_numpy(ref["rows"]).to(DEV)] if rows is not None else y
    # the first tokens attend over a handful of keys, so their outputs reach
    # ~11 RMS of the whole output, where the bf16 rounding of y alone is half
    # an ulp: that rounding is allowed on top of the usual bar
    return check_output(yg, ref["y"], out_rounding_slack=True)


@pytest.mark.parametrize("global_layer", [False, True])
@pytest.mark.parametrize("T", [1, 7, 130, 700])
def test_attention_small(bm, T, global_layer):
    print(run_case(bm, T, 256, global_layer, case=T))


@pytest.mark.parametrize("T,window", [(300, 1), (300, 64), (300, 127), (400, 129), (200, 4096)])
def test_attention_windows(bm, T, window):
    print(run_case(bm, T, 256, False, window=window, case=window))


def test_attention_rope_base(bm):
    print(run_case(bm, 260, 320, False, window=100, theta=500000.0, case=3))


def test_attention_empty_sequence(bm):
    w_qkvg, w_o = bm.pack_attention_weights(*[w.to(DEV) for w in MI.make_attention_weights(256)])
    y = bm.attention(torch.empty((0, 256), dtype=torch.bfloat16, device=DEV), w_qkvg, w_o, False)
    sync()
    assert y.shape == (0, 256)


def test_attention_repeat_calls_are_identical(bm):
    """The tile counters and workspace are reset by every call."""
    u = MI.make_attention_input(700, 256, case=9).to(DEV)
    w_qkvg, w_o = bm.pack_attention_weights(*[w.to(DEV) for w in
                                              MI.make_attention_weights(256, case=9)])
    y1 = bm.attention(u, w_qkvg, w_o, True).clone()
    bm.attention(u[:130].contiguous(), w_qkvg, w_o, False)
    y2 = bm.attention(u, w_qkvg, w_o, True)
    sync()
    assert torch.equal(y1, y2)


FULL_ROWS = [0, 1, 63, 127, 128, 511, 512, 513, 1000, 4095, 4096, 6143, 8190, 8191]


@pytest.mark.slow
@pytest.mark.parametrize("global_layer", [False, True])
def test_attention_full_shape_sampled_rows(bm, global_layer):
    print(run_case(bm, 8192, 5120, global_layer, rows=FULL_ROWS))


@pytest.mark.slow
@pytest.mark.parametrize("global_layer", [False, True])
def test_attention_long_sequence_sampled_rows(bm, global_layer):
    """Positions up to 20000 (RoPE angles far beyond FP32 resolution of the
    product pos * theta^(-i/64)); T not a multiple of the 128-query tile."""
    rows = [0, 511, 512, 10000, 19487, 19488, 19999]
    print(run_case(bm, 20000, 1024, global_layer, rows=rows, case=7))
