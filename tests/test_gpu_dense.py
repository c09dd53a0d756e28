"""GPU parity of the dense SwiGLU layer (beam_dense_mlp) against the FP64
oracle, through the C ABI.

The layer runs as the expert path over `chunks` pieces of its intermediate
dimension.  Small shapes are compared element by element for 1, 2 and 8
chunks (8 chunks of 64 rows), sequence lengths from 1 to 1000 tokens, on the
streaming and the tiled GEMM schedule, with bf16 and with FP8 weights (the
oracle on its own dequantised E4M3 encoding); the Beam shape (H = 5120, I = 20480)
in full at T = 64 (8 chunks) and on sampled rows at T = 8192 (1 and 8
chunks: the configurations the benchmark times)."""
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
    yield bm
    bm.set_schedule("auto")


def fp8_oracle_weights(wg, wu, wd, chunks):
    """The oracle's own E4M3 encoding, dequantised: one scale per row of gate
    and up, and per row of each chunk of down (its columns split in chunks)."""
    deq = lambda m: O.dequantize_rows(*O.quantize_rows(m))
    d = bf16_bits(wd)
    Ic = d.shape[1] // chunks
    dq = np.concatenate([deq(np.ascontiguousarray(d[:, c * Ic:(c + 1) * Ic])) for c in range(chunks)], axis=1)
    return deq(bf16_bits(wg)), deq(bf16_bits(wu)), dq


def run(bm, T, H, I, chunks, schedule="auto", case=0, rows=None, fp8=False):
    print(f"[case] dense T={T} H={H} I={I} chunks={chunks} schedule={schedule} fp8={fp8}", flush=True)
    x = MI.make_x(T, H, case=case).to(DEV)
    wg, wu, wd = MI.make_dense_weights(H, I, DEV, case=case)
    packed = bm.pack_dense(wg, wu, wd, chunks=chunks, fp8=fp8)
    bm.set_schedule(schedule)
    try:
        y = bm.dense_mlp(x, *packed)
        sync()
    finally:
        bm.set_schedule("auto")
    xs = x if rows is None else x[torch.as_tensor(rows, device=DEV)]
    ws = fp8_oracle_weights(wg, wu, wd, chunks) if fp8 else (bf16_bits(wg), bf16_bits(wu), bf16_bits(wd))
    ref = O.dense_mlp(bf16_bits(xs), *ws)
    yg = y if rows is None else y[torch.as_tensor(rows, device=DEV)]
    return y, check_output(yg, ref)


@pytest.mark.parametrize("schedule", ["stream", "tiled"])
@pytest.mark.parametrize("chunks", [1, 2, 8])
@pytest.mark.parametrize("T", [1, 7, 130, 1000])
def test_dense_small(bm, T, chunks, schedule):
    print(run(bm, T, 256, 512, chunks, schedule, case=T)[1])


@pytest.mark.parametrize("schedule", ["stream", "tiled"])
@pytest.mark.parametrize("chunks", [1, 2])
@pytest.mark.parametrize("T", [7, 130, 1000])
def test_dense_small_fp8(bm, T, chunks, schedule):
    print(run(bm, T, 256, 512, chunks, schedule, case=T + 1, fp8=True)[1])


def test_dense_chunking_changes_only_summation_order(bm):
    """1, 2 and 8 chunks of the same layer agree to FP32 summation order."""
    ys = [run(bm, 300, 320, 1024, c, case=5)[0].float() for c in (1, 2, 8)]
    for y in ys[1:]:
        assert torch.allclose(y, ys[0], rtol=1e-2, atol=1e-2 * ys[0].abs().max().item())


def test_dense_empty(bm):
    wg, wu, wd = MI.make_dense_weights(256, 512, DEV)
    y = bm.dense_mlp(torch.empty((0, 256), dtype=torch.bfloat16, device=DEV), *bm.pack_dense(wg, wu, wd))
    sync()
    assert y.shape == (0, 256)


@pytest.mark.slow
def test_dense_beam_decode_T64(bm):
    print(run(bm, 64, 5120, 20480, 8)[1])


@pytest.mark.slow
def test_dense_beam_decode_T64_fp8(bm):
    print(run(bm, 64, 5120, 20480, 8, fp8=True)[1])


@pytest.mark.slow
@pytest.mark.parametrize("chunks", [1, 8])
def test_dense_beam_prefill_T8192_sampled(bm, chunks):
    rows = [0, 1, 221, 222, 319, 320, 4095, 4096, 8190, 8191]
    print(run(bm, 8192, 5120, 20480, chunks, rows=rows)[1])
