"""The seeded input generator: determinism, shapes and value recipe."""
import numpy as np
import torch

import moe_inputs as MI


def test_seed_is_deterministic_and_keyed():
    assert MI.seed_for(1, 2, 3) == MI.seed_for(1, 2, 3)
    assert MI.seed_for(1, 2, 3) != MI.seed_for(1, 2, 4)


def test_x_and_router_are_reproducible():
    a = MI.make_x(16, 256)
    b = MI.make_x(16, 256)
    assert a.dtype == torch.bfloat16 and a.shape == (16, 256)
    assert torch.equal(a, b)
    assert not torch.equal(MI.make_x(16, 256, layer=1), a)
    wr = MI.make_router(256, 512)
    assert wr.shape == (256, 512)
    assert abs(wr.float().std().item() - 0.02) < 0.001


def test_expert_weights_cpu_recipe():
    wg, wu, wd = MI.make_expert_weights(4, 128, 64, "cpu")
    assert wg.shape == (4, 64, 128) and wu.shape == (4, 64, 128) and wd.shape == (4, 128, 64)
    for w in (wg, wu, wd):
        assert abs(w.float().std().item() - 0.02) < 0.001
    wg2, _, _ = MI.make_expert_weights(4, 128, 64, "cpu")
    assert torch.equal(wg, wg2)
    assert not torch.equal(wg[0], wg[1])


def test_zipf_offsets_file():
    off = MI.load_zipf_offsets(256)
    assert off.dtype == torch.float32 and off.shape == (256,)
    assert float(off.min()) >= -8.0 and float(off.max()) <= 6.0
    ranks = MI.zipf_rank_permutation(256)
    # hotter ranks get larger offsets on average
    order = np.argsort(ranks)
    o = off.numpy()[order]
    assert o[:16].mean() > o[-16:].mean()


def test_bf16_bits_roundtrip():
    t = MI.make_x(3, 64)
    bits = MI.bf16_bits(t)
    assert bits.dtype == np.uint16
    back = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    assert torch.equal(back, t)
