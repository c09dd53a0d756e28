"""Pins of the dense SwiGLU layer oracle against torch's SiLU and bf16
conversion, the chunk decomposition the device uses, and trivial inputs."""
import numpy as np
import torch

import oracle as O


def bits(a):
    return O.f64_to_bf16_bits(a)


def layer(seed, T=9, H=64, I=256):
    rng = np.random.default_rng(seed)
    x = bits(rng.standard_normal((T, H)))
    wg, wu = bits(rng.standard_normal((I, H)) * 0.2), bits(rng.standard_normal((I, H)) * 0.2)
    wd = bits(rng.standard_normal((H, I)) * 0.2)
    return x, wg, wu, wd


def torch_of(b):
    return torch.from_numpy(O.bf16_bits_to_f64(b))


def test_dense_matches_torch_silu_and_bf16_rounding():
    x, wg, wu, wd = layer(1)
    X, G, U, D = (torch_of(b) for b in (x, wg, wu, wd))
    h = torch.nn.functional.silu(X @ G.T) * (X @ U.T)
    h = h.to(torch.bfloat16).to(torch.float64)          # torch's own RNE conversion
    ref = (h @ D.T).numpy()
    assert np.allclose(O.dense_mlp(x, wg, wu, wd), ref, rtol=1e-12, atol=1e-12)


def test_dense_chunk_decomposition():
    """The intermediate dimension split into C chunks (rows of gate/up, columns
    of down): the chunks' outputs sum to the whole layer's output."""
    x, wg, wu, wd = layer(2, I=512)
    full = O.dense_mlp(x, wg, wu, wd)
    for C in (2, 4, 8):
        Ic = 512 // C
        parts = sum(O.dense_mlp(x, wg[c * Ic:(c + 1) * Ic], wu[c * Ic:(c + 1) * Ic],
                                np.ascontiguousarray(wd[:, c * Ic:(c + 1) * Ic])) for c in range(C))
        assert np.allclose(parts, full, rtol=1e-12, atol=1e-12)


def test_dense_zero_cases():
    x, wg, wu, wd = layer(3)
    assert np.all(O.dense_mlp(np.zeros_like(x), wg, wu, wd) == 0.0)
    assert np.all(O.dense_mlp(x, wg, np.zeros_like(wu), wd) == 0.0)


def test_dense_width_reading():
    assert O.DENSE_INTERMEDIATE == 20480
