"""Packed-weight layouts as the tests read them back (numpy index arithmetic).
The GPU tests check the library's packing against these bit for bit."""
import numpy as np


def fp8_chunk_swizzle(j):
    """Row j of a 128-row FP8 block stores its logical 8-byte chunk c (k
    offsets 8c .. 8c+7 of the 32-k block) at chunk position c ^ s(j), with
    s(j) = (bit2(j) ^ bit4(j)) + 2 bit3(j)."""
    j = np.asarray(j)
    return (((j >> 2) ^ (j >> 4)) & 1) | ((j >> 2) & 2)


def bf16_chunk_swizzle(j):
    """Row j of a 128-row bf16 block stores its logical 16-byte chunk c (k
    offsets 8c .. 8c+7 of the 32-k block) at chunk position c ^ s(j), with
    s(j) = ((j >> 1) ^ (j >> 2)) & 3."""
    j = np.asarray(j)
    return ((j >> 1) ^ (j >> 2)) & 3
