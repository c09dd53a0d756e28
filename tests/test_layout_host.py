"""Host checks of the packed layouts' LDS behaviour.

The tiled GEMM copies each k-step of packed FP8 weights into LDS unchanged
and then reads an MFMA weight operand as 8 bytes per lane: lane l reads row
l % 32 of a 32-row block (32-byte rows), chunk (2s + l // 32) ^ s(row) for
the half s of the step.  Depending on how the LDS serves 8-byte reads (a
group of lanes per cycle over a number of 4-byte banks), the swizzle must
keep every group free of bank conflicts.  The swizzle is the one the GPU
tests pin to the library's packing (layouts.fp8_chunk_swizzle)."""
import numpy as np
import pytest

from layouts import bf16_chunk_swizzle, fp8_chunk_swizzle


def conflict_ways(addrs, lanes, banks, width=8):
    """Largest number of accesses to one bank within a group of `lanes`
    consecutive lanes, each lane reading `width` bytes at its address."""
    worst = 1
    for g0 in range(0, len(addrs), lanes):
        count = {}
        for a in addrs[g0:g0 + lanes]:
            for w in range(width // 4):
                b = (a // 4 + w) % banks
                count[b] = count.get(b, 0) + 1
        worst = max(worst, max(count.values()))
    return worst


def operand_addrs(swz, s):
    return [32 * (l % 32) + 8 * ((2 * s + l // 32) ^ int(swz(l % 32))) for l in range(64)]


@pytest.mark.parametrize("lanes,banks", [(8, 32), (16, 32), (16, 64), (32, 64)])
def test_fp8_operand_reads_conflict_free(lanes, banks):
    for s in (0, 1):
        assert conflict_ways(operand_addrs(fp8_chunk_swizzle, s), lanes, banks) == 1


def test_bank_model_sees_a_swizzle_by_bits_3_and_4_conflict():
    """The model is sharp enough to see the conflict a swizzle by row bits
    3..4 alone has when 16 lanes share 32 banks (rows r and r + 4 collide)."""
    old = lambda j: (j >> 3) & 3
    assert conflict_ways(operand_addrs(old, 0), 16, 32) == 2
    assert conflict_ways(operand_addrs(old, 0), 32, 64) == 1


def test_fp8_swizzle_repeats_every_32_rows():
    """The kernel reads row r of every 32-row block with the same offsets."""
    j = np.arange(128)
    np.testing.assert_array_equal(fp8_chunk_swizzle(j), fp8_chunk_swizzle(j % 32))
    assert set(np.unique(fp8_chunk_swizzle(j)).tolist()) == {0, 1, 2, 3}


@pytest.mark.parametrize("lanes,banks", [(8, 32), (16, 64)])
def test_bf16_operand_reads_conflict_free(lanes, banks):
    """bf16 operands are 16-byte reads of 64-byte rows: lane l reads row
    l % 32, chunk (2s + l // 32) ^ s(row); the token slab of the tiled GEMM
    uses the same swizzle."""
    for s in (0, 1):
        addrs = [64 * (l % 32) + 16 * ((2 * s + l // 32) ^ int(bf16_chunk_swizzle(l % 32))) for l in range(64)]
        assert conflict_ways(addrs, lanes, banks, width=16) == 1
