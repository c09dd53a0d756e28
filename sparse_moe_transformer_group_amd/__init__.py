"""Beam Mixture-of-Experts block on AMD Instinct MI355X (gfx950).

The block (router, group-limited top-k, token permutation, grouped SwiGLU
expert GEMMs, combine) runs in the HIP kernels of libbeam_moe.so behind the C
ABI declared in include/beam_moe.h; this package is its ctypes binding.
Importing it fails if the library has not been built.
"""
from ._lib import (  # noqa: F401
    BeamMoeError, NOALLOC_SCRATCH_BYTES, PackedFP8, PackedMatrix, StageTimer, attention,
    attention_workspace_bytes, block, block_noalloc,
    dense_mlp, dense_workspace_bytes, pack_dense, forward, get_workspace, lib,
    pack_attention_weights, pack_experts, pack_experts_fp8, pack_weights, pack_weights_fp8, packed_fp8_bytes,
    packed_weight_bytes, permute, release_workspaces, residual_update, rmsnorm, route,
    set_schedule, stage_names, stream_init, sublayer, version, workspace_bytes,
)
from .build import LIB_PATH  # noqa: F401
