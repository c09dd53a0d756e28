"""C ABI checks that need no GPU: the library loads, exports every function
include/beam_moe.h declares, and rejects bad arguments on the host before any
HIP call (so these calls are safe without a device)."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_moe_transformer_group_amd as bm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "beam_moe.h")

lib = bm.lib
P = 0x10000  # a 16-byte aligned fake device pointer; never dereferenced here
BIG = 1 << 40


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(beam_(?:moe|attn|dense)_\w+)\s*\(", src)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ("beam_moe_route", "beam_moe_permute", "beam_moe_forward", "beam_moe_block",
              "beam_moe_workspace_bytes", "beam_moe_status_string", "beam_moe_sublayer",
              "beam_attn_forward", "beam_attn_workspace_bytes", "beam_dense_mlp",
              "beam_dense_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", bm.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert hasattr(ctypes.CDLL(bm.LIB_PATH), n)


def test_status_strings():
    for code in range(-6, 1):
        assert lib.beam_moe_status_string(code)
    assert lib.beam_moe_status_string(-99) == b"unknown status"


def test_workspace_bytes():
    n = lib.beam_moe_workspace_bytes(8192, 5120, 2560, 256, 8)
    # o partials (fp32) and h (bf16) dominate
    assert n >= 8192 * 8 * (5120 * 4 + 2560 * 2)
    assert lib.beam_moe_workspace_bytes(64, 5120, 2560, 256, 8) > 0
    assert lib.beam_moe_workspace_bytes(64, 100, 2560, 256, 8) == 0   # H not a multiple of 64
    assert lib.beam_moe_workspace_bytes(-1, 5120, 2560, 256, 8) == 0
    assert lib.beam_moe_workspace_bytes(64, 5120, 2560, 600, 8) == 0  # E > 512
    assert lib.beam_moe_workspace_bytes(64, 5120, 2560, 256, 33) == 0  # k > 32


def route(T=64, H=5120, E=256, G=8, KG=4, k=8, scale=2.5, x=P, wr=P, off=None, ids=P, w=P,
          counts=None, ws=P, wsb=BIG):
    return lib.beam_moe_route(None, T, H, E, G, KG, k, scale, x, wr, off, ids, w, counts, ws, wsb)


def test_route_validation():
    assert route(H=100) == -1
    assert route(E=255) == -1            # not divisible by 8 groups
    assert route(E=16, G=16) == -1       # groups of one expert
    assert route(KG=9) == -1
    assert route(KG=0) == -1
    assert route(k=0) == -1
    assert route(k=33) == -1
    assert route(E=16, G=8, KG=1, k=3) == -1   # only 2 eligible experts
    assert route(scale=float("inf")) == -1
    assert route(T=-5) == -1
    assert route(x=None) == -2
    assert route(ws=None) == -2
    assert route(wr=P + 8) == -3
    assert route(off=P + 4) == -3
    assert route(counts=P + 2) == -3
    assert route(wsb=16) == -4
    assert route(T=0) == 0                # no-op, no device touched


def forward(T=64, H=5120, I=2560, E=256, k=8, x=P, ids=P, w=P, wg=P, wu=P, wd=P, y=P,
            counts=None, ws=P, wsb=BIG):
    return lib.beam_moe_forward(None, T, H, I, E, k, x, ids, w, wg, wu, wd, y, counts, ws, wsb)


def test_forward_validation():
    assert forward(I=100) == -1
    assert forward(H=0) == -1
    assert forward(k=0) == -1
    assert forward(E=0) == -1
    assert forward(wd=None) == -2
    assert forward(y=P + 2) == -3
    assert forward(wsb=1024) == -4
    assert forward(T=0) == 0


def block(T=64, H=5120, I=2560, E=256, G=8, KG=4, k=8, scale=2.5, ws=P, wsb=BIG, **kw):
    a = dict(x=P, wr=P, off=None, wg=P, wu=P, wd=P, y=P, ids=None, w=None, counts=None)
    a.update(kw)
    return lib.beam_moe_block(None, T, H, I, E, G, KG, k, scale, a["x"], a["wr"], a["off"], a["wg"],
                              a["wu"], a["wd"], a["y"], a["ids"], a["w"], a["counts"], ws, wsb)


def test_block_validation():
    assert block(G=3) == -1
    assert block(I=96) == -1
    assert block(k=40) == -1
    assert block(wr=None) == -2
    assert block(ids=P + 4) == -3
    need = lib.beam_moe_workspace_bytes(64, 5120, 2560, 256, 8)
    assert block(wsb=need - 1) == -4
    assert block(T=0, wsb=need) == 0


def test_pack_validation_and_sizes():
    # one packed expert matrix: ceil(N/128) row blocks x K/32 k-blocks of 8 KB
    assert lib.beam_moe_packed_weight_bytes(2560, 5120) == 20 * 160 * 8192
    assert lib.beam_moe_packed_weight_bytes(5120, 2560) == 40 * 80 * 8192
    assert lib.beam_moe_packed_weight_bytes(192, 64) == 2 * 2 * 8192      # padded to 256 rows
    assert lib.beam_moe_packed_weight_bytes(100, 64) == 0
    assert lib.beam_moe_packed_weight_bytes(128, 0) == 0
    big = 1 << 36
    assert lib.beam_moe_pack_weights(None, 0, 128, 128, P, big) == -1       # E < 1
    assert lib.beam_moe_pack_weights(None, 4, 96, 128, P, big) == -1       # N not a multiple of 64
    assert lib.beam_moe_pack_weights(None, 4, 128, 128, None, big) == -2
    assert lib.beam_moe_pack_weights(None, 4, 128, 128, P + 8, big) == -3
    assert lib.beam_moe_pack_weights(None, 4, 128, 128, P, P + 4096) == -1  # overlapping buffers


def test_permute_and_helpers_validation():
    assert lib.beam_moe_permute(None, 10, 0, 8, P, P, P, P, P, P, BIG) == -1
    assert lib.beam_moe_permute(None, 10, 256, 8, P, P, None, P, P, P, BIG) == -2
    assert lib.beam_moe_permute(None, 10, 256, 8, P, P, P, P, P, P, 8) == -4
    assert lib.beam_moe_permute(None, 0, 256, 8, P, P, P, P, P, P, BIG) == 0
    assert lib.beam_moe_rmsnorm(None, 4, 100, 1e-6, P, P) == -1
    assert lib.beam_moe_rmsnorm(None, 4, 128, -1.0, P, P) == -1
    assert lib.beam_moe_rmsnorm(None, 0, 128, 1e-6, P, P) == 0
    assert lib.beam_moe_residual_update(None, 4, 128, 1e-6, 1, P, P) == -1   # step 1 is the embedding
    assert lib.beam_moe_residual_update(None, 4, 128, 1e-6, 2, None, P) == -2
    assert lib.beam_moe_stream_init(None, 4, 128, P + 1, P) == -3
    assert lib.beam_moe_sublayer(None, 4, 128, 64, 16, 4, 2, 2, 2.5, 1e-6, 1, P, P, P, P, P,
                                 None, None, None, None, None, P, BIG) == -1
    assert lib.beam_moe_set_schedule(3) == -1
    assert lib.beam_moe_set_schedule(0) == 0


def test_timer_api_without_device():
    assert lib.beam_moe_stage_count() == 10
    assert lib.beam_moe_stage_name(0) == b"router_logits"
    assert [lib.beam_moe_stage_name(i) for i in (6, 7, 8, 9)] == [
        b"attn_proj", b"attn_prep", b"attn_flash", b"attn_out"]
    assert lib.beam_moe_stage_name(99) == b""
    assert lib.beam_moe_timer_begin(0) == -1
    assert lib.beam_moe_timer_begin_stages(0, 1) == -1
    assert lib.beam_moe_timer_begin_stages(4, 0) == -1                # no stage
    assert lib.beam_moe_timer_begin_stages(4, 1 << 10) == -1          # no such stage
    n = ctypes.c_int(0)
    arr = (ctypes.c_double * 10)()
    assert lib.beam_moe_timer_end(arr, 10, ctypes.byref(n)) == -1   # not started


def test_product_path_does_not_import_oracle():
    """The HIP binding must not reach the CPU oracle (no fallback)."""
    pkg = os.path.join(ROOT, "sparse_moe_transformer_group_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "oracle" not in src.replace("oracle is", ""), f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            src = open(os.path.join(ROOT, "oracle", f), encoding="utf-8").read()
            assert "sparse_moe_transformer_group_amd" not in src, f


def test_attention_rejects_bad_arguments_on_host():
    assert lib.beam_attn_workspace_bytes(8192, 5120) >= 8192 * 14336 * 4   # FP32 projections
    assert lib.beam_attn_workspace_bytes(8192, 100) == 0
    assert lib.beam_attn_workspace_bytes(-1, 5120) == 0
    assert lib.beam_attn_workspace_bytes((1 << 16) + 1, 5120) == 0
    assert lib.beam_attn_workspace_bytes(1 << 15, 32768) == 0         # T * H >= 2^30
    assert lib.beam_attn_workspace_bytes((1 << 15) - 1, 32768) > 0
    ws = lib.beam_attn_workspace_bytes(64, 256)
    f = lib.beam_attn_forward

    def call(T=64, H=256, g=0, win=512, theta=1e4, u=P, wqkvg=P, wo=P, y=P, w=P, nb=ws):
        return f(None, T, H, g, win, theta, u, wqkvg, wo, y, w, nb)
    assert call(H=100) == -1
    assert call(T=-1) == -1
    assert call(g=2) == -1
    assert call(win=0) == -1
    assert call(theta=0.0) == -1
    assert call(theta=float("nan")) == -1
    assert call(T=0) == 0                                   # empty sequence: nothing to do
    assert call(u=None) != 0
    assert call(nb=ws - 1) == -4
    assert call(g=1, win=0, theta=0.0, nb=ws - 1) == -4     # window/theta unused on global layers


def test_dense_rejects_bad_arguments_on_host():
    n = lib.beam_dense_workspace_bytes(8192, 5120, 20480, 8)
    assert n >= 8192 * 8 * 5120 * 4        # FP32 chunk outputs
    assert lib.beam_dense_workspace_bytes(64, 5120, 20480, 3) == 0     # I % chunks
    assert lib.beam_dense_workspace_bytes(64, 5120, 20480, 33) == 0    # chunks > 32
    assert lib.beam_dense_workspace_bytes(64, 5120, 20480 + 64, 8) == 0  # I / chunks not a multiple of 64
    assert lib.beam_dense_workspace_bytes(64, 100, 2048, 1) == 0
    ws = lib.beam_dense_workspace_bytes(64, 256, 512, 2)
    f = lib.beam_dense_mlp

    def call(T=64, H=256, I=512, C=2, x=P, g=P, u=P, d=P, y=P, w=P, nb=ws):
        return f(None, T, H, I, C, x, g, u, d, y, w, nb)
    assert call(C=0) == -1
    assert call(I=500) == -1
    assert call(T=-1) == -1
    assert call(T=0) == 0
    assert call(g=None) == -2
    assert call(y=P + 2) == -3
    assert call(nb=ws - 1) == -4
    f8 = lib.beam_dense_mlp_fp8
    assert f8(None, 64, 256, 512, 2, P, P, None, P, P, P, P, P, P, ws) == -2      # gate scales missing
    assert f8(None, 64, 256, 512, 3, P, P, P, P, P, P, P, P, P, ws) == -1         # I % chunks
    assert f8(None, 0, 256, 512, 2, P, P, P, P, P, P, P, P, P, ws) == 0


def block_noalloc(T=64, H=5120, I=2560, E=256, G=8, KG=4, k=8, scale=2.5, **kw):
    a = dict(x=P, wr=P, off=None, wg=P, wu=P, wd=P, y=P, ids=None, w=None, counts=None)
    a.update(kw)
    return lib.beam_moe_block_noalloc(None, T, H, I, E, G, KG, k, scale, a["x"], a["wr"], a["off"],
                                      a["wg"], a["wu"], a["wd"], a["y"], a["ids"], a["w"],
                                      a["counts"])


def test_block_noalloc_validation_and_scratch_limit():
    """Host-side checks of the no-allocation block (nothing reaches a device):
    dimension, pointer and alignment errors as in beam_moe_block, and sizes
    beyond the static scratch rejected before any launch."""
    assert bm.NOALLOC_SCRATCH_BYTES == 64 << 20
    assert block_noalloc(G=3) == -1
    assert block_noalloc(k=40) == -1
    assert block_noalloc(wr=None) == -2
    assert block_noalloc(y=None) == -2
    assert block_noalloc(ids=P + 4) == -3
    assert block_noalloc(T=0) == 0
    # the largest Beam-shape batch that fits, and the first that does not
    fits = max(T for T in range(1, 400)
               if lib.beam_moe_workspace_bytes(T, 5120, 2560, 256, 8) <= bm.NOALLOC_SCRATCH_BYTES)
    assert fits == 259
    assert block_noalloc(T=fits + 1) == -4
    assert block_noalloc(T=8192) == -4
