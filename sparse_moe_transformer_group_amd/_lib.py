"""ctypes binding of libbeam_moe.so (declarations in include/beam_moe.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, and their device pointers, the sizes and torch's current HIP
stream are passed to the C ABI.  Every step of the block runs in the HIP
kernels of the library.  There is no fallback: if the library is missing or
cannot be loaded, importing this module raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional

import torch

from .build import LIB_PATH

_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_f = ctypes.c_float
_c_vp = ctypes.c_void_p
_c_sz = ctypes.c_size_t

STATUS = {
    0: "ok", -1: "invalid dimension", -2: "null pointer", -3: "misaligned pointer",
    -4: "workspace too small", -5: "unsupported device", -6: "HIP error",
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python -m sparse_moe_transformer_group_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "beam_moe_status_string": (ctypes.c_char_p, [_c_int]),
        "beam_moe_version": (ctypes.c_char_p, []),
        "beam_moe_workspace_bytes": (_c_sz, [_c_i64, _c_int, _c_int, _c_int, _c_int]),
        "beam_moe_packed_weight_bytes": (_c_sz, [_c_int, _c_int]),
        "beam_moe_pack_weights": (_c_int, [_c_vp, _c_int, _c_int, _c_int, _c_vp, _c_vp]),
        "beam_moe_packed_fp8_bytes": (_c_sz, [_c_int, _c_int]),
        "beam_moe_pack_weights_fp8": (_c_int, [_c_vp, _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_vp]),
        "beam_moe_route": (_c_int, [_c_vp, _c_i64, _c_int, _c_int, _c_int, _c_int, _c_int, _c_f,
                                    _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz]),
        "beam_moe_permute": (_c_int, [_c_vp, _c_i64, _c_int, _c_int, _c_vp, _c_vp, _c_vp, _c_vp,
                                      _c_vp, _c_vp, _c_sz]),
        "beam_moe_forward": (_c_int, [_c_vp, _c_i64, _c_int, _c_int, _c_int, _c_int, _c_vp, _c_vp,
                                      _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz]),
        "beam_moe_block": (_c_int, [_c_vp, _c_i64, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                    _c_f, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                    _c_vp, _c_vp, _c_vp, _c_sz]),
        "beam_moe_block_noalloc": (_c_int, [_c_vp, _c_i64, _c_int, _c_int, _c_int, _c_int, _c_int,
                                            _c_int, _c_f, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                            _c_vp, _c_vp, _c_vp, _c_vp]),
        "beam_moe_forward_fp8": (_c_int, [_c_vp, _c_i64, _c_int, _c_int, _c_int, _c_int, _c_vp,
                                          _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                          _c_vp, _c_vp, _c_vp, _c_vp, _c_sz]),
        "beam_moe_block_fp8": (_c_int, [_c_vp, _c_i64, _c_int, _c_int, _c_int, _c_int, _c_int,
                                        _c_int, _c_f, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                        _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                        _c_sz]),
        "beam_moe_stream_init": (_c_int, [_c_vp, _c_i64, _c_int, _c_vp, _c_vp]),
        "beam_moe_rmsnorm": (_c_int, [_c_vp, _c_i64, _c_int, _c_f, _c_vp, _c_vp]),
        "beam_moe_residual_update": (_c_int, [_c_vp, _c_i64, _c_int, _c_f, _c_int, _c_vp, _c_vp]),
        "beam_moe_sublayer": (_c_int, [_c_vp, _c_i64, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_f, _c_f, _c_int, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                       _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz]),
        "beam_attn_workspace_bytes": (_c_sz, [_c_i64, _c_int]),
        "beam_attn_forward": (_c_int, [_c_vp, _c_i64, _c_int, _c_int, _c_int, _c_f, _c_vp, _c_vp,
                                       _c_vp, _c_vp, _c_vp, _c_sz]),
        "beam_dense_workspace_bytes": (_c_sz, [_c_i64, _c_int, _c_int, _c_int]),
        "beam_dense_mlp": (_c_int, [_c_vp, _c_i64, _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_vp,
                                    _c_vp, _c_vp, _c_vp, _c_sz]),
        "beam_dense_mlp_fp8": (_c_int, [_c_vp, _c_i64, _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_vp,
                                        _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz]),
        "beam_moe_sublayer_fp8": (_c_int, [_c_vp, _c_i64, _c_int, _c_int, _c_int, _c_int, _c_int,
                                           _c_int, _c_f, _c_f, _c_int, _c_vp, _c_vp, _c_vp, _c_vp,
                                           _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                           _c_vp, _c_vp, _c_sz]),
        "beam_moe_set_schedule": (_c_int, [_c_int]),
        "beam_moe_stage_count": (_c_int, []),
        "beam_moe_stage_name": (ctypes.c_char_p, [_c_int]),
        "beam_moe_timer_begin": (_c_int, [_c_int]),
        "beam_moe_timer_begin_stages": (_c_int, [_c_int, ctypes.c_uint]),
        "beam_moe_timer_end": (_c_int, [ctypes.POINTER(ctypes.c_double), _c_int,
                                        ctypes.POINTER(_c_int)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class BeamMoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib.beam_moe_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


def _check(fn: str, status: int):
    if status != 0:
        if status in (-1, -2, -3, -4):
            raise ValueError(f"{fn}: {lib.beam_moe_status_string(status).decode()} ({status})")
        raise BeamMoeError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev_tensor(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, found {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, found {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, found {tuple(t.shape)}")
    return t


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_ws_lock = threading.Lock()
_ws_cache = {}


def workspace_bytes(T: int, H: int, I: int, E: int, k: int) -> int:
    n = lib.beam_moe_workspace_bytes(T, H, I, E, k)
    if n == 0 and T >= 0:
        raise ValueError("dimensions break the library's rules")
    return int(n)


def get_workspace(device: torch.device, nbytes: int, workspace: Optional[torch.Tensor] = None
                  ) -> torch.Tensor:
    """Workspace for one call on `device` and torch's current stream there.

    With `workspace` (a caller-owned uint8 device tensor) that tensor is used
    as is.  While the stream is being captured into a graph, a fresh buffer
    is taken from torch's allocator (the graph's private pool, which keeps
    the memory for the graph's replays) and nothing is cached.  Otherwise
    one buffer per (device, stream) is kept and reused, so calls on
    different streams never share one; it grows on demand, and no captured
    graph ever addresses a cached buffer, so growing frees nothing a graph
    still uses."""
    if workspace is not None:
        _dev_tensor(workspace, "workspace", torch.uint8)
        if workspace.device != device:
            raise ValueError(f"workspace is on {workspace.device}, the call on {device}")
        if workspace.numel() < nbytes:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, the call needs {nbytes}")
        return workspace
    if torch.cuda.is_current_stream_capturing():
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    with _ws_lock:
        buf = _ws_cache.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            _ws_cache[key] = buf
        return buf


def release_workspaces():
    with _ws_lock:
        _ws_cache.clear()


def version() -> str:
    return lib.beam_moe_version().decode()


def set_schedule(mode: str):
    """'auto', 'stream' or 'tiled' expert-GEMM schedule for later calls."""
    code = {"auto": 0, "stream": 1, "tiled": 2}[mode]
    _check("beam_moe_set_schedule", lib.beam_moe_set_schedule(code))


def route(x, w_router, groups=8, topk_groups=4, k=8, scale=2.5, logit_offset=None,
          return_counts=True, workspace=None):
    """Router + group-limited top-k.  Returns (ids int32 [T,k], weights fp32 [T,k], counts)."""
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    _dev_tensor(x, "x", torch.bfloat16, (T, H))
    _dev_tensor(w_router, "w_router", torch.bfloat16, (E, H))
    if logit_offset is not None:
        _dev_tensor(logit_offset, "logit_offset", torch.float32, (E,))
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty((E,), dtype=torch.int32, device=dev) if return_counts else None
    nbytes = workspace_bytes(T, H, 64, E, k)
    ws = get_workspace(dev, nbytes, workspace)
    rc = lib.beam_moe_route(_stream(dev), T, H, E, groups, topk_groups, k, float(scale), _ptr(x),
                            _ptr(w_router), _ptr(logit_offset), _ptr(ids), _ptr(w), _ptr(counts),
                            _ptr(ws), ws.numel())
    _check("beam_moe_route", rc)
    return ids, w, counts


def permute(topk_ids, E, workspace=None):
    """Expert-major order of the assignments: (counts, offsets, sorted_tokens, row_of)."""
    T, k = topk_ids.shape
    dev = topk_ids.device
    _dev_tensor(topk_ids, "topk_ids", torch.int32, (T, k))
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    sorted_tokens = torch.full((max(T * k, 1),), -1, dtype=torch.int32, device=dev)[:T * k]
    row_of = torch.empty((T * k,), dtype=torch.int32, device=dev)
    ws = get_workspace(dev, workspace_bytes(T, 64, 64, E, k), workspace)
    rc = lib.beam_moe_permute(_stream(dev), T, E, k, _ptr(topk_ids), _ptr(counts), _ptr(offsets),
                              _ptr(sorted_tokens), _ptr(row_of), _ptr(ws), ws.numel())
    _check("beam_moe_permute", rc)
    return counts, offsets, sorted_tokens, row_of


class PackedMatrix:
    """E expert matrices of N x K in the library's packed block layout
    (see beam_moe_pack_weights in include/beam_moe.h); `data` is the device
    buffer (uint8)."""

    __slots__ = ("data", "E", "N", "K")

    def __init__(self, data: torch.Tensor, E: int, N: int, K: int):
        self.data, self.E, self.N, self.K = data, E, N, K

    @property
    def shape(self):
        return (self.E, self.N, self.K)

    @property
    def device(self):
        return self.data.device


def packed_weight_bytes(N: int, K: int) -> int:
    """Bytes of one packed N x K expert matrix."""
    n = lib.beam_moe_packed_weight_bytes(int(N), int(K))
    if n == 0:
        raise ValueError(f"unsupported matrix shape {N} x {K} (multiples of 64 up to 32768)")
    return n


def pack_weights(w: torch.Tensor) -> PackedMatrix:
    """Packed copy of expert matrices w [E, N, K] bf16 (nn.Linear layout)."""
    E, N, K = w.shape
    _dev_tensor(w, "w", torch.bfloat16, (E, N, K))
    out = torch.empty((E * packed_weight_bytes(N, K),), dtype=torch.uint8, device=w.device)
    _check("beam_moe_pack_weights",
           lib.beam_moe_pack_weights(_stream(w.device), E, N, K, _ptr(w), _ptr(out)))
    return PackedMatrix(out, E, N, K)


class PackedFP8:
    """E expert matrices of N x K as FP8 (E4M3) codes in the packed block
    layout plus one fp32 power-of-two scale per row (beam_moe_pack_weights_fp8)."""

    __slots__ = ("data", "scales", "E", "N", "K")

    def __init__(self, data: torch.Tensor, scales: torch.Tensor, E: int, N: int, K: int):
        self.data, self.scales, self.E, self.N, self.K = data, scales, E, N, K

    @property
    def shape(self):
        return (self.E, self.N, self.K)

    @property
    def device(self):
        return self.data.device


def packed_fp8_bytes(N: int, K: int) -> int:
    """Bytes of one packed N x K FP8 expert matrix."""
    n = lib.beam_moe_packed_fp8_bytes(int(N), int(K))
    if n == 0:
        raise ValueError(f"unsupported matrix shape {N} x {K} (multiples of 64 up to 32768)")
    return n


def pack_weights_fp8(w: torch.Tensor) -> PackedFP8:
    """FP8 codes + row scales of expert matrices w [E, N, K] bf16."""
    E, N, K = w.shape
    _dev_tensor(w, "w", torch.bfloat16, (E, N, K))
    out = torch.empty((E * packed_fp8_bytes(N, K),), dtype=torch.uint8, device=w.device)
    sc = torch.empty((E, N), dtype=torch.float32, device=w.device)
    _check("beam_moe_pack_weights_fp8",
           lib.beam_moe_pack_weights_fp8(_stream(w.device), E, N, K, _ptr(w), _ptr(out), _ptr(sc)))
    return PackedFP8(out, sc, E, N, K)


def pack_experts_fp8(w_gate, w_up, w_down):
    """(gate, up, down) as FP8 for the *_fp8 compute calls."""
    return pack_weights_fp8(w_gate), pack_weights_fp8(w_up), pack_weights_fp8(w_down)


def pack_experts(w_gate, w_up, w_down):
    """(gate, up, down) in the packed layout the compute calls take."""
    return pack_weights(w_gate), pack_weights(w_up), pack_weights(w_down)


def _expert_shapes(w_gate, w_up, w_down, allow_fp8=True):
    kind = PackedFP8 if isinstance(w_gate, PackedFP8) and allow_fp8 else PackedMatrix
    for name, m in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        if not isinstance(m, kind):
            raise TypeError(f"{name} must be packed with pack_weights / pack_experts"
                            + (" or pack_experts_fp8 (all three alike)" if allow_fp8 else ""))
        if not m.data.is_cuda:
            raise ValueError(f"{name} must be a device buffer")
    E, I, H = w_gate.shape
    if w_up.shape != (E, I, H) or w_down.shape != (E, H, I):
        raise ValueError(f"expert shapes disagree: gate {w_gate.shape}, up {w_up.shape}, "
                         f"down {w_down.shape}")
    return E, I, H


def forward(x, topk_ids, topk_weights, w_gate, w_up, w_down, return_counts=False, workspace=None):
    """Experts + combine with given routing; expert weights packed (pack_experts).
    Returns y bf16 [T,H] (and counts)."""
    E, I, H = _expert_shapes(w_gate, w_up, w_down)
    T, k = topk_ids.shape
    dev = x.device
    _dev_tensor(x, "x", torch.bfloat16, (T, H))
    _dev_tensor(topk_ids, "topk_ids", torch.int32, (T, k))
    _dev_tensor(topk_weights, "topk_weights", torch.float32, (T, k))
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    counts = torch.empty((E,), dtype=torch.int32, device=dev) if return_counts else None
    ws = get_workspace(dev, workspace_bytes(T, H, I, E, k), workspace)
    if isinstance(w_gate, PackedFP8):
        rc = lib.beam_moe_forward_fp8(_stream(dev), T, H, I, E, k, _ptr(x), _ptr(topk_ids),
                                      _ptr(topk_weights), _ptr(w_gate.data), _ptr(w_gate.scales),
                                      _ptr(w_up.data), _ptr(w_up.scales), _ptr(w_down.data),
                                      _ptr(w_down.scales), _ptr(y), _ptr(counts), _ptr(ws),
                                      ws.numel())
        _check("beam_moe_forward_fp8", rc)
        return (y, counts) if return_counts else y
    rc = lib.beam_moe_forward(_stream(dev), T, H, I, E, k, _ptr(x), _ptr(topk_ids),
                              _ptr(topk_weights), _ptr(w_gate.data), _ptr(w_up.data),
                              _ptr(w_down.data), _ptr(y), _ptr(counts), _ptr(ws), ws.numel())
    _check("beam_moe_forward", rc)
    return (y, counts) if return_counts else y


def block(x, w_router, w_gate, w_up, w_down, groups=8, topk_groups=4, k=8, scale=2.5,
          logit_offset=None, out=None, return_routing=True, workspace=None):
    """Whole MoE block; expert weights packed (pack_experts).
    Returns (y, ids, weights, counts) or y."""
    E, I, H = _expert_shapes(w_gate, w_up, w_down)
    T = x.shape[0]
    dev = x.device
    _dev_tensor(x, "x", torch.bfloat16, (T, H))
    _dev_tensor(w_router, "w_router", torch.bfloat16, (E, H))
    if logit_offset is not None:
        _dev_tensor(logit_offset, "logit_offset", torch.float32, (E,))
    y = out if out is not None else torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _dev_tensor(y, "out", torch.bfloat16, (T, H))
    ids = w = counts = None
    if return_routing:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        counts = torch.empty((E,), dtype=torch.int32, device=dev)
    ws = get_workspace(dev, workspace_bytes(T, H, I, E, k), workspace)
    if isinstance(w_gate, PackedFP8):
        rc = lib.beam_moe_block_fp8(_stream(dev), T, H, I, E, groups, topk_groups, k, float(scale),
                                    _ptr(x), _ptr(w_router), _ptr(logit_offset), _ptr(w_gate.data),
                                    _ptr(w_gate.scales), _ptr(w_up.data), _ptr(w_up.scales),
                                    _ptr(w_down.data), _ptr(w_down.scales), _ptr(y), _ptr(ids),
                                    _ptr(w), _ptr(counts), _ptr(ws), ws.numel())
        _check("beam_moe_block_fp8", rc)
        return (y, ids, w, counts) if return_routing else y
    rc = lib.beam_moe_block(_stream(dev), T, H, I, E, groups, topk_groups, k, float(scale), _ptr(x),
                            _ptr(w_router), _ptr(logit_offset), _ptr(w_gate.data), _ptr(w_up.data),
                            _ptr(w_down.data), _ptr(y), _ptr(ids), _ptr(w), _ptr(counts), _ptr(ws),
                            ws.numel())
    _check("beam_moe_block", rc)
    return (y, ids, w, counts) if return_routing else y


NOALLOC_SCRATCH_BYTES = 64 << 20   # BEAM_MOE_NOALLOC_SCRATCH_BYTES of include/beam_moe.h


def block_noalloc(x, w_router, w_gate, w_up, w_down, out, groups=8, topk_groups=4, k=8, scale=2.5,
                  logit_offset=None, topk_ids=None, topk_weights=None, counts=None):
    """The whole MoE block (as `block`, bf16 packed weights) with the library's
    static device scratch as workspace (beam_moe_block_noalloc): nothing is
    allocated, by the library or here, so every output is the caller's
    (`out` y [T, H] bf16; optional ids int32 [T, k], weights fp32 [T, k],
    counts int32 [E]).  Calls on one GPU share the scratch: calls that overlap
    (different streams) race.  Sizes that need more scratch than the library
    holds raise ValueError.  Returns `out`."""
    E, I, H = _expert_shapes(w_gate, w_up, w_down, allow_fp8=False)
    T = x.shape[0]
    dev = x.device
    _dev_tensor(x, "x", torch.bfloat16, (T, H))
    _dev_tensor(w_router, "w_router", torch.bfloat16, (E, H))
    _dev_tensor(out, "out", torch.bfloat16, (T, H))
    if logit_offset is not None:
        _dev_tensor(logit_offset, "logit_offset", torch.float32, (E,))
    if topk_ids is not None:
        _dev_tensor(topk_ids, "topk_ids", torch.int32, (T, k))
    if topk_weights is not None:
        _dev_tensor(topk_weights, "topk_weights", torch.float32, (T, k))
    if counts is not None:
        _dev_tensor(counts, "counts", torch.int32, (E,))
    rc = lib.beam_moe_block_noalloc(_stream(dev), T, H, I, E, groups, topk_groups, k, float(scale),
                                    _ptr(x), _ptr(w_router), _ptr(logit_offset), _ptr(w_gate.data),
                                    _ptr(w_up.data), _ptr(w_down.data), _ptr(out), _ptr(topk_ids),
                                    _ptr(topk_weights), _ptr(counts))
    if rc == -4:
        raise ValueError(f"beam_moe_block_noalloc: T={T} needs "
                         f"{workspace_bytes(T, H, I, E, k)} bytes of scratch, more than the "
                         f"library's {NOALLOC_SCRATCH_BYTES}")
    _check("beam_moe_block_noalloc", rc)
    return out


def stream_init(x):
    T, H = x.shape
    _dev_tensor(x, "x", torch.bfloat16, (T, H))
    s = torch.empty((T, H), dtype=torch.float32, device=x.device)
    _check("beam_moe_stream_init", lib.beam_moe_stream_init(_stream(x.device), T, H, _ptr(x), _ptr(s)))
    return s


def rmsnorm(v, eps=1e-6):
    T, H = v.shape
    _dev_tensor(v, "in", torch.float32, (T, H))
    out = torch.empty((T, H), dtype=torch.bfloat16, device=v.device)
    _check("beam_moe_rmsnorm", lib.beam_moe_rmsnorm(_stream(v.device), T, H, float(eps), _ptr(v), _ptr(out)))
    return out


def residual_update(stream_io, y, step, eps=1e-6):
    T, H = stream_io.shape
    _dev_tensor(stream_io, "stream", torch.float32, (T, H))
    _dev_tensor(y, "y", torch.bfloat16, (T, H))
    _check("beam_moe_residual_update",
           lib.beam_moe_residual_update(_stream(y.device), T, H, float(eps), int(step), _ptr(y),
                                        _ptr(stream_io)))
    return stream_io


def sublayer(stream_io, step, w_router, w_gate, w_up, w_down, groups=8, topk_groups=4, k=8,
             scale=2.5, eps=1e-6, keep_io=True, workspace=None):
    """One sandwich-normed MoE sublayer + residual update, in place on stream_io
    (expert weights from pack_experts or pack_experts_fp8).  Returns
    (moe_input, moe_output, ids, weights, counts) when keep_io."""
    E, I, H = _expert_shapes(w_gate, w_up, w_down)
    T = stream_io.shape[0]
    dev = stream_io.device
    _dev_tensor(stream_io, "stream", torch.float32, (T, H))
    _dev_tensor(w_router, "w_router", torch.bfloat16, (E, H))
    xin = yb = ids = w = counts = None
    if keep_io:
        xin = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        yb = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        counts = torch.empty((E,), dtype=torch.int32, device=dev)
    ws = get_workspace(dev, workspace_bytes(T, H, I, E, k), workspace)
    if isinstance(w_gate, PackedFP8):
        rc = lib.beam_moe_sublayer_fp8(_stream(dev), T, H, I, E, groups, topk_groups, k, float(scale),
                                       float(eps), int(step), _ptr(stream_io), _ptr(w_router),
                                       _ptr(w_gate.data), _ptr(w_gate.scales), _ptr(w_up.data),
                                       _ptr(w_up.scales), _ptr(w_down.data), _ptr(w_down.scales),
                                       _ptr(xin), _ptr(yb), _ptr(ids), _ptr(w), _ptr(counts), _ptr(ws),
                                       ws.numel())
        _check("beam_moe_sublayer_fp8", rc)
        return (xin, yb, ids, w, counts) if keep_io else None
    rc = lib.beam_moe_sublayer(_stream(dev), T, H, I, E, groups, topk_groups, k, float(scale),
                               float(eps), int(step), _ptr(stream_io), _ptr(w_router), _ptr(w_gate.data),
                               _ptr(w_up.data), _ptr(w_down.data), _ptr(xin), _ptr(yb), _ptr(ids), _ptr(w),
                               _ptr(counts), _ptr(ws), ws.numel())
    _check("beam_moe_sublayer", rc)
    return (xin, yb, ids, w, counts) if keep_io else None


ATTN_Q_HEADS, ATTN_KV_HEADS, ATTN_HEAD_DIM = 48, 8, 128
ATTN_PROJ_ROWS = (2 * ATTN_Q_HEADS + 2 * ATTN_KV_HEADS) * ATTN_HEAD_DIM     # 14336


def pack_attention_weights(wq, wk, wv, wg, wo):
    """Packed attention weights (nn.Linear layouts, bf16): [Wq; Wk; Wv; Wg]
    stacked into one [14336, H] matrix and Wo [H, 6144], each as one packed
    matrix (E = 1).  Returns (w_qkvg, w_o)."""
    H = wq.shape[1]
    qd, kd = ATTN_Q_HEADS * ATTN_HEAD_DIM, ATTN_KV_HEADS * ATTN_HEAD_DIM
    for name, t, shape in [("wq", wq, (qd, H)), ("wk", wk, (kd, H)), ("wv", wv, (kd, H)),
                           ("wg", wg, (qd, H)), ("wo", wo, (H, qd))]:
        _dev_tensor(t, name, torch.bfloat16, shape)
    w_qkvg = pack_weights(torch.cat([wq, wk, wv, wg], dim=0).unsqueeze(0))
    w_o = pack_weights(wo.unsqueeze(0))
    return w_qkvg, w_o


def attention_workspace_bytes(T: int, H: int) -> int:
    n = lib.beam_attn_workspace_bytes(T, H)
    if n == 0:
        raise ValueError("dimensions break the library's rules")
    return int(n)


def attention(u, w_qkvg, w_o, global_layer, window=512, theta=10000.0, out=None, workspace=None):
    """Attention sublayer of one sequence at positions 0..T-1 (beam_attn_forward).
    u bf16 [T, H]; weights from pack_attention_weights.  Returns y bf16 [T, H]."""
    T, H = u.shape
    dev = u.device
    _dev_tensor(u, "u", torch.bfloat16, (T, H))
    if not (isinstance(w_qkvg, PackedMatrix) and isinstance(w_o, PackedMatrix)):
        raise TypeError("weights must come from pack_attention_weights")
    if (w_qkvg.E, w_qkvg.N, w_qkvg.K) != (1, ATTN_PROJ_ROWS, H) or \
            (w_o.E, w_o.N, w_o.K) != (1, H, ATTN_Q_HEADS * ATTN_HEAD_DIM):
        raise ValueError("packed attention weights do not match the hidden size")
    y = out if out is not None else torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _dev_tensor(y, "out", torch.bfloat16, (T, H))
    ws = get_workspace(dev, attention_workspace_bytes(T, H), workspace)
    rc = lib.beam_attn_forward(_stream(dev), T, H, int(bool(global_layer)), int(window),
                               float(theta), _ptr(u), _ptr(w_qkvg.data), _ptr(w_o.data), _ptr(y),
                               _ptr(ws), ws.numel())
    _check("beam_attn_forward", rc)
    return y


DENSE_CHUNKS = 8


def pack_dense(w_gate, w_up, w_down, chunks=DENSE_CHUNKS, fp8=False):
    """Packed weights of a dense SwiGLU layer (nn.Linear layouts, bf16):
    gate and up [I, H] as `chunks` row blocks, down [H, I] as `chunks`
    column blocks (beam_dense_mlp).  Returns (gate, up, down) PackedMatrix,
    or PackedFP8 (E4M3 codes, a power-of-two scale per row of each chunk)
    with fp8=True."""
    I, H = w_gate.shape
    if I % chunks:
        raise ValueError(f"I = {I} is not a multiple of chunks = {chunks}")
    _dev_tensor(w_gate, "w_gate", torch.bfloat16, (I, H))
    _dev_tensor(w_up, "w_up", torch.bfloat16, (I, H))
    _dev_tensor(w_down, "w_down", torch.bfloat16, (H, I))
    Ic = I // chunks
    wd = w_down.view(H, chunks, Ic).permute(1, 0, 2).contiguous()     # [chunks, H, Ic]
    pack = pack_weights_fp8 if fp8 else pack_weights
    return pack(w_gate.view(chunks, Ic, H)), pack(w_up.view(chunks, Ic, H)), pack(wd)


def dense_workspace_bytes(T: int, H: int, I: int, chunks: int) -> int:
    n = lib.beam_dense_workspace_bytes(T, H, I, chunks)
    if n == 0:
        raise ValueError("dimensions break the library's rules")
    return int(n)


def dense_mlp(x, w_gate, w_up, w_down, out=None, workspace=None):
    """Dense SwiGLU layer on packed weights from pack_dense.  Returns y bf16 [T, H]."""
    T, H = x.shape
    dev = x.device
    _dev_tensor(x, "x", torch.bfloat16, (T, H))
    kind = PackedFP8 if isinstance(w_gate, PackedFP8) else PackedMatrix
    for name, m in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        if not isinstance(m, kind):
            raise TypeError(f"{name} must come from pack_dense")
    C, Ic = w_gate.E, w_gate.N
    if (w_gate.K, w_up.E, w_up.N, w_up.K) != (H, C, Ic, H) or (w_down.E, w_down.N, w_down.K) != (C, H, Ic):
        raise ValueError("packed dense weights do not match each other or the hidden size")
    y = out if out is not None else torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _dev_tensor(y, "out", torch.bfloat16, (T, H))
    ws = get_workspace(dev, dense_workspace_bytes(T, H, C * Ic, C), workspace)
    if kind is PackedFP8:
        rc = lib.beam_dense_mlp_fp8(_stream(dev), T, H, C * Ic, C, _ptr(x), _ptr(w_gate.data),
                                    _ptr(w_gate.scales), _ptr(w_up.data), _ptr(w_up.scales),
                                    _ptr(w_down.data), _ptr(w_down.scales), _ptr(y), _ptr(ws), ws.numel())
        _check("beam_dense_mlp_fp8", rc)
        return y
    rc = lib.beam_dense_mlp(_stream(dev), T, H, C * Ic, C, _ptr(x), _ptr(w_gate.data), _ptr(w_up.data),
                            _ptr(w_down.data), _ptr(y), _ptr(ws), ws.numel())
    _check("beam_dense_mlp", rc)
    return y


def stage_names():
    return [lib.beam_moe_stage_name(i).decode() for i in range(lib.beam_moe_stage_count())]


class StageTimer:
    """Per-stage hipEvent timing of the next `max_calls` block/forward calls;
    `stages` (names from stage_names()) limits the events to those stages,
    and the result then holds only them."""

    def __init__(self, max_calls: int, stages=None):
        self.max_calls = max_calls
        self.stages = None if stages is None else list(stages)
        self.result = None

    def __enter__(self):
        if self.stages is None:
            _check("beam_moe_timer_begin", lib.beam_moe_timer_begin(self.max_calls))
        else:
            names = stage_names()
            unknown = [n for n in self.stages if n not in names]
            if unknown or not self.stages:
                raise ValueError(f"unknown or no stages {unknown}; known: {names}")
            mask = sum(1 << names.index(n) for n in set(self.stages))
            _check("beam_moe_timer_begin_stages", lib.beam_moe_timer_begin_stages(self.max_calls, mask))
        return self

    def __exit__(self, *exc):
        n = lib.beam_moe_stage_count()
        arr = (ctypes.c_double * n)()
        calls = _c_int(0)
        rc = lib.beam_moe_timer_end(arr, n, ctypes.byref(calls))
        if exc[0] is None:
            _check("beam_moe_timer_end", rc)
        names = stage_names()
        self.calls = calls.value
        self.result = {names[i]: arr[i] for i in range(n)
                       if self.stages is None or names[i] in self.stages}
        return False
