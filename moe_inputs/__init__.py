"""Seeded synthetic inputs for one Beam Mixture-of-Experts block.

This module only draws random numbers and names workload shapes.  It holds
none of the block's arithmetic (no routing, no expert MLP, no combine), so
both the HIP path and the CPU oracle may take their inputs from it.

Workloads follow the shapes the Beam pages state (hidden size 5120, 256 SwiGLU
experts of intermediate size 2560 in 8 groups of 32, 4 kept groups, top-8,
combine scale 2.5; pages "Willkommen Beam: ein offenes 501B-Modell, das Sie
besitzen, anpassen und skalieren können", sections "Attention" and
"Mixture of Experts").  Token counts are the synthetic decode / prefill /
skewed / stacked batches this repository measures.

Value recipe (no trained weights exist here):
  * attention input u ~ N(0, 1) and Wq, Wk, Wv, Wg, Wo ~ N(0, 0.02) -> bf16
  * dense layer gate, up [I, H] and down [H, I] ~ N(0, 0.02) -> bf16
  * x            ~ N(0, 1)    -> bf16 (round to nearest even)
  * router Wr    ~ N(0, 0.02) -> bf16, layout [E, H]
  * gate, up     ~ N(0, 0.02) -> bf16, layout [E, I, H]
  * down         ~ N(0, 0.02) -> bf16, layout [E, H, I]
x and Wr are always drawn on the CPU with torch's CPU generator, so they are
the same on every machine; the large expert tensors are drawn on the target
device one expert at a time (a device generator seeded per tensor), and any
check that needs them on the host copies them back.
"""
from __future__ import annotations

import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

SEED = 20261016

# Tensor ids used to derive independent seeds.
TID_X, TID_WR, TID_WG, TID_WU, TID_WD, TID_ZIPF_PERM, TID_ZIPF_CAL = range(7)
TID_ATT_U, TID_ATT_WQ, TID_ATT_WK, TID_ATT_WV, TID_ATT_WG, TID_ATT_WO = range(7, 13)
TID_DENSE_WG, TID_DENSE_WU, TID_DENSE_WD = range(13, 16)

# attention: 48 query heads and 8 key/value heads of 128 dims
ATT_Q_DIM, ATT_KV_DIM = 48 * 128, 8 * 128

WEIGHT_SIGMA = 0.02
X_SIGMA = 1.0

_DATA_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "data")
ZIPF_OFFSETS_FILE = os.path.join(_DATA_DIR, "zipf_offsets_h5120_e256.txt")


@dataclass(frozen=True)
class BlockShape:
    """Dimensions of one MoE block call."""
    T: int
    H: int
    I: int
    E: int = 256
    groups: int = 8
    topk_groups: int = 4
    k: int = 8
    scale: float = 2.5
    offset: Optional[str] = None      # None or "zipf"
    layers: int = 1                    # > 1 only for the stacked workload
    name: str = ""

    def asdict(self):
        return {f: getattr(self, f) for f in self.__dataclass_fields__}


WORKLOADS = {
    # small case the oracle finishes in seconds
    "tiny": BlockShape(T=128, H=256, I=128, name="tiny"),
    # Beam shape, decode-size batch: expert-weight streaming
    "decode": BlockShape(T=64, H=5120, I=2560, name="decode"),
    # Beam shape, speculative-verify batch: 16 sequences x 16 tokens (a
    # drafter proposes up to 15 tokens and the model checks them plus the
    # current one in a single forward pass; page "Reflection 发布 501B 开放模型
    # Beam，支持自托管定制与扩展" (sihot.dev), section vLLM)
    "verify": BlockShape(T=256, H=5120, I=2560, name="verify"),
    # Beam shape, prefill chunk with near-uniform load
    "prefill": BlockShape(T=8192, H=5120, I=2560, name="prefill"),
    # Beam shape, Zipf(1.1)-skewed expert load through per-expert logit offsets
    "skewed": BlockShape(T=16384, H=5120, I=2560, offset="zipf", name="skewed"),
    # four stacked sublayers RMSNorm -> MoE -> RMSNorm -> scaled residual
    "stack": BlockShape(T=4096, H=5120, I=2560, layers=4, name="stack"),
}


def seed_for(*key: int) -> int:
    """Deterministic 63-bit seed from an integer key (numpy SeedSequence)."""
    ss = np.random.SeedSequence([SEED, *[int(v) for v in key]])
    return int(ss.generate_state(1, dtype=np.uint64)[0]) & 0x7FFF_FFFF_FFFF_FFFF


def _cpu_normal(shape, sigma, *key) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_for(*key))
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if sigma != 1.0:
        t.mul_(sigma)
    return t.to(torch.bfloat16)


def make_x(T: int, H: int, layer: int = 0, tid: int = TID_X, case: int = 0) -> torch.Tensor:
    """Token activations [T, H] bf16 on the CPU."""
    return _cpu_normal((T, H), X_SIGMA, case, layer, tid, T, H)


def make_router(E: int, H: int, layer: int = 0, case: int = 0) -> torch.Tensor:
    """Router weight [E, H] bf16 on the CPU."""
    return _cpu_normal((E, H), WEIGHT_SIGMA, case, layer, TID_WR, E, H)


def make_expert_weights(E: int, H: int, I: int, device, layer: int = 0, case: int = 0):
    """Gate [E,I,H], up [E,I,H], down [E,H,I] bf16, drawn on `device`."""
    device = torch.device(device)
    out = []
    for tid, shape in ((TID_WG, (I, H)), (TID_WU, (I, H)), (TID_WD, (H, I))):
        w = torch.empty((E, *shape), dtype=torch.bfloat16, device=device)
        g = torch.Generator(device=device)
        g.manual_seed(seed_for(case, layer, tid, E, H, I))
        for e in range(E):
            tmp = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
            tmp.mul_(WEIGHT_SIGMA)
            w[e].copy_(tmp.to(torch.bfloat16))
            del tmp
        out.append(w)
    return tuple(out)


def load_zipf_offsets(E: int = 256) -> torch.Tensor:
    """Per-expert fp32 logit offsets for the skewed workload (stored file)."""
    vals = np.loadtxt(ZIPF_OFFSETS_FILE, dtype=np.float64, comments="#")
    if vals.shape != (E,):
        raise ValueError(f"{ZIPF_OFFSETS_FILE}: expected {E} values, found {vals.shape}")
    return torch.from_numpy(vals.astype(np.float32))


def zipf_rank_permutation(E: int = 256) -> np.ndarray:
    """Seeded rank of each expert (rank 1 = hottest) for the Zipf load."""
    rng = np.random.default_rng(seed_for(0, 0, TID_ZIPF_PERM, E))
    return 1 + rng.permutation(E)


def zipf_calibration_x(Tc: int, H: int) -> torch.Tensor:
    """Calibration token batch [Tc, H] bf16 for fitting the Zipf offsets."""
    return make_x(Tc, H, tid=TID_ZIPF_CAL)


@dataclass
class BlockInputs:
    shape: BlockShape
    x: torch.Tensor
    wr: torch.Tensor
    wg: torch.Tensor
    wu: torch.Tensor
    wd: torch.Tensor
    offset: Optional[torch.Tensor] = None
    extra: dict = field(default_factory=dict)


def make_block_inputs(shape: BlockShape, device, layer: int = 0, case: int = 0,
                      T: Optional[int] = None) -> BlockInputs:
    """All inputs of one block call, resident on `device`."""
    T = shape.T if T is None else T
    device = torch.device(device)
    x = make_x(T, shape.H, layer=layer, case=case).to(device)
    wr = make_router(shape.E, shape.H, layer=layer, case=case).to(device)
    wg, wu, wd = make_expert_weights(shape.E, shape.H, shape.I, device, layer=layer, case=case)
    off = None
    if shape.offset == "zipf":
        off = load_zipf_offsets(shape.E).to(device)
    return BlockInputs(shape, x, wr, wg, wu, wd, off)


def make_attention_input(T: int, H: int, layer: int = 0, case: int = 0) -> torch.Tensor:
    """Normalised attention-layer input u [T, H] bf16 on the CPU, ~ N(0, 1)."""
    return make_x(T, H, layer=layer, tid=TID_ATT_U, case=case)


def make_attention_weights(H: int, layer: int = 0, case: int = 0):
    """Wq [6144, H], Wk [1024, H], Wv [1024, H], Wg [6144, H], Wo [H, 6144]
    bf16 on the CPU (nn.Linear layouts), each ~ N(0, 0.02)."""
    shapes = ((TID_ATT_WQ, (ATT_Q_DIM, H)), (TID_ATT_WK, (ATT_KV_DIM, H)),
              (TID_ATT_WV, (ATT_KV_DIM, H)), (TID_ATT_WG, (ATT_Q_DIM, H)),
              (TID_ATT_WO, (H, ATT_Q_DIM)))
    return tuple(_cpu_normal(shape, WEIGHT_SIGMA, case, layer, tid, *shape) for tid, shape in shapes)


def make_dense_weights(H: int, I: int, device, layer: int = 0, case: int = 0):
    """Dense SwiGLU layer: gate [I, H], up [I, H], down [H, I] bf16 ~ N(0, 0.02),
    drawn on `device` (a device generator seeded per tensor)."""
    device = torch.device(device)
    out = []
    for tid, shape in ((TID_DENSE_WG, (I, H)), (TID_DENSE_WU, (I, H)), (TID_DENSE_WD, (H, I))):
        g = torch.Generator(device=device)
        g.manual_seed(seed_for(case, layer, tid, H, I))
        w = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
        out.append(w.mul_(WEIGHT_SIGMA).to(torch.bfloat16))
        del w
    return tuple(out)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a bf16 tensor as uint16 bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
