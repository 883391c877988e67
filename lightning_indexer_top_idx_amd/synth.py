"""Seeded synthetic inputs for the lightning-indexer decode step.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, so both the HIP path and the CPU oracle can consume what
it produces. Everything is drawn with ``torch.Generator`` on the device the
caller names (CPU for small cases, the GPU for full-size ones: the same seed
gives different numbers on different devices, so a test always hands ONE
generated set to both sides).

Distributions (the pages give only shapes; the workloads fix the rest):
  index queries q_idx ~ N(0,1); head weights w ~ U(0,1) (fp32);
  index keys k_idx ~ N(0, 1/128); a fraction of "planted" entries gets
  alpha * q_idx[0]/|q_idx[0]| added (positions uniform without replacement);
  attention queries q ~ N(0,1); latent rows kv ~ N(0,1);
  bf16 storage is round-to-nearest-even from the fp32 draw.
FP8 rows: per row and 64-dim group, scale exponent e = ceil(log2(amax/448)),
byte = e + 127, and the group divided by 2^e is rounded to E4M3 (never above 448).
Gate weights: wq_a ~ N(0, 1/d_model), wq_b ~ N(0, 1/rank), w_proj ~ N(0, 1/d_model)
(bf16), hidden state h ~ N(0,1) (fp32).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

IDX_DIM = 128
KV_DIM = 512
FP8_DIMS = 448
ROPE_DIMS = 64
FP8_GROUP = 64
SCALE_STRIDE = 8


def seed_of(*parts: int) -> int:
    """Deterministic 63-bit seed from a tuple of small ints (config, layer, ...)."""
    s = 0x9E3779B97F4A7C15
    for p in parts:
        s ^= (int(p) + 0x632BE59BD9B4E019 + ((s << 6) & (2**64 - 1)) + (s >> 2)) & (2**64 - 1)
        s = (s * 0xBF58476D1CE4E5B9) & (2**64 - 1)
    return s & (2**63 - 1)


def generator(device, *parts: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*parts))
    return g


@dataclass
class IndexerInputs:
    q_idx: torch.Tensor  # [B,H,128] f32 or bf16
    w: torch.Tensor  # [B,H] f32
    k_idx: torch.Tensor  # [B,N,128] f32 or bf16
    planted: List[torch.Tensor] = field(default_factory=list)  # per sequence, int64 positions


@dataclass
class KVRows:
    dtype: str  # "f32" | "bf16" | "fp8"
    data: torch.Tensor  # [B,N,512] (f32/bf16) or [B,N,448] uint8
    rope: Optional[torch.Tensor] = None  # [B,N,64] bf16 (fp8 only)
    scale: Optional[torch.Tensor] = None  # [B,N,8] uint8 (fp8 only)

    @property
    def n_rows(self) -> int:
        return self.data.shape[1]

    @property
    def batch(self) -> int:
        return self.data.shape[0]


def _store(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return x.float().contiguous()
    if dtype == "bf16":
        return x.to(torch.bfloat16).contiguous()
    raise ValueError(dtype)


def planted_counts(fracs, N: int) -> List[int]:
    return [int(round(float(f) * N)) for f in fracs]


def make_indexer(B: int, N: int, H: int, dtype: str, g: torch.Tensor, device, planted_frac=0.0,
                 alpha: float = 0.4, planted_count=None, planted_positions=None) -> IndexerInputs:
    """Index queries, head weights and keys for B sequences of N entries.

    planted_frac: one float, or a sequence of B floats; planted_count overrides it
    with exact counts; planted_positions (list of B index tensors) overrides both."""
    q = torch.randn(B, H, IDX_DIM, generator=g, device=device)
    w = torch.rand(B, H, generator=g, device=device)
    k = torch.randn(B, N, IDX_DIM, generator=g, device=device) / math.sqrt(IDX_DIM)
    if planted_positions is None:
        if planted_count is None:
            fr = planted_frac if hasattr(planted_frac, "__len__") else [planted_frac] * B
            planted_count = planted_counts(fr, N)
        elif not hasattr(planted_count, "__len__"):
            planted_count = [planted_count] * B
        planted_positions = []
        for b in range(B):
            perm = torch.randperm(N, generator=g, device=device)
            planted_positions.append(perm[: planted_count[b]].sort().values)
    for b in range(B):
        pos = planted_positions[b]
        if pos.numel():
            qb = _store(q[b, 0], dtype).float()
            unit = qb / qb.norm()
            k[b, pos] += alpha * unit
    return IndexerInputs(_store(q, dtype), w.float().contiguous(), _store(k, dtype), planted_positions)


def fp8_encode(x: torch.Tensor):
    """Encode fp32 rows [..., 448] as E4M3 bytes + one E8M0 byte per 64 dims.

    Input preparation only (the decode is part of the method and lives on each
    side separately). Exponent e = ceil(log2(amax/448)) so the scaled group
    never exceeds 448; all-zero groups get e = 0."""
    shp = x.shape[:-1]
    grp = x.float().reshape(*shp, FP8_DIMS // FP8_GROUP, FP8_GROUP)
    amax = grp.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.ceil(torch.log2(amax / 448.0)), torch.zeros_like(amax))
    # guard the log2 rounding: make sure amax / 2^e <= 448
    e = torch.where(amax / torch.exp2(e) > 448.0, e + 1, e)
    scaled = grp / torch.exp2(e).unsqueeze(-1)
    codes = scaled.to(torch.float8_e4m3fn).view(torch.uint8).reshape(*shp, FP8_DIMS)
    sc = torch.zeros(*shp, SCALE_STRIDE, dtype=torch.uint8, device=x.device)
    sc[..., : FP8_DIMS // FP8_GROUP] = (e + 127).to(torch.uint8)
    return codes.contiguous(), sc.contiguous()


def make_kv(B: int, N: int, dtype: str, g: torch.Tensor, device) -> KVRows:
    x = torch.randn(B, N, KV_DIM, generator=g, device=device)
    if dtype in ("f32", "bf16"):
        return KVRows(dtype, _store(x, dtype))
    if dtype == "fp8":
        codes, sc = fp8_encode(x[..., :FP8_DIMS])
        rope = x[..., FP8_DIMS:].to(torch.bfloat16).contiguous()
        return KVRows("fp8", codes, rope, sc)
    raise ValueError(dtype)


def make_q(B: int, Hq: int, dtype: str, g, device) -> torch.Tensor:
    return _store(torch.randn(B, Hq, KV_DIM, generator=g, device=device), dtype)


def make_exact_grid(B: int, N: int, H: int, g, device, dtype="bf16") -> IndexerInputs:
    """q, k in {0, +-0.5, +-1}, w in {0, 1/4, 1/2, 3/4, 1}: every partial sum of a
    score is a multiple of 1/16 far below 2^24, so fp32 sums are exact in any
    order and ties are frequent."""
    vals = torch.tensor([0.0, 0.5, -0.5, 1.0, -1.0], device=device)
    q = vals[torch.randint(0, 5, (B, H, IDX_DIM), generator=g, device=device)]
    k = vals[torch.randint(0, 5, (B, N, IDX_DIM), generator=g, device=device)]
    w = torch.randint(0, 5, (B, H), generator=g, device=device).float() / 4.0
    return IndexerInputs(_store(q, dtype), w.contiguous(), _store(k, dtype), [])


@dataclass
class GateLayer:
    h: torch.Tensor  # [B, d_model] f32
    wq_a: torch.Tensor  # [rank, d_model] bf16
    wq_b: torch.Tensor  # [H*128, rank] bf16
    w_proj: torch.Tensor  # [H, d_model] bf16
    k: torch.Tensor  # [B, N, 128] bf16 (this layer's frozen index keys)

    def as_dict(self):
        return {"h": self.h, "wq_a": self.wq_a, "wq_b": self.wq_b, "w_proj": self.w_proj, "k": self.k}


def make_gate_weights(B: int, H: int, d_model: int, rank: int, g, device):
    h = torch.randn(B, d_model, generator=g, device=device)
    wq_a = (torch.randn(rank, d_model, generator=g, device=device) / math.sqrt(d_model)).to(torch.bfloat16)
    wq_b = (torch.randn(H * IDX_DIM, rank, generator=g, device=device) / math.sqrt(rank)).to(torch.bfloat16)
    w_proj = (torch.randn(H, d_model, generator=g, device=device) / math.sqrt(d_model)).to(torch.bfloat16)
    return h.contiguous(), wq_a.contiguous(), wq_b.contiguous(), w_proj.contiguous()
