"""The synthetic workloads of the decode step and their input builders.

Shapes follow the pages: [ARCH] (ai-muninn.com Part 6, "(A) 壓縮你存的" and
"(B) 只讀你需要的"): 4:1 compression gives N = T/4 CSA entries, 128:1 gives
ceil(T/128) HCA entries; 128-dim index keys; top-512 (1024 Pro); SWA window 128;
512-wide latent rows. Head counts, distributions and planting come from the
workload descriptions (see synth.py for the draws).

  tiny     : 1 seq, N=1024, 4 index heads, top-64, window 16, 8 query heads, fp32
  ctx64k   : 1 seq, N=16384, 64 index heads, top-512, window 128, 64 heads, bf16
  ctx64k_b : 32 seqs x 21 CSA layers (sequential), per-sequence planted fraction U(1%,5%)
  ctx500k  : 4 seqs, N=125000 CSA (planted 0.5%) + one HCA layer of N=3907 rows read densely
  gate64k  : 8 seqs x 21 CSA layers, FP8 rows, top-1024, gate at layers 10/12/20
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from . import synth

CSA_LAYERS = tuple(range(2, 43, 2))  # even layers 2..42: the 21 CSA layers
GATE_LAYERS = (10, 12, 20)
SCALE = 1.0 / math.sqrt(512)


def csa_entries(tokens: int) -> int:
    return -(-tokens // 4)


def hca_entries(tokens: int) -> int:
    return -(-tokens // 128)


@dataclass(frozen=True)
class Workload:
    name: str
    cid: int
    B: int
    N: int
    H: int
    k: int
    window: int
    Hq: int
    idx_dtype: str
    kv_dtype: str
    layers: int = 1
    planted: Tuple = ("frac", 0.02)  # ("count", n) | ("frac", f) | ("uniform", lo, hi)
    alpha: float = 0.4
    hca_N: int = 0
    shared_plant: bool = False  # one set of planted positions per sequence, shared by its layers

    def planted_spec(self, g, device):
        kind = self.planted[0]
        if kind == "count":
            return dict(planted_count=self.planted[1])
        if kind == "frac":
            return dict(planted_frac=self.planted[1])
        lo, hi = self.planted[1], self.planted[2]
        fr = (lo + (hi - lo) * torch.rand(self.B, generator=g, device=device)).tolist()
        return dict(planted_frac=fr)


TINY = Workload("tiny", 0, 1, 1024, 4, 64, 16, 8, "f32", "f32", planted=("count", 32), alpha=0.5)
CTX64K = Workload("ctx64k", 1, 1, csa_entries(65536), 64, 512, 128, 64, "bf16", "bf16")
CTX64K_B = Workload("ctx64k_b", 2, 32, csa_entries(65536), 64, 512, 128, 64, "bf16", "bf16", layers=21,
                    planted=("uniform", 0.01, 0.05))
CTX500K = Workload("ctx500k", 3, 4, csa_entries(500000), 64, 512, 128, 64, "bf16", "bf16",
                   planted=("frac", 0.005), hca_N=hca_entries(500000))
GATE64K = Workload("gate64k", 4, 8, csa_entries(65536), 64, 1024, 128, 64, "bf16", "fp8", layers=21,
                   shared_plant=True)

ALL = {w.name: w for w in (TINY, CTX64K, CTX64K_B, CTX500K, GATE64K)}


@dataclass
class LayerInputs:
    idx: synth.IndexerInputs
    q: torch.Tensor
    kv: synth.KVRows


def layer_inputs(wl: Workload, layer: int = 0, device="cpu", B: Optional[int] = None, N: Optional[int] = None,
                 planted_positions=None) -> LayerInputs:
    """Inputs of one layer of a workload (B and N may be shrunk for tests)."""
    B = wl.B if B is None else B
    N = wl.N if N is None else N
    if wl.shared_plant and planted_positions is None:
        planted_positions = shared_planted(wl, device, B, N)
    if wl.cid == 0:
        g = torch.Generator(device=device)
        g.manual_seed(0)
    else:
        g = synth.generator(device, wl.cid, layer)
    spec = {} if planted_positions is not None else wl.planted_spec(g, device)
    if wl.planted[0] == "uniform" and B != wl.B and planted_positions is None:
        spec = dict(planted_frac=spec["planted_frac"][:B])
    if wl.planted[0] == "count" and N != wl.N:
        spec = dict(planted_count=max(1, round(wl.planted[1] * N / wl.N)))
    idx = synth.make_indexer(B, N, wl.H, wl.idx_dtype, g, device, alpha=wl.alpha,
                             planted_positions=planted_positions, **spec)
    q = synth.make_q(B, wl.Hq, wl.idx_dtype if wl.kv_dtype != "fp8" else "bf16", g, device)
    kv = synth.make_kv(B, N, wl.kv_dtype, g, device)
    return LayerInputs(idx, q, kv)


def hca_inputs(wl: Workload, device="cpu", B: Optional[int] = None) -> Tuple[torch.Tensor, synth.KVRows]:
    B = wl.B if B is None else B
    g = synth.generator(device, wl.cid, 1000)
    q = synth.make_q(B, wl.Hq, "bf16", g, device)
    kv = synth.make_kv(B, wl.hca_N, "bf16", g, device)
    return q, kv


def shared_planted(wl: Workload, device="cpu", B: Optional[int] = None, N: Optional[int] = None):
    """Planted positions shared by all layers of a sequence (relevance belongs to
    the context, not to a layer; with positions drawn per layer no entry would
    be relevant in enough layers to win the cross-layer vote). The fraction is
    the workload's planted fraction; sequence b's positions do not depend on B."""
    B = wl.B if B is None else B
    N = wl.N if N is None else N
    g = synth.generator(device, wl.cid, 999)
    cnt = int(round(wl.planted[1] * N))
    return [torch.randperm(N, generator=g, device=device)[:cnt].sort().values for _ in range(B)]


def gate_layer(wl: Workload, layer: int, keys: torch.Tensor, device="cpu", d_model: int = 4096, rank: int = 2048,
               H: Optional[int] = None) -> synth.GateLayer:
    H = wl.H if H is None else H
    g = synth.generator(device, wl.cid, 2000 + layer)
    h, wa, wb, wp = synth.make_gate_weights(keys.shape[0], H, d_model, rank, g, device)
    return synth.GateLayer(h, wa, wb, wp, keys)


# The other attention layers of a decode step ([ARCH] (A), the layer table):
# SWA on layers 0-1 keeps the last W uncompressed rows, HCA on the odd layers
# 3-41 keeps ceil(T/128) rows read densely. Their inputs come from streams of
# their own (config id 5), one per layer.
SCHEDULE_CID = 5


def dense_layer_inputs(B: int, rows: int, Hq: int, layer: int, device="cpu") -> Tuple[torch.Tensor, synth.KVRows]:
    """Attention query [B,Hq,512] bf16 and bf16 rows [B,rows,512] of an SWA or HCA layer."""
    g = synth.generator(device, SCHEDULE_CID, layer)
    q = synth.make_q(B, Hq, "bf16", g, device)
    kv = synth.make_kv(B, rows, "bf16", g, device)
    return q, kv


# Several queries per sequence (the multi-query indexer): the index queries of
# nearby tokens share a component, q_j = rho * q_0 + sqrt(1 - rho^2) * z_j
# (z_j drawn like q_0), so the planted entries, aligned with q_0's head 0, stay
# strong for every query; head weights are drawn afresh per query. Config id 6.
MQ_CID = 6
MQ_RHO = 0.8
# depth-1 MTP: the current token and its draft, 32 sequences at 64K context
MTP_Q = 2
# a prefill chunk: the last 2048 tokens of a 64K prompt, one sequence
PREFILL_Q = 2048
PREFILL_T = 65536


def extra_queries(idx: synth.IndexerInputs, Q: int, layer: int, device="cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """Q index queries per sequence [B,Q,H,128] and weights [B,Q,H] around the
    single query of `idx` (which becomes query 0)."""
    B, H = idx.q_idx.shape[0], idx.q_idx.shape[1]
    g = synth.generator(device, MQ_CID, layer)
    q0 = idx.q_idx.float()
    z = torch.randn(B, Q, H, synth.IDX_DIM, generator=g, device=device)
    q = MQ_RHO * q0[:, None] + math.sqrt(1.0 - MQ_RHO ** 2) * z
    q[:, 0] = q0
    w = torch.rand(B, Q, H, generator=g, device=device)
    w[:, 0] = idx.w
    return q.to(idx.q_idx.dtype).contiguous(), w.contiguous()


def mq_inputs(wl: Workload, Q: int, layer: int = 0, device="cpu", B: Optional[int] = None,
              N: Optional[int] = None) -> synth.IndexerInputs:
    """Index queries [B,Q,H,128], weights [B,Q,H] and the keys [B,N,128] of
    layer_inputs(wl, layer) (whose own query is query 0)."""
    L = layer_inputs(wl, layer, device, B=B, N=N)
    q, w = extra_queries(L.idx, Q, layer, device)
    return synth.IndexerInputs(q, w, L.idx.k_idx, L.idx.planted)


def causal_lengths(B: int, Q: int, t0: int, device="cpu") -> torch.Tensor:
    """Entries visible to the queries of tokens t0 .. t0+Q-1 (0-based positions):
    a 4:1 compressed entry exists once its four tokens do, so token t sees
    floor((t + 1) / 4) entries. [B,Q] int32."""
    t = torch.arange(t0, t0 + Q, device=device, dtype=torch.int64)
    return ((t + 1) // 4).to(torch.int32).expand(B, Q).contiguous()


# The lookahead golden: the attention queries of the next TAU decode steps,
# drawn like the multi-query index queries (step 0 is the layer's own query,
# step t >= 1 mixes it with a fresh draw: rho * q_0 + sqrt(1 - rho^2) * z_t).
TAU = 64


def horizon_queries(q0: torch.Tensor, T: int, layer: int, device="cpu") -> torch.Tensor:
    """[B,T,Hq,512] attention queries of a T-step horizon around q0 [B,Hq,512]."""
    B, Hq, D = q0.shape
    g = synth.generator(device, MQ_CID, 1000 + layer)
    z = torch.randn(B, T, Hq, D, generator=g, device=device)
    q = MQ_RHO * q0.float()[:, None] + math.sqrt(1.0 - MQ_RHO ** 2) * z
    q[:, 0] = q0.float()
    return q.to(q0.dtype).contiguous()
