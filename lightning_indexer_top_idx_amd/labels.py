"""The gate-stress recall measurement: gate, gated and native selections, vote labels.

zhichai.net, "FlashMemory-DeepSeek-V4 深度解读": section 2.2 (a sigmoid chunk gate,
kept at 0.5, restricts what the native indexer may pick), section 3.2 (labels:
each CSA layer's softmax, a top-p cut at 0.6, and a vote that keeps entries
chosen by at least 3 of the 21 CSA layers), section 4.1 (gate layers 10, 12 and
20, their kept sets OR-ed). ai-muninn.com, "FlashMemory can't improve
DeepSeek-V4-Flash's own lightning indexer", "The setup" (the gate only narrows
the native indexer's candidates) and "Act 3" (recall against a golden set).

The chain, for one batch of sequences over the CSA layers of one decode step:
  1. gate  A = OR over the gate layers of lit_lsa_gate's keep sets;
  2. per CSA layer l: native S_l = exact top-k of the indexer scores; gated
     S'_l = exact top-k inside A;
  3. labels from two sources (the pages leave open which softmax section 3.2
     means): R1 = the softmax of layer l's exact indexer logits, R2 = the
     head-averaged dense attention probabilities (the golden of "Act 3");
     per source a top-p cut per layer and the vote give the golden set G;
  4. recall: #(S'_l & G) / #G and #(S'_l & S_l) / #S_l, with #G and the gate's
     keep fraction beside them.

Every step is a call of the C ABI on the current stream (lit_lsa_gate,
lit_idx_score, lit_topk_select, lit_idx_score_exact, lit_golden_topk,
lit_golden_topp_vote, lit_recall); this module only sequences the calls and
stacks their outputs.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Dict, List, Sequence

from . import golden_topk, golden_topp_vote, idx_score, idx_score_exact, lsa_gate, recall, topk_select


@dataclass
class RecallChain:
    """Outputs of one run of the chain (device tensors; L layers, B sequences, N entries)."""

    gate: object  # [B,N] u8, the OR of the gate layers' keep sets
    gate_count: object  # [B]
    native_mask: object  # [L,B,N] u8, S_l
    native_count: object  # [L,B]
    gated_mask: object  # [L,B,N] u8, S'_l
    gated_count: object  # [L,B]
    votes: Dict[str, object]  # source -> [B,N] int32 (layers whose top-p set holds the entry)
    gold: Dict[str, object]  # source -> [B,N] u8
    gold_count: Dict[str, object]  # source -> [B]
    inter: Dict[str, object]  # "gated&R1", "gated&R2", "native&R1", "native&R2", "gated&native" -> [L,B]
    x: Dict[str, object]  # source -> [L,B,N] fp64: R1 the exact indexer logits, R2 the dense attention pbar


def run_chain(layer_inputs: Sequence[Callable[[], object]], gate_layers: Sequence, k: int, threshold: float = 0.5,
              top_p: float = 0.6, min_votes: int = 3, scale: float = 1.0 / 512 ** 0.5) -> RecallChain:
    """layer_inputs: one callable per CSA layer (in layer order) returning that
    layer's inputs on the GPU (idx: q_idx, w, k_idx; q; kv); gate_layers: the
    gate layers' GateLayer inputs. Inputs are built one layer at a time, so the
    whole decode step never has to be resident."""
    import torch

    gate, gate_count = lsa_gate(gate_layers, threshold)
    Ln = len(layer_inputs)
    B, N = gate.shape
    dev = gate.device
    X1 = torch.empty(Ln, B, N, dtype=torch.float64, device=dev)  # exact indexer logits (R1)
    X2 = torch.empty(Ln, B, N, dtype=torch.float64, device=dev)  # dense attention pbar (R2)
    nmask = torch.empty(Ln, B, N, dtype=torch.uint8, device=dev)
    gmask = torch.empty(Ln, B, N, dtype=torch.uint8, device=dev)
    ncount = torch.empty(Ln, B, dtype=torch.int32, device=dev)
    gcount = torch.empty(Ln, B, dtype=torch.int32, device=dev)
    for i, make in enumerate(layer_inputs):
        L = make()
        q, w, kk = L.idx.q_idx, L.idx.w, L.idx.k_idx
        s, h = idx_score(q, w, kk)
        _, ncount[i], nmask[i] = topk_select(s, k, exact=(q, w, kk), hints=h)
        s, h = idx_score(q, w, kk, allowed=gate)
        _, gcount[i], gmask[i] = topk_select(s, k, exact=(q, w, kk), hints=h)
        X1[i] = idx_score_exact(q, w, kk)
        _, _, _, X2[i] = golden_topk(L.q, L.kv, k, scale, want_mask=False)
        del L, s, h
    votes, gold, gold_count = {}, {}, {}
    for src, X, is_logits in (("R1", X1, True), ("R2", X2, False)):
        gold[src], gold_count[src], votes[src] = golden_topp_vote(X, is_logits, top_p, min_votes)
    inter = {name: torch.empty(Ln, B, dtype=torch.int32, device=dev)
             for name in ("gated&R1", "gated&R2", "native&R1", "native&R2", "gated&native")}
    for i in range(Ln):
        for src in ("R1", "R2"):
            inter[f"gated&{src}"][i] = recall(gmask[i], gold[src])[0]
            inter[f"native&{src}"][i] = recall(nmask[i], gold[src])[0]
        inter["gated&native"][i] = recall(gmask[i], nmask[i])[0]
    return RecallChain(gate, gate_count, nmask, ncount, gmask, gcount, votes, gold, gold_count, inter,
                       {"R1": X1, "R2": X2})


def summary(r: RecallChain, N: int) -> Dict[str, object]:
    """The reported figures: recalls averaged over layers and sequences, #G and
    the gate's keep fraction (a recall against an empty golden set is undefined
    and left out, with the number of such sequences reported)."""
    out: Dict[str, object] = {"keep_frac": round(float(r.gate_count.float().mean().item()) / N, 4)}
    nc = r.native_count.double()
    out["recall_gated_vs_native"] = round(float((r.inter["gated&native"].double() / nc).mean().item()), 4)
    for src in ("R1", "R2"):
        g = r.gold_count[src].double()  # [B]
        ok = g > 0
        out[f"gold_count_{src}"] = [int(x) for x in r.gold_count[src].tolist()]
        # each layer's top-p set size, averaged (the votes sum to the sets' sizes)
        out[f"topp_set_mean_{src}"] = round(float(r.votes[src].double().sum().item()) / (len(r.x[src]) * len(g)), 1)
        out[f"gold_empty_sequences_{src}"] = int((~ok).sum().item())
        if ok.any():
            for who in ("gated", "native"):
                rec = r.inter[f"{who}&{src}"].double()[:, ok] / g[ok]
                out[f"recall_{who}_vs_{src}"] = round(float(rec.mean().item()), 4)
    return out
