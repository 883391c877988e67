"""The gate-stress recall chain on the GPU against the oracle's chain.

zhichai.net, "FlashMemory-DeepSeek-V4 深度解读", sections 2.2, 3.2 and 4.1: the gate
of layers 10/12/20 (OR-ed), the native and the gated exact top-k of every CSA
layer, the labels (softmax -> top-p 0.6 -> at least 3 of 21 layers) from two
sources (R1: the indexer logits, R2: dense attention), and the recall counts.
Bars: gate, selections, votes, golden sets and recall counts bit-exact; the
exact logits bit-exact; the dense-attention probabilities within 1e-11.
"""
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import lightning_indexer_top_idx_amd as lit
import oracle
from lightning_indexer_top_idx_amd import labels, synth
from lightning_indexer_top_idx_amd import workloads as W

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(512)
SOURCES = ("R1", "R2")


@pytest.fixture(scope="module", autouse=True)
def _dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lit.load()
    oracle.build()


def _cpu_seq(L, b):
    """Sequence b of a layer's device inputs, on the host."""
    kv = L.kv
    return {"q_idx": L.idx.q_idx[b:b + 1].cpu(), "w": L.idx.w[b:b + 1].cpu(), "k_idx": L.idx.k_idx[b:b + 1].cpu(),
            "q": L.q[b:b + 1].cpu(),
            "kv": synth.KVRows(kv.dtype, kv.data[b:b + 1].cpu(), None if kv.rope is None else kv.rope[b:b + 1].cpu(),
                               None if kv.scale is None else kv.scale[b:b + 1].cpu())}


def oracle_chain(seq_layers, gate_dicts, k, threads=16):
    """The chain for one sequence on the oracle: seq_layers = per CSA layer the
    sequence's inputs (as _cpu_seq gives them); gate_dicts = its gate layers."""
    gate, gc = oracle.lsa_gate(gate_dicts, 0.5)

    def layer(x):
        s = oracle.idx_score(x["q_idx"], x["w"], x["k_idx"])
        _, nc, nm = oracle.topk(s, k)
        sg = oracle.idx_score(x["q_idx"], x["w"], x["k_idx"], gate)
        _, gcn, gm = oracle.topk(sg, k)
        _, _, _, pbar = oracle.golden(x["q"], x["kv"], SCALE, k)
        return s[0], nc[0], nm[0], gcn[0], gm[0], pbar[0]

    with ThreadPoolExecutor(max_workers=threads) as ex:
        res = list(ex.map(layer, seq_layers))
    X1 = np.stack([r[0] for r in res])[:, None]
    X2 = np.stack([r[5] for r in res])[:, None]
    out = {"gate": gate[0], "gate_count": int(gc[0]), "X1": X1[:, 0], "X2": X2[:, 0],
           "native_count": np.array([r[1] for r in res]), "native_mask": np.stack([r[2] for r in res]),
           "gated_count": np.array([r[3] for r in res]), "gated_mask": np.stack([r[4] for r in res])}
    for src, X, lg in (("R1", X1, True), ("R2", X2, False)):
        g, c, v = oracle.topp_vote(X, lg, 0.6, 3)
        out[f"gold_{src}"], out[f"gold_count_{src}"], out[f"votes_{src}"] = g[0], int(c[0]), v[0]
        for who in ("gated", "native"):
            out[f"{who}&{src}"] = np.array([oracle.recall(m[None], g)[0][0] for m in out[f"{who}_mask"]])
    out["gated&native"] = np.array([oracle.recall(a[None], b[None])[0][0]
                                    for a, b in zip(out["gated_mask"], out["native_mask"])])
    return out


def check_against_oracle(r, b, ref):
    assert np.array_equal(r.gate[b].cpu().numpy(), ref["gate"]), f"seq {b}: gate"
    assert np.array_equal(r.x["R1"][:, b].cpu().numpy(), ref["X1"]), f"seq {b}: exact logits"
    np.testing.assert_allclose(r.x["R2"][:, b].cpu().numpy(), ref["X2"], rtol=1e-11, atol=0)
    assert int(r.gate_count[b]) == ref["gate_count"]
    for what in ("native", "gated"):
        cnt = getattr(r, f"{what}_count")[:, b].cpu().numpy()
        msk = getattr(r, f"{what}_mask")[:, b].cpu().numpy()
        bad = [l for l in range(len(cnt)) if cnt[l] != ref[f"{what}_count"][l]
               or not np.array_equal(msk[l], ref[f"{what}_mask"][l])]
        assert not bad, f"seq {b}: {what} selection differs in layers {bad}"
    for src in SOURCES:
        votes = r.votes[src][b].cpu().numpy()
        if not np.array_equal(votes, ref[f"votes_{src}"]):
            diff = np.flatnonzero(votes != ref[f"votes_{src}"])[:8]
            raise AssertionError(f"seq {b}: {src} votes differ at {diff.tolist()}: "
                                 f"{votes[diff].tolist()} vs {ref[f'votes_{src}'][diff].tolist()}")
        assert np.array_equal(r.gold[src][b].cpu().numpy(), ref[f"gold_{src}"])
        assert int(r.gold_count[src][b]) == ref[f"gold_count_{src}"]
        for who in ("gated", "native"):
            assert r.inter[f"{who}&{src}"][:, b].cpu().tolist() == ref[f"{who}&{src}"].tolist(), f"{who}&{src}"
    assert r.inter["gated&native"][:, b].cpu().tolist() == ref["gated&native"].tolist()


def _run(B, N, k, d_model, rank, layers, keep_seqs):
    """The chain on the GPU with the gate workload's generators; returns the
    chain's outputs, the kept sequences' inputs per layer (host) and their gates."""
    wl = W.GATE64K
    keys = [W.layer_inputs(wl, l, "cuda", B=B, N=N).idx.k_idx for l in W.GATE_LAYERS]
    gl = [W.gate_layer(wl, l, kk, "cuda", d_model=d_model, rank=rank) for l, kk in zip(W.GATE_LAYERS, keys)]
    kept = {b: [] for b in keep_seqs}

    def maker(l):
        def make():
            L = W.layer_inputs(wl, l, "cuda", B=B, N=N)
            for b in keep_seqs:
                kept[b].append(_cpu_seq(L, b))
            return L
        return make

    r = labels.run_chain([maker(l) for l in layers], gl, k)
    torch.cuda.synchronize()
    gates = {b: [{"h": Ly.h[b:b + 1].cpu(), "wq_a": Ly.wq_a.cpu(), "wq_b": Ly.wq_b.cpu(), "w_proj": Ly.w_proj.cpu(),
                  "k": Ly.k[b:b + 1].cpu()} for Ly in gl] for b in keep_seqs}
    return r, kept, gates


def test_recall_chain_reduced_shapes_every_sequence():
    # 2 sequences x 3000 entries, the 21 CSA layers, top-256, gate projections at
    # d_model 512 / rank 256: every output of every sequence against the oracle
    B, N, k = 2, 3000, 256
    print("case recall chain B=2 N=3000 k=256", flush=True)
    r, kept, gates = _run(B, N, k, 512, 256, W.CSA_LAYERS, (0, 1))
    for b in range(B):
        ref = oracle_chain(kept[b], gates[b], k)
        check_against_oracle(r, b, ref)
    # the chain's invariants: gated selections lie inside the gate and never
    # exceed the native count; recall counts are bounded by the set sizes
    g = r.gate.cpu().numpy()
    gm = r.gated_mask.cpu().numpy()
    assert (gm <= g[None]).all()
    assert (r.gated_count <= r.native_count).all()
    for src in SOURCES:
        assert (r.inter[f"gated&{src}"] <= r.gold_count[src][None]).all()


def test_recall_chain_gate_workload_full_size_sampled_sequences():
    # the gate workload as the bench measures it: 8 sequences x 16384 entries,
    # FP8 rows, top-1024, the gate at d_model 4096 / rank 2048; every sequence's
    # outputs are checked for consistency, sequences 0 and 5 against the oracle
    wl = W.GATE64K
    print("case recall chain gate64k full size", flush=True)
    r, kept, gates = _run(wl.B, wl.N, wl.k, 4096, 2048, W.CSA_LAYERS, (0, 5))
    gm, nm = r.gated_mask.cpu().numpy(), r.native_mask.cpu().numpy()
    gate = r.gate.cpu().numpy()
    assert (gm <= gate[None]).all()
    assert np.array_equal(gm.sum(-1), r.gated_count.cpu().numpy())
    assert np.array_equal(nm.sum(-1), r.native_count.cpu().numpy())
    assert (r.native_count == wl.k).all()
    gc = r.gate_count.cpu().numpy()
    assert (r.gated_count.cpu().numpy() == np.minimum(wl.k, gc)[None]).all()
    for src in SOURCES:
        v = r.votes[src].cpu().numpy()
        assert np.array_equal((v >= 3).astype(np.uint8), r.gold[src].cpu().numpy())
        assert np.array_equal(r.gold[src].cpu().numpy().sum(-1), r.gold_count[src].cpu().numpy())
    for b in (0, 5):
        print(f"case recall chain gate64k oracle seq {b}", flush=True)
        check_against_oracle(r, b, oracle_chain(kept[b], gates[b], wl.k))
    s = labels.summary(r, wl.N)
    print("summary", s, flush=True)
    assert 0.0 < s["keep_frac"] < 1.0
