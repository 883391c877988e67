"""Parity at the measured workloads' full sizes, in the launch configurations
the benchmark times (the same batch and entry counts, hence the same grids,
chunking, head groups and row slices).

Every sequence is checked for what holds at any size (count, ascending unique
ids in range, the mask agreeing with the ids); sampled sequences are checked
against the CPU oracle one by one: ids bit-exact, attention within 2e-2 of
the largest |output| of each head.
"""
import math

import numpy as np
import pytest
import torch

import lightning_indexer_top_idx_amd as lit
import oracle
from lightning_indexer_top_idx_amd import synth
from lightning_indexer_top_idx_amd import workloads as W

pytestmark = pytest.mark.gpu

ATTN_TOL = 2e-2
SCALE = 1.0 / math.sqrt(512)


@pytest.fixture(scope="module", autouse=True)
def _dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lit.load()
    oracle.build()


def kv_dev(kv):
    return synth.KVRows(kv.dtype, kv.data.cuda(), None if kv.rope is None else kv.rope.cuda(),
                        None if kv.scale is None else kv.scale.cuda())


def gpu_step(L, k, window, allowed=None):
    q, w, kk = L.idx.q_idx, L.idx.w, L.idx.k_idx
    scores, hints = lit.idx_score(q, w, kk, allowed)
    ids, cnt, mask = lit.topk_select(scores, k, exact=(q, w, kk), hints=hints)
    out, lse = lit.sparse_attn_decode(L.q, L.kv, ids, cnt, window, SCALE)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), cnt.cpu().numpy(), mask.cpu().numpy(), out.double().cpu().numpy()


def check_valid(ids, cnt, mask, N, k, selectable=None):
    B = ids.shape[0]
    for b in range(B):
        want = min(k, N if selectable is None else int(selectable[b]))
        assert cnt[b] == want, f"b={b}: count {cnt[b]} != {want}"
        sel = ids[b, :want]
        assert (np.diff(sel) > 0).all() and sel[0] >= 0 and sel[-1] < N, f"b={b}: ids not ascending in range"
        assert (ids[b, want:] == -1).all(), f"b={b}: tail not -1"
        assert mask[b].sum() == want and mask[b][sel].all(), f"b={b}: mask disagrees with ids"


def seq_cpu(L, b):
    """Sequence b of a layer as a B=1 CPU layer (same bits)."""
    one = lambda x: None if x is None else x[b:b + 1].cpu()
    idx = synth.IndexerInputs(one(L.idx.q_idx), one(L.idx.w), one(L.idx.k_idx))
    kv = synth.KVRows(L.kv.dtype, one(L.kv.data), one(L.kv.rope), one(L.kv.scale))
    return idx, one(L.q), kv


def check_oracle(L, b, k, window, ids, out, allowed=None):
    idx, q, kv = seq_cpu(L, b)
    al = None if allowed is None else allowed[b:b + 1].cpu().numpy()
    s64 = oracle.idx_score(idx.q_idx, idx.w, idx.k_idx, al)
    rids, rcnt, _ = oracle.topk(s64, k)
    assert np.array_equal(ids[b], rids[0]), f"b={b}: ids differ from the oracle"
    ref, _ = oracle.attend(q, kv, rids, rcnt, window, SCALE)
    err = np.abs(out[b] - ref[0]).max(-1)
    scale = np.abs(ref[0]).max(-1)
    assert (err <= ATTN_TOL * np.maximum(scale, 1e-30)).all(), f"b={b}: attention off by {np.max(err / scale):.3g}"


@pytest.mark.parametrize("layer", [0, 20])
def test_ctx64k_batched_headline(layer):
    # 32 sequences x N = 16384, top-512 + window 128: one layer of the timed step
    wl = W.CTX64K_B
    print(f"case ctx64k_b layer {layer}", flush=True)
    L = W.layer_inputs(wl, layer, "cuda")
    ids, cnt, mask, out = gpu_step(L, wl.k, wl.window)
    check_valid(ids, cnt, mask, wl.N, wl.k)
    for b in (0, 13, 31):
        check_oracle(L, b, wl.k, wl.window, ids, out)


def test_ctx500k_batch4_csa_and_hca():
    # 4 sequences x N = 125000 (CSA), then the HCA layer's 3907 rows read densely
    wl = W.CTX500K
    print("case ctx500k_b4", flush=True)
    L = W.layer_inputs(wl, 0, "cuda")
    ids, cnt, mask, out = gpu_step(L, wl.k, wl.window)
    check_valid(ids, cnt, mask, wl.N, wl.k)
    for b in (0, 3):
        check_oracle(L, b, wl.k, wl.window, ids, out)
    q, kv = W.hca_inputs(wl, "cuda")
    dense, _ = lit.sparse_attn_decode(q, kv, None, None, 0, SCALE)
    torch.cuda.synchronize()
    ref, _ = oracle.attend(q.cpu(), synth.KVRows(kv.dtype, kv.data.cpu(), None, None), None, None, 0, SCALE)
    d = dense.double().cpu().numpy()
    err = np.abs(d - ref).max(-1)
    assert (err <= ATTN_TOL * np.abs(ref).max(-1)).all()


def test_gate_stress_batch8_fp8_top1024_gated():
    # 8 sequences x N = 16384, FP8 rows, top-1024 inside the gated set of layers 10/12/20
    wl = W.GATE64K
    print("case gate64k_b8", flush=True)
    keys = [W.layer_inputs(wl, l, "cuda").idx.k_idx for l in W.GATE_LAYERS]
    gl = [W.gate_layer(wl, l, kk, "cuda") for l, kk in zip(W.GATE_LAYERS, keys)]
    gate, gcnt = lit.lsa_gate(gl, 0.5)
    L = W.layer_inputs(wl, 10, "cuda")
    ids, cnt, mask, out = gpu_step(L, wl.k, wl.window, allowed=gate)
    gc = gcnt.cpu().numpy()
    # the gate of sequence 0 at full size against the oracle's (fp64 projections)
    g0 = [{"h": Ly.h[:1].cpu(), "wq_a": Ly.wq_a.cpu(), "wq_b": Ly.wq_b.cpu(), "w_proj": Ly.w_proj.cpu(),
           "k": Ly.k[:1].cpu()} for Ly in gl]
    rg, rc = oracle.lsa_gate(g0, 0.5)
    assert np.array_equal(gate[:1].cpu().numpy(), rg) and gc[0] == rc[0]
    assert 0 < gc.min() and gc.max() < wl.N
    check_valid(ids, cnt, mask, wl.N, wl.k, selectable=gc)
    assert (mask <= gate.cpu().numpy()).all()
    for b in (0, 7):
        check_oracle(L, b, wl.k, wl.window, ids, out, allowed=gate)
