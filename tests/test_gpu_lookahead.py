"""The lookahead golden on the GPU: the golden set of every step of a horizon
(fp64 logits on the matrix cores), the per-entry step counts and their union,
against the oracle."""
import math

import numpy as np
import pytest
import torch

import lightning_indexer_top_idx_amd as lit
import oracle
from lightning_indexer_top_idx_amd import synth
from lightning_indexer_top_idx_amd import workloads as W

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(512)


@pytest.fixture(scope="module", autouse=True)
def _dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lit.load()
    oracle.build()


def _assert_same_sets(ids, rids, pbar_ref, k):
    """Each step's golden ids equal the oracle's; where they differ, only by
    entries whose pbar ties the k-th value within 1e-12 (relative): the two
    sides add the fp64 logits in different orders."""
    for idx in np.ndindex(ids.shape[:-1]):
        a, r = ids[idx], rids[idx]
        if np.array_equal(a, r):
            continue
        p = pbar_ref[idx]
        kth = np.sort(p)[::-1][k - 1]
        diff = set(a.tolist()) ^ set(r.tolist())
        assert all(abs(p[n] - kth) <= 1e-12 * kth for n in diff if n >= 0), (idx, diff)


@pytest.mark.parametrize("kv_dtype,B,T,Hq,N,k", [("bf16", 2, 8, 8, 1500, 64), ("fp8", 1, 5, 16, 2049, 128),
                                                 ("f32", 1, 3, 5, 300, 16), ("bf16", 3, 64, 1, 777, 8)])
def test_lookahead_golden_matches_oracle(kv_dtype, B, T, Hq, N, k):
    print(f"case lookahead {kv_dtype} B={B} T={T} Hq={Hq} N={N} k={k}", flush=True)
    g = synth.generator("cuda", 99, N)
    qd = "f32" if kv_dtype == "f32" else "bf16"
    q0 = synth.make_q(B, Hq, qd, g, "cuda")
    q = W.horizon_queries(q0, T, 7, "cuda")
    kv = synth.make_kv(B, N, kv_dtype, g, "cuda")
    ids, hits, um, uc, pbar = lit.lookahead_golden(q, kv, k, SCALE, want_pbar=True)
    torch.cuda.synchronize()
    rids, rhits, rum, ruc, rpbar = oracle.lookahead_golden(q.cpu(), kv, SCALE, k)
    np.testing.assert_allclose(pbar.cpu().numpy(), rpbar, rtol=1e-11, atol=0)
    ids_np = ids.cpu().numpy()
    _assert_same_sets(ids_np, rids, rpbar, k)
    if np.array_equal(ids_np, rids):
        assert np.array_equal(hits.cpu().numpy(), rhits)
        assert np.array_equal(um.cpu().numpy(), rum) and np.array_equal(uc.cpu().numpy(), ruc)
    # the union and the counts follow from the step sets the GPU chose
    mine = np.zeros((B, N), np.int32)
    for b in range(B):
        for t in range(T):
            sel = ids_np[b, t][ids_np[b, t] >= 0]
            mine[b, sel] += 1
    assert np.array_equal(hits.cpu().numpy(), mine)
    assert np.array_equal(um.cpu().numpy(), (mine > 0).astype(np.uint8))
    assert np.array_equal(uc.cpu().numpy(), (mine > 0).sum(-1))


def test_lookahead_single_step_equals_golden_topk():
    print("case lookahead T=1 vs golden", flush=True)
    g = synth.generator("cuda", 98, 1)
    q0 = synth.make_q(2, 16, "bf16", g, "cuda")
    kv = synth.make_kv(2, 3000, "bf16", g, "cuda")
    ids, hits, um, uc, pbar = lit.lookahead_golden(q0[:, None].contiguous(), kv, 100, SCALE, want_pbar=True)
    gids, gcnt, gmask, gpbar = lit.golden_topk(q0, kv, 100, SCALE)
    torch.cuda.synchronize()
    np.testing.assert_allclose(pbar[:, 0].cpu().numpy(), gpbar.cpu().numpy(), rtol=1e-12, atol=0)
    assert torch.equal(ids[:, 0], gids) and torch.equal(um, gmask) and torch.equal(uc, gcnt)


def test_lookahead_full_size_sampled_steps():
    # the benchmark's configuration: the gate workload's layer 10 (8 sequences x
    # 16384 FP8 rows, 64 heads, top-1024) over a 64-step horizon; every
    # sequence's union and hits must follow from its step sets, and sampled
    # steps must equal the oracle's golden sets
    wl = W.GATE64K
    print("case lookahead full size gate64k T=64", flush=True)
    L = W.layer_inputs(wl, 10, "cuda")
    q = W.horizon_queries(L.q, W.TAU, 10, "cuda")
    ids, hits, um, uc, _ = lit.lookahead_golden(q, L.kv, wl.k, SCALE)
    torch.cuda.synchronize()
    ic = ids.cpu().numpy()
    assert (ic >= 0).all() and (np.diff(ic, axis=-1) > 0).all()  # k ascending ids per step
    mine = np.zeros((wl.B, wl.N), np.int32)
    for b in range(wl.B):
        for t in range(W.TAU):
            mine[b, ic[b, t]] += 1
    assert np.array_equal(hits.cpu().numpy(), mine)
    assert np.array_equal(uc.cpu().numpy(), (mine > 0).sum(-1))
    for b, t in ((0, 0), (0, 63), (5, 31)):
        qb = q[b:b + 1, t:t + 1].cpu()
        kv = synth.KVRows("fp8", L.kv.data[b:b + 1].cpu(), L.kv.rope[b:b + 1].cpu(), L.kv.scale[b:b + 1].cpu())
        rids, _, _, _, rp = oracle.lookahead_golden(qb, kv, SCALE, wl.k)
        _assert_same_sets(ic[b:b + 1, t:t + 1], rids, rp, wl.k)
