"""The multi-query indexer on the GPU (several queries per sequence sharing its
keys: MTP's draft token, a prefill chunk): scores against the oracle, the
per-query exact top-k bit for bit, and Q = 1 equal to the single-query call."""
import numpy as np
import pytest
import torch

import lightning_indexer_top_idx_amd as lit
import oracle
from lightning_indexer_top_idx_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lit.load()
    oracle.build()


def _score_bound(q, w, k, hid):
    """The rounding bound of the fp32 scores (the one the single-query parity
    tests use), per row: 4 * 2^-24 * (128 + H + 2) * sum_h |w_h| ||q_h|| * max ||k||."""
    H = q.shape[2]
    Qs = (w.double().cpu().abs() * q.double().cpu().norm(dim=-1)).sum(-1)  # [B,Q]
    K = k.double().cpu().norm(dim=-1).amax(-1)                             # [B]
    return (4 * 2.0 ** -24 * (128 + H + 2) * Qs * K[:, None]).numpy()


def _check_scores(s, s64, bound):
    s = s.double().cpu().numpy()
    fin = np.isfinite(s64)
    assert np.array_equal(np.isfinite(s), fin), "the -inf entries differ"
    err = np.where(fin, np.abs(np.where(fin, s, 0) - np.where(fin, s64, 0)), 0).max(-1)
    assert (err <= bound).all(), (err.max(), bound.min())


def _check_hints(s, h, N):
    # group maxima of the written scores, per row
    nch = -(-N // 256)
    G = -(-N // 16)
    s = s.cpu()
    pad = torch.full(s.shape[:-1] + (G * 16 - N,), float("-inf"))
    gm = torch.cat([s, pad], -1).view(*s.shape[:-1], G, 16).amax(-1)
    assert torch.equal(h.cpu()[..., nch:nch + G], gm)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_query_equals_lit_idx_score(dtype):
    wl = W.CTX64K_B if dtype == "bf16" else W.TINY
    print(f"case Q=1 {dtype}", flush=True)
    L = W.layer_inputs(wl, 3, "cuda", B=4 if dtype == "bf16" else 1, N=3001)
    q, w, k = L.idx.q_idx, L.idx.w, L.idx.k_idx
    s1, h1 = lit.idx_score(q, w, k)
    sm, hm = lit.idx_score_mq(q[:, None].contiguous(), w[:, None].contiguous(), k)
    torch.cuda.synchronize()
    # bit for bit (the hints end with fp64 word pairs, which may read as NaN floats)
    assert torch.equal(sm[:, 0], s1) and torch.equal(hm[:, 0].view(torch.int32), h1.view(torch.int32))


@pytest.mark.parametrize("Q,B,N,causal", [(2, 3, 5003, False), (2, 2, 4100, True), (5, 2, 2000, True),
                                          (9, 1, 1500, False), (37, 2, 1500, True), (16, 1, 2049, False),
                                          (2, 8, 1500, True), (3, 16, 700, False), (2, 2, 20000, False)])
def test_mq_scores_and_exact_topk_match_oracle(Q, B, N, causal):
    wl = W.CTX64K_B
    print(f"case mq Q={Q} B={B} N={N} causal={causal}", flush=True)
    idx = W.mq_inputs(wl, Q, 5, "cuda", B=B, N=N)
    q, w, k = idx.q_idx, idx.w, idx.k_idx
    lengths = W.causal_lengths(B, Q, 4 * N - Q - 37, "cuda") if causal else None
    s, h = lit.idx_score_mq(q, w, k, lengths)
    ids, cnt, mask = lit.topk_select_mq(s, wl.k, exact=(q, w, k), hints=h)
    torch.cuda.synchronize()
    s64 = oracle.idx_score_mq(q.cpu(), w.cpu(), k.cpu(), None if lengths is None else lengths.cpu())
    _check_scores(s, s64, _score_bound(q, w, k, None))
    _check_hints(s, h, N)
    rids, rcnt, rmask = oracle.topk_mq(s64, wl.k)
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert np.array_equal(mask.cpu().numpy(), rmask)


def test_mq_fp32_inputs_with_lengths_and_allowed():
    wl = W.TINY
    Q, B, N = 3, 2, 1000
    print("case mq f32 Q=3 allowed+lengths", flush=True)
    idx = W.mq_inputs(wl, Q, 0, "cuda", B=B, N=N)
    q, w, k = idx.q_idx, idx.w, idx.k_idx
    lengths = torch.tensor([[1000, 999, 70], [0, 1, 2000]], dtype=torch.int32, device="cuda")
    g = torch.Generator().manual_seed(5)
    allowed = (torch.rand(B, N, generator=g) < 0.7).to(torch.uint8).cuda()
    s, h = lit.idx_score_mq(q, w, k, lengths, allowed)
    ids, cnt, _ = lit.topk_select_mq(s, wl.k, exact=(q, w, k), hints=h)
    torch.cuda.synchronize()
    s64 = oracle.idx_score_mq(q.cpu(), w.cpu(), k.cpu(), lengths.cpu(), allowed.cpu())
    _check_scores(s, s64, _score_bound(q, w, k, None))
    rids, rcnt, _ = oracle.topk_mq(s64, wl.k)
    assert cnt.cpu().tolist() == rcnt.tolist() and cnt[1, 0].item() == 0
    assert np.array_equal(ids.cpu().numpy(), rids)


def test_mq_argument_errors():
    q = torch.zeros(1, 2, 4, 128, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(1, 2, 4, device="cuda")
    k = torch.zeros(1, 64, 128, dtype=torch.bfloat16, device="cuda")
    s = torch.empty(1, 2, 64, device="cuda")
    desc = lit.idx_in_mq(q, w, k)
    import ctypes
    C = lit.load()
    assert C.lit_idx_score_mq(ctypes.byref(desc), 0, None, None, 1, 64, s.data_ptr(), None, None) == 2
    assert C.lit_idx_score_mq(ctypes.byref(desc), 65537, None, None, 1, 64, s.data_ptr(), None, None) == 2
    assert C.lit_idx_score_mq(ctypes.byref(desc), 2, None, None, 1, 64, None, None, None) == 1
    assert C.lit_topk_select_mq(s.data_ptr(), 1, 0, 64, 8, None, None, s.data_ptr(), s.data_ptr(), None, None, 0,
                                None) == 2


def test_mtp_full_size_sampled_rows():
    # the MTP workload at full size, in the launch configuration the benchmark
    # times: 32 sequences x 2 queries x 16384 entries; every row's count and the
    # selection's invariants, and sampled rows against the oracle
    wl = W.CTX64K_B
    print("case mtp full size", flush=True)
    idx = W.mq_inputs(wl, W.MTP_Q, 2, "cuda")
    q, w, k = idx.q_idx, idx.w, idx.k_idx
    s, h = lit.idx_score_mq(q, w, k)
    ids, cnt, _ = lit.topk_select_mq(s, wl.k, exact=(q, w, k), hints=h, want_mask=False)
    torch.cuda.synchronize()
    assert (cnt == wl.k).all()
    ic = ids.cpu()
    assert (ic[..., 1:] > ic[..., :-1]).all()
    for b, j in ((0, 0), (0, 1), (17, 1), (31, 0)):
        s64 = oracle.idx_score_mq(q[b:b + 1, j:j + 1].cpu(), w[b:b + 1, j:j + 1].cpu(), k[b:b + 1].cpu())
        rids, _, _ = oracle.topk_mq(s64, wl.k)
        assert np.array_equal(ic[b, j].numpy(), rids[0, 0]), (b, j)


def test_prefill_chunk_sampled_rows():
    # a 2048-token prefill chunk at the end of a 64K prompt, causal lengths
    wl = W.CTX64K
    Q = W.PREFILL_Q
    print("case prefill chunk", flush=True)
    idx = W.mq_inputs(wl, Q, 0, "cuda")
    q, w, k = idx.q_idx, idx.w, idx.k_idx
    lengths = W.causal_lengths(1, Q, W.PREFILL_T - Q, "cuda")
    s, h = lit.idx_score_mq(q, w, k, lengths)
    ids, cnt, _ = lit.topk_select_mq(s, wl.k, exact=(q, w, k), hints=h, want_mask=False)
    torch.cuda.synchronize()
    assert (cnt == wl.k).all()
    lc = lengths.cpu()
    ic = ids.cpu()
    assert (ic.max(-1).values < lc).all()
    for j in (0, 1, 2, 3, 1000, 2047):
        s64 = oracle.idx_score_mq(q[:, j:j + 1].cpu(), w[:, j:j + 1].cpu(), k.cpu(), lc[:, j:j + 1])
        rids, _, _ = oracle.topk_mq(s64, wl.k)
        assert np.array_equal(ic[0, j].numpy(), rids[0, 0]), j


def test_many_query_arrangement_equals_few_query_arrangement():
    # 32 queries take the GEMM arrangement (16 queries per workgroup, key tiles
    # in LDS); 8 at a time take the key-streaming one. Both accumulate each head
    # over the same four K-steps, so scores and group maxima agree bit for bit.
    wl = W.CTX64K_B
    print("case mq arrangements Q=32 vs 4 x 8", flush=True)
    idx = W.mq_inputs(wl, 32, 9, "cuda", B=2, N=3001)
    q, w, k = idx.q_idx, idx.w, idx.k_idx
    lengths = W.causal_lengths(2, 32, 4 * 3001 - 40, "cuda")
    s, h = lit.idx_score_mq(q, w, k, lengths)
    nch, G = -(-3001 // 256), -(-3001 // 16)
    for j0 in range(0, 32, 8):
        sj, hj = lit.idx_score_mq(q[:, j0:j0 + 8].contiguous(), w[:, j0:j0 + 8].contiguous(), k,
                                  lengths[:, j0:j0 + 8].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(s[:, j0:j0 + 8], sj)
        assert torch.equal(h[:, j0:j0 + 8, nch:nch + G], hj[..., nch:nch + G])
        # the query-side sums agree to their stated accuracy, the key-norm bounds bound the same norms
        qa = h[:, j0:j0 + 8, nch + G:].contiguous().view(torch.float64)
        qb = hj[..., nch + G:].contiguous().view(torch.float64)
        assert torch.allclose(qa, qb, rtol=2.0 ** -40, atol=0)
        kn = k.double().norm(dim=-1)
        kn = torch.cat([kn, kn[:, -1:].expand(2, nch * 256 - 3001)], 1).view(2, nch, 256).amax(-1)
        assert (h[:, j0:j0 + 8, :nch].double() >= kn[:, None]).all() and (hj[..., :nch].double() >= kn[:, None]).all()
