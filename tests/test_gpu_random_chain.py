"""Seeded random shapes through the whole decode chain (score -> exact top-k ->
sparse attention) against the oracle.

Each case draws the batch, the number of entries, the index and query head
counts (including counts that are not multiples of 16), k (also past N), the
window, the index dtype, the KV dtype and signed head weights (the pages' index
weights come from a projection and may be negative), then compares ids, counts
and masks bit for bit and the attention output to the usual bar.
"""
import math

import numpy as np
import pytest
import torch

import lightning_indexer_top_idx_amd as lit
import oracle
from lightning_indexer_top_idx_amd import synth

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(512)
ATTN_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lit.load()
    oracle.build()


def _case(seed):
    r = np.random.default_rng(1000 + seed)
    # the sizes cycle through their lists (every one is met), the rest is drawn
    N = [1, 17, 256, 1000, 2049, 3001, 4097, 5003, 8191, 16384][seed % 10]
    H = [1, 5, 16, 17, 33, 48, 64][seed % 7]
    Hq = [1, 3, 16, 20, 64][seed % 5]
    B = int(r.choice([1, 2, 3, 5])) if N <= 5003 else int(r.choice([1, 2]))
    k = N + int(r.integers(1, 21)) if r.random() < 0.15 else int(r.integers(1, min(N, 1024) + 1))
    window = int(r.choice([0, 1, 64, 128, min(N + 5, 300)]))
    idx_dtype = str(r.choice(["bf16", "bf16", "f32"]))
    kv_dtype = str(r.choice(["bf16", "fp8"]))
    return B, N, H, Hq, k, window, idx_dtype, kv_dtype


CASES = [_case(s) for s in range(16)]


@pytest.mark.parametrize("B,N,H,Hq,k,window,idx_dtype,kv_dtype", CASES,
                         ids=[f"s{i}_B{c[0]}_N{c[1]}_H{c[2]}_Hq{c[3]}_k{c[4]}_W{c[5]}_{c[6]}_{c[7]}" for i, c in enumerate(CASES)])
def test_random_chain(B, N, H, Hq, k, window, idx_dtype, kv_dtype):
    print(f"case B={B} N={N} H={H} Hq={Hq} k={k} W={window} {idx_dtype} {kv_dtype}", flush=True)
    g = torch.Generator().manual_seed(B * 1_000_003 + N * 101 + H * 7 + k)
    inp = synth.make_indexer(B, N, H, idx_dtype, g, "cpu", planted_frac=0.01)
    w = (torch.randn(B, H, generator=g) * 0.5).float()  # signed head weights
    kv = synth.make_kv(B, N, kv_dtype, g, "cpu")
    q = synth.make_q(B, Hq, "bf16", g, "cpu")
    qi, wi, ki = inp.q_idx.cuda(), w.cuda(), inp.k_idx.cuda()

    scores, hints = lit.idx_score(qi, wi, ki)
    ids, cnt, mask = lit.topk_select(scores, k, exact=(qi, wi, ki), hints=hints)
    kv_d = synth.KVRows(kv.dtype, kv.data.cuda(), None if kv.rope is None else kv.rope.cuda(),
                        None if kv.scale is None else kv.scale.cuda())
    out, lse = lit.sparse_attn_decode(q.cuda(), kv_d, ids, cnt, window, SCALE)
    torch.cuda.synchronize()

    s64 = oracle.idx_score(inp.q_idx, w, inp.k_idx)
    rids, rcnt, rmask = oracle.topk(s64, k)
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert np.array_equal(mask.cpu().numpy(), rmask)

    ref, rlse = oracle.attend(q, kv, rids, rcnt, window, SCALE)
    o = out.double().cpu().numpy()
    err = np.abs(o - ref).max(-1)
    bar = ATTN_TOL * np.maximum(np.abs(ref).max(-1), 1e-30)
    assert not (err > bar).any(), f"worst relative error {np.max(err / np.maximum(np.abs(ref).max(-1), 1e-30)):.3g}"
    np.testing.assert_allclose(lse.double().cpu().numpy(), rlse, atol=2e-3, rtol=0)
