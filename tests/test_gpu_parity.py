"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: selected ids, masks, counts, golden sets, recall counts and gate masks
bit-exact; attention outputs within 2e-2 of the largest |output| of each
(sequence, head) row (bf16 inputs, fp32 accumulation); fp32 indexer scores
within the proven rounding bound of the fp64 scores.
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


def dev(x):
    return None if x is None else x.cuda()


def kv_dev(kv):
    return synth.KVRows(kv.dtype, kv.data.cuda(), dev(kv.rope), dev(kv.scale))


def score_bound(q, w, k):
    """The rounding bound the exact selection relies on (per sequence)."""
    qd = q.double().cpu()
    Q = (w.double().cpu().abs() * qd.norm(dim=-1)).sum(-1)
    K = k.double().cpu().norm(dim=-1).amax(-1)
    H = q.shape[1]
    return 4 * 2.0**-24 * (128 + H + 2) * Q * K


def assert_attn_close(out, ref, tol=ATTN_TOL):
    out = out.double().cpu().numpy()
    err = np.abs(out - ref).max(-1)
    scale = np.abs(ref).max(-1)
    bad = err > tol * np.maximum(scale, 1e-30)
    assert not bad.any(), f"attention mismatch: worst rel {np.max(err / np.maximum(scale, 1e-30)):.3g}"


def run_select(inp, k, exact=True, allowed=None):
    q, w, kk = dev(inp.q_idx), dev(inp.w), dev(inp.k_idx)
    scores, hints = lit.idx_score(q, w, kk, dev(allowed))
    ids, cnt, mask = lit.topk_select(scores, k, exact=(q, w, kk) if exact else None, hints=hints)
    torch.cuda.synchronize()
    return scores, hints, ids, cnt, mask


def oracle_select(inp, k, allowed=None):
    s = oracle.idx_score(inp.q_idx, inp.w, inp.k_idx, allowed)
    ids, cnt, mask = oracle.topk(s, k)
    return s, ids, cnt, mask


def check_selection(ids, cnt, mask, rids, rcnt, rmask, s64=None, what=""):
    ids, cnt, mask = ids.cpu().numpy(), cnt.cpu().numpy(), mask.cpu().numpy()
    if not (np.array_equal(cnt, rcnt) and np.array_equal(ids, rids)):
        msg = [f"{what}: selection differs"]
        for b in range(len(cnt)):
            a, r = set(ids[b][: max(cnt[b], 0)].tolist()), set(rids[b][: rcnt[b]].tolist())
            if a != r:
                extra, miss = sorted(a - r)[:5], sorted(r - a)[:5]
                gap = ""
                if s64 is not None and extra and miss:
                    gap = f" fp64 gap {s64[b][miss[0]] - s64[b][extra[0]]:.3e}"
                msg.append(f" b={b} cnt {cnt[b]} vs {rcnt[b]} extra {extra} missing {miss}{gap}")
        pytest.fail("\n".join(msg))
    assert np.array_equal(mask, rmask), f"{what}: mask differs"


# ---------------------------------------------------------------- a1 + a2


SEL_CASES = [
    # name, workload, B, N, k
    ("tiny", W.TINY, None, None, 64),
    ("ctx64k_b1", W.CTX64K, None, None, 512),
    ("ragged_b2", W.CTX64K, 2, 5003, 512),
    ("k_above_n", W.CTX64K, 1, 300, 512),
    ("n_one", W.CTX64K, 1, 1, 1),
    ("n40000", W.CTX64K, 1, 40000, 512),
    ("pro_k1024", W.CTX64K, 3, 16384, 1024),
    ("ctx500k", W.CTX500K, 1, None, 512),
    ("full_scan_140k", W.CTX64K, 1, 140000, 512),
    # the two-kernel path for long rows: several rows, and more than eight rows
    # (the candidate grid pads each group of eight)
    ("wide_b3_n40000", W.CTX64K, 3, 40000, 512),
    ("wide_b9_n20000", W.CTX64K, 9, 20000, 256),
]


@pytest.mark.parametrize("name,wl,B,N,k", SEL_CASES, ids=[c[0] for c in SEL_CASES])
def test_score_and_exact_topk(name, wl, B, N, k):
    print(f"case {name}", flush=True)
    inp = W.layer_inputs(wl, 0, "cpu", B=B, N=N).idx
    scores, hints, ids, cnt, mask = run_select(inp, k)
    s64, rids, rcnt, rmask = oracle_select(inp, k)
    # fp32 scores within the bound of the fp64 ones; empirically far tighter
    err = np.abs(scores.double().cpu().numpy() - s64).max(-1)
    bound = score_bound(inp.q_idx, inp.w, inp.k_idx).numpy()
    assert (err <= bound).all(), f"score error {err} above bound {bound}"
    assert (err <= 1e-5 * np.abs(s64).max(-1) + 1e-30).all()
    # hints: key-norm chunk bounds cover every chunk's largest norm tightly, and
    # the group maxima are exactly the maxima of the scores written
    norms = inp.k_idx.double().norm(dim=-1)
    Nn = norms.shape[1]
    nch = -(-Nn // 256)
    pad = (-Nn) % 256
    cm = torch.nn.functional.pad(norms, (0, pad)).reshape(norms.shape[0], -1, 256).amax(-1).numpy()
    hn = hints.double().cpu()
    km = hn[:, :nch].numpy()
    assert (km >= cm).all() and (km <= cm * (1 + 1e-4) + 1e-30).all()
    sc = scores.cpu()
    gpad = (-Nn) % 16
    gref = torch.nn.functional.pad(sc, (0, gpad), value=float("-inf")).reshape(sc.shape[0], -1, 16).amax(-1)
    ng = gref.shape[1]
    assert hints.shape[1] == nch + ng + 4
    assert torch.equal(hints.cpu()[:, nch:nch + ng], gref)
    # the query-side bound sums, fp64 word pairs at the end: sum |w| ||q|| and sum |w|
    qb = np.ascontiguousarray(hints.cpu()[:, nch + ng:].numpy()).view(np.float64)
    q64 = inp.q_idx.double().cpu()
    w64 = inp.w.double().cpu().abs()
    qref = (w64 * q64.norm(dim=-1)).sum(-1).numpy()
    wref = w64.sum(-1).numpy()
    assert np.allclose(qb[:, 0], qref, rtol=2.0 ** -40, atol=0), (qb[:, 0], qref)
    assert np.allclose(qb[:, 1], wref, rtol=2.0 ** -40, atol=0), (qb[:, 1], wref)
    check_selection(ids, cnt, mask, rids, rcnt, rmask, s64, name)


def test_exact_grid_ties_bit_exact_scores_and_selection():
    g = torch.Generator().manual_seed(7)
    inp = synth.make_exact_grid(2, 4000, 8, g, "cpu")
    scores, hints, ids, cnt, mask = run_select(inp, 100)
    s64, rids, rcnt, rmask = oracle_select(inp, 100)
    np.testing.assert_array_equal(scores.double().cpu().numpy(), s64)  # exact in any order
    check_selection(ids, cnt, mask, rids, rcnt, rmask, s64, "exact_grid")


def test_all_zero_keys_select_first_k():
    inp = W.layer_inputs(W.CTX64K, 0, "cpu", B=1, N=2000).idx
    inp.k_idx.zero_()
    scores, hints, ids, cnt, mask = run_select(inp, 64)
    assert (scores.cpu() == 0).all()
    assert ids.cpu()[0].tolist() == list(range(64)) and cnt.item() == 64


def test_gated_candidate_set():
    inp = W.layer_inputs(W.CTX64K, 0, "cpu", B=2, N=4000).idx
    allowed = torch.zeros(2, 4000, dtype=torch.uint8)
    allowed[0, torch.randperm(4000, generator=torch.Generator().manual_seed(1))[:300]] = 1  # fewer than k
    allowed[1, torch.randperm(4000, generator=torch.Generator().manual_seed(2))[:2500]] = 1
    scores, hints, ids, cnt, mask = run_select(inp, 512, allowed=allowed)
    s64, rids, rcnt, rmask = oracle_select(inp, 512, allowed.numpy())
    assert torch.isneginf(scores.cpu()[allowed == 0]).all()
    check_selection(ids, cnt, mask, rids, rcnt, rmask, s64, "gated")
    assert cnt.cpu().tolist() == [300, 512]
    assert (mask.cpu() <= allowed).all()


def test_gated_candidate_set_long_rows():
    # the two-kernel path with a gate: a row with fewer selectable entries than
    # k (its candidates are every selectable entry) and a row gated to 3/4
    N = 40000
    inp = W.layer_inputs(W.CTX64K, 0, "cpu", B=2, N=N).idx
    allowed = torch.zeros(2, N, dtype=torch.uint8)
    allowed[0, torch.randperm(N, generator=torch.Generator().manual_seed(3))[:300]] = 1
    allowed[1, torch.randperm(N, generator=torch.Generator().manual_seed(4))[:30000]] = 1
    scores, hints, ids, cnt, mask = run_select(inp, 512, allowed=allowed)
    s64, rids, rcnt, rmask = oracle_select(inp, 512, allowed.numpy())
    check_selection(ids, cnt, mask, rids, rcnt, rmask, s64, "gated long rows")
    assert cnt.cpu().tolist() == [300, 512]


def test_long_rows_with_a_block_of_equal_top_scores():
    # 400 entries of row 0 share the key of its best entry: their exact scores
    # tie at the top and top-300 takes the 300 lowest indices among them. The
    # two-kernel path cannot rescore them all in one slice and takes its
    # in-row fallback; row 1 is ordinary
    N, k = 40000, 300
    inp = W.layer_inputs(W.CTX64K, 2, "cpu", B=2, N=N).idx
    s = oracle.idx_score(inp.q_idx, inp.w, inp.k_idx)
    best = int(np.argmax(s[0]))
    inp.k_idx[0, 1000:1400] = inp.k_idx[0, best]
    scores, hints, ids, cnt, mask = run_select(inp, k)
    s64, rids, rcnt, rmask = oracle_select(inp, k)
    check_selection(ids, cnt, mask, rids, rcnt, rmask, s64, "equal top block")
    sel = set(ids.cpu().numpy()[0].tolist())
    assert set(range(1000, 1300)) <= sel | {best}


def test_topk_on_given_scores_with_heavy_ties():
    g = torch.Generator().manual_seed(9)
    for N, k in ((1000, 64), (16384, 512), (70000, 512)):
        s = torch.round(torch.randn(3, N, generator=g) * 4) / 4  # many exact ties
        s[0, :50] = float("-inf")
        s[1, 7] = float("nan")
        # row 2: the k-th score is zero and +0.0 / -0.0 (equal values) are mixed:
        # the lower index must win between them as between any equal scores
        z = torch.where(torch.rand(N, generator=g) < 0.5, torch.tensor(-0.0), torch.tensor(0.0))
        z[torch.randperm(N, generator=g)[: k // 2]] = torch.rand(k // 2, generator=g) + 1.0
        s[2] = z
        ids, cnt, mask = lit.topk_select(s.cuda(), k)
        torch.cuda.synchronize()
        rids, rcnt, rmask = oracle.topk(s.double().numpy(), k)
        check_selection(ids, cnt, mask, rids, rcnt, rmask, None, f"given_scores N={N}")


def test_topk_with_hints_on_fp32_order():
    # without `exact` the fp32 scores define the order; the hinted path must agree
    for B, N, k in ((2, 16384, 512), (1, 5000, 4000), (1, 125000, 1024), (4, 125000, 512)):
        inp = W.layer_inputs(W.CTX64K, 3, "cpu", B=B, N=N).idx
        q, w, kk = dev(inp.q_idx), dev(inp.w), dev(inp.k_idx)
        scores, hints = lit.idx_score(q, w, kk)
        ids, cnt, mask = lit.topk_select(scores, k, hints=hints)
        torch.cuda.synchronize()
        rids, rcnt, rmask = oracle.topk(scores.double().cpu().numpy(), k)
        check_selection(ids, cnt, mask, rids, rcnt, rmask, None, f"fp32 order N={N} k={k}")


def test_topk_with_hints_of_other_scores_falls_back():
    # hints computed for other scores: their group maxima may lie below or above
    # these scores' own; the selection detects that (a key above the hinted
    # largest, or fewer than k entries above the hinted bound) and takes the
    # full scan, so the result is still the exact top-k of the scores given;
    # above 16384 entries the two-kernel path's checks send it there
    for N, k in ((16384, 512), (4000, 256), (40000, 512)):
        a = W.layer_inputs(W.CTX64K, 1, "cpu", B=2, N=N).idx
        o = W.layer_inputs(W.CTX64K, 2, "cpu", B=2, N=N).idx
        scores, _ = lit.idx_score(dev(a.q_idx), dev(a.w), dev(a.k_idx))
        for scale in (0.25, 4.0):
            _, hints = lit.idx_score(dev(o.q_idx), dev(o.w) * scale, dev(o.k_idx))
            ids, cnt, mask = lit.topk_select(scores, k, hints=hints)
            torch.cuda.synchronize()
            rids, rcnt, rmask = oracle.topk(scores.double().cpu().numpy(), k)
            check_selection(ids, cnt, mask, rids, rcnt, rmask, None, f"other hints N={N} x{scale}")


def test_score_launch_arrangements_agree_bit_for_bit():
    # the headline batch (32 sequences, four chunks per workgroup, each
    # sequence on one XCD) and sequences of it scored in smaller batches (one
    # chunk per workgroup; or four chunks on a two-dimensional grid, 20
    # sequences) run the same per-entry arithmetic
    inp = W.layer_inputs(W.CTX64K_B, 3, "cuda").idx
    s32, h32 = lit.idx_score(inp.q_idx, inp.w, inp.k_idx)
    for lo, hi in ((0, 8), (16, 24), (29, 30), (5, 25)):
        s, h = lit.idx_score(inp.q_idx[lo:hi].contiguous(), inp.w[lo:hi].contiguous(), inp.k_idx[lo:hi].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(s, s32[lo:hi]), (lo, hi)
        assert torch.equal(h.view(torch.int32), h32[lo:hi].view(torch.int32)), (lo, hi)


def test_idx_score_exact_matches_oracle_bit_for_bit():
    for wl, B, N in ((W.TINY, None, None), (W.CTX64K, 2, 3001)):
        inp = W.layer_inputs(wl, 0, "cpu", B=B, N=N).idx
        got = lit.idx_score_exact(dev(inp.q_idx), dev(inp.w), dev(inp.k_idx)).cpu().numpy()
        np.testing.assert_array_equal(got, oracle.idx_score(inp.q_idx, inp.w, inp.k_idx))


# ---------------------------------------------------------------- a3/a4/a5


def oracle_ids(inp, k):
    return oracle.topk(oracle.idx_score(inp.q_idx, inp.w, inp.k_idx), k)


@pytest.mark.parametrize("name,wl,B,N,k,window", [
    ("tiny_f32", W.TINY, None, None, 64, 16),
    ("ctx64k_b2", W.CTX64K, 2, 16384, 512, 128),
    ("ragged", W.CTX64K, 3, 2049, 512, 128),
    ("window_over_n", W.CTX64K, 1, 100, 512, 300),
    ("no_window", W.CTX64K, 2, 3000, 256, 0),
    # k beyond N: the selection's capacity exceeds the rows; the workspace the
    # binding takes from lit_attn_workspace_bytes(B, Hq, N) must still suffice
    ("kcap_over_n", W.CTX64K, 2, 300, 512, 128),
    ("kcap_over_n_b1", W.CTX64K, 1, 100, 512, 128),
])
def test_sparse_attention(name, wl, B, N, k, window):
    print(f"case {name}", flush=True)
    L = W.layer_inputs(wl, 0, "cpu", B=B, N=N)
    rids, rcnt, _ = oracle_ids(L.idx, k)
    out, lse = lit.sparse_attn_decode(dev(L.q), kv_dev(L.kv), dev(torch.from_numpy(rids)),
                                      dev(torch.from_numpy(rcnt)), window, SCALE)
    torch.cuda.synchronize()
    ref, rlse = oracle.attend(L.q, L.kv, rids, rcnt, window, SCALE)
    assert_attn_close(out, ref)
    np.testing.assert_allclose(lse.double().cpu().numpy(), rlse, atol=2e-3, rtol=0)


def test_attention_head_counts():
    # one head block per workgroup (Hq <= 16), two (Hq > 16), and a partial
    # second block (Hq = 48: heads 48..63 of the last group are not written)
    L = W.layer_inputs(W.CTX64K, 1, "cpu", B=3, N=2500)
    rids, rcnt, _ = oracle_ids(L.idx, 512)
    for Hq in (8, 16, 48, 64):
        print(f"case attention Hq={Hq}", flush=True)
        q = synth.make_q(3, Hq, "bf16", torch.Generator().manual_seed(40 + Hq), "cpu")
        out, lse = lit.sparse_attn_decode(q.cuda(), kv_dev(L.kv), dev(torch.from_numpy(rids)),
                                          dev(torch.from_numpy(rcnt)), 128, SCALE)
        dense, dlse = lit.sparse_attn_decode(q.cuda(), kv_dev(L.kv), None, None, 0, SCALE)
        torch.cuda.synchronize()
        ref, rlse = oracle.attend(q, L.kv, rids, rcnt, 128, SCALE)
        assert_attn_close(out, ref)
        np.testing.assert_allclose(lse.double().cpu().numpy(), rlse, atol=2e-3, rtol=0)
        dref, drlse = oracle.attend(q, L.kv, None, None, 0, SCALE)
        assert_attn_close(dense, dref)
        np.testing.assert_allclose(dlse.double().cpu().numpy(), drlse, atol=2e-3, rtol=0)


def test_attention_counts_below_cap_duplicates_and_empty():
    L = W.layer_inputs(W.CTX64K, 0, "cpu", B=4, N=1000)
    ids = np.full((4, 64), -1, np.int32)
    ids[0, :10] = np.arange(990, 1000)  # all inside the window of 16
    ids[1, :5] = [0, 1, 2, 500, 999]
    ids[2, :64] = np.arange(0, 640, 10)
    cnt = np.array([10, 5, 64, 0], np.int32)
    for window in (16, 0):
        out, lse = lit.sparse_attn_decode(dev(L.q), kv_dev(L.kv), dev(torch.from_numpy(ids)),
                                          dev(torch.from_numpy(cnt)), window, SCALE)
        torch.cuda.synchronize()
        ref, rlse = oracle.attend(L.q, L.kv, ids, cnt, window, SCALE)
        if window == 0:  # sequence 3 selects nothing and has no window
            assert (out[3] == 0).all() and torch.isneginf(lse[3]).all()
            ref[3] = 0
        assert_attn_close(out, ref)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_attention_scores_rising_far_past_the_first_tile(kv_dtype):
    # Sixteen sequences split into four slices of two tiles each. In every
    # sequence one row in a slice's second tile is 120 x head 0's unit query, so
    # head 0's score there exceeds its first tile's maximum by ~170 in log2
    # units: the slice's running softmax reference has to move that far and
    # rescale what it holds. The sparse list holds it at position 266 (slice
    # 0's second tile), the dense layout at position 300; the other sequences
    # plant it elsewhere.
    B, N, Hq = 16, 2000, 64
    print(f"case rising scores {kv_dtype}", flush=True)
    g = torch.Generator().manual_seed(91)
    x = torch.randn(B, N, 512, generator=g)
    q = synth.make_q(B, Hq, "bf16", g, "cpu")
    ids = np.stack([np.sort(np.random.default_rng(b).choice(N, 512, replace=False)) for b in range(B)]).astype(np.int32)
    cnt = np.full(B, 512, np.int32)
    for b in range(B):
        unit = q[b, 0].float() / q[b, 0].float().norm()
        for r in {int(ids[b, 266 - 7 * b]), 300 + 17 * b}:
            x[b, r] = 120.0 * unit
    if kv_dtype == "bf16":
        kv = synth.KVRows("bf16", x.to(torch.bfloat16).contiguous())
    else:
        codes, sc = synth.fp8_encode(x[..., :synth.FP8_DIMS])
        kv = synth.KVRows("fp8", codes, x[..., synth.FP8_DIMS:].to(torch.bfloat16).contiguous(), sc)
    for sparse in (True, False):
        a_ids, a_cnt = (dev(torch.from_numpy(ids)), dev(torch.from_numpy(cnt))) if sparse else (None, None)
        out, lse = lit.sparse_attn_decode(q.cuda(), kv_dev(kv), a_ids, a_cnt, 0, SCALE)
        torch.cuda.synchronize()
        ref, rlse = oracle.attend(q, kv, ids if sparse else None, cnt if sparse else None, 0, SCALE)
        assert np.isfinite(out.cpu().numpy()).all()
        assert_attn_close(out, ref)
        np.testing.assert_allclose(lse.double().cpu().numpy(), rlse, atol=2e-3, rtol=0)


def test_failed_selection_gives_nan_for_its_sequence_only():
    # count[b] = -1 (the exact selection's failure sign): that sequence's out
    # and lse are NaN, the others match the oracle; on the split path (slices
    # + combine), the single-slice path and the FP32 kernel
    for name, wl, B, N, k, window, bad in (("split", W.CTX64K, 2, 3000, 256, 128, 0),
                                             ("one_slice", W.CTX64K, 64, 1000, 64, 16, 3),
                                             ("f32", W.TINY, 3, 1024, 64, 16, 1)):
        print(f"case failed selection {name}", flush=True)
        L = W.layer_inputs(wl, 0, "cpu", B=B, N=N)
        rids, rcnt, _ = oracle_ids(L.idx, k)
        cnt = rcnt.copy()
        cnt[bad] = -1
        out, lse = lit.sparse_attn_decode(dev(L.q), kv_dev(L.kv), dev(torch.from_numpy(rids)),
                                          dev(torch.from_numpy(cnt)), window, SCALE)
        torch.cuda.synchronize()
        assert torch.isnan(out[bad]).all() and torch.isnan(lse[bad]).all(), name
        keep = [b for b in range(out.shape[0]) if b != bad]
        ref, rlse = oracle.attend(L.q, L.kv, rids, rcnt, window, SCALE)
        assert_attn_close(out[keep], ref[keep])
        np.testing.assert_allclose(lse[keep].double().cpu().numpy(), rlse[keep], atol=2e-3, rtol=0)


def test_full_selection_equals_dense_and_hca_mode():
    L = W.layer_inputs(W.CTX64K, 0, "cpu", B=2, N=3907)
    q, kv = dev(L.q), kv_dev(L.kv)
    dense, dlse = lit.sparse_attn_decode(q, kv, None, None, 0, SCALE)
    allids = torch.arange(3907, dtype=torch.int32).repeat(2, 1).cuda()
    full, flse = lit.sparse_attn_decode(q, kv, allids, torch.full((2,), 3907, dtype=torch.int32).cuda(), 128, SCALE)
    torch.cuda.synchronize()
    ref, rlse = oracle.attend(L.q, L.kv, None, None, 0, SCALE)
    assert_attn_close(dense, ref)
    assert_attn_close(full, ref)
    np.testing.assert_allclose(dlse.double().cpu().numpy(), rlse, atol=2e-3, rtol=0)


def test_fp8_rows_attention():
    L = W.layer_inputs(W.GATE64K, 2, "cpu", B=2, N=3000)
    rids, rcnt, _ = oracle_ids(L.idx, 1024)
    out, lse = lit.sparse_attn_decode(dev(L.q), kv_dev(L.kv), dev(torch.from_numpy(rids)),
                                      dev(torch.from_numpy(rcnt)), 128, SCALE)
    torch.cuda.synchronize()
    ref, rlse = oracle.attend(L.q, L.kv, rids, rcnt, 128, SCALE)
    assert_attn_close(out, ref)


def _fp8_rows_wide_exponents(B, N, seed):
    # FP8 rows whose 64-dim groups span scale exponents from 2^-14 to 2^3, with
    # every 7th group all zero (scale byte 127, zero codes) and every 11th row's
    # RoPE part zero: the widening must be exact for each scale
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, N, 7, 64, generator=g)
    x = x * torch.exp2(torch.randint(-14, 4, (B, N, 7, 1), generator=g).float())
    x.view(-1, 64)[::7] = 0
    codes, sc = synth.fp8_encode(x.view(B, N, 448))
    rope = torch.randn(B, N, 64, generator=g).to(torch.bfloat16)
    rope[:, ::11] = 0
    return synth.KVRows("fp8", codes, rope.contiguous(), sc)


def test_fp8_rows_dense_ragged_and_sparse_with_window():
    B, N, Hq = 3, 3001, 64
    kv = _fp8_rows_wide_exponents(B, N, 21)
    assert (kv.scale[..., :7] == 127).any() and (kv.scale[..., :7] < 127 - 10).any()
    q = synth.make_q(B, Hq, "bf16", torch.Generator().manual_seed(22), "cpu")
    # dense: every row (47 tiles of 64, the last one 57 rows)
    out, lse = lit.sparse_attn_decode(q.cuda(), kv_dev(kv), None, None, 0, SCALE)
    torch.cuda.synchronize()
    ref, rlse = oracle.attend(q, kv, None, None, 0, SCALE)
    assert_attn_close(out, ref)
    np.testing.assert_allclose(lse.double().cpu().numpy(), rlse, atol=2e-3, rtol=0)
    # sparse: counts below the cap, ids inside the window (counted once), an empty selection
    ids = np.full((B, 300), -1, np.int32)
    ids[0, :300] = np.arange(0, 3000, 10)
    ids[1, :40] = np.arange(2961, 3001)
    ids[2, :0] = 0
    cnt = np.array([300, 40, 0], np.int32)
    out, lse = lit.sparse_attn_decode(q.cuda(), kv_dev(kv), torch.from_numpy(ids).cuda(),
                                      torch.from_numpy(cnt).cuda(), 128, SCALE)
    torch.cuda.synchronize()
    ref, rlse = oracle.attend(q, kv, ids, cnt, 128, SCALE)
    assert_attn_close(out, ref)
    np.testing.assert_allclose(lse.double().cpu().numpy(), rlse, atol=2e-3, rtol=0)


# ---------------------------------------------------------------- a6 / a7 / a9


@pytest.mark.parametrize("name,wl,B,N,k", [
    ("tiny", W.TINY, None, None, 64),
    ("bf16", W.CTX64K, 2, 4096, 512),
    ("fp8", W.GATE64K, 1, 2048, 1024),
])
def test_golden_topk(name, wl, B, N, k):
    L = W.layer_inputs(wl, 0, "cpu", B=B, N=N)
    ids, cnt, mask, pbar = lit.golden_topk(dev(L.q), kv_dev(L.kv), k, SCALE)
    torch.cuda.synchronize()
    rids, rcnt, rmask, rp = oracle.golden(L.q, L.kv, SCALE, k)
    np.testing.assert_allclose(pbar.cpu().numpy(), rp, rtol=1e-11, atol=0)
    ids_np = ids.cpu().numpy()
    if np.array_equal(ids_np, rids):
        check_selection(ids, cnt, mask, rids, rcnt, rmask, rp, f"golden {name}")
        return
    # the logits are fp64 sums on the matrix cores, added in another order than
    # the oracle's: a set may differ only at a tie with the k-th value within that
    # rounding, and the count and mask follow the ids the GPU chose
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    for b in range(ids_np.shape[0]):
        kth = np.sort(rp[b])[::-1][k - 1]
        diff = set(ids_np[b].tolist()) ^ set(rids[b].tolist())
        assert all(abs(rp[b][n] - kth) <= 1e-12 * kth for n in diff if n >= 0), (b, diff)
        m = np.zeros(rp.shape[1], np.uint8)
        m[ids_np[b][ids_np[b] >= 0]] = 1
        assert np.array_equal(mask.cpu().numpy()[b], m)


def test_recall_counts():
    g = torch.Generator().manual_seed(4)
    a = (torch.rand(5, 3000, generator=g) < 0.2).to(torch.uint8)
    m = (torch.rand(5, 3000, generator=g) < 0.3).to(torch.uint8)
    inter, ca, cb = lit.recall(a.cuda(), m.cuda())
    ri, rca, rcb = oracle.recall(a, m)
    assert inter.cpu().tolist() == ri.tolist() and ca.cpu().tolist() == rca.tolist() and cb.cpu().tolist() == rcb.tolist()


def test_topp_vote_probabilities_and_logits():
    g = torch.Generator().manual_seed(8)
    L_, B, N = 21, 2, 3000
    x = torch.randn(L_, B, N, generator=g, dtype=torch.float64) * 2
    p = torch.softmax(x, dim=-1)
    gold, gc, votes = lit.golden_topp_vote(p.cuda(), False, 0.6, 3)
    rg, rc, rv = oracle.topp_vote(p.numpy(), False, 0.6, 3)
    assert np.array_equal(votes.cpu().numpy(), rv) and np.array_equal(gold.cpu().numpy(), rg)
    assert gc.cpu().tolist() == rc.tolist()
    gold2, gc2, votes2 = lit.golden_topp_vote(x.cuda(), True, 0.6, 3)
    rg2, rc2, rv2 = oracle.topp_vote(x.numpy(), True, 0.6, 3)
    # the softmax exp of two libraries may differ in the last ulp: votes may only
    # differ where the oracle's running sum sits within 1e-12 of the cut
    assert np.array_equal(votes2.cpu().numpy(), rv2)
    assert np.array_equal(gold2.cpu().numpy(), rg2)


# ---------------------------------------------------------------- a8 gate


def test_lsa_gate_layers_or():
    B, N = 2, 2048
    keys = [W.layer_inputs(W.GATE64K, l, "cpu", B=B, N=N).idx.k_idx for l in W.GATE_LAYERS]
    layers = [W.gate_layer(W.GATE64K, l, kk, "cpu") for l, kk in zip(W.GATE_LAYERS, keys)]
    rg, rc = oracle.lsa_gate([Ly.as_dict() for Ly in layers], 0.5)
    dl = [synth.GateLayer(dev(Ly.h), dev(Ly.wq_a), dev(Ly.wq_b), dev(Ly.w_proj), dev(Ly.k)) for Ly in layers]
    gate, cnt = lit.lsa_gate(dl, 0.5)
    torch.cuda.synchronize()
    assert np.array_equal(gate.cpu().numpy(), rg)
    assert cnt.cpu().tolist() == rc.tolist()
    assert 0 < rc.sum() < B * N


# ---------------------------------------------------------------- the chained step


def test_tiny_end_to_end_step():
    L = W.layer_inputs(W.TINY, 0, "cpu")
    q_idx, w, k_idx = dev(L.idx.q_idx), dev(L.idx.w), dev(L.idx.k_idx)
    scores, hints = lit.idx_score(q_idx, w, k_idx)
    ids, cnt, mask = lit.topk_select(scores, 64, exact=(q_idx, w, k_idx), hints=hints)
    out, lse = lit.sparse_attn_decode(dev(L.q), kv_dev(L.kv), ids, cnt, 16, SCALE)
    gids, gcnt, gmask, _ = lit.golden_topk(dev(L.q), kv_dev(L.kv), 64, SCALE)
    inter, _, _ = lit.recall(mask, gmask)
    torch.cuda.synchronize()
    job = dict(q_idx=L.idx.q_idx[0].numpy(), w=L.idx.w[0].numpy(), k_idx=L.idx.k_idx[0].numpy(), k=64,
               q=L.q[0].numpy(), kv_dtype=oracle.F32, data=L.kv.data[0].numpy(), window=16, scale_f=SCALE)
    c, rids, rout, rlse = oracle.decode_queries([job])[0]
    assert c == 64 and ids.cpu()[0].tolist() == rids.tolist()
    assert_attn_close(out, rout[None])
    _, _, rgmask, _ = oracle.golden(L.q, L.kv, SCALE, 64)
    ri, _, _ = oracle.recall(oracle.topk(oracle.idx_score(L.idx.q_idx, L.idx.w, L.idx.k_idx), 64)[2], rgmask)
    assert inter.item() == ri[0]
