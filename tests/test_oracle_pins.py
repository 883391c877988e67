"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own loops: they use hand-worked fixtures,
closed forms, brute force, special cases that reduce to a library routine
(numpy / scipy / torch's float8 decoder) and invariants, chosen so that a
dropped term, a wrong sign or index, or a transposed operand fails one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from lightning_indexer_top_idx_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def bf16(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16)


# ---------------------------------------------------------------- FP8 codec


def test_fp8_e4m3_all_codes_match_torch_float8():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = np.array([oracle.fp8_e4m3(c) for c in range(256)])
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    assert (nan_ref == nan_got).all()
    assert set(np.flatnonzero(nan_got)) == {0x7F, 0xFF}
    np.testing.assert_array_equal(got[~nan_got], ref[~nan_ref])


def test_fp8_e4m3_spot_values_from_the_format_definition():
    assert oracle.fp8_e4m3(0x38) == 1.0  # exponent field 7 = bias
    assert oracle.fp8_e4m3(0x7E) == 448.0  # largest finite: 1.75 * 2^8
    assert oracle.fp8_e4m3(0x08) == 2.0**-6  # smallest normal
    assert oracle.fp8_e4m3(0x01) == 2.0**-9  # smallest subnormal
    assert oracle.fp8_e4m3(0xB8) == -1.0
    assert oracle.e8m0(127) == 1.0 and oracle.e8m0(128) == 2.0 and oracle.e8m0(120) == 2.0**-7
    assert math.isnan(oracle.e8m0(255))


def test_kv_dequant_fp8_matches_torch_float8_times_scale():
    g = torch.Generator().manual_seed(5)
    kv = synth.make_kv(1, 9, "fp8", g, "cpu")
    got = oracle.kv_dequant(kv, 0)
    codes = kv.data[0].view(torch.float8_e4m3fn).double()
    sc = torch.exp2(kv.scale[0, :, :7].double() - 127.0).repeat_interleave(64, dim=1)
    ref = torch.cat([codes * sc, kv.rope[0].double()], dim=1).numpy()
    np.testing.assert_array_equal(got, ref)


# ---------------------------------------------------------------- a1 score


def _tiny_from_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "score_tiny.json")))
    H = fx["H"]
    q = np.zeros((1, H, 128), np.float32)
    q[0, :, :2] = fx["q_dims01"]
    k = np.zeros((1, len(fx["k_dims01"]), 128), np.float32)
    k[0, :, :2] = fx["k_dims01"]
    w = np.array([fx["w"]], np.float32)
    return fx, q, w, k


def test_score_hand_worked_fixture():
    fx, q, w, k = _tiny_from_fixture()
    s = oracle.idx_score(q, w, k)
    assert s[0].tolist() == fx["scores"]
    ids, cnt, mask = oracle.topk(s, 2)
    assert ids[0].tolist() == fx["top2_ids"] and cnt[0] == 2 and mask[0].tolist() == [1, 1, 0]


def test_score_single_head_unit_query_selects_a_coordinate():
    # w = 1, q = e_j: s_n = max(0, k[n][j]) (catches a transposed q/k or a wrong dim index)
    k = rng.standard_normal((1, 40, 128)).astype(np.float32)
    for j in (0, 5, 127):
        q = np.zeros((1, 1, 128), np.float32)
        q[0, 0, j] = 1.0
        s = oracle.idx_score(q, np.ones((1, 1), np.float32), k)
        np.testing.assert_array_equal(s[0], np.maximum(k[0, :, j].astype(np.float64), 0.0))


def test_score_relu_identity_with_negated_queries():
    # relu(x) + relu(-x) = |x|: s(q) + s(-q) = sum_h w_h |q_h . k|
    q = rng.standard_normal((1, 6, 128)).astype(np.float32)
    k = rng.standard_normal((1, 50, 128)).astype(np.float32)
    w = rng.random((1, 6)).astype(np.float32)
    s = oracle.idx_score(q, w, k) + oracle.idx_score(-q, w, k)
    ref = (np.abs(q[0].astype(np.float64) @ k[0].astype(np.float64).T) * w[0, :, None]).sum(0)
    np.testing.assert_allclose(s[0], ref, rtol=1e-12, atol=1e-12)


def test_score_exact_grid_equals_integer_arithmetic():
    # q,k in {0,+-1/2,+-1}, w in {0,1/4,..,1}: 16*s is an integer computed exactly in int64
    g = torch.Generator().manual_seed(3)
    inp = synth.make_exact_grid(2, 300, 7, g, "cpu")
    s = oracle.idx_score(inp.q_idx, inp.w, inp.k_idx)
    q2 = (inp.q_idx.float().numpy() * 2).astype(np.int64)
    k2 = (inp.k_idx.float().numpy() * 2).astype(np.int64)
    w4 = (inp.w.numpy() * 4).astype(np.int64)
    for b in range(2):
        dots4 = q2[b] @ k2[b].T  # 4 * (q . k)
        ref16 = (w4[b][:, None] * np.maximum(dots4, 0)).sum(0)  # 16 * s
        np.testing.assert_array_equal(s[b] * 16.0, ref16.astype(np.float64))


def test_score_bf16_reads_the_same_values_as_fp32():
    q = bf16(rng.standard_normal((2, 3, 128)))
    k = bf16(rng.standard_normal((2, 20, 128)) / 11)
    w = torch.tensor(rng.random((2, 3)), dtype=torch.float32)
    np.testing.assert_array_equal(oracle.idx_score(q, w, k), oracle.idx_score(q.float(), w, k.float()))


def test_score_close_to_float64_library_matmul():
    q = rng.standard_normal((3, 64, 128)).astype(np.float32)
    k = (rng.standard_normal((3, 200, 128)) / 11).astype(np.float32)
    w = rng.random((3, 64)).astype(np.float32)
    s = oracle.idx_score(q, w, k)
    for b in range(3):
        ref = (w[b].astype(np.float64)[:, None] * np.maximum(q[b].astype(np.float64) @ k[b].T.astype(np.float64), 0)).sum(0)
        np.testing.assert_allclose(s[b], ref, rtol=1e-13)


def test_score_allowed_mask_gives_minus_inf():
    q = rng.standard_normal((1, 2, 128)).astype(np.float32)
    k = rng.standard_normal((1, 10, 128)).astype(np.float32)
    w = np.ones((1, 2), np.float32)
    allowed = np.array([[1, 0, 1, 1, 0, 0, 1, 1, 1, 0]], np.uint8)
    s = oracle.idx_score(q, w, k, allowed)
    full = oracle.idx_score(q, w, k)
    assert np.all(np.isneginf(s[0][allowed[0] == 0]))
    np.testing.assert_array_equal(s[0][allowed[0] == 1], full[0][allowed[0] == 1])


# ---------------------------------------------------------------- a2 top-k


def _brute_force_topk(s, k):
    """The unique set S with |S| = min(k, #finite) such that every member beats
    every finite non-member by (score desc, index asc); found by enumeration."""
    finite = [i for i in range(len(s)) if np.isfinite(s[i]) or s[i] == np.inf]
    m = min(k, len(finite))
    hits = []
    for S in itertools.combinations(finite, m):
        Sset = set(S)
        ok = all((s[i] > s[j]) or (s[i] == s[j] and i < j) for i in S for j in finite if j not in Sset)
        if ok:
            hits.append(S)
    assert len(hits) == 1
    return list(hits[0])


def test_topk_brute_force_small_with_ties():
    for trial in range(60):
        N = int(rng.integers(1, 11))
        s = rng.integers(0, 4, N).astype(np.float64)
        if trial % 3 == 0:
            s[rng.random(N) < 0.3] = -np.inf
        for k in range(1, N + 2):
            ids, cnt, mask = oracle.topk(s[None, :], k)
            ref = _brute_force_topk(s, k)
            assert cnt[0] == len(ref)
            assert ids[0, : cnt[0]].tolist() == ref
            assert (ids[0, cnt[0]:] == -1).all()
            assert mask[0].nonzero()[0].tolist() == ref


def test_topk_against_python_sorted_with_ties():
    for _ in range(20):
        N = int(rng.integers(20, 400))
        s = np.round(rng.standard_normal(N), 1)
        k = int(rng.integers(1, N))
        ids, cnt, _ = oracle.topk(s[None, :], k)
        ref = sorted(sorted(range(N), key=lambda i: (-s[i], i))[:k])
        assert ids[0].tolist() == ref and cnt[0] == k


def test_topk_nan_never_selected_and_k_beyond_n():
    s = np.array([[1.0, np.nan, 3.0, -np.inf, 2.0]])
    ids, cnt, mask = oracle.topk(s, 10)
    assert cnt[0] == 3 and ids[0, :3].tolist() == [0, 2, 4] and (ids[0, 3:] == -1).all()
    assert mask[0].tolist() == [1, 0, 1, 0, 1]


def test_topk_permutation_equivariance_without_ties():
    s = rng.standard_normal(300)
    perm = rng.permutation(300)
    a = set(oracle.topk(s[None, :], 40)[0][0].tolist())
    b = set(oracle.topk(s[perm][None, :], 40)[0][0].tolist())
    assert {int(perm[i]) for i in b} == a


# ---------------------------------------------------------------- a3 attention


def _dense_attention(qv, rows, scale):
    x = scale * (qv.astype(np.float64) @ rows.astype(np.float64).T)
    p = scipy.special.softmax(x, axis=-1)
    return p @ rows.astype(np.float64), scipy.special.logsumexp(x, axis=-1)


def _kv(data):
    return oracle.KV(oracle.F32, data.astype(np.float32))


def test_attention_full_selection_equals_dense_softmax():
    N, Hq = 37, 3
    kv = rng.standard_normal((1, N, 512)).astype(np.float32)
    q = rng.standard_normal((1, Hq, 512)).astype(np.float32)
    ids = np.arange(N, dtype=np.int32)[None, :]
    out, lse = oracle.attend(q, _kv(kv), ids, np.array([N]), window=0, scale=0.125)
    ref, rl = _dense_attention(q[0], kv[0], float(np.float32(0.125)))
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[0], rl, rtol=1e-12)
    out2, _ = oracle.attend(q, _kv(kv), None, None, window=0, scale=0.125)  # ids=None: every row
    np.testing.assert_array_equal(out2, out)


def test_attention_single_row_returns_the_row():
    kv = rng.standard_normal((1, 20, 512)).astype(np.float32)
    q = rng.standard_normal((1, 2, 512)).astype(np.float32)
    out, lse = oracle.attend(q, _kv(kv), np.array([[7, -1, -1]], np.int32), np.array([1]), window=0, scale=0.3)
    np.testing.assert_array_equal(out[0, 0], kv[0, 7].astype(np.float64))
    np.testing.assert_allclose(lse[0, 0], float(np.float32(0.3)) * float(q[0, 0].astype(np.float64) @ kv[0, 7]), rtol=1e-12)


def test_attention_window_union_counts_each_row_once():
    N = 30
    kv = rng.standard_normal((1, N, 512)).astype(np.float32)
    q = rng.standard_normal((1, 2, 512)).astype(np.float32)
    sel = np.array([[3, 11, 27, 29]], np.int32)  # 27, 29 also in the window of 5
    out, lse = oracle.attend(q, _kv(kv), sel, np.array([4]), window=5, scale=0.05)
    rows = sorted({3, 11, 27, 29} | set(range(25, 30)))
    ref, rl = _dense_attention(q[0], kv[0, rows], float(np.float32(0.05)))
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[0], rl, rtol=1e-12)


def test_attention_zero_query_is_the_mean_row():
    kv = rng.standard_normal((1, 12, 512)).astype(np.float32)
    q = np.zeros((1, 1, 512), np.float32)
    out, lse = oracle.attend(q, _kv(kv), np.array([[0, 4, 9]], np.int32), np.array([3]), window=2, scale=0.5)
    ref = kv[0, [0, 4, 9, 10, 11]].astype(np.float64).mean(0)
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], math.log(5.0), rtol=1e-14)


def test_attention_split_lse_combine_invariance():
    N = 40
    kv = rng.standard_normal((1, N, 512)).astype(np.float32)
    q = rng.standard_normal((1, 2, 512)).astype(np.float32)
    A = np.array([[1, 5, 8, 20]], np.int32)
    Bs = np.array([[2, 9, 33]], np.int32)
    AB = np.array([[1, 2, 5, 8, 9, 20, 33]], np.int32)
    oa, la = oracle.attend(q, _kv(kv), A, [4], 0, 0.07)
    ob, lb = oracle.attend(q, _kv(kv), Bs, [3], 0, 0.07)
    oab, lab = oracle.attend(q, _kv(kv), AB, [7], 0, 0.07)
    M = np.maximum(la, lb)
    wa, wb = np.exp(la - M), np.exp(lb - M)
    comb = (oa * wa[..., None] + ob * wb[..., None]) / (wa + wb)[..., None]
    np.testing.assert_allclose(oab, comb, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lab, M + np.log(wa + wb), rtol=1e-13)


def test_attention_empty_selection():
    kv = rng.standard_normal((1, 5, 512)).astype(np.float32)
    q = rng.standard_normal((1, 2, 512)).astype(np.float32)
    out, lse = oracle.attend(q, _kv(kv), np.full((1, 3), -1, np.int32), np.array([0]), window=0, scale=0.1)
    assert (out == 0).all() and np.isneginf(lse).all()


def test_attention_fp8_rows_equal_decoded_rows():
    g = torch.Generator().manual_seed(11)
    kv = synth.make_kv(1, 25, "fp8", g, "cpu")
    q = synth.make_q(1, 2, "bf16", g, "cpu")
    codes = kv.data[0].view(torch.float8_e4m3fn).double()
    sc = torch.exp2(kv.scale[0, :, :7].double() - 127.0).repeat_interleave(64, dim=1)
    dense = torch.cat([codes * sc, kv.rope[0].double()], dim=1).numpy()
    ids = np.array([[0, 3, 4, 17]], np.int32)
    out, lse = oracle.attend(q, kv, ids, [4], 3, 0.044)
    rows = [0, 3, 4, 17, 22, 23, 24]
    ref, rl = _dense_attention(q[0].double().numpy(), dense[rows], float(np.float32(0.044)))
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- a6 golden


def test_golden_single_head_is_the_library_softmax():
    N = 60
    kv = rng.standard_normal((1, N, 512)).astype(np.float32)
    q = rng.standard_normal((1, 1, 512)).astype(np.float32)
    ids, cnt, mask, pbar = oracle.golden(q, _kv(kv), 0.044, 10)
    ref = scipy.special.softmax(float(np.float32(0.044)) * (q[0, 0].astype(np.float64) @ kv[0].astype(np.float64).T))
    np.testing.assert_allclose(pbar[0], ref, rtol=1e-12)
    assert ids[0].tolist() == sorted(np.argsort(-ref, kind="stable")[:10].tolist())


def test_golden_head_average_and_normalisation():
    N, Hq = 50, 4
    kv = rng.standard_normal((1, N, 512)).astype(np.float32)
    q = rng.standard_normal((1, Hq, 512)).astype(np.float32)
    _, _, _, pbar = oracle.golden(q, _kv(kv), 0.044, 5)
    x = float(np.float32(0.044)) * (q[0].astype(np.float64) @ kv[0].astype(np.float64).T)
    ref = scipy.special.softmax(x, axis=-1).mean(0)
    np.testing.assert_allclose(pbar[0], ref, rtol=1e-12)
    assert abs(pbar[0].sum() - 1.0) < 1e-12


def test_golden_uniform_attention_picks_first_k():
    kv = rng.standard_normal((1, 30, 512)).astype(np.float32)
    q = np.zeros((1, 3, 512), np.float32)
    ids, cnt, _, pbar = oracle.golden(q, _kv(kv), 0.1, 7)
    np.testing.assert_allclose(pbar[0], 1 / 30, rtol=1e-14)
    assert ids[0].tolist() == list(range(7))


# ---------------------------------------------------------------- a7 recall


def test_recall_counts_and_bounds():
    N, k = 200, 60
    a = np.zeros((3, N), np.uint8)
    m = np.zeros((3, N), np.uint8)
    for b in range(3):
        a[b, rng.choice(N, k, replace=False)] = 1
        m[b, rng.choice(N, k, replace=False)] = 1
    inter, ca, cb = oracle.recall(a, m)
    assert (ca == k).all() and (cb == k).all()
    np.testing.assert_array_equal(inter, (a & m).sum(1))
    assert (inter >= max(0, 2 * k - N)).all()
    i2, _, _ = oracle.recall(a, a)
    assert (i2 == k).all()


def test_recall_random_selector_expectation_is_k_over_n():
    # hypergeometric mean k/N; the pages' random baselines are this ratio
    N, k, T = 800, 512, 400
    gold = np.zeros((T, N), np.uint8)
    sel = np.zeros((T, N), np.uint8)
    for t in range(T):
        gold[t, rng.choice(N, k, replace=False)] = 1
        sel[t, rng.choice(N, k, replace=False)] = 1
    inter, _, _ = oracle.recall(sel, gold)
    mean = inter.mean() / k
    sd = math.sqrt(k * (k / N) * (1 - k / N) * (N - k) / (N - 1)) / k / math.sqrt(T)
    assert abs(mean - k / N) < 5 * sd
    # the pages' baselines: 512 kept of ~889 chunks -> 0.576 (Act 1), of ~764 -> 0.67 (Act 3)
    assert round(512 / 889, 3) == 0.576 and round(512 / 764, 2) == 0.67


# ---------------------------------------------------------------- a8 gate


def _gate_inputs(B=2, N=40, H=3, d_model=32, rank=16, seed=0):
    g = torch.Generator().manual_seed(seed)
    k = (torch.randn(B, N, 128, generator=g) / 11).to(torch.bfloat16)
    h, wa, wb, wp = synth.make_gate_weights(B, H, d_model, rank, g, "cpu")
    return dict(h=h, wq_a=wa, wq_b=wb, w_proj=wp, k=k)


def test_gate_matches_library_matmuls_and_sigmoid():
    L = _gate_inputs()
    gate, cnt, zs = oracle.lsa_gate([L], 0.5, return_z=True)
    h = L["h"].double().numpy()
    wa, wb, wp = (L[n].double().numpy() for n in ("wq_a", "wq_b", "w_proj"))
    k = L["k"].double().numpy()
    for b in range(2):
        u = wa @ h[b]
        q = (wb @ u).reshape(-1, 128)
        w = wp @ h[b]
        z = (w[:, None] * np.maximum(q @ k[b].T, 0)).sum(0)
        np.testing.assert_allclose(zs[0][b], z, rtol=1e-10, atol=1e-12)
        sig = scipy.special.expit(zs[0][b])
        assert (gate[b] == (sig >= 0.5)).all()
    np.testing.assert_array_equal(cnt, gate.sum(1))


def test_gate_zero_weights_keep_everything_and_or_across_layers():
    L0 = _gate_inputs(seed=1)
    L0["w_proj"] = torch.zeros_like(L0["w_proj"])  # w = 0 -> z = 0 -> sigmoid = 0.5 -> kept
    gate, cnt = oracle.lsa_gate([L0])
    assert gate.all() and (cnt == 40).all()
    L1, L2 = _gate_inputs(seed=2), _gate_inputs(seed=3)
    g1, _ = oracle.lsa_gate([L1])
    g2, _ = oracle.lsa_gate([L2])
    g12, c12 = oracle.lsa_gate([L1, L2])
    np.testing.assert_array_equal(g12, g1 | g2)
    assert 0 < c12.sum() < g12.size  # non-trivial


def test_gate_threshold_maps_to_logit():
    L = _gate_inputs(seed=4)
    gate, _, zs = oracle.lsa_gate([L], 0.7, return_z=True)
    assert (gate == (scipy.special.expit(zs[0]) >= 0.7)).all()


# ---------------------------------------------------------------- a9 top-p + vote


def test_topp_uniform_takes_first_ceil_of_p_times_n():
    N = 8  # p = 1/8 exactly: running sums are exact
    x = np.full((1, 1, N), 1 / N)
    gold, cnt, votes = oracle.topp_vote(x, False, 0.6, 1)
    assert gold[0].tolist() == [1] * 5 + [0] * 3  # ceil(0.6 * 8) = 5, ties by index


def test_topp_one_hot_and_identical_layers():
    N = 20
    x = np.zeros((21, 1, N))
    x[:, 0, 13] = 1.0
    gold, cnt, votes = oracle.topp_vote(x, False, 0.6, 3)
    assert gold[0].nonzero()[0].tolist() == [13] and cnt[0] == 1 and votes[0, 13] == 21


def test_topp_vote_threshold_counts_layers():
    N = 10
    x = np.zeros((5, 1, N))
    # layer l puts all mass on entries {l, l+1}: top-p 0.6 keeps the larger, index l
    for l in range(5):
        x[l, 0, l] = 0.7
        x[l, 0, (l + 1) % N] = 0.3
    x[3, 0, 0] = 0.9  # layer 3: mass 0.9 on entry 0, 0.7 on entry 3 -> top-p keeps {0} (0.9 >= 0.6)
    x[3, 0, 3] = 0.0
    x[3, 0, 4] = 0.1
    gold, cnt, votes = oracle.topp_vote(x, False, 0.6, 2)
    assert votes[0].tolist()[:5] == [2, 1, 1, 0, 1]
    assert gold[0].nonzero()[0].tolist() == [0]


def test_topp_logits_path_uses_softmax():
    N = 30
    x = rng.standard_normal((2, 1, N)) * 3
    gold, cnt, votes = oracle.topp_vote(x, True, 0.6, 1)
    for l in range(2):
        p = scipy.special.softmax(x[l, 0])
        order = sorted(range(N), key=lambda i: (-p[i], i))
        run, keep = 0.0, []
        for i in order:
            keep.append(i)
            run += p[i]
            if run >= 0.6:
                break
        for i in keep:
            assert votes[0, i] >= 1


# ---------------------------------------------------------------- counts and the KV byte model


def test_entry_counts_from_the_pages():
    from lightning_indexer_top_idx_amd import workloads as W

    assert W.csa_entries(65536) == 16384 and W.hca_entries(65536) == 512  # ~16K / ~512 at 64K
    assert round(512 / 16384 * 100, 1) == 3.1  # top-512 is ~3% of the CSA entries
    assert W.csa_entries(500000) == 125000 and W.hca_entries(500000) == 3907  # ceil, not floor
    assert len(W.CSA_LAYERS) == 21 and W.CSA_LAYERS[0] == 2 and W.CSA_LAYERS[-1] == 42


def test_kv_cache_871_mib_reconstruction():
    # 21 CSA layers x 16384 entries x (512 + 128) fp32, 20 HCA layers x 512 x 512 fp32,
    # 43 windows x 128 x 512 fp32 = 870.75 MiB, the page's "~871 MiB" at 64K
    csa = 21 * 16384 * (512 + 128) * 4
    hca = 20 * 512 * 512 * 4
    swa = 43 * 128 * 512 * 4
    assert (csa + hca + swa) / 2**20 == 870.75


# ---------------------------------------------------------------- cold-pool plan


def test_pool_plan_hand_worked_cases():
    # nothing gated: only the window (the last W entries) is kept, right-aligned
    m, c, a = oracle.pool_plan(np.zeros((1, 10), np.uint8), 3, 5)
    assert m.tolist() == [[-1, -1, 7, 8, 9]] and c.tolist() == [3] and a.tolist() == [[0, 0, 0, 0, 0]]
    # everything gated: every entry, all allowed
    m, c, a = oracle.pool_plan(np.ones((1, 6), np.uint8), 2, 8)
    assert m.tolist() == [[-1, -1, 0, 1, 2, 3, 4, 5]] and c.tolist() == [6]
    assert a.tolist() == [[0, 0, 1, 1, 1, 1, 1, 1]]
    # gated {0, 3, 7}, window {6, 7}: union {0, 3, 6, 7} fills C = 4 exactly;
    # 6 is kept for the window only, so it is not a scoring candidate
    g = np.array([[1, 0, 0, 1, 0, 0, 0, 1]], np.uint8)
    m, c, a = oracle.pool_plan(g, 2, 4)
    assert m.tolist() == [[0, 3, 6, 7]] and c.tolist() == [4] and a.tolist() == [[1, 1, 0, 1]]
    # one slot short: nothing fits, the count says how many were needed
    m, c, a = oracle.pool_plan(g, 2, 3)
    assert m.tolist() == [[-1, -1, -1]] and c.tolist() == [4] and a.sum() == 0
    # a window longer than the sequence keeps the whole sequence
    m, c, _ = oracle.pool_plan(np.zeros((1, 3), np.uint8), 16, 3)
    assert m.tolist() == [[0, 1, 2]] and c.tolist() == [3]
    # no window: the gated entries alone
    m, c, _ = oracle.pool_plan(g, 0, 5)
    assert m.tolist() == [[-1, -1, 0, 3, 7]] and c.tolist() == [3]


def test_pool_plan_invariants_on_random_gates():
    g = (rng.random((5, 300)) < np.array([0.0, 0.05, 0.3, 0.9, 1.0])[:, None]).astype(np.uint8)
    m, c, a = oracle.pool_plan(g, 32, 300)
    for b in range(5):
        kept = m[b][m[b] >= 0]
        assert len(kept) == c[b] and (np.diff(kept) > 0).all()            # ascending, distinct
        assert (m[b][: 300 - c[b]] == -1).all()                             # right-aligned
        assert set(range(268, 300)) <= set(kept.tolist())                   # the window is in
        assert set(np.flatnonzero(g[b]).tolist()) <= set(kept.tolist())     # every gated entry is in
        assert (a[b][300 - c[b]:] == g[b][kept]).all() and a[b][: 300 - c[b]].sum() == 0
        assert c[b] == len(set(np.flatnonzero(g[b]).tolist()) | set(range(268, 300)))


# ---------------------------------------------------------------- multi-query indexer

def _unit_keys(B, N):
    # key n of sequence b = (b + 1) * e_(n mod 128): the head dot products read
    # one coordinate of the query, scaled by the sequence's number
    k = np.zeros((B, N, 128), np.float32)
    for b in range(B):
        for n in range(N):
            k[b, n, n % 128] = b + 1
    return k


def test_mq_score_closed_form_rows_keys_weights_and_lengths():
    # two heads per query: head 0 = a, head 1 = -a, weights (r+1, 10(r+1)) for
    # row r = b*Q + j. Against key (b+1) e_i the score is
    #   (b+1)(r+1) * (a_i if a_i > 0 else -10 a_i)
    # (ReLU keeps exactly one head), and -inf from lengths[b][j] on.
    B, Q, N = 2, 3, 150
    a = rng.integers(-4, 5, size=(B, Q, 128)).astype(np.float32) / 4
    q = np.stack([a, -a], axis=2)  # [B,Q,2,128]
    r = np.arange(B * Q, dtype=np.float32).reshape(B, Q) + 1
    w = np.stack([r, 10 * r], axis=2)
    lengths = np.array([[150, 7, 0], [129, 1, 200]], np.int32)
    s = oracle.idx_score_mq(q, w, _unit_keys(B, N), lengths)
    for b in range(B):
        for j in range(Q):
            for n in range(N):
                ai = a[b, j, n % 128]
                want = (b + 1) * r[b, j] * (ai if ai > 0 else -10 * ai)
                if n >= min(lengths[b, j], N):
                    want = -np.inf
                assert s[b, j, n] == want, (b, j, n)


def test_mq_score_allowed_is_shared_by_the_queries_of_a_sequence():
    B, Q, N = 2, 2, 40
    a = np.abs(rng.standard_normal((B, Q, 1, 128))).astype(np.float32) + 0.5
    w = np.ones((B, Q, 1), np.float32)
    allowed = np.zeros((B, N), np.uint8)
    allowed[0, ::3] = 1
    allowed[1, 5:9] = 1
    s = oracle.idx_score_mq(a, w, _unit_keys(B, N), None, allowed)
    for b in range(B):
        for j in range(Q):
            assert (np.isfinite(s[b, j]) == (allowed[b] == 1)).all()
            vis = np.flatnonzero(allowed[b])
            assert np.array_equal(s[b, j, vis], (b + 1) * a[b, j, 0, vis % 128])


def test_mq_topk_rows_select_among_visible_entries():
    # query j sees j+2 entries with scores 1..; its top-3 are the best of those
    B, Q, N = 1, 4, 12
    s = np.full((B, Q, N), 0.0)
    s[0] = np.arange(N)[None, :] % 5 + 1.0
    for j in range(Q):
        s[0, j, j + 2:] = -np.inf
    ids, cnt, mask = oracle.topk_mq(s, 3)
    for j in range(Q):
        vis = list(range(j + 2))
        want = sorted(sorted(vis, key=lambda n: (-s[0, j, n], n))[:3])
        assert cnt[0, j] == min(3, j + 2)
        assert ids[0, j, : cnt[0, j]].tolist() == want and (ids[0, j, cnt[0, j]:] == -1).all()
        assert mask[0, j].sum() == cnt[0, j]


# ---------------------------------------------------------------- lookahead golden

def test_lookahead_sharp_queries_give_known_sets_union_and_hits():
    # rows are 4 * e_i (i < 512); step t's query points at rows a_t and c_t on
    # every head with a large weight, so its top-2 is {a_t, c_t} exactly; the
    # union is the set of all a_t, c_t and hits counts repeats across steps
    B, T, Hq, N = 2, 5, 3, 40
    kv = np.zeros((B, N, 512), np.float32)
    for n in range(N):
        kv[:, n, n] = 4.0
    targets = [[(3, 7), (7, 9), (3, 7), (0, 39), (12, 9)], [(1, 2), (1, 2), (1, 2), (1, 2), (5, 6)]]
    q = np.zeros((B, T, Hq, 512), np.float32)
    for b in range(B):
        for t, (a, c) in enumerate(targets[b]):
            q[b, t, :, a] = 8.0
            q[b, t, :, c] = 8.0
    ids, hits, um, uc, pbar = oracle.lookahead_golden(q, _kv(kv), 0.5, 2)
    for b in range(B):
        want_hits = np.zeros(N, int)
        for t, (a, c) in enumerate(targets[b]):
            assert ids[b, t].tolist() == sorted([a, c])
            want_hits[a] += 1
            want_hits[c] += 1
        assert hits[b].tolist() == want_hits.tolist()
        assert um[b].tolist() == (want_hits > 0).astype(int).tolist()
        assert uc[b] == len({x for ac in targets[b] for x in ac})
    # two targets share the mass: each gets (1 - 38 eps) / 2 with eps = e^-16 / (2 + 38 e^-16)
    e = math.exp(-16.0)
    np.testing.assert_allclose(pbar[0, 0, 3], 1.0 / (2 + 38 * e), rtol=1e-12)
    np.testing.assert_allclose(pbar[0, 0, 5], e / (2 + 38 * e), rtol=1e-12)


def test_lookahead_one_step_is_the_current_golden_and_union_grows_with_the_horizon():
    B, T, Hq, N, k = 1, 6, 4, 80, 9
    kv = rng.standard_normal((B, N, 512)).astype(np.float32)
    q = rng.standard_normal((B, T, Hq, 512)).astype(np.float32)
    ids, hits, um, uc, pbar = oracle.lookahead_golden(q, _kv(kv), 0.044, k)
    # each step: the library softmax's head average, its top-k
    for t in range(T):
        x = float(np.float32(0.044)) * (q[0, t].astype(np.float64) @ kv[0].astype(np.float64).T)
        ref = scipy.special.softmax(x, axis=-1).mean(0)
        np.testing.assert_allclose(pbar[0, t], ref, rtol=1e-12)
        assert ids[0, t].tolist() == sorted(np.argsort(-ref, kind="stable")[:k].tolist())
    assert hits.sum() == T * k and k <= uc[0] <= min(N, T * k)
    # the union of a prefix of the horizon is contained in the union of the whole horizon
    _, h3, _, u3, _ = oracle.lookahead_golden(q[:, :3], _kv(kv), 0.044, k)
    assert (h3 <= hits).all() and u3[0] <= uc[0]


# ---------------------------------------------------------------- the chained step


def _decode_tiny_job(k, window):
    """Inputs of tests/golden/decode_tiny.json: the score_tiny indexer, three
    marker rows and two hand-chosen attention heads plus one random head."""
    _, q, w, kk = _tiny_from_fixture()
    rows = np.zeros((3, 512), np.float32)
    for r in range(3):
        rows[r, 0], rows[r, 1], rows[r, 2 + r] = r, 1.0, 1.0
    qa = np.zeros((3, 512), np.float32)
    qa[1, 0] = 1.0
    qa[2] = rng.standard_normal(512).astype(np.float32)
    return {"q_idx": q[0], "w": w[0], "k_idx": kk[0], "k": k, "q": qa, "kv_dtype": oracle.F32, "data": rows,
            "window": window, "scale_f": math.log(2.0)}, rows, qa


def test_decode_query_hand_worked_chain():
    fx = json.load(open(os.path.join(GOLDEN, "decode_tiny.json")))
    ln = {"ln 2": math.log(2), "ln 3": math.log(3), "ln 6": math.log(6), "ln 7": math.log(7)}
    frac = {"10/7": 10 / 7, "5/3": 5 / 3, "2/3": 2 / 3}
    for case in fx["cases"]:
        job, rows, qa = _decode_tiny_job(case["k"], case["window"])
        (c, ids, out, lse), = oracle.decode_queries([job])
        assert c == case["count"], case["work"]
        assert ids.tolist() == case["ids"], case["work"]
        # head 0: uniform weights over R; head 1: weights proportional to 2^r
        np.testing.assert_allclose(out[0, 2:5], case["head0_weights"], rtol=0, atol=1e-15)
        w1 = np.array(case["head1_weights_unnormalised"], np.float64)
        np.testing.assert_allclose(out[1, 2:5], w1 / w1.sum(), rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(out[1, 0], frac[case["head1_dim0"]], rtol=1e-14)
        np.testing.assert_allclose(out[:2, 1], 1.0, rtol=1e-15)
        np.testing.assert_allclose(lse[:2], [ln[s] for s in case["lse"]], rtol=1e-14)
        # every head against the library softmax over the hand-listed rows
        x = math.log(2.0) * (qa.astype(np.float64) @ rows[case["rows"]].astype(np.float64).T)
        ref = scipy.special.softmax(x, axis=-1) @ rows[case["rows"]].astype(np.float64)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse, scipy.special.logsumexp(x, axis=-1), rtol=1e-13)


def test_decode_query_equals_the_three_steps():
    # the chain's wiring: the same count, ids and attention as score -> topk ->
    # attend called one by one, for counts below and at k and windows past N
    g = torch.Generator().manual_seed(21)
    sc = float(np.float32(1.0 / math.sqrt(512)))  # the attention call takes its scale as fp32
    for N, k, window in ((50, 8, 5), (50, 80, 7), (30, 10, 40)):
        idx = synth.make_indexer(1, N, 4, "bf16", g, "cpu", planted_count=3)
        kv = synth.make_kv(1, N, "bf16", g, "cpu")
        q = synth.make_q(1, 3, "bf16", g, "cpu")
        job = {"q_idx": oracle.np_of(idx.q_idx)[0], "w": oracle.np_of(idx.w)[0], "k_idx": oracle.np_of(idx.k_idx)[0],
               "k": k, "q": oracle.np_of(q)[0], "kv_dtype": oracle.BF16, "data": oracle.np_of(kv.data)[0],
               "window": window, "scale_f": sc}
        (c, ids, out, lse), = oracle.decode_queries([job])
        s = oracle.idx_score(idx.q_idx, idx.w, idx.k_idx)
        rids, rc, _ = oracle.topk(s, k)
        rout, rlse = oracle.attend(q, kv, rids, rc, window, sc)
        assert c == rc[0] == min(k, N)
        np.testing.assert_array_equal(ids, rids[0])
        np.testing.assert_array_equal(out, rout[0])
        np.testing.assert_array_equal(lse, rlse[0])
