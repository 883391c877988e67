"""The LSA cold-pool fetch on the GPU: plan, gather, and the decode step on the
compact pool, against the oracle and against the same step on the resident
arrays with the gate as the allowed set."""
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


def test_pool_plan_matches_oracle():
    g = torch.Generator().manual_seed(11)
    B, N = 4, 5003
    frac = torch.tensor([0.0, 0.1, 0.5, 1.0])[:, None]
    gate = (torch.rand(B, N, generator=g) < frac).to(torch.uint8)
    for window, C in ((128, N), (128, 2600), (0, 700), (5003, N)):
        print(f"case window={window} C={C}", flush=True)
        m, cnt, ac = lit.pool_plan(gate.cuda(), window, C)
        torch.cuda.synchronize()
        rm, rc, rac = oracle.pool_plan(gate.numpy(), window, C)
        assert np.array_equal(cnt.cpu().numpy(), rc)
        assert np.array_equal(m.cpu().numpy(), rm)
        assert np.array_equal(ac.cpu().numpy(), rac)


@pytest.mark.parametrize("where", ["device", "pinned"])
def test_pool_gather_rows_bit_exact(where):
    g = torch.Generator().manual_seed(12)
    B, R, C = 3, 700, 500
    # row widths that take 16-, 8- and 4-byte pieces
    for tail, dt in (((128,), torch.bfloat16), ((448,), torch.uint8), ((8,), torch.uint8), ((3,), torch.float32)):
        print(f"case {where} row {tail} {dt}", flush=True)
        src = torch.randint(0, 255, (B, R) + tail, generator=g, dtype=torch.uint8)
        src = src.view(dt) if dt.itemsize == 1 else torch.randn((B, R) + tail, generator=g).to(dt)
        m = torch.randint(-1, R, (B, C), generator=g, dtype=torch.int32)
        m[:, :7] = -1
        ref = torch.zeros((B, C) + tail, dtype=dt)
        for b in range(B):
            ok = m[b] >= 0
            ref[b][ok] = src[b][m[b][ok].long()]
        s = src.cuda() if where == "device" else src.pin_memory()
        dst = lit.pool_gather(s, m.cuda())
        torch.cuda.synchronize()
        assert torch.equal(dst.cpu().view(torch.uint8), ref.view(torch.uint8))


def test_pool_gather_refuses_pageable_host_memory():
    src = np.zeros((2, 10, 16), np.uint8)  # pageable
    m = torch.zeros(2, 4, dtype=torch.int32, device="cuda")
    dst = torch.empty(2, 4, 16, dtype=torch.uint8, device="cuda")
    st = lit.load().lit_pool_gather(src.ctypes.data, 10, 16, 2, m.data_ptr(), 4, dst.data_ptr(), None)
    assert st == 7 and "page-locked" in lit.last_error()
    with pytest.raises(ValueError):
        lit.pool_gather(torch.zeros(2, 10, 16, dtype=torch.uint8), m)


def test_offload_step_equals_resident_gated_step():
    # the gate64k workload (FP8 rows, top-1024, gate at layers 10/12/20) at 4
    # sequences: the cold pool lives in pinned host memory and only the kept
    # entries are fetched; score -> select -> attend on the compact pool must
    # give the resident gated step's ids and, bit for bit, its outputs
    wl = W.GATE64K
    B = 4
    print("case gate64k offload B=4", flush=True)
    keys = [W.layer_inputs(wl, l, "cuda", B=B).idx.k_idx for l in W.GATE_LAYERS]
    gl = [W.gate_layer(wl, l, kk, "cuda") for l, kk in zip(W.GATE_LAYERS, keys)]
    gate, gcnt = lit.lsa_gate(gl, 0.5)
    L = W.layer_inputs(wl, 10, "cuda", B=B)
    q, w, kk = L.idx.q_idx, L.idx.w, L.idx.k_idx
    s, h = lit.idx_score(q, w, kk, gate)
    ids, cnt, _ = lit.topk_select(s, wl.k, exact=(q, w, kk), hints=h)
    out, lse = lit.sparse_attn_decode(L.q, L.kv, ids, cnt, wl.window, SCALE)
    # the cold pool, and the compact pool sized to the largest kept set
    _, pc, _ = lit.pool_plan(gate, wl.window, wl.N)
    need = min(wl.N, int((pc.max().item() + 63) // 64 * 64))
    m, pc, ac = lit.pool_plan(gate, wl.window, need)
    assert (pc.cpu() <= need).all()
    host = [t.cpu().pin_memory() for t in (kk, L.kv.data, L.kv.rope, L.kv.scale)]
    kc, dc, rc, sc = (lit.pool_gather(t, m) for t in host)
    s_c, h_c = lit.idx_score(q, w, kc, ac)
    ids_c, cnt_c, _ = lit.topk_select(s_c, wl.k, exact=(q, w, kc), hints=h_c)
    out_c, lse_c = lit.sparse_attn_decode(L.q, synth.KVRows("fp8", dc, rc, sc), ids_c, cnt_c, wl.window, SCALE)
    ids_o = lit.pool_remap_ids(ids_c, cnt_c, m)
    torch.cuda.synchronize()
    assert torch.equal(cnt_c.cpu(), cnt.cpu()) and torch.equal(cnt.cpu(), gcnt.clamp(max=wl.k).cpu())
    assert torch.equal(ids_o.cpu(), ids.cpu())
    assert torch.equal(out_c.cpu(), out.cpu()) and torch.equal(lse_c.cpu(), lse.cpu())
    # sequence 0 against the oracle (gated selection, then attention)
    one = lambda x: x[:1].cpu()
    s64 = oracle.idx_score(one(q), one(w), one(kk), gate[:1].cpu().numpy())
    rids, rcnt, _ = oracle.topk(s64, wl.k)
    assert np.array_equal(ids_o[:1].cpu().numpy(), rids)
    kv0 = synth.KVRows("fp8", one(L.kv.data), one(L.kv.rope), one(L.kv.scale))
    ref, _ = oracle.attend(one(L.q), kv0, rids, rcnt, wl.window, SCALE)
    err = np.abs(out_c[:1].double().cpu().numpy() - ref).max(-1)
    assert (err <= 2e-2 * np.abs(ref).max(-1)).all()
