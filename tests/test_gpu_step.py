"""One token's decode step over all 43 attention layers (2 SWA + 21 CSA + 20
HCA, in layer order) on the GPU, eager and replayed from a HIP graph, each
layer's output against the oracle."""
import math

import numpy as np
import pytest
import torch

import lightning_indexer_top_idx_amd as lit
import oracle
from lightning_indexer_top_idx_amd import workloads as W
from lightning_indexer_top_idx_amd.step import CsaLayer, DenseLayer, TokenSchedule, layer_kind

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(512)
ATTN_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lit.load()
    oracle.build()


def _schedule(T, B):
    """The layers of one step at context T: CSA over ceil(T/4) entries (the
    64K workload's heads, top-512, window 128), HCA over ceil(T/128) rows, SWA
    over the last 128 rows."""
    wl = W.CTX64K_B
    n_csa, n_hca = -(-T // 4), -(-T // 128)
    layers = []
    for l in range(43):
        kind = layer_kind(l)
        if kind == "csa":
            L = W.layer_inputs(wl, l, "cuda", B=B, N=n_csa)
            layers.append(CsaLayer(L, wl.k, wl.window, SCALE, "cuda"))
        else:
            rows = 128 if kind == "swa" else n_hca
            layers.append(DenseLayer(*W.dense_layer_inputs(B, rows, wl.Hq, l, "cuda"), SCALE, "cuda"))
    return TokenSchedule(layers)


def _check_layer(l, Ly):
    one = lambda x: x.cpu()
    if layer_kind(l) == "csa":
        q, w, k = Ly.L.idx.q_idx, Ly.L.idx.w, Ly.L.idx.k_idx
        s64 = oracle.idx_score(one(q), one(w), one(k))
        rids, rcnt, _ = oracle.topk(s64, Ly.k)
        assert np.array_equal(Ly.count.cpu().numpy(), rcnt), f"layer {l}: counts"
        assert np.array_equal(Ly.ids.cpu().numpy(), rids), f"layer {l}: ids"
        ref, rlse = oracle.attend(one(Ly.L.q), Ly.L.kv, rids, rcnt, Ly.window, SCALE)
    else:
        ref, rlse = oracle.attend(one(Ly.q), Ly.kv, None, None, 0, SCALE)
    out = Ly.out.double().cpu().numpy()
    err = np.abs(out - ref).max(-1)
    assert (err <= ATTN_TOL * np.abs(ref).max(-1)).all(), f"layer {l} ({layer_kind(l)}): attention"
    np.testing.assert_allclose(Ly.lse.double().cpu().numpy(), rlse, atol=2e-3, rtol=0, err_msg=f"layer {l}")


def test_token_step_matches_oracle_layer_by_layer():
    # 8K context: 2048 CSA entries (several top-k tiles), 64 HCA rows, 128 SWA rows
    print("case token step T=8192 B=2", flush=True)
    sched = _schedule(8192, 2)
    s = torch.cuda.current_stream().cuda_stream
    sched.run(s)
    torch.cuda.synchronize()
    for l, Ly in enumerate(sched.layers):
        _check_layer(l, Ly)


def test_token_step_graph_replays_equal_eager():
    # 10001 tokens: ragged CSA (2501 entries) and HCA (79 rows) counts
    print("case token step graph T=10001 B=3", flush=True)
    sched = _schedule(10001, 3)
    s0 = torch.cuda.current_stream().cuda_stream
    sched.run(s0)
    torch.cuda.synchronize()
    ref = [(Ly.out.clone(), Ly.lse.clone()) for Ly in sched.layers]
    ref_ids = [Ly.ids.clone() for Ly in sched.layers if isinstance(Ly, CsaLayer)]
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=st):
        sched.run(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        for Ly in sched.layers:
            Ly.out.fill_(float("nan"))
            if isinstance(Ly, CsaLayer):
                Ly.ids.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (o, ls), Ly in zip(ref, sched.layers):
            assert torch.equal(Ly.out, o) and torch.equal(Ly.lse, ls), f"replay {rep}"
        for ri, Ly in zip(ref_ids, [Ly for Ly in sched.layers if isinstance(Ly, CsaLayer)]):
            assert torch.equal(Ly.ids, ri), f"replay {rep}"
    # and the layers against the oracle, after the replays
    for l in (0, 2, 3, 42):
        _check_layer(l, sched.layers[l])


def test_token_step_full_size_sampled():
    # the benchmark's 64K token step: 32 sequences, CSA layers over 16384
    # entries (the timed workload's layers), HCA layers over 512 rows, SWA over
    # 128, replayed from one graph; sampled (layer, sequence) pairs of each kind
    # against the oracle
    print("case token step full size T=65536 B=32", flush=True)
    sched = _schedule(65536, 32)
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        sched.run(torch.cuda.current_stream().cuda_stream)  # warm
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=st):
        sched.run(torch.cuda.current_stream().cuda_stream)
    g.replay()
    torch.cuda.synchronize()
    for l, b in ((0, 3), (2, 0), (3, 7), (42, 31), (41, 30)):
        Ly = sched.layers[l]
        one = lambda x: x[b:b + 1].cpu()
        if layer_kind(l) == "csa":
            assert (Ly.count.cpu() == Ly.k).all()
            q, w, k = Ly.L.idx.q_idx, Ly.L.idx.w, Ly.L.idx.k_idx
            rids, rcnt, _ = oracle.topk(oracle.idx_score(one(q), one(w), one(k)), Ly.k)
            assert np.array_equal(Ly.ids[b:b + 1].cpu().numpy(), rids), (l, b)
            kv = type(Ly.L.kv)(Ly.L.kv.dtype, one(Ly.L.kv.data))
            ref, _ = oracle.attend(one(Ly.L.q), kv, rids, rcnt, Ly.window, SCALE)
        else:
            kv = type(Ly.kv)(Ly.kv.dtype, one(Ly.kv.data))
            ref, _ = oracle.attend(one(Ly.q), kv, None, None, 0, SCALE)
        err = np.abs(Ly.out[b:b + 1].double().cpu().numpy() - ref).max(-1)
        assert (err <= ATTN_TOL * np.abs(ref).max(-1)).all(), (l, b)
