"""The allocation-free attention call against the workspace call, on the GPU.

lit_sparse_attn_decode_noalloc runs the same kernels as lit_sparse_attn_decode
with the library's own scratch array in place of the caller's workspace, so the
two must agree bit for bit. Two calls in a row (the second on a smaller input,
over the scratch the first one left behind), then FP8 rows and a dense call,
and a plan larger than the scratch array, which must be refused.
"""
import ctypes
import math

import pytest
import torch

import lightning_indexer_top_idx_amd as lit
from lightning_indexer_top_idx_amd import synth

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(512)


@pytest.fixture(scope="module")
def C():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    L = lit.load()
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    L.lit_sparse_attn_decode_noalloc.argtypes = [vp, ctypes.c_int, i32, ctypes.POINTER(lit.KVDesc), i32, vp, vp, i32,
                                                 i32, f32, vp, vp, vp]
    L.lit_sparse_attn_decode_noalloc.restype = ctypes.c_int
    return L


def _selection(B, N, k, g, short=()):
    """Ascending distinct ids [B,k] (tail -1) and counts; sequences in `short` keep fewer."""
    ids = torch.full((B, k), -1, dtype=torch.int32)
    cnt = torch.empty(B, dtype=torch.int32)
    for b in range(B):
        c = min(k, N) - (17 * (b + 1) if b in short else 0)
        ids[b, :c] = torch.randperm(N, generator=g)[:c].sort().values.to(torch.int32)
        cnt[b] = c
    return ids.cuda(), cnt.cuda()


def _both(C, q, kv, ids, cnt, k_cap, window):
    """The workspace call and the allocation-free call on the same inputs."""
    B, Hq = q.shape[0], q.shape[1]
    ref, rlse = lit.sparse_attn_decode(q, kv, ids, cnt, window, SCALE)
    out = torch.full_like(ref, float("nan"))
    lse = torch.full_like(rlse, float("nan"))
    desc = lit.kv_desc(kv)
    st = C.lit_sparse_attn_decode_noalloc(q.data_ptr(), lit.LIT_BF16, Hq, ctypes.byref(desc), B,
                                          None if ids is None else ids.data_ptr(),
                                          None if cnt is None else cnt.data_ptr(), k_cap, window, SCALE,
                                          out.data_ptr(), lse.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, lit.last_error()
    torch.cuda.synchronize()
    return ref, rlse, out, lse


def test_noalloc_equals_workspace_call_two_calls_then_smaller(C):
    g = torch.Generator().manual_seed(3)
    # 1: the headline shape (32 sequences x 16384 rows, top-512 + window 128:
    #    two row slices per sequence, 8.5 MB of partial results in the scratch)
    print("case noalloc B=32 N=16384 k=512", flush=True)
    B, N, k, Hq = 32, 16384, 512, 64
    gd = torch.Generator(device="cuda").manual_seed(5)
    q = synth.make_q(B, Hq, "bf16", gd, "cuda")
    kv = synth.make_kv(B, N, "bf16", gd, "cuda")
    ids, cnt = _selection(B, N, k, g, short=(3, 17))
    ref, rlse, out, lse = _both(C, q, kv, ids, cnt, k, 128)
    assert torch.equal(out, ref) and torch.equal(lse, rlse)
    # 2: a smaller call right after, over what the first left in the scratch
    print("case noalloc B=4 N=3000 k=256", flush=True)
    B, N, k = 4, 3000, 256
    q = synth.make_q(B, Hq, "bf16", gd, "cuda")
    kv = synth.make_kv(B, N, "bf16", gd, "cuda")
    ids, cnt = _selection(B, N, k, g, short=(1,))
    ref, rlse, out, lse = _both(C, q, kv, ids, cnt, k, 64)
    assert torch.equal(out, ref) and torch.equal(lse, rlse)


def test_noalloc_fp8_rows_and_dense(C):
    g = torch.Generator().manual_seed(4)
    gd = torch.Generator(device="cuda").manual_seed(6)
    print("case noalloc fp8 B=8 N=16384 k=1024", flush=True)
    B, N, k, Hq = 8, 16384, 1024, 64
    q = synth.make_q(B, Hq, "bf16", gd, "cuda")
    kv = synth.make_kv(B, N, "fp8", gd, "cuda")
    ids, cnt = _selection(B, N, k, g, short=(2,))
    ref, rlse, out, lse = _both(C, q, kv, ids, cnt, k, 128)
    assert torch.equal(out, ref) and torch.equal(lse, rlse)
    print("case noalloc dense B=4 N=3907", flush=True)
    q = synth.make_q(4, Hq, "bf16", gd, "cuda")
    kv = synth.make_kv(4, 3907, "bf16", gd, "cuda")
    ref, rlse, out, lse = _both(C, q, kv, None, None, 0, 0)
    assert torch.equal(out, ref) and torch.equal(lse, rlse)


def test_noalloc_refuses_a_plan_beyond_its_scratch(C):
    # 32 sequences whose selections hold 8192 ids plus a window of 8192 rows need
    # 15 row slices each: 63 MB of partial results, beyond the library's array
    print("case noalloc refusal", flush=True)
    B, N, Hq, k = 32, 16384, 64, 8192
    q = torch.zeros(B, Hq, 512, dtype=torch.bfloat16, device="cuda")
    kv = synth.KVRows("bf16", torch.zeros(B, N, 512, dtype=torch.bfloat16, device="cuda"))
    ids = torch.full((B, k), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, Hq, 512, dtype=torch.float32, device="cuda")
    desc = lit.kv_desc(kv)
    st = C.lit_sparse_attn_decode_noalloc(q.data_ptr(), lit.LIT_BF16, Hq, ctypes.byref(desc), B, ids.data_ptr(),
                                          cnt.data_ptr(), k, 8192, SCALE, out.data_ptr(), None,
                                          torch.cuda.current_stream().cuda_stream)
    assert st == 5, (st, lit.last_error())
    assert "scratch" in lit.last_error()
    # the same call with a workspace of the queried size is accepted
    o2, _ = lit.sparse_attn_decode(q, kv, ids, cnt, 8192, SCALE)
    torch.cuda.synchronize()
    assert torch.isfinite(o2).all()
