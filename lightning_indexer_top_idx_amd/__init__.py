"""lightning_indexer_top_idx_amd - the lightning-indexer decode step on MI355X.

A thin ctypes binding over liblit.so (include/lit.h). Every function here only
marshals torch device tensors into the C ABI: it allocates the outputs and the
workspace with torch, passes raw pointers and the current HIP stream, and
raises LitError when the library reports a failure. All arithmetic runs in the
HIP kernels; there is no fallback: if the library is not built, every call
raises.

Functions (same names as the C entry points, without the lit_ prefix):
  idx_score, topk_select, sparse_attn_decode, sparse_attn_decode_noalloc, golden_topk, golden_topp_vote,
  idx_score_exact, recall, lsa_gate, pool_plan, pool_gather, pool_remap_ids.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
# LIT_LIBRARY names another build of the same library (the tests' sanitized
# host build); there is no other implementation behind this binding
LIB_PATH = os.environ.get("LIT_LIBRARY", os.path.join(_HERE, "liblit.so"))

LIT_F32, LIT_BF16, LIT_FP8 = 0, 1, 2
IDX_DIM = 128
KV_DIM = 512
KNORM_CHUNK = 256
DEFAULT_SCALE = 1.0 / math.sqrt(KV_DIM)

_STATUS = {0: "LIT_OK", 1: "LIT_ERR_NULL", 2: "LIT_ERR_SHAPE", 3: "LIT_ERR_ALIGN", 4: "LIT_ERR_DTYPE",
           5: "LIT_ERR_WORKSPACE", 6: "LIT_ERR_LAUNCH", 7: "LIT_ERR_MEMORY"}

EXPORTS = [
    "lit_abi_version", "lit_last_error", "lit_idx_hints_len", "lit_idx_score", "lit_topk_workspace_bytes", "lit_topk_select",
    "lit_attn_workspace_bytes", "lit_sparse_attn_decode", "lit_sparse_attn_decode_noalloc", "lit_golden_workspace_bytes", "lit_golden_topk",
    "lit_topp_workspace_bytes", "lit_golden_topp_vote", "lit_idx_score_exact", "lit_recall",
    "lit_gate_workspace_bytes", "lit_lsa_gate", "lit_pool_plan", "lit_pool_gather", "lit_pool_remap_ids",
    "lit_idx_score_mq", "lit_topk_select_mq", "lit_lookahead_workspace_bytes", "lit_lookahead_golden",
]


class LitError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class IdxIn(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("w", ctypes.c_void_p), ("k", ctypes.c_void_p),
                ("dtype", ctypes.c_int), ("H", ctypes.c_int32)]


class KVDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("n_rows", ctypes.c_int32), ("data", ctypes.c_void_p),
                ("rope", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("seq_stride", ctypes.c_int64), ("row_stride", ctypes.c_int64),
                ("rope_seq_stride", ctypes.c_int64), ("rope_row_stride", ctypes.c_int64),
                ("scale_seq_stride", ctypes.c_int64), ("scale_row_stride", ctypes.c_int64)]


class GateLayerDesc(ctypes.Structure):
    _fields_ = [("h", ctypes.c_void_p), ("wq_a", ctypes.c_void_p), ("wq_b", ctypes.c_void_p),
                ("w_proj", ctypes.c_void_p), ("k", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH):
    """Loads liblit.so (raises if it is missing: there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m lightning_indexer_top_idx_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, sz, f32, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float, ctypes.c_double
    L.lit_abi_version.restype = ctypes.c_int
    L.lit_last_error.restype = ctypes.c_char_p
    L.lit_idx_hints_len.argtypes = [i32]
    L.lit_idx_hints_len.restype = i32
    L.lit_idx_score.argtypes = [ctypes.POINTER(IdxIn), vp, i32, i32, vp, vp, vp]
    L.lit_topk_workspace_bytes.argtypes = [i32, i32, i32]
    L.lit_topk_workspace_bytes.restype = sz
    L.lit_topk_select.argtypes = [vp, i32, i32, i32, ctypes.POINTER(IdxIn), vp, vp, vp, vp, vp, sz, vp]
    L.lit_attn_workspace_bytes.argtypes = [i32, i32, i32]
    L.lit_attn_workspace_bytes.restype = sz
    L.lit_sparse_attn_decode.argtypes = [vp, ctypes.c_int, i32, ctypes.POINTER(KVDesc), i32, vp, vp, i32, i32, f32,
                                         vp, vp, vp, sz, vp]
    L.lit_sparse_attn_decode_noalloc.argtypes = [vp, ctypes.c_int, i32, ctypes.POINTER(KVDesc), i32, vp, vp, i32,
                                                 i32, f32, vp, vp, vp]
    L.lit_golden_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.lit_golden_workspace_bytes.restype = sz
    L.lit_golden_topk.argtypes = [vp, ctypes.c_int, i32, ctypes.POINTER(KVDesc), i32, f32, i32, vp, vp, vp, vp, vp,
                                  sz, vp]
    L.lit_topp_workspace_bytes.argtypes = [i32, i32, i32]
    L.lit_topp_workspace_bytes.restype = sz
    L.lit_golden_topp_vote.argtypes = [vp, i32, i32, i32, i32, f64, i32, vp, vp, vp, vp, sz, vp]
    L.lit_idx_score_exact.argtypes = [ctypes.POINTER(IdxIn), vp, i32, i32, vp, vp]
    L.lit_recall.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp]
    L.lit_gate_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.lit_gate_workspace_bytes.restype = sz
    L.lit_lsa_gate.argtypes = [ctypes.POINTER(GateLayerDesc), i32, i32, i32, i32, i32, i32, f64, vp, vp, vp, sz, vp]
    L.lit_pool_plan.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp]
    L.lit_pool_gather.argtypes = [vp, i32, ctypes.c_int64, i32, vp, i32, vp, vp]
    L.lit_pool_remap_ids.argtypes = [vp, vp, i32, i32, vp, i32, vp, vp]
    L.lit_idx_score_mq.argtypes = [ctypes.POINTER(IdxIn), i32, vp, vp, i32, i32, vp, vp, vp]
    L.lit_topk_select_mq.argtypes = [vp, i32, i32, i32, i32, ctypes.POINTER(IdxIn), vp, vp, vp, vp, vp, sz, vp]
    L.lit_lookahead_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.lit_lookahead_workspace_bytes.restype = sz
    L.lit_lookahead_golden.argtypes = [vp, ctypes.c_int, i32, i32, ctypes.POINTER(KVDesc), i32, f32, i32, vp, vp, vp,
                                       vp, vp, vp, sz, vp]
    for name in ("lit_idx_score", "lit_topk_select", "lit_sparse_attn_decode", "lit_sparse_attn_decode_noalloc",
                 "lit_golden_topk",
                 "lit_golden_topp_vote", "lit_idx_score_exact", "lit_recall", "lit_lsa_gate", "lit_pool_plan",
                 "lit_pool_gather", "lit_pool_remap_ids", "lit_idx_score_mq", "lit_topk_select_mq", "lit_lookahead_golden"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def last_error() -> str:
    return load().lit_last_error().decode()


def _check(status: int):
    if status != 0:
        raise LitError(status, last_error())


# ---------------------------------------------------------------------------
# marshalling helpers


def _torch():
    import torch

    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t=None) -> int:
    torch = _torch()
    dev = t.device if t is not None else None
    return torch.cuda.current_stream(dev).cuda_stream


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return LIT_F32
    if t.dtype == torch.bfloat16:
        return LIT_BF16
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _need_cuda(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def workspace(nbytes: int, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def idx_in(q_idx, w, k_idx) -> IdxIn:
    _need_cuda(q_idx, w, k_idx)
    return IdxIn(q_idx.data_ptr(), w.data_ptr(), k_idx.data_ptr(), _dtype_code(q_idx), q_idx.shape[1])


def _row_strides(t):
    """Byte strides (sequence, row) of a [B][N][row] tensor whose rows are contiguous;
    (0, 0) for none. A dimension of size one takes 0 (the dense value)."""
    if t is None:
        return 0, 0
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if t.dim() != 3 or (t.shape[2] > 1 and t.stride(2) != 1):
        raise ValueError("KV arrays must be [B][N][row] with contiguous rows")
    out = []
    for d in (0, 1):
        if t.shape[d] == 1:
            out.append(0)
        elif t.stride(d) <= 0:
            raise ValueError("KV arrays cannot be broadcast over sequences or rows")
        else:
            out.append(t.stride(d) * t.element_size())
    return tuple(out)


def kv_desc(kv) -> KVDesc:
    """kv: object with dtype in {"f32","bf16","fp8"} and data/rope/scale tensors of shape
    [B][N][row]; a view (N rows of a longer cache, rows inside wider records) is described
    by its strides and read in place."""
    code = {"f32": LIT_F32, "bf16": LIT_BF16, "fp8": LIT_FP8}[kv.dtype]
    rope, scale = getattr(kv, "rope", None), getattr(kv, "scale", None)
    strides = _row_strides(kv.data) + _row_strides(rope) + _row_strides(scale)
    return KVDesc(code, kv.data.shape[1], kv.data.data_ptr(), _ptr(rope), _ptr(scale), *strides)


# ---------------------------------------------------------------------------
# the calls


def hints_len(N: int) -> int:
    return load().lit_idx_hints_len(N)


def idx_score(q_idx, w, k_idx, allowed=None, want_hints: bool = True, out=None):
    """a1: scores [B,N] fp32 and the selection hints [B, hints_len(N)] (key-norm
    chunk bounds, then per-16-entry score maxima)."""
    torch = _torch()
    B, N = k_idx.shape[0], k_idx.shape[1]
    _need_cuda(allowed)
    scores = out if out is not None else torch.empty(B, N, dtype=torch.float32, device=k_idx.device)
    hints = torch.empty(B, hints_len(N), dtype=torch.float32, device=k_idx.device) if want_hints else None
    desc = idx_in(q_idx, w, k_idx)
    _check(load().lit_idx_score(ctypes.byref(desc), _ptr(allowed), B, N, scores.data_ptr(), _ptr(hints),
                                _stream(k_idx)))
    return scores, hints


def topk_select(scores, k: int, exact=None, hints=None, want_mask: bool = True, ws=None):
    """a2: ids [B,k] ascending (tail -1), count [B], mask [B,N] u8.
    exact: (q_idx, w, k_idx) that produced the scores -> fp64-exact selection;
    hints: the second output of idx_score for these scores."""
    torch = _torch()
    _need_cuda(scores, hints)
    B, N = scores.shape
    dev = scores.device
    ids = torch.empty(B, k, dtype=torch.int32, device=dev)
    count = torch.empty(B, dtype=torch.int32, device=dev)
    mask = torch.empty(B, N, dtype=torch.uint8, device=dev) if want_mask else None
    L = load()
    need = L.lit_topk_workspace_bytes(B, N, k)
    if ws is None:
        ws = workspace(need, dev)
    desc = idx_in(*exact) if exact is not None else None
    _check(L.lit_topk_select(scores.data_ptr(), B, N, k, ctypes.byref(desc) if desc is not None else None,
                             _ptr(hints), ids.data_ptr(), count.data_ptr(), _ptr(mask), ws.data_ptr(), ws.numel(),
                             _stream(scores)))
    return ids, count, mask


def idx_in_mq(q_idx, w, k_idx) -> IdxIn:
    """Descriptor of Q queries per sequence: q_idx [B,Q,H,128], w [B,Q,H], k_idx [B,N,128]."""
    _need_cuda(q_idx, w, k_idx)
    if q_idx.dim() != 4 or w.shape != q_idx.shape[:3] or k_idx.shape[0] != q_idx.shape[0]:
        raise ValueError("q_idx [B,Q,H,128], w [B,Q,H] and k_idx [B,N,128] disagree")
    return IdxIn(q_idx.data_ptr(), w.data_ptr(), k_idx.data_ptr(), _dtype_code(q_idx), q_idx.shape[2])


def idx_score_mq(q_idx, w, k_idx, lengths=None, allowed=None, want_hints: bool = True, out=None):
    """Multi-query indexer scores: [B,Q,N] fp32 and hints [B,Q,hints_len(N)].
    lengths [B,Q] int32: entries visible to each query (None: all)."""
    torch = _torch()
    B, Q, N = q_idx.shape[0], q_idx.shape[1], k_idx.shape[1]
    _need_cuda(allowed, lengths)
    if lengths is not None and (lengths.dtype != torch.int32 or tuple(lengths.shape) != (B, Q)):
        raise ValueError("lengths must be int32 [B,Q]")
    scores = out if out is not None else torch.empty(B, Q, N, dtype=torch.float32, device=k_idx.device)
    hints = torch.empty(B, Q, hints_len(N), dtype=torch.float32, device=k_idx.device) if want_hints else None
    desc = idx_in_mq(q_idx, w, k_idx)
    _check(load().lit_idx_score_mq(ctypes.byref(desc), Q, _ptr(lengths), _ptr(allowed), B, N, scores.data_ptr(),
                                   _ptr(hints), _stream(k_idx)))
    return scores, hints


def topk_select_mq(scores, k: int, exact=None, hints=None, want_mask: bool = True, ws=None):
    """Per-row top-k of idx_score_mq's scores [B,Q,N]: ids [B,Q,k], count [B,Q],
    mask [B,Q,N]. exact: (q_idx [B,Q,H,128], w, k_idx) -> fp64-exact selection."""
    torch = _torch()
    _need_cuda(scores, hints)
    B, Q, N = scores.shape
    dev = scores.device
    ids = torch.empty(B, Q, k, dtype=torch.int32, device=dev)
    count = torch.empty(B, Q, dtype=torch.int32, device=dev)
    mask = torch.empty(B, Q, N, dtype=torch.uint8, device=dev) if want_mask else None
    L = load()
    if ws is None:
        ws = workspace(L.lit_topk_workspace_bytes(B * Q, N, k), dev)
    desc = idx_in_mq(*exact) if exact is not None else None
    _check(L.lit_topk_select_mq(scores.data_ptr(), B, Q, N, k, ctypes.byref(desc) if desc is not None else None,
                                _ptr(hints), ids.data_ptr(), count.data_ptr(), _ptr(mask), ws.data_ptr(), ws.numel(),
                                _stream(scores)))
    return ids, count, mask


def sparse_attn_decode(q, kv, ids=None, count=None, window: int = 128, scale: float = DEFAULT_SCALE,
                       want_lse: bool = True, ws=None, out=None):
    """a3/a4/a5: out [B,Hq,512] fp32, lse [B,Hq]. ids None = every row (HCA)."""
    torch = _torch()
    _need_cuda(q, ids, count)
    B, Hq = q.shape[0], q.shape[1]
    dev = q.device
    o = out if out is not None else torch.empty(B, Hq, KV_DIM, dtype=torch.float32, device=dev)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev) if want_lse else None
    desc = kv_desc(kv)
    L = load()
    if ws is None:
        ws = workspace(L.lit_attn_workspace_bytes(B, Hq, desc.n_rows), dev)
    k_cap = ids.shape[1] if ids is not None else 0
    _check(L.lit_sparse_attn_decode(q.data_ptr(), _dtype_code(q), Hq, ctypes.byref(desc), B, _ptr(ids), _ptr(count),
                                    k_cap, int(window), float(scale), o.data_ptr(), _ptr(lse), ws.data_ptr(),
                                    ws.numel(), _stream(q)))
    return o, lse


def sparse_attn_decode_noalloc(q, kv, ids=None, count=None, window: int = 128, scale: float = DEFAULT_SCALE,
                               out=None, lse=None):
    """sparse_attn_decode without a workspace: the partial results go to the
    library's scratch array on this GPU (the call allocates no device memory
    beyond the outputs created here when `out` / `lse` are not given)."""
    torch = _torch()
    _need_cuda(q, ids, count, out, lse)
    B, Hq = q.shape[0], q.shape[1]
    o = out if out is not None else torch.empty(B, Hq, KV_DIM, dtype=torch.float32, device=q.device)
    desc = kv_desc(kv)
    k_cap = ids.shape[1] if ids is not None else 0
    _check(load().lit_sparse_attn_decode_noalloc(q.data_ptr(), _dtype_code(q), Hq, ctypes.byref(desc), B, _ptr(ids),
                                                 _ptr(count), k_cap, int(window), float(scale), o.data_ptr(), _ptr(lse),
                                                 _stream(q)))
    return o, lse


def golden_topk(q, kv, k: int, scale: float = DEFAULT_SCALE, want_pbar: bool = True, want_mask: bool = True, ws=None):
    """a6: golden ids [B,k], count [B], mask [B,N], pbar [B,N] fp64."""
    torch = _torch()
    _need_cuda(q)
    B, Hq = q.shape[0], q.shape[1]
    desc = kv_desc(kv)
    N = desc.n_rows
    dev = q.device
    ids = torch.empty(B, k, dtype=torch.int32, device=dev)
    count = torch.empty(B, dtype=torch.int32, device=dev)
    mask = torch.empty(B, N, dtype=torch.uint8, device=dev) if want_mask else None
    pbar = torch.empty(B, N, dtype=torch.float64, device=dev) if want_pbar else None
    L = load()
    if ws is None:
        ws = workspace(L.lit_golden_workspace_bytes(B, Hq, N, k), dev)
    _check(L.lit_golden_topk(q.data_ptr(), _dtype_code(q), Hq, ctypes.byref(desc), B, float(scale), k,
                             ids.data_ptr(), count.data_ptr(), _ptr(mask), _ptr(pbar), ws.data_ptr(), ws.numel(),
                             _stream(q)))
    return ids, count, mask, pbar


def lookahead_golden(q, kv, k: int, scale: float = DEFAULT_SCALE, want_step_ids: bool = True,
                     want_pbar: bool = False, ws=None):
    """Lookahead golden of the T queries q [B,T,Hq,512] against kv: step_ids
    [B,T,k], hits [B,N] int32, union_mask [B,N] u8, union_count [B], pbar [B,T,N]."""
    torch = _torch()
    _need_cuda(q)
    B, T, Hq = q.shape[0], q.shape[1], q.shape[2]
    desc = kv_desc(kv)
    N = desc.n_rows
    dev = q.device
    step_ids = torch.empty(B, T, k, dtype=torch.int32, device=dev) if want_step_ids else None
    hits = torch.empty(B, N, dtype=torch.int32, device=dev)
    umask = torch.empty(B, N, dtype=torch.uint8, device=dev)
    ucount = torch.empty(B, dtype=torch.int32, device=dev)
    pbar = torch.empty(B, T, N, dtype=torch.float64, device=dev) if want_pbar else None
    L = load()
    if ws is None:
        ws = workspace(L.lit_lookahead_workspace_bytes(B, T, Hq, N, k), dev)
    _check(L.lit_lookahead_golden(q.data_ptr(), _dtype_code(q), T, Hq, ctypes.byref(desc), B, float(scale), k,
                                  _ptr(step_ids), hits.data_ptr(), umask.data_ptr(), ucount.data_ptr(), _ptr(pbar),
                                  ws.data_ptr(), ws.numel(), _stream(q)))
    return step_ids, hits, umask, ucount, pbar


def golden_topp_vote(x, is_logits: bool, top_p: float = 0.6, min_votes: int = 3, want_votes: bool = True, ws=None):
    """a9: x [L,B,N] fp64 -> gold [B,N] u8, gold_count [B], votes [B,N]."""
    torch = _torch()
    _need_cuda(x)
    L_, B, N = x.shape
    dev = x.device
    gold = torch.empty(B, N, dtype=torch.uint8, device=dev)
    gc = torch.empty(B, dtype=torch.int32, device=dev)
    votes = torch.empty(B, N, dtype=torch.int32, device=dev) if want_votes else None
    L = load()
    if ws is None:
        ws = workspace(L.lit_topp_workspace_bytes(L_, B, N), dev)
    _check(L.lit_golden_topp_vote(x.data_ptr(), 1 if is_logits else 0, L_, B, N, float(top_p), int(min_votes),
                                  gold.data_ptr(), gc.data_ptr(), _ptr(votes), ws.data_ptr(), ws.numel(), _stream(x)))
    return gold, gc, votes


def idx_score_exact(q_idx, w, k_idx, allowed=None):
    """fp64 canonical indexer scores [B,N] (slow; the label pipeline's input)."""
    torch = _torch()
    B, N = k_idx.shape[0], k_idx.shape[1]
    _need_cuda(allowed)
    out = torch.empty(B, N, dtype=torch.float64, device=k_idx.device)
    desc = idx_in(q_idx, w, k_idx)
    _check(load().lit_idx_score_exact(ctypes.byref(desc), _ptr(allowed), B, N, out.data_ptr(), _stream(k_idx)))
    return out


def recall(a, m):
    """a7: intersection [B], |a| [B], |m| [B] of two u8 masks [B,N]."""
    torch = _torch()
    _need_cuda(a, m)
    B, N = a.shape
    dev = a.device
    inter = torch.empty(B, dtype=torch.int32, device=dev)
    ca = torch.empty(B, dtype=torch.int32, device=dev)
    cb = torch.empty(B, dtype=torch.int32, device=dev)
    _check(load().lit_recall(a.data_ptr(), m.data_ptr(), B, N, inter.data_ptr(), ca.data_ptr(), cb.data_ptr(),
                             _stream(a)))
    return inter, ca, cb


def lsa_gate(layers: Sequence, threshold: float = 0.5, ws=None):
    """a8: layers = GateLayer-like objects (h, wq_a, wq_b, w_proj, k). Returns gate [B,N] u8, count [B]."""
    torch = _torch()
    descs = (GateLayerDesc * len(layers))()
    for i, Ly in enumerate(layers):
        g = Ly if not isinstance(Ly, dict) else type("G", (), Ly)
        _need_cuda(g.h, g.wq_a, g.wq_b, g.w_proj, g.k)
        descs[i] = GateLayerDesc(g.h.data_ptr(), g.wq_a.data_ptr(), g.wq_b.data_ptr(), g.w_proj.data_ptr(),
                                 g.k.data_ptr())
    g0 = layers[0] if not isinstance(layers[0], dict) else type("G", (), layers[0])
    B, d_model = g0.h.shape
    rank = g0.wq_a.shape[0]
    H = g0.w_proj.shape[0]
    N = g0.k.shape[1]
    dev = g0.h.device
    gate = torch.empty(B, N, dtype=torch.uint8, device=dev)
    count = torch.empty(B, dtype=torch.int32, device=dev)
    L = load()
    if ws is None:
        ws = workspace(L.lit_gate_workspace_bytes(len(layers), B, H, rank, N), dev)
    _check(L.lit_lsa_gate(descs, len(layers), B, N, H, d_model, rank, float(threshold), gate.data_ptr(),
                          count.data_ptr(), ws.data_ptr(), ws.numel(), _stream(g0.h)))
    return gate, count


def pool_plan(gate, window: int, C: int, want_allowed: bool = True):
    """The compact pool of the LSA fetch: gate [B,N] u8 -> map [B,C] int32 (the
    gated entries plus the window, ascending, right-aligned; -1 before them),
    count [B] int32 (> C: the pool is too small), allowed_c [B,C] u8."""
    torch = _torch()
    _need_cuda(gate)
    B, N = gate.shape
    dev = gate.device
    m = torch.empty(B, C, dtype=torch.int32, device=dev)
    count = torch.empty(B, dtype=torch.int32, device=dev)
    ac = torch.empty(B, C, dtype=torch.uint8, device=dev) if want_allowed else None
    _check(load().lit_pool_plan(gate.data_ptr(), B, N, int(window), int(C), m.data_ptr(), count.data_ptr(), _ptr(ac),
                                _stream(gate)))
    return m, count, ac


def pool_gather(src, m, out=None):
    """Rows of src [B,src_rows,...] (a GPU tensor, or a pinned CPU tensor read in
    place over the host link) through map m [B,C] -> [B,C,...] on the GPU
    (zeros for empty slots)."""
    torch = _torch()
    _need_cuda(m)
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    if not src.is_cuda and not src.is_pinned():
        raise ValueError("a CPU src must be pinned (page-locked)")
    B, C = m.shape
    rows = src.shape[1]
    row_bytes = src[0, 0].numel() * src.element_size() if src.dim() > 2 else src.element_size()
    dst = out if out is not None else torch.empty((B, C) + tuple(src.shape[2:]), dtype=src.dtype, device=m.device)
    _check(load().lit_pool_gather(src.data_ptr(), rows, row_bytes, B, m.data_ptr(), C, dst.data_ptr(), _stream(m)))
    return dst


def pool_remap_ids(ids_c, count, m):
    """Selected compact ids [B,k] (with their count [B]) -> original entry ids [B,k]."""
    torch = _torch()
    _need_cuda(ids_c, count, m)
    B, k = ids_c.shape
    ids = torch.empty_like(ids_c)
    _check(load().lit_pool_remap_ids(ids_c.data_ptr(), count.data_ptr(), B, k, m.data_ptr(), m.shape[1],
                                     ids.data_ptr(), _stream(ids_c)))
    return ids
