"""CPU oracle of the lightning-indexer decode step (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its binding) never does, and this package imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, loops in index order);
this module compiles it with gcc and marshals numpy / torch CPU arrays into it,
one sequence at a time. Each wrapper names the page passage its C function
follows; see the header of ``oracle.c`` for the page titles.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# ORACLE_SANITIZED=1: the same source built with AddressSanitizer and
# UndefinedBehaviorSanitizer (loaded with the sanitizer runtime preloaded)
_SANITIZED = os.environ.get("ORACLE_SANITIZED") == "1"
if _SANITIZED:
    _LIB_PATH = os.path.join(_HERE, "..", "_build", "liboracle_sanitized.so")

F32, BF16, FP8 = 0, 1, 2
IDX_DIM = 128
KV_DIM = 512
FP8_DIMS = 448
ROPE_DIMS = 64
SCALE_STRIDE = 8

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no FP contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
        os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             *(san if _SANITIZED else []), "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, ip, dp, i32, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        L.or_fp8_e4m3.argtypes = [ctypes.c_uint8]
        L.or_fp8_e4m3.restype = f64
        L.or_e8m0.argtypes = [ctypes.c_uint8]
        L.or_e8m0.restype = f64
        L.or_kv_dequant.argtypes = [i32, vp, vp, vp, i32, dp]
        L.or_idx_score.argtypes = [vp, vp, vp, i32, i32, i32, vp, dp]
        L.or_topk.argtypes = [dp, i32, i32, vp, vp]
        L.or_topk.restype = i32
        L.or_attend.argtypes = [vp, i32, i32, i32, vp, vp, vp, i32, vp, i32, i32, f64, dp, dp]
        L.or_golden.argtypes = [vp, i32, i32, i32, vp, vp, vp, i32, f64, i32, dp, vp, vp]
        L.or_golden.restype = i32
        L.or_recall.argtypes = [vp, vp, i32, vp, vp, vp]
        L.or_gate_layer.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f64, dp, vp]
        L.or_topp_vote.argtypes = [dp, i32, i32, i32, f64, i32, vp, vp]
        L.or_topp_vote.restype = i32
        L.or_decode_query.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, i32, i32, i32, vp, vp, vp,
                                      i32, f64, vp, dp, dp]
        L.or_decode_query.restype = i32
        _lib = L
    return _lib


# ---------------------------------------------------------------------------
# marshalling helpers


def np_of(x):
    """numpy view of a CPU array; torch bf16 becomes its uint16 bit pattern."""
    if x is None:
        return None
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16)
            if x.dtype == torch.float8_e4m3fn:
                return x.view(torch.uint8).numpy()
            return x.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x)


def dtype_code(arr) -> int:
    a = np_of(arr)
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"unsupported element type {a.dtype}")


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class KV:
    """Compressed latent rows of one batch: dtype F32/BF16 with data [B,N,512],
    or FP8 with data [B,N,448] u8, rope [B,N,64] bf16, scale [B,N,8] u8."""

    def __init__(self, dtype, data, rope=None, scale=None):
        self.dtype = dtype
        self.data = np.ascontiguousarray(np_of(data))
        self.rope = None if rope is None else np.ascontiguousarray(np_of(rope))
        self.scale = None if scale is None else np.ascontiguousarray(np_of(scale))

    @property
    def n_rows(self):
        return self.data.shape[1]

    def seq(self, b):
        return (self.data[b], None if self.rope is None else self.rope[b],
                None if self.scale is None else self.scale[b])


def kv_from(kv) -> KV:
    """Accept an oracle.KV or any object with dtype/data/rope/scale fields."""
    if isinstance(kv, KV):
        return kv
    code = {"f32": F32, "bf16": BF16, "fp8": FP8}.get(kv.dtype, kv.dtype)
    return KV(code, kv.data, getattr(kv, "rope", None), getattr(kv, "scale", None))


# ---------------------------------------------------------------------------
# the oracle, one function per step; B is looped here, each call is one sequence


def fp8_e4m3(code: int) -> float:
    """OCP E4M3FN decode of one byte ([ARCH] KV precision)."""
    return lib().or_fp8_e4m3(code)


def e8m0(code: int) -> float:
    return lib().or_e8m0(code)


def kv_dequant(kv, b: int = 0) -> np.ndarray:
    kv = kv_from(kv)
    data, rope, scale = kv.seq(b)
    out = np.empty((kv.n_rows, KV_DIM), np.float64)
    lib().or_kv_dequant(kv.dtype, _p(data), _p(rope), _p(scale), kv.n_rows, _p(out))
    return out


def idx_score(q, w, k, allowed=None) -> np.ndarray:
    """a1 ([ARCH] (B); [LSA] reply equation without its sigmoid): fp64 scores [B,N]."""
    q, w, k = np_of(q), np.ascontiguousarray(np_of(w), np.float32), np_of(k)
    allowed = None if allowed is None else np.ascontiguousarray(np_of(allowed), np.uint8)
    dt = dtype_code(q)
    assert dtype_code(k) == dt
    B, H, _ = q.shape
    N = k.shape[1]
    out = np.empty((B, N), np.float64)
    for b in range(B):
        lib().or_idx_score(_p(np.ascontiguousarray(q[b])), _p(np.ascontiguousarray(w[b])),
                           _p(np.ascontiguousarray(k[b])), dt, H, N,
                           None if allowed is None else _p(np.ascontiguousarray(allowed[b])),
                           _p(out[b]))
    return out


def topk(scores64, k: int):
    """a2 ([ARCH] (B)): ids [B,k] ascending (tail -1), count [B], mask [B,N]."""
    s = np.ascontiguousarray(np_of(scores64), np.float64)
    B, N = s.shape
    ids = np.empty((B, k), np.int32)
    cnt = np.empty((B,), np.int32)
    mask = np.empty((B, N), np.uint8)
    for b in range(B):
        cnt[b] = lib().or_topk(_p(s[b]), N, k, _p(ids[b]), _p(mask[b]))
    return ids, cnt, mask


def attend(q, kv, ids, count, window: int, scale: float):
    """a3/a4/a5 ([ARCH] (A), (B)): out [B,Hq,512] fp64, lse [B,Hq]. ids None = all rows."""
    q = np_of(q)
    kv = kv_from(kv)
    qdt = dtype_code(q)
    B, Hq, _ = q.shape
    out = np.empty((B, Hq, KV_DIM), np.float64)
    lse = np.empty((B, Hq), np.float64)
    ids = None if ids is None else np.ascontiguousarray(np_of(ids), np.int32)
    count = None if count is None else np_of(count)
    for b in range(B):
        data, rope, sc = kv.seq(b)
        lib().or_attend(_p(np.ascontiguousarray(q[b])), qdt, Hq, kv.dtype, _p(data), _p(rope), _p(sc),
                        kv.n_rows, None if ids is None else _p(ids[b]),
                        0 if ids is None else int(count[b]), int(window), float(np.float32(scale)),
                        _p(out[b]), _p(lse[b]))
    return out, lse


def golden(q, kv, scale: float, k: int):
    """a6 ([FMEN] "Act 3"): ids [B,k], count [B], mask [B,N], pbar [B,N] fp64."""
    q = np_of(q)
    kv = kv_from(kv)
    qdt = dtype_code(q)
    B, Hq, _ = q.shape
    N = kv.n_rows
    ids = np.empty((B, k), np.int32)
    cnt = np.empty((B,), np.int32)
    mask = np.empty((B, N), np.uint8)
    pbar = np.empty((B, N), np.float64)
    for b in range(B):
        data, rope, sc = kv.seq(b)
        cnt[b] = lib().or_golden(_p(np.ascontiguousarray(q[b])), qdt, Hq, kv.dtype, _p(data), _p(rope),
                                 _p(sc), N, float(np.float32(scale)), k, _p(pbar[b]), _p(ids[b]),
                                 _p(mask[b]))
    return ids, cnt, mask, pbar


def lookahead_golden(q, kv, scale: float, k: int):
    """The lookahead golden ([FMEN] "The one caveat I didn't test: lookahead";
    [LSA] 2.2: the gate predicts what the next 64 steps need): for every step t
    of the horizon, the a6 golden set of its query q[:, t] against the same rows;
    hits[b][n] counts the steps whose set holds n, the union is hits > 0.
    q [B,T,Hq,512] -> step_ids [B,T,k], hits [B,N], union_mask [B,N] u8,
    union_count [B], pbar [B,T,N]."""
    q = np_of(q)
    kv = kv_from(kv)
    B, T = q.shape[0], q.shape[1]
    N = kv.n_rows
    step_ids = np.empty((B, T, k), np.int32)
    hits = np.zeros((B, N), np.int32)
    pbar = np.empty((B, T, N), np.float64)
    for t in range(T):
        ids, _, mask, pb = golden(np.ascontiguousarray(q[:, t]), kv, scale, k)
        step_ids[:, t] = ids
        hits += mask.astype(np.int32)
        pbar[:, t] = pb
    umask = (hits > 0).astype(np.uint8)
    return step_ids, hits, umask, umask.sum(-1).astype(np.int32), pbar


def recall(a, m):
    """a7 ([FMEN] "Act 1", "Act 3"): intersection and set sizes per sequence."""
    a = np.ascontiguousarray(np_of(a), np.uint8)
    m = np.ascontiguousarray(np_of(m), np.uint8)
    B, N = a.shape
    inter = np.empty(B, np.int32)
    ca = np.empty(B, np.int32)
    cb = np.empty(B, np.int32)
    for b in range(B):
        i, x, y = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        lib().or_recall(_p(a[b]), _p(m[b]), N, ctypes.byref(i), ctypes.byref(x), ctypes.byref(y))
        inter[b], ca[b], cb[b] = i.value, x.value, y.value
    return inter, ca, cb


def gate_threshold_logit(threshold: float) -> float:
    """sigmoid(z) >= t  <=>  z >= log(t / (1 - t)); exactly 0 for t = 0.5."""
    return 0.0 if threshold == 0.5 else math.log(threshold / (1.0 - threshold))


def lsa_gate(layers, threshold: float = 0.5, return_z: bool = False):
    """a8 ([LSA] 2.2, 4.1, reply equation): OR over layers of the per-layer keep
    sets. layers: list of dicts with h [B,d_model] f32, wq_a, wq_b, w_proj, k (bf16)."""
    thr = gate_threshold_logit(threshold)
    gate = None
    zs = []
    for L in layers:
        h = np.ascontiguousarray(np_of(L["h"]), np.float32)
        wa, wb, wp = np_of(L["wq_a"]), np_of(L["wq_b"]), np_of(L["w_proj"])
        k = np_of(L["k"])
        B, d_model = h.shape
        rank = wa.shape[0]
        H = wp.shape[0]
        N = k.shape[1]
        keep = np.empty((B, N), np.uint8)
        z = np.empty((B, N), np.float64)
        for b in range(B):
            lib().or_gate_layer(_p(h[b]), _p(wa), _p(wb), _p(wp), _p(np.ascontiguousarray(k[b])), H,
                                d_model, rank, N, thr, _p(z[b]), _p(keep[b]))
        gate = keep.copy() if gate is None else (gate | keep)
        zs.append(z)
    count = gate.sum(axis=1).astype(np.int32)
    return (gate, count, zs) if return_z else (gate, count)


def pool_plan(gate, window: int, C: int):
    """The LSA cold-pool fetch ([LSA] 2.2: the kept blocks move to the GPU, the
    steps in between attend only inside them). Per sequence the kept entries are
    the gated ones and the last min(window, N) ones (the SWA window is always
    attended), in ascending order, placed in the last |K| of C slots, -1 in the
    slots before; allowed_c marks the gated ones. When |K| > C nothing fits: the
    map is all -1. Returns map [B,C] int32, count [B] int32, allowed_c [B,C] u8."""
    g = np.asarray(np_of(gate)) != 0
    B, N = g.shape
    W = min(window, N)
    m = np.full((B, C), -1, np.int32)
    ac = np.zeros((B, C), np.uint8)
    cnt = np.zeros(B, np.int32)
    for b in range(B):
        kept = sorted(set(np.flatnonzero(g[b]).tolist()) | set(range(N - W, N)))
        cnt[b] = len(kept)
        if len(kept) <= C:
            m[b, C - len(kept):] = kept
            ac[b, C - len(kept):] = g[b, kept]
    return m, cnt, ac


def idx_score_mq(q, w, k, lengths=None, allowed=None) -> np.ndarray:
    """The multi-query indexer: Q queries per sequence scored against that
    sequence's keys (depth-1 MTP verifies the draft token with the current one;
    a prefill chunk scores every token; [ARCH], the series list and (A)). Query
    j of sequence b is row (b, j) and sees the entries n < lengths[b][j] (all N
    when lengths is None); each row is the a1 score of that query against k[b],
    -inf where the entry is hidden or not allowed. q [B,Q,H,128], w [B,Q,H],
    k [B,N,128], lengths [B,Q], allowed [B,N] -> fp64 [B,Q,N]."""
    q, w, k = np_of(q), np.ascontiguousarray(np_of(w), np.float32), np_of(k)
    B, Q = q.shape[0], q.shape[1]
    N = k.shape[1]
    al = None if allowed is None else np.asarray(np_of(allowed)) != 0
    ln = None if lengths is None else np.asarray(np_of(lengths), np.int64)
    out = np.empty((B, Q, N), np.float64)
    for b in range(B):
        for j in range(Q):
            vis = np.ones(N, bool) if al is None else al[b].copy()
            if ln is not None:
                vis[max(int(ln[b, j]), 0):] = False
            out[b, j] = idx_score(q[b, j][None], w[b, j][None], k[b][None], vis[None].astype(np.uint8))[0]
    return out


def topk_mq(scores64, k: int):
    """The per-query top-k of idx_score_mq's rows: ids [B,Q,k], count [B,Q], mask [B,Q,N]."""
    s = np.ascontiguousarray(np_of(scores64), np.float64)
    B, Q, N = s.shape
    ids, cnt, mask = topk(s.reshape(B * Q, N), k)
    return ids.reshape(B, Q, k), cnt.reshape(B, Q), mask.reshape(B, Q, N)


def topp_vote(x, is_logits: bool, top_p: float = 0.6, min_votes: int = 3):
    """a9 ([LSA] 3.2): x [L,B,N] fp64 -> gold [B,N] u8, gold_count [B], votes [B,N]."""
    x = np.ascontiguousarray(np_of(x), np.float64)
    L, B, N = x.shape
    gold = np.empty((B, N), np.uint8)
    votes = np.empty((B, N), np.int32)
    cnt = np.empty(B, np.int32)
    for b in range(B):
        xb = np.ascontiguousarray(x[:, b, :])
        cnt[b] = lib().or_topp_vote(_p(xb), 1 if is_logits else 0, L, N, float(top_p), int(min_votes),
                                    _p(gold[b]), _p(votes[b]))
    return gold, cnt, votes


def decode_queries(jobs, threads: int = 1):
    """Score -> select -> attend for a list of single-sequence jobs (dicts of numpy
    arrays), spread over `threads` host threads (ctypes releases the GIL).
    Returns a list of (count, ids, out, lse)."""

    def one(j):
        H = j["q_idx"].shape[0]
        N = j["k_idx"].shape[0]
        Hq = j["q"].shape[0]
        ids = np.empty(j["k"], np.int32)
        out = np.empty((Hq, KV_DIM), np.float64)
        lse = np.empty(Hq, np.float64)
        c = lib().or_decode_query(_p(j["q_idx"]), _p(j["w"]), _p(j["k_idx"]), dtype_code(j["q_idx"]), H, N,
                                  j["k"], _p(j["q"]), dtype_code(j["q"]), Hq, j["kv_dtype"], _p(j["data"]),
                                  _p(j.get("rope")), _p(j.get("scale")), j["window"], float(j["scale_f"]),
                                  _p(ids), _p(out), _p(lse))
        return c, ids, out, lse

    lib()
    if threads <= 1:
        return [one(j) for j in jobs]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(one, jobs))
