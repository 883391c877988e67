"""One decode step of the attention layers, on preallocated buffers.

[ARCH] (ai-muninn.com, "284B 塞得進 128GB、長 context 還跑得動", section "(A) 壓縮你存的",
the layer table): the model interleaves three kinds of attention layer - SWA
(a small sliding window, uncompressed) on layers 0-1, CSA (4:1 compressed
entries, indexer + top-k + sparse attention) on the even layers 2-42, and HCA
(128:1 compressed entries, read densely, no top-k) on the odd layers 3-41.
Every layer below only issues calls of the C ABI (liblit.so) on the stream it
is given, with outputs and workspaces allocated once up front, so that a step
can be captured in a HIP graph and replayed.

  CsaLayer       score (a1) -> exact top-k (a2) -> sparse attention (a3)
  DenseLayer     attention over every row it is given (HCA rows, or the SWA window)
  TokenSchedule  the layers of one token's step, in layer order
"""
from __future__ import annotations

import ctypes
from typing import List, Sequence

from . import _dtype_code, hints_len, idx_in, kv_desc, last_error, load


def layer_kind(layer: int) -> str:
    """[ARCH] (A): SWA on layers 0-1, CSA on even layers 2-42, HCA on odd layers 3-41."""
    if layer < 2:
        return "swa"
    return "csa" if layer % 2 == 0 else "hca"


class CsaLayer:
    """Preallocated buffers of one CSA layer of B sequences and the three calls.
    L: LayerInputs (idx: q_idx/w/k_idx, q, kv); allowed: optional [B,N] u8."""

    def __init__(self, L, k: int, window: int, scale: float, dev, allowed=None):
        import torch

        self.L, self.allowed = L, allowed
        self.B, self.N = L.idx.k_idx.shape[0], L.idx.k_idx.shape[1]
        self.H, self.Hq = L.idx.q_idx.shape[1], L.q.shape[1]
        self.k, self.window, self.scale = k, window, scale
        B, N = self.B, self.N
        self.scores = torch.empty(B, N, dtype=torch.float32, device=dev)
        self.hints = torch.empty(B, hints_len(N), dtype=torch.float32, device=dev)
        self.ids = torch.empty(B, k, dtype=torch.int32, device=dev)
        self.count = torch.empty(B, dtype=torch.int32, device=dev)
        self.out = torch.empty(B, self.Hq, 512, dtype=torch.float32, device=dev)
        self.lse = torch.empty(B, self.Hq, dtype=torch.float32, device=dev)
        C = load()
        self.ws_topk = torch.empty(C.lit_topk_workspace_bytes(B, N, k), dtype=torch.uint8, device=dev)
        self.ws_attn = torch.empty(C.lit_attn_workspace_bytes(B, self.Hq, N), dtype=torch.uint8, device=dev)
        self.idx_desc = idx_in(L.idx.q_idx, L.idx.w, L.idx.k_idx)
        self.kv_desc = kv_desc(L.kv)
        self.q_dtype = _dtype_code(L.q)
        self.C = C

    def score(self, stream):
        st = self.C.lit_idx_score(ctypes.byref(self.idx_desc),
                                  None if self.allowed is None else self.allowed.data_ptr(), self.B, self.N,
                                  self.scores.data_ptr(), self.hints.data_ptr(), stream)
        assert st == 0, last_error()

    def select(self, stream):
        st = self.C.lit_topk_select(self.scores.data_ptr(), self.B, self.N, self.k, ctypes.byref(self.idx_desc),
                                    self.hints.data_ptr(), self.ids.data_ptr(), self.count.data_ptr(), None,
                                    self.ws_topk.data_ptr(), self.ws_topk.numel(), stream)
        assert st == 0, last_error()

    def attend(self, stream):
        st = self.C.lit_sparse_attn_decode(self.L.q.data_ptr(), self.q_dtype, self.Hq, ctypes.byref(self.kv_desc),
                                           self.B, self.ids.data_ptr(), self.count.data_ptr(), self.k, self.window,
                                           self.scale, self.out.data_ptr(), self.lse.data_ptr(),
                                           self.ws_attn.data_ptr(), self.ws_attn.numel(), stream)
        assert st == 0, last_error()

    def run(self, stream):
        self.score(stream)
        self.select(stream)
        self.attend(stream)

    def check(self):
        """Raise if a sequence's exact selection failed (count < 0: the rounding
        bound was violated; attention then wrote NaN for it). Waits for the
        device; meant for an eager step, not inside a captured one."""
        bad = (self.count < 0).nonzero().flatten().tolist()
        if bad:
            raise RuntimeError(f"exact top-k failed (count < 0) for sequences {bad}")


class DenseLayer:
    """Attention over every row given: the HCA layer's compressed rows, or an
    SWA layer's window (its last W uncompressed rows). q [B,Hq,512]; kv rows."""

    def __init__(self, q, kv, scale: float, dev):
        import torch

        self.q, self.kv = q, kv
        self.B, self.Hq = q.shape[0], q.shape[1]
        self.scale = scale
        self.out = torch.empty(self.B, self.Hq, 512, dtype=torch.float32, device=dev)
        self.lse = torch.empty(self.B, self.Hq, dtype=torch.float32, device=dev)
        self.kv_desc = kv_desc(kv)
        C = load()
        self.ws = torch.empty(C.lit_attn_workspace_bytes(self.B, self.Hq, self.kv_desc.n_rows), dtype=torch.uint8,
                              device=dev)
        self.q_dtype = _dtype_code(q)
        self.C = C

    def run(self, stream):
        st = self.C.lit_sparse_attn_decode(self.q.data_ptr(), self.q_dtype, self.Hq, ctypes.byref(self.kv_desc), self.B,
                                           None, None, 0, 0, self.scale, self.out.data_ptr(), self.lse.data_ptr(),
                                           self.ws.data_ptr(), self.ws.numel(), stream)
        assert st == 0, last_error()


class TokenSchedule:
    """The attention layers of one decode step, run in layer order."""

    def __init__(self, layers: Sequence):
        self.layers: List = list(layers)

    def run(self, stream):
        for Ly in self.layers:
            Ly.run(stream)

    def check(self):
        """Raise if any CSA layer's exact selection failed (see CsaLayer.check)."""
        for Ly in self.layers:
            if isinstance(Ly, CsaLayer):
                Ly.check()
