"""Thin Python binding of ``libmisa_indexer.so`` (C ABI in include/misa_indexer.h).

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the indexer runs in the library's gfx950
kernels.  There is no fallback: if the library is missing or no GPU is
visible, the calls raise.

Tensor formats (all on the GPU, contiguous):
  keys  bf16 [S][Lmax][128]   q bf16 [T][H][128]   w fp32 [T][H]
  seq_lens, q_seq, q_pos int32
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmisa_indexer.so")

(MISA_OP_DENSE, MISA_OP_ROUTE, MISA_OP_SCORE_TOPK, MISA_OP_RERANK, MISA_OP_TOPK, MISA_OP_INDEXER,
 MISA_OP_HISA) = range(7)

# Every entry point include/misa_indexer.h declares.
EXPORTS = ("misa_workspace_bytes", "misa_pool", "misa_pool_append", "misa_route", "misa_score", "misa_topk",
           "misa_score_topk", "misa_score_topk_ev", "indexer_dense", "misa_rerank",
           "misa_indexer", "misa_indexer_ev", "misa_indexer_noalloc", "hisa_indexer",
           "hisa_indexer_ev", "hisa_blocks", "misa_stream_read", "misa_status_str")

MISA_ERR_TOO_LARGE = -6
# bytes of misa_indexer_noalloc's static scratch (MISA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024


class MisaBatch(ctypes.Structure):
    _fields_ = [("keys", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("q", ctypes.c_void_p), ("w", ctypes.c_void_p),
                ("q_seq", ctypes.c_void_p), ("q_pos", ctypes.c_void_p),
                ("S", ctypes.c_int32), ("Lmax", ctypes.c_int32), ("d", ctypes.c_int32),
                ("T", ctypes.c_int32), ("H", ctypes.c_int32)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t
_lib = None


def load():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmisa_indexer.so is not built; run "
                              "`python -m long_context_sparse_05_amd.build_lib`")
        L = ctypes.CDLL(LIB_PATH)
        BP = ctypes.POINTER(MisaBatch)
        L.misa_workspace_bytes.argtypes = [BP, _I, _I, _I, _I, _I, ctypes.POINTER(_SZ)]
        L.misa_pool.argtypes = [BP, _I, _P, _P]
        L.misa_route.argtypes = [BP, _P, _I, _I, _I, _P, _P, _P, _SZ, _P]
        L.misa_score.argtypes = [BP, _P, _I, _P, _P]
        L.misa_topk.argtypes = [_P, _I, _I, _P, _I, _P, _P, _P, _SZ, _P]
        L.misa_score_topk.argtypes = [BP, _P, _I, _I, _P, _P, _P, _SZ, _P]
        L.misa_score_topk_ev.argtypes = [BP, _P, _I, _I, _P, _P, _P, _SZ, _P, _P, _P]
        L.indexer_dense.argtypes = [BP, _I, _P, _P, _P, _SZ, _P]
        L.misa_rerank.argtypes = [BP, _P, _I, _I, _P, _P, _P, _SZ, _P]
        L.misa_indexer.argtypes = [BP, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P]
        L.misa_indexer_ev.argtypes = [BP, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P, _P, _P]
        L.misa_indexer_noalloc.argtypes = [BP, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P]
        L.misa_pool_append.argtypes = [BP, _I, _P, _I, _P, _P]
        L.hisa_indexer.argtypes = [BP, _P, _I, _I, _P, _I, _I, _P, _P, _P, _SZ, _P]
        L.hisa_indexer_ev.argtypes = [BP, _P, _I, _I, _P, _I, _I, _P, _P, _P, _SZ, _P, _P, _P]
        L.hisa_blocks.argtypes = [BP, _P, _I, _I, _P, _I, _P, _P, _P, _SZ, _P]
        L.misa_stream_read.argtypes = [_P, _SZ, _I, _P, _P, _P, _P]
        for name in EXPORTS:
            getattr(L, name).restype = ctypes.c_int
        L.misa_status_str.argtypes = [ctypes.c_int]
        L.misa_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(code: int) -> str:
    return load().misa_status_str(int(code)).decode()


def _check(code, what):
    if code != 0:
        raise RuntimeError("%s: %s (status %d)" % (what, status_str(code), code))


def _torch():
    import torch
    return torch


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims" % (name, ndim))
    return t


class Batch:
    """Device-resident indexer inputs plus the ABI struct describing them."""

    def __init__(self, keys, q, w, q_seq, q_pos, seq_lens=None):
        torch = _torch()
        self.keys = _need(keys, torch.bfloat16, "keys", 3)
        self.q = _need(q, torch.bfloat16, "q", 3)
        self.w = _need(w, torch.float32, "w", 2)
        self.q_seq = _need(q_seq, torch.int32, "q_seq", 1)
        self.q_pos = _need(q_pos, torch.int32, "q_pos", 1)
        S, Lmax, d = self.keys.shape
        T, H, dq = self.q.shape
        if dq != d or tuple(self.w.shape) != (T, H) or self.q_seq.numel() != T or self.q_pos.numel() != T:
            raise ValueError("inconsistent batch shapes")
        if seq_lens is None:
            seq_lens = torch.full((S,), Lmax, dtype=torch.int32, device=self.keys.device)
        self.seq_lens = _need(seq_lens, torch.int32, "seq_lens", 1)
        self.S, self.Lmax, self.d, self.T, self.H = S, Lmax, d, T, H
        self.c = MisaBatch(self.keys.data_ptr(), self.seq_lens.data_ptr(), self.q.data_ptr(),
                           self.w.data_ptr(), self.q_seq.data_ptr(), self.q_pos.data_ptr(),
                           S, Lmax, d, T, H)

    @classmethod
    def from_numpy(cls, case, device="cuda"):
        """Upload a case from :mod:`synth` (bf16 bits as uint16)."""
        torch = _torch()
        import numpy as np

        def bf(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

        def i32(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)

        return cls(bf(case["keys"]), bf(case["q"]),
                   torch.from_numpy(np.ascontiguousarray(case["w"], dtype=np.float32)).to(device),
                   i32(case["q_seq"]), i32(case["q_pos"]), i32(case["seq_lens"]))

    def workspace_bytes(self, op, B=1, h=1, k=1, kc=1):
        n = _SZ(0)
        _check(load().misa_workspace_bytes(ctypes.byref(self.c), op, B, h, k, kc, ctypes.byref(n)),
               "misa_workspace_bytes")
        return n.value

    def workspace(self, op, B=1, h=1, k=1, kc=1):
        torch = _torch()
        return torch.empty(self.workspace_bytes(op, B, h, k, kc), dtype=torch.uint8,
                           device=self.keys.device)


def _ws(batch, ws, op, **kw):
    if ws is None:
        ws = batch.workspace(op, **kw)
    return ws, _SZ(ws.numel() * ws.element_size())


def pool(batch: Batch, B: int, out=None, stream=None):
    torch = _torch()
    M = (batch.Lmax + B - 1) // B
    if out is None:
        out = torch.empty((batch.S, M, batch.d), dtype=torch.float32, device=batch.keys.device)
    _need(out, torch.float32, "pooled")
    _check(load().misa_pool(ctypes.byref(batch.c), B, _ptr(out), _stream(stream)), "misa_pool")
    return out


def pool_append(batch: Batch, B: int, old_lens, max_new: int, pooled, stream=None):
    """Bring `pooled` (misa_pool's output) up to date in place after keys were
    appended: the batch's seq_lens hold the new lengths, old_lens (int32 [S] on
    the device) the lengths pooled reflects, max_new bounds the keys appended
    to any sequence.  Only the blocks that hold an appended key are rewritten."""
    torch = _torch()
    _need(pooled, torch.float32, "pooled")
    _need(old_lens, torch.int32, "old_lens", 1)
    _check(load().misa_pool_append(ctypes.byref(batch.c), B, _ptr(old_lens), int(max_new), _ptr(pooled),
                                   _stream(stream)), "misa_pool_append")
    return pooled


def route(batch: Batch, pooled, B: int, h: int, mode: int = 0, heads=None, head_score=None,
          want_score=False, ws=None, stream=None):
    torch = _torch()
    dev = batch.keys.device
    if heads is None:
        heads = torch.empty((batch.T, h), dtype=torch.int32, device=dev)
    if head_score is None and want_score:
        head_score = torch.empty((batch.T, batch.H), dtype=torch.float32, device=dev)
    ws, nws = _ws(batch, ws, MISA_OP_ROUTE, B=B, h=h)
    _check(load().misa_route(ctypes.byref(batch.c), _ptr(pooled), B, h, mode, _ptr(heads),
                             _ptr(head_score), _ptr(ws), nws, _stream(stream)), "misa_route")
    return (heads, head_score) if want_score or head_score is not None else heads


def score(batch: Batch, heads=None, out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty((batch.T, batch.Lmax), dtype=torch.float32, device=batch.keys.device)
    h = 0 if heads is None else heads.shape[1]
    _check(load().misa_score(ctypes.byref(batch.c), _ptr(heads), h, _ptr(out), _stream(stream)),
           "misa_score")
    return out


def _sel_out(batch_T, k, dev, idx, val, want_val):
    torch = _torch()
    if idx is None:
        idx = torch.empty((batch_T, k), dtype=torch.int32, device=dev)
    if val is None and want_val:
        val = torch.empty((batch_T, k), dtype=torch.float32, device=dev)
    return idx, val


def score_topk(batch: Batch, heads, k: int, idx=None, val=None, want_val=True, ws=None,
               stream=None, events=None):
    """misa_score_topk; `events` = (start, stop) raw hipEvent_t handles (ints)
    recorded around the scoring kernel (misa_score_topk_ev)."""
    idx, val = _sel_out(batch.T, k, batch.keys.device, idx, val, want_val)
    h = 0 if heads is None else heads.shape[1]
    ws, nws = _ws(batch, ws, MISA_OP_SCORE_TOPK, h=max(h, 1), k=k)
    if events is None:
        _check(load().misa_score_topk(ctypes.byref(batch.c), _ptr(heads), h, k, _ptr(idx),
                                      _ptr(val), _ptr(ws), nws, _stream(stream)),
               "misa_score_topk")
    else:
        _check(load().misa_score_topk_ev(ctypes.byref(batch.c), _ptr(heads), h, k, _ptr(idx),
                                         _ptr(val), _ptr(ws), nws, _stream(stream),
                                         ctypes.c_void_p(events[0]), ctypes.c_void_p(events[1])),
               "misa_score_topk_ev")
    return idx, val


def indexer_dense(batch: Batch, k: int, idx=None, val=None, want_val=True, ws=None, stream=None):
    idx, val = _sel_out(batch.T, k, batch.keys.device, idx, val, want_val)
    ws, nws = _ws(batch, ws, MISA_OP_DENSE, k=k)
    _check(load().indexer_dense(ctypes.byref(batch.c), k, _ptr(idx), _ptr(val), _ptr(ws), nws,
                                _stream(stream)), "indexer_dense")
    return idx, val


def indexer(batch: Batch, pooled, B: int, h: int, k: int, mode: int = 0, heads=None,
            head_score=None, idx=None, val=None, want_val=True, ws=None, stream=None,
            events=None):
    """misa_indexer: router + routed scoring + top-k in one call.
    Returns (heads, idx, val)."""
    torch = _torch()
    dev = batch.keys.device
    if heads is None:
        heads = torch.empty((batch.T, h), dtype=torch.int32, device=dev)
    idx, val = _sel_out(batch.T, k, dev, idx, val, want_val)
    ws, nws = _ws(batch, ws, MISA_OP_INDEXER, B=B, h=h, k=k)
    if events is None:
        _check(load().misa_indexer(ctypes.byref(batch.c), _ptr(pooled), B, h, mode, k, _ptr(heads),
                                   _ptr(head_score), _ptr(idx), _ptr(val), _ptr(ws), nws,
                                   _stream(stream)), "misa_indexer")
    else:
        _check(load().misa_indexer_ev(ctypes.byref(batch.c), _ptr(pooled), B, h, mode, k,
                                      _ptr(heads), _ptr(head_score), _ptr(idx), _ptr(val),
                                      _ptr(ws), nws, _stream(stream), ctypes.c_void_p(events[0]),
                                      ctypes.c_void_p(events[1])), "misa_indexer_ev")
    return heads, idx, val


def indexer_noalloc(batch: Batch, pooled, B: int, h: int, k: int, mode: int = 0, heads=None,
                    head_score=None, idx=None, val=None, want_val=True, stream=None):
    """misa_indexer_noalloc: misa_indexer with the library's static device
    scratch instead of a workspace (nothing is allocated by the call; the
    outputs are allocated here only when not passed).  Returns (heads, idx, val)."""
    torch = _torch()
    dev = batch.keys.device
    if heads is None:
        heads = torch.empty((batch.T, h), dtype=torch.int32, device=dev)
    idx, val = _sel_out(batch.T, k, dev, idx, val, want_val)
    _check(load().misa_indexer_noalloc(ctypes.byref(batch.c), _ptr(pooled), B, h, mode, k,
                                       _ptr(heads), _ptr(head_score), _ptr(idx), _ptr(val),
                                       _stream(stream)), "misa_indexer_noalloc")
    return heads, idx, val


def hisa_indexer(batch: Batch, pooled, B: int, m: int, k: int, heads=None, idx=None, val=None,
                 want_val=True, ws=None, stream=None, events=None):
    """hisa_indexer: block scores, the m best blocks, the indexer over their
    tokens, top-k.  heads=None uses all heads; an int32 [T][h] tensor uses
    those heads in both stages (MISA composed with HISA).  Returns (idx, val)."""
    torch = _torch()
    idx, val = _sel_out(batch.T, k, batch.keys.device, idx, val, want_val)
    h = 0 if heads is None else heads.shape[1]
    if heads is not None:
        _need(heads, torch.int32, "heads", 2)
    ws, nws = _ws(batch, ws, MISA_OP_HISA, B=B, h=max(h, 1), k=k, kc=m)
    args = (ctypes.byref(batch.c), _ptr(pooled), B, m, _ptr(heads), h, k, _ptr(idx), _ptr(val),
            _ptr(ws), nws, _stream(stream))
    if events is None:
        _check(load().hisa_indexer(*args), "hisa_indexer")
    else:
        _check(load().hisa_indexer_ev(*args, ctypes.c_void_p(events[0]), ctypes.c_void_p(events[1])),
               "hisa_indexer_ev")
    return idx, val


def hisa_blocks(batch: Batch, pooled, B: int, m: int, heads=None, ws=None, stream=None):
    """hisa_indexer's coarse stage: (block_scores [T][ceil(Lmax/B)], kept
    blocks [T][m], a set)."""
    torch = _torch()
    dev = batch.keys.device
    M = (batch.Lmax + B - 1) // B
    scores = torch.empty((batch.T, M), dtype=torch.float32, device=dev)
    blocks = torch.empty((batch.T, m), dtype=torch.int32, device=dev)
    h = 0 if heads is None else heads.shape[1]
    ws, nws = _ws(batch, ws, MISA_OP_HISA, B=B, h=max(h, 1), k=1, kc=m)
    _check(load().hisa_blocks(ctypes.byref(batch.c), _ptr(pooled), B, m, _ptr(heads), h, _ptr(scores),
                              _ptr(blocks), _ptr(ws), nws, _stream(stream)), "hisa_blocks")
    return scores, blocks


def rerank(batch: Batch, cand, k: int, idx=None, val=None, want_val=True, ws=None, stream=None):
    torch = _torch()
    _need(cand, torch.int32, "cand", 2)
    kc = cand.shape[1]
    idx, val = _sel_out(batch.T, k, batch.keys.device, idx, val, want_val)
    ws, nws = _ws(batch, ws, MISA_OP_RERANK, k=k, kc=kc)
    _check(load().misa_rerank(ctypes.byref(batch.c), _ptr(cand), kc, k, _ptr(idx), _ptr(val),
                              _ptr(ws), nws, _stream(stream)), "misa_rerank")
    return idx, val


def stream_read(buf, wgs: int, sink=None, stream=None, events=None):
    """misa_stream_read: one plain streaming read of the GPU tensor `buf`
    (its bytes, a multiple of 16) by `wgs` workgroups; `events` = (start,
    stop) raw hipEvent_t handles stamped with the kernel's begin and end."""
    torch = _torch()
    if sink is None:
        sink = torch.zeros(wgs, dtype=torch.int32, device=buf.device)
    ev = (None, None) if events is None else (ctypes.c_void_p(events[0]), ctypes.c_void_p(events[1]))
    _check(load().misa_stream_read(_ptr(buf), _SZ(buf.numel() * buf.element_size()), wgs, _ptr(sink),
                                   _stream(stream), *ev), "misa_stream_read")
    return sink


def topk(scores, row_len, k: int, idx=None, val=None, want_val=True, ws=None, stream=None):
    torch = _torch()
    _need(scores, torch.float32, "scores", 2)
    _need(row_len, torch.int32, "row_len", 1)
    rows, ld = scores.shape
    idx, val = _sel_out(rows, k, scores.device, idx, val, want_val)
    if ws is None:
        shape = MisaBatch(1, 0, 0, 0, 0, 0, 1, ld, 128, rows, 1)
        n = _SZ(0)
        _check(load().misa_workspace_bytes(ctypes.byref(shape), MISA_OP_TOPK, 1, 1, k, 1,
                                           ctypes.byref(n)), "misa_workspace_bytes")
        ws = torch.empty(n.value, dtype=torch.uint8, device=scores.device)
    _check(load().misa_topk(_ptr(scores), rows, ld, _ptr(row_len), k, _ptr(idx), _ptr(val),
                            _ptr(ws), _SZ(ws.numel()), _stream(stream)), "misa_topk")
    return idx, val
