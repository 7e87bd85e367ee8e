"""ctypes wrapper of the CPU oracle in ``misa_oracle.c``.

TEST INFRASTRUCTURE ONLY: only the tests, the package smoke check and the
benchmark's CPU-baseline leg import this module.  It shares no code with the
GPU path and never imports it.

Every function takes numpy arrays (keys and q as uint16 holding bf16 bits,
w as float32, positions as int32) and returns numpy results in float64 /
int32.  Each wraps one C function; the citation of the passage it follows is
on the C function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "misa_oracle.c")
_LIB = os.path.join(_HERE, "libmisa_oracle.so")

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
            "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm",
        ])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        L.orc_topk.argtypes = [_P, _I64, _I64, _P, _P]
        L.orc_topk_f32.argtypes = [_P, _I64, _I64, _P]
        L.orc_scores.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I, _P]
        L.orc_pool.argtypes = [_P, _P, _I, _I, _I, _I, _P]
        L.orc_route.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P]
        L.orc_dsa.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P]
        L.orc_misa.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                               _P, _P, _P, _P, _P]
        L.orc_rerank.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I, _I, _P, _P]
        L.orc_misa_dagger.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                      _I, _I, _P, _P, _P, _P]
        L.orc_hisa.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _I, _I,
                               _P, _P, _P, _P]
        L.orc_num_threads.restype = _I
        L.orc_set_num_threads.argtypes = [_I]
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(_P)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError("oracle %s failed with code %d" % (what, rc))


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


class Batch:
    """Host copy of one batch: keys [S][Lmax][d] and q [T][H][d] as bf16 bits."""

    def __init__(self, keys, q, w, q_seq, q_pos, seq_lens=None):
        self.keys, self.pk = _c(keys, np.uint16)
        self.q, self.pq = _c(q, np.uint16)
        self.w, self.pw = _c(w, np.float32)
        self.q_seq, self.ps = _c(q_seq, np.int32)
        self.q_pos, self.pp = _c(q_pos, np.int32)
        self.S, self.Lmax, self.d = self.keys.shape
        self.T, self.H, dq = self.q.shape
        assert dq == self.d and self.w.shape == (self.T, self.H)
        if seq_lens is None:
            seq_lens = np.full(self.S, self.Lmax, np.int32)
        self.seq_lens, self.pl = _c(seq_lens, np.int32)

    @classmethod
    def from_case(cls, case):
        return cls(case["keys"], case["q"], case["w"], case["q_seq"], case["q_pos"],
                   case.get("seq_lens"))

    def dims(self):
        return (self.S, self.Lmax, self.d, self.T, self.H)

    def head(self):
        return (self.pk, self.pq, self.pw, self.ps, self.pp) + self.dims()


def topk(v, k):
    """Indices of the k largest of v by (value desc, index asc), -1 padded."""
    v, pv = _c(v, np.float64)
    idx = np.empty(k, np.int32)
    val = np.empty(k, np.float64)
    _check(lib().orc_topk(pv, v.size, k, idx.ctypes.data_as(_P), val.ctypes.data_as(_P)), "topk")
    return idx, val


def topk_f32(v, k):
    """The same ranking taken on fp32 values (the GPU's own precision)."""
    v, pv = _c(v, np.float32)
    idx = np.empty(k, np.int32)
    _check(lib().orc_topk_f32(pv, v.size, k, idx.ctypes.data_as(_P)), "topk_f32")
    return idx


def scores(b: Batch, heads=None):
    out = np.empty((b.T, b.Lmax), np.float64)
    if heads is None:
        ph, h = None, 0
    else:
        heads, ph = _c(heads, np.int32)
        h = heads.shape[1]
    _check(lib().orc_scores(*b.head(), ph, h, out.ctypes.data_as(_P)), "scores")
    return out


def pool(b: Batch, B):
    M = (b.Lmax + B - 1) // B
    out = np.empty((b.S, M, b.d), np.float64)
    _check(lib().orc_pool(b.pk, b.pl, b.S, b.Lmax, b.d, B, out.ctypes.data_as(_P)), "pool")
    return out


def route(b: Batch, B, h, mode=0):
    g = np.empty((b.T, b.H), np.float64)
    heads = np.empty((b.T, h), np.int32)
    _check(lib().orc_route(*b.head(), B, h, mode, g.ctypes.data_as(_P),
                           heads.ctypes.data_as(_P)), "route")
    return heads, g


def dsa(b: Batch, k, want_scores=False):
    idx = np.empty((b.T, k), np.int32)
    val = np.empty((b.T, k), np.float64)
    sc = np.empty((b.T, b.Lmax), np.float64) if want_scores else None
    _check(lib().orc_dsa(*b.head(), k, idx.ctypes.data_as(_P), val.ctypes.data_as(_P),
                         sc.ctypes.data_as(_P) if sc is not None else None), "dsa")
    return (idx, val, sc) if want_scores else (idx, val)


def misa(b: Batch, B, h, k, mode=0, want_scores=False):
    heads = np.empty((b.T, h), np.int32)
    g = np.empty((b.T, b.H), np.float64)
    idx = np.empty((b.T, k), np.int32)
    val = np.empty((b.T, k), np.float64)
    sc = np.empty((b.T, b.Lmax), np.float64) if want_scores else None
    _check(lib().orc_misa(*b.head(), B, h, mode, k, heads.ctypes.data_as(_P),
                          g.ctypes.data_as(_P), idx.ctypes.data_as(_P),
                          val.ctypes.data_as(_P),
                          sc.ctypes.data_as(_P) if sc is not None else None), "misa")
    out = dict(heads=heads, g=g, idx=idx, val=val)
    if want_scores:
        out["scores"] = sc
    return out


def rerank(b: Batch, cand, k):
    cand, pc = _c(cand, np.int32)
    idx = np.empty((b.T, k), np.int32)
    val = np.empty((b.T, k), np.float64)
    _check(lib().orc_rerank(*b.head(), pc, cand.shape[1], k, idx.ctypes.data_as(_P),
                            val.ctypes.data_as(_P)), "rerank")
    return idx, val


def hisa(b: Batch, B, m, k, heads=None):
    """The hierarchical block-to-token indexer (orc_hisa): all heads, or the
    given heads [T][h] in both stages.  Returns dict(idx, val, blocks, bscore)."""
    Mmax = (b.Lmax + B - 1) // B
    idx = np.empty((b.T, k), np.int32)
    val = np.empty((b.T, k), np.float64)
    blocks = np.empty((b.T, m), np.int32)
    bscore = np.empty((b.T, Mmax), np.float64)
    if heads is None:
        ph, h = None, 0
    else:
        heads, ph = _c(heads, np.int32)
        h = heads.shape[1]
    _check(lib().orc_hisa(*b.head(), B, m, ph, h, k, idx.ctypes.data_as(_P), val.ctypes.data_as(_P),
                          blocks.ctypes.data_as(_P), bscore.ctypes.data_as(_P)), "hisa")
    return dict(idx=idx, val=val, blocks=blocks, bscore=bscore)


def misa_dagger(b: Batch, B, h, kc, k, mode=0):
    heads = np.empty((b.T, h), np.int32)
    cand = np.empty((b.T, kc), np.int32)
    idx = np.empty((b.T, k), np.int32)
    val = np.empty((b.T, k), np.float64)
    _check(lib().orc_misa_dagger(*b.head(), B, h, mode, kc, k, heads.ctypes.data_as(_P),
                                 cand.ctypes.data_as(_P), idx.ctypes.data_as(_P),
                                 val.ctypes.data_as(_P)), "misa_dagger")
    return dict(heads=heads, cand=cand, idx=idx, val=val)
