"""fp64 CPU oracle for block/page-sparse decode attention -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product library never does, and it shares
no code with it.  The arithmetic lives in ``oracle.c`` (plain C, IEEE double,
sums in index order); this file only marshals numpy arrays through ctypes.

Each function follows one step of the method as the pages state it; the C
file's header lists the passages.  Parity pins for every function are in
``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

QUEST, MEAN, CENTROID, COMPRESSED = 0, 1, 2, 3


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Cache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("B", "Hq", "Hkv", "hd", "P", "max_pages", "num_phys", "dtype")] + [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.orc_run.restype = ctypes.c_int
        lib.orc_run.argtypes = [P, ctypes.c_int, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_double, P, P, ctypes.c_int, P, P, P, P, P, P, P, ctypes.c_int]
        lib.orc_page_summary.restype = ctypes.c_int
        lib.orc_page_summary.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, P]
        lib.orc_page_score.restype = ctypes.c_double
        lib.orc_page_score.argtypes = [ctypes.c_int, P, P, ctypes.c_int]
        lib.orc_topk.restype = ctypes.c_int
        lib.orc_topk.argtypes = [P, P, ctypes.c_int, ctypes.c_int, P]
        lib.orc_merge.restype = None
        lib.orc_merge.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, P, P]
        lib.orc_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


class _Bound:
    """Keeps the numpy buffers of a cache alive while C holds their pointers."""

    def __init__(self, cache):
        self.k = np.ascontiguousarray(cache.k)
        self.v = np.ascontiguousarray(cache.v)
        self.bt = np.ascontiguousarray(cache.block_table, dtype=np.int32)
        self.sl = np.ascontiguousarray(cache.seq_lens, dtype=np.int32)
        self.s = _Cache(cache.B, cache.Hq, cache.Hkv, cache.hd, cache.P, cache.max_pages, cache.num_phys,
                        cache.dtype, self.k.ctypes.data, self.v.ctypes.data, self.bt.ctypes.data,
                        self.sl.ctypes.data)


def max_threads() -> int:
    return int(_load().orc_max_threads())


def summary_size(mode: int, hd: int) -> int:
    return 2 * hd if mode == QUEST else hd


def page_summary(cache, mode: int, b: int, kvh: int, page: int):
    """Summary of one logical page over its valid tokens; returns (summary, n_valid).
    Quest: [min(hd), max(hd)]; mean: [hd]; centroid: unit-norm [hd]."""
    lib = _load()
    bc = _Bound(cache)
    out = np.zeros(summary_size(mode, cache.hd), dtype=np.float64)
    n = lib.orc_page_summary(ctypes.byref(bc.s), mode, b, kvh, page, _ptr(out))
    return out, int(n)


def page_score(mode: int, summ: np.ndarray, q: np.ndarray) -> float:
    summ = np.ascontiguousarray(summ, dtype=np.float64)
    q = np.ascontiguousarray(q, dtype=np.float64)
    return float(_load().orc_page_score(mode, _ptr(summ), _ptr(q), q.size))


def topk(score: np.ndarray, cand: np.ndarray, k: int) -> np.ndarray:
    score = np.ascontiguousarray(score, dtype=np.float64)
    cand = np.ascontiguousarray(cand, dtype=np.uint8)
    sel = np.zeros(max(1, score.size), dtype=np.int32)
    n = _load().orc_topk(_ptr(score), _ptr(cand), score.size, k, _ptr(sel))
    return sel[:n].copy()


def merge(o: np.ndarray, m: np.ndarray, l: np.ndarray):
    """Log-sum-exp merge of partial states o[n][hd] (normalised), m[n], l[n]."""
    o = np.ascontiguousarray(o, dtype=np.float64)
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    out = np.zeros(o.shape[1], dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    _load().orc_merge(o.shape[0], o.shape[1], _ptr(o), _ptr(m), _ptr(l), _ptr(out), _ptr(lse))
    return out, float(lse[0])


@dataclass
class Result:
    sel: np.ndarray  # int32 [B][Hkv][Q][kmax], ascending, -1 padded
    cnt: np.ndarray  # int32 [B][Hkv][Q]
    out: np.ndarray  # float64 [B][Hq][Q][hd]
    lse: np.ndarray  # float64 [B][Hq][Q]
    ntok: np.ndarray  # int32 [B][Hq][Q]
    scores: Optional[np.ndarray] = None  # float64 [B][Hkv][Q][max_pages], NaN = not a candidate
    head_scores: Optional[np.ndarray] = None  # float64 [B][Hq][Q][max_pages]


def run(cache, q: np.ndarray, *, mode: int, Q: int, sink: int, window: int, budget: int,
        scale: Optional[float] = None, sel: Optional[np.ndarray] = None, cnt: Optional[np.ndarray] = None,
        want_scores: bool = False, want_head_scores: bool = False, threads: int = 0) -> Result:
    """Summaries -> scores -> per-KV-head top-k -> token set -> exact attention.
    With `sel`/`cnt` given, the selection steps are skipped and that page set
    is attended instead."""
    lib = _load()
    bc = _Bound(cache)
    q = np.ascontiguousarray(q)
    B, Hq, Hkv, hd, P = cache.B, cache.Hq, cache.Hkv, cache.hd, cache.P
    assert q.shape == (B, Hq, Q, hd)
    kmax = budget // P
    scale = 1.0 / np.sqrt(hd) if scale is None else float(scale)
    sel_out = np.full((B, Hkv, Q, max(kmax, 1)), -1, dtype=np.int32)
    cnt_out = np.zeros((B, Hkv, Q), dtype=np.int32)
    out = np.zeros((B, Hq, Q, hd), dtype=np.float64)
    lse = np.zeros((B, Hq, Q), dtype=np.float64)
    ntok = np.zeros((B, Hq, Q), dtype=np.int32)
    scores = np.zeros((B, Hkv, Q, cache.max_pages), dtype=np.float64) if want_scores else None
    hscores = np.zeros((B, Hq, Q, cache.max_pages), dtype=np.float64) if want_head_scores else None
    kmax_in = 0
    if sel is not None:
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        cnt = np.ascontiguousarray(cnt, dtype=np.int32)
        kmax_in = sel.shape[-1]
        assert sel.shape[:3] == (B, Hkv, Q) and cnt.shape == (B, Hkv, Q)
    rc = lib.orc_run(ctypes.byref(bc.s), mode, _ptr(q), Q, sink, window, budget, scale, _ptr(sel), _ptr(cnt),
                     kmax_in, _ptr(sel_out), _ptr(cnt_out), _ptr(scores), _ptr(hscores), _ptr(out), _ptr(lse),
                     _ptr(ntok), threads)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return Result(sel=sel_out[..., :kmax], cnt=cnt_out, out=out, lse=lse, ntok=ntok, scores=scores,
                  head_scores=hscores)
