"""Test-only numpy references, written independently of the oracle.

`dense_keys_values` gathers a sequence's keys and values through its block
table; `masked_attention` is textbook softmax attention with an additive
-inf mask (course module 14, exercise 14.1 computes attention the same way:
logits q.k/sqrt(d) plus a mask, max-subtracted, exponentiated, normalised).
"""
from __future__ import annotations

import numpy as np

from block_sparse_long_page_amd.synth import to_f32


def dense_keys_values(cache, b: int, kvh: int):
    L = int(cache.seq_lens[b])
    n_pages = -(-L // cache.P)
    phys = cache.block_table[b, :n_pages]
    K = to_f32(cache.k[phys, kvh], cache.dtype).astype(np.float64).reshape(-1, cache.hd)[:L]
    V = to_f32(cache.v[phys, kvh], cache.dtype).astype(np.float64).reshape(-1, cache.hd)[:L]
    return K, V


def masked_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, allowed: np.ndarray, scale: float):
    """q [hd]; K, V [L][hd]; allowed bool [L].  Returns (out [hd], lse)."""
    logits = (K @ q) * scale + np.where(allowed, 0.0, -np.inf)
    m = logits.max()
    w = np.exp(logits - m)
    s = w.sum()
    return (w @ V) / s, m + np.log(s)


def query(problem, b: int, h: int, i: int) -> np.ndarray:
    return to_f32(problem.q[b, h, i], problem.cache.dtype).astype(np.float64)


def seq_dot(a: np.ndarray, b: np.ndarray) -> float:
    """a.b summed strictly in index order (cumsum is sequential)."""
    return float(np.cumsum(np.asarray(a, np.float64) * np.asarray(b, np.float64))[-1])
