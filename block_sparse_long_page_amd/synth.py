"""Seeded synthetic inputs: paged K/V caches, block tables and queries.

This module only draws inputs.  It holds none of the method's arithmetic
(no summaries, scores, selection or attention) and is shared by the tests,
the smoke check and the benchmark on both sides of every parity check.

Conventions
-----------
* K and V are stored paged, each ``[num_phys_pages][Hkv][P][hd]``; one
  (page, KV head) slab is ``P*hd`` contiguous elements.
* ``block_table[b][p]`` maps logical page p of sequence b to a physical page;
  entries past the sequence's last page are -1.
* bf16 values are the round-to-nearest-even image of fp32 draws and are kept
  as their uint16 bit patterns; fp32 values are kept as float32.
* ``q`` is ``[B][Hq][Q][hd]`` in the cache dtype; query row i of sequence b
  sits at position ``seq_lens[b] - Q + i``.
* Draws use ``numpy.random.default_rng(seed)`` (the generator family the
  course module's needle exercise uses).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

from .configs import BF16, DTYPE_NAMES, F32, MODE_NAMES, Workload


# ---------------------------------------------------------------------------
# bf16 bit patterns
# ---------------------------------------------------------------------------

def _round_chunk(c: np.ndarray, o: np.ndarray) -> None:
    r = c >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += c
    r >>= np.uint32(16)
    nan = (c & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        r[nan] = (c[nan] >> np.uint32(16)) | np.uint32(0x40)
    o[:] = r


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 20
    spans = [(s, min(flat_u.size, s + step)) for s in range(0, flat_u.size, step)]
    if len(spans) <= 1:
        for s, e in spans:
            _round_chunk(flat_u[s:e], flat_o[s:e])
    else:
        with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(lambda se: _round_chunk(flat_u[se[0]:se[1]], flat_o[se[0]:se[1]]), spans))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f32(arr: np.ndarray, dtype: int) -> np.ndarray:
    """The float32 value of stored elements (exact for both dtypes)."""
    return bf16_bits_to_f32(arr) if dtype == BF16 else np.asarray(arr, dtype=np.float32)


def store(x: np.ndarray, dtype: int) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == BF16 else np.ascontiguousarray(x, dtype=np.float32)


# ---------------------------------------------------------------------------
# containers
# ---------------------------------------------------------------------------

@dataclass
class Cache:
    B: int
    Hq: int
    Hkv: int
    hd: int
    P: int
    max_pages: int
    num_phys: int
    dtype: int  # F32 | BF16
    k: np.ndarray  # [num_phys][Hkv][P][hd]
    v: np.ndarray
    block_table: np.ndarray  # int32 [B][max_pages]
    seq_lens: np.ndarray  # int32 [B]


@dataclass
class Problem:
    cache: Cache
    q: np.ndarray  # [B][Hq][Q][hd] in the cache dtype
    Q: int
    sink: int
    window: int
    budget: int
    mode: int
    needles: List[Tuple[int, int, int]] = field(default_factory=list)  # (b, kvh, logical page)
    name: str = ""

    @property
    def k_pages(self) -> int:
        return self.budget // self.cache.P


# ---------------------------------------------------------------------------
# samplers
# ---------------------------------------------------------------------------

def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def _unit(rng: np.random.Generator, n: int, d: int) -> np.ndarray:
    g = rng.standard_normal((n, d))
    return g / np.linalg.norm(g, axis=1, keepdims=True)


def sample_vmf(rng: np.random.Generator, mu: np.ndarray, kappa: float, n: int) -> np.ndarray:
    """n unit vectors from the von Mises-Fisher law with concentration kappa
    and mean direction mu ([d], or one row per sample [n][d]), by Wood's
    (1994) rejection sampler for the cosine w and a uniform direction in the
    tangent space of the mean."""
    mu = np.asarray(mu, dtype=np.float64)
    d = mu.shape[-1]
    mus = np.broadcast_to(mu, (n, d)) if mu.ndim == 1 else mu
    assert mus.shape == (n, d)
    m1 = d - 1.0
    b = (-2.0 * kappa + np.sqrt(4.0 * kappa * kappa + m1 * m1)) / m1
    x0 = (1.0 - b) / (1.0 + b)
    c = kappa * x0 + m1 * np.log(1.0 - x0 * x0)
    w = np.empty(n)
    filled = 0
    while filled < n:
        m = max(16, int((n - filled) * 1.3))
        z = rng.beta(m1 / 2.0, m1 / 2.0, size=m)
        u = rng.random(m)
        ww = (1.0 - (1.0 + b) * z) / (1.0 - (1.0 - b) * z)
        ok = kappa * ww + m1 * np.log(1.0 - x0 * ww) - c >= np.log(u)
        got = ww[ok][: n - filled]
        w[filled:filled + got.size] = got
        filled += got.size
    g = rng.standard_normal((n, d))
    g -= np.einsum("nd,nd->n", g, mus)[:, None] * mus
    g /= np.linalg.norm(g, axis=1, keepdims=True)
    return w[:, None] * mus + np.sqrt(np.maximum(0.0, 1.0 - w * w))[:, None] * g


_CHUNK_PAGES = 64


def _fill_pages(k: np.ndarray, v: np.ndarray, rng: np.random.Generator, dt: int, *, mu=None,
                cluster_noise: float = 0.5, out_ch=None, outlier_scale: float = 8.0) -> None:
    """Fill k and v ([num_phys][Hkv][P][hd]) chunk by chunk of physical pages.
    Each chunk draws from its own child generator (spawned from `rng`), so the
    result depends only on the seed, and chunks fill in parallel threads."""
    num_phys, Hkv, P, hd = v.shape
    starts = list(range(0, num_phys, _CHUNK_PAGES))
    children = rng.spawn(len(starts))

    def fill(i):
        s = starts[i]
        e = min(num_phys, s + _CHUNK_PAGES)
        r = children[i]
        if k is None:
            pass
        elif mu is not None:
            ids = r.integers(0, mu.shape[1], size=(e - s, Hkv, P))
            kk = _normal(r, (e - s, Hkv, P, hd))
            kk *= np.float32(cluster_noise)
            kk += mu[np.arange(Hkv)[None, :, None], ids]
        else:
            kk = _normal(r, (e - s, Hkv, P, hd))
        if out_ch is not None:
            kk[..., out_ch] *= np.float32(outlier_scale)
        if k is not None:
            k[s:e] = store(kk, dt)
        v[s:e] = store(_normal(r, (e - s, Hkv, P, hd)), dt)

    workers = min(16, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, range(len(starts))))


# ---------------------------------------------------------------------------
# generic random problem
# ---------------------------------------------------------------------------

def _block_table(rng, B, max_pages, P, seq_lens, shuffle: bool, spare_pages: int):
    used = [-(-int(L) // P) for L in seq_lens]
    num_phys = B * max_pages + spare_pages
    bt = np.full((B, max_pages), -1, dtype=np.int32)
    if shuffle:
        perm = rng.permutation(num_phys).astype(np.int32)
        i = 0
        for b in range(B):
            bt[b, : used[b]] = perm[i:i + used[b]]
            i += used[b]
    else:
        for b in range(B):
            bt[b, : used[b]] = b * max_pages + np.arange(used[b], dtype=np.int32)
    return bt, num_phys


def random_problem(
    *, B: int, Hq: int, Hkv: int, hd: int, P: int, seq_lens: Sequence[int], sink: int, window: int,
    budget: int, mode: str = "quest", dtype: str = "bf16", Q: int = 1, seed: int = 0,
    max_pages: Optional[int] = None, shuffle: bool = False, spare_pages: int = 0,
    needles_per_head: int = 0, outlier_channels: int = 0, outlier_scale: float = 8.0,
    clusters: int = 0, cluster_noise: float = 0.5, name: str = "",
) -> Problem:
    """K, V, q ~ N(0,1) (optionally clustered keys, outlier channels, needles)."""
    rng = np.random.default_rng(seed)
    dt = DTYPE_NAMES[dtype]
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.shape == (B,)
    if max_pages is None:
        max_pages = int(-(-int(seq_lens.max()) // P))
    bt, num_phys = _block_table(rng, B, max_pages, P, seq_lens, shuffle, spare_pages)

    q32 = _normal(rng, (B, Hq, Q, hd))
    q = store(q32, dt)
    qv = to_f32(q, dt)

    k = np.empty((num_phys, Hkv, P, hd), dtype=np.uint16 if dt == BF16 else np.float32)
    v = np.empty_like(k)
    mu = _normal(rng, (Hkv, clusters, hd)) if clusters else None
    out_ch = rng.choice(hd, size=outlier_channels, replace=False) if outlier_channels else None
    _fill_pages(k, v, rng, dt, mu=mu, cluster_noise=cluster_noise, out_ch=out_ch, outlier_scale=outlier_scale)

    needles: List[Tuple[int, int, int]] = []
    G = Hq // Hkv
    if needles_per_head:
        for b in range(B):
            L = int(seq_lens[b])
            lo = -(-sink // P)  # first page wholly after the sink
            hi = (L - window) // P  # pages wholly before the window
            for kvh in range(Hkv):
                if hi - lo < needles_per_head:
                    continue
                pages = rng.choice(np.arange(lo, hi), size=needles_per_head, replace=False)
                for p in sorted(int(x) for x in pages):
                    phys = bt[b, p]
                    # keys of the page point along the group's first q-head: k = 3 q + z
                    z = _normal(rng, (P, hd))
                    kk = np.float32(3.0) * qv[b, kvh * G, Q - 1][None, :] + z
                    k[phys, kvh] = store(kk, dt)
                    needles.append((b, kvh, p))

    cache = Cache(B=B, Hq=Hq, Hkv=Hkv, hd=hd, P=P, max_pages=max_pages, num_phys=num_phys, dtype=dt,
                  k=k, v=v, block_table=bt, seq_lens=seq_lens)
    return Problem(cache=cache, q=q, Q=Q, sink=sink, window=window, budget=budget, mode=MODE_NAMES[mode],
                   needles=needles, name=name)


# ---------------------------------------------------------------------------
# the named workloads
# ---------------------------------------------------------------------------

def workload_problem(wl: Workload, *, seed: Optional[int] = None, batch: Optional[int] = None,
                     context: Optional[int] = None, shuffle: bool = False) -> Problem:
    """Inputs of a single-layer workload (not the multi-layer schedule)."""
    seed = wl.seed if seed is None else seed
    B = wl.batch if batch is None else batch
    L = wl.context if context is None else context
    common = dict(B=B, Hq=wl.num_q_heads, Hkv=wl.num_kv_heads, hd=wl.head_dim, P=wl.page_size,
                  seq_lens=[L] * B, sink=wl.sink, window=wl.window, budget=wl.budget, mode=wl.mode,
                  dtype=wl.dtype, Q=wl.q_rows, seed=seed, shuffle=shuffle, name=wl.name)
    if wl.name.startswith("tiny"):
        return random_problem(**common, needles_per_head=1)
    if wl.name.startswith("qwen3"):
        return random_problem(**common, needles_per_head=4, outlier_channels=4, outlier_scale=8.0)
    if wl.name.startswith("llama3"):
        return random_problem(**common, clusters=64, cluster_noise=0.5)
    if wl.name.startswith("keydiff"):
        return random_problem(**common, clusters=64, cluster_noise=0.5, needles_per_head=4)
    if wl.name.startswith("semantic"):
        return semantic_problem(wl, seed=seed, batch=B)
    raise ValueError(f"no single-layer generator for {wl.name}")


def semantic_problem(wl: Workload, *, seed: Optional[int] = None, batch: Optional[int] = None,
                     blocks: int = 256, block_tokens: int = 2048, kappa: float = 100.0,
                     q_kappa: float = 50.0, topics: int = 4, scatter: bool = False) -> Problem:
    """Keys from `blocks` von Mises-Fisher clusters per (b, KV head) on the unit
    sphere scaled by sqrt(hd), exactly `block_tokens` per cluster, stored
    cluster by cluster (the permuted, block-contiguous layout), one cluster per
    page of P = block_tokens.  With `scatter` the prefix tokens of each
    (b, KV head) are instead placed in a seeded random order (a document in
    which the semantic blocks are interleaved; the index builder's input).
    The current chunk of Q queries is appended as a final partial page; each
    query row and chunk key follows one of `topics` clusters drawn per
    (b, KV head)."""
    seed = wl.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    B = wl.batch if batch is None else batch
    Hq, Hkv, hd, P, Q = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size, wl.q_rows
    assert P == block_tokens
    L = blocks * block_tokens + Q
    max_pages = blocks + 1
    dt = DTYPE_NAMES[wl.dtype]
    bt, num_phys = _block_table(rng, B, max_pages, P, [L] * B, False, 0)
    k = np.empty((num_phys, Hkv, P, hd), dtype=np.uint16)
    v = np.empty_like(k)
    q = np.empty((B, Hq, Q, hd), dtype=np.uint16)
    G = Hq // Hkv
    scale = np.float32(np.sqrt(hd))
    per = 32  # clusters drawn per batch
    children = rng.spawn(B * Hkv + 1)

    def head(i):
        b, kvh = divmod(i, Hkv)
        r = children[i]
        mus = _unit(r, blocks, hd)
        order = r.permutation(blocks * block_tokens) if scatter else None  # position of each clustered token
        for j0 in range(0, blocks, per):
            j1 = min(blocks, j0 + per)
            u = sample_vmf(r, np.repeat(mus[j0:j1], block_tokens, axis=0), kappa, (j1 - j0) * block_tokens)
            kk = store(u.astype(np.float32).reshape(j1 - j0, block_tokens, hd) * scale, dt)
            if order is None:
                for j in range(j0, j1):
                    k[bt[b, j], kvh] = kk[j - j0]
            else:
                pos = order[j0 * block_tokens:j1 * block_tokens]
                k[bt[b, pos // P], kvh, pos % P] = kk.reshape(-1, hd)
        topic = r.choice(blocks, size=topics, replace=False)
        row_topic = topic[r.integers(0, topics, size=Q)]
        ck = np.zeros((P, hd), dtype=np.float32)
        ck[:Q] = sample_vmf(r, mus[row_topic], kappa, Q).astype(np.float32) * scale
        k[bt[b, blocks], kvh] = store(ck, dt)
        qq = sample_vmf(r, np.tile(mus[row_topic], (G, 1)), q_kappa, G * Q).astype(np.float32) * scale
        q[b, kvh * G:(kvh + 1) * G] = store(qq.reshape(G, Q, hd), dt)

    with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(head, range(B * Hkv)))
    _fill_pages(None, v, children[-1], dt)
    cache = Cache(B=B, Hq=Hq, Hkv=Hkv, hd=hd, P=P, max_pages=max_pages, num_phys=num_phys, dtype=dt,
                  k=k, v=v, block_table=bt, seq_lens=np.full(B, L, dtype=np.int32))
    return Problem(cache=cache, q=q, Q=Q, sink=wl.sink, window=wl.window, budget=wl.budget,
                   mode=MODE_NAMES[wl.mode], name=wl.name)


@dataclass
class HybridSchedule:
    """Inputs of the multi-layer decode schedule: one cache per layer holding
    all tokens up to the last step (the first `context` are the prompt, one
    more is appended per step), and one query per (step, layer)."""

    caches: List[Cache]
    q: List[np.ndarray]  # per layer: [steps][B][Hq][1][hd]
    context: int
    steps: int
    refresh: int
    sink: int
    windows: List[int]
    budgets: List[int]
    mode: int
    name: str = ""


def hybrid_schedule(wl: Workload, *, seed: Optional[int] = None, batch: Optional[int] = None,
                    context: Optional[int] = None, steps: Optional[int] = None) -> HybridSchedule:
    seed = wl.seed if seed is None else seed
    B = wl.batch if batch is None else batch
    L0 = wl.context if context is None else context
    T = wl.steps if steps is None else steps
    caches, qs = [], []
    for li, layer in enumerate(wl.layers):
        pr = random_problem(B=B, Hq=wl.num_q_heads, Hkv=wl.num_kv_heads, hd=wl.head_dim, P=wl.page_size,
                            seq_lens=[L0 + T] * B, sink=wl.sink, window=layer.window, budget=layer.budget,
                            mode=wl.mode, dtype=wl.dtype, Q=1, seed=seed * 1000 + li)
        rng = np.random.default_rng(seed * 1000 + 100 + li)
        qs.append(store(_normal(rng, (T, B, wl.num_q_heads, 1, wl.head_dim)), DTYPE_NAMES[wl.dtype]))
        caches.append(pr.cache)
    return HybridSchedule(caches=caches, q=qs, context=L0, steps=T, refresh=wl.refresh, sink=wl.sink,
                          windows=[l.window for l in wl.layers], budgets=[l.budget for l in wl.layers],
                          mode=MODE_NAMES[wl.mode], name=wl.name)


def prefill_queries(pr: Problem, *, seed: int = 0, topics: int = 4, q_kappa: float = 50.0) -> np.ndarray:
    """Query rows for every position of a problem's cache (a prompt to
    prefill): per (b, KV head) `topics` directions, the unit keys at random
    positions (a key lies close to its cluster's direction); each row follows
    one of them for every head of the group (von Mises-Fisher, concentration
    q_kappa), scaled by sqrt(hd).  [B][Hq][L][hd] in the cache dtype."""
    c = pr.cache
    L = int(c.seq_lens[0])
    G = c.Hq // c.Hkv
    n_pages = -(-L // c.P)
    q = np.empty((c.B, c.Hq, L, c.hd), dtype=np.uint16 if c.dtype == BF16 else np.float32)
    children = np.random.default_rng(seed).spawn(c.B * c.Hkv)

    def head(i):
        b, kvh = divmod(i, c.Hkv)
        r = children[i]
        keys = to_f32(c.k[c.block_table[b, :n_pages], kvh], c.dtype).reshape(-1, c.hd)[:L]
        dirs = keys[r.integers(0, L, size=topics)].astype(np.float64)
        dirs /= np.maximum(np.linalg.norm(dirs, axis=1, keepdims=True), 1e-30)
        row_topic = r.integers(0, topics, size=L)
        for g in range(G):
            u = sample_vmf(r, dirs[row_topic], q_kappa, L).astype(np.float32) * np.float32(np.sqrt(c.hd))
            q[b, kvh * G + g] = store(u, c.dtype)

    with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(head, range(c.B * c.Hkv)))
    return q

