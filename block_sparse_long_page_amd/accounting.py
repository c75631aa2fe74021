"""Byte and FLOP accounting of one decode step (host arithmetic only).

Algorithmic bytes are what the method must move: the deduplicated K and V of
the attended token set (sink, window and selected pages, once per (sequence,
KV head)), the page summaries that selection reads, the query, the split
partials and the output.  They are *not* the dense cache the method avoids.

The KV-size formula is the pages' own: 2 (K and V) x layers x KV heads x head
dim x bytes per element per token (self-indexing attention page, "How much
memory the KV cache eats"; course module 14, section 14.1).  The FLOP ratio of
a block-sparse pattern follows course module 14, exercise 14.1.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Sequence

ELEM_BYTES = {0: 4, 1: 2}  # F32, BF16


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * layers * kv_heads * head_dim * elem_bytes


def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, elem_bytes: int, tokens: int, batch: int = 1) -> int:
    return kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes) * tokens * batch


def dense_flops(n: int, d: int) -> int:
    """QK^T and PV over a causal-free n x n square: 2 n^2 d each."""
    return 4 * n * n * d


def block_sparse_flops(n: int, d: int, block: int, topk: int) -> int:
    """The same two products restricted to topk key blocks per query block."""
    return 4 * (n // block) * topk * block * block * d


def regions(L: int, S: int, W: int):
    """(sink end, window start): sink [0, se), middle [se, ws), window [ws, L)."""
    se = min(S, L)
    ws = max(se, L - W)
    return se, ws


def candidate_pages(L: int, P: int, S: int, W: int) -> int:
    """Pages with at least one token in the middle region."""
    se, ws = regions(L, S, W)
    if ws <= se:
        return 0
    return (ws - 1) // P - se // P + 1


def attended_tokens(L: int, P: int, S: int, W: int, k: int) -> int:
    """Tokens attended by the last position when the k selected pages are whole
    middle pages (the usual case; exact when S and L-W are page-aligned)."""
    se, ws = regions(L, S, W)
    mid = ws - se
    return se + min(mid, k * P) + (L - ws)


@dataclass
class StepBytes:
    kv: int  # attended K + V
    meta: int  # page summaries read by selection
    q: int
    partials: int  # split partials written by decode and read by combine (x2)
    out: int

    @property
    def total(self) -> int:
        return self.kv + self.meta + self.q + self.partials + self.out

    def as_dict(self) -> Dict[str, int]:
        return dict(kv=self.kv, meta=self.meta, q=self.q, partials=self.partials, out=self.out, total=self.total)


def summary_bytes_per_page(mode: int, head_dim: int, elem_bytes: int) -> int:
    """Per (page, KV head): Quest min+max in the KV dtype, mean/centroid fp32."""
    return 2 * head_dim * elem_bytes if mode == 0 else 4 * head_dim


def decode_step_bytes(*, B: int, Hq: int, Hkv: int, hd: int, elem_bytes: int, L: int, P: int, S: int, W: int,
                      budget: int, mode: int, splits: int, Q: int = 1, attended: Sequence[int] = None,
                      out_bytes: int = None) -> StepBytes:
    """Algorithmic bytes of select + decode + combine for one step.
    `attended` (optional) gives the exact attended-token count per (b, kvh)."""
    k = budget // P
    if attended is None:
        ntok = B * Hkv * attended_tokens(L, P, S, W, k)
    else:
        ntok = int(sum(attended))
    kv = ntok * 2 * hd * elem_bytes
    meta = B * Hkv * Q * candidate_pages(L, P, S, W) * summary_bytes_per_page(mode, hd, elem_bytes)
    qb = B * Hq * Q * hd * elem_bytes
    rows = B * Hq * Q
    partials = 2 * rows * splits * (hd + 2) * 4
    ob = rows * hd * (elem_bytes if out_bytes is None else out_bytes) + rows * 4
    return StepBytes(kv=kv, meta=meta, q=qb, partials=partials, out=ob)


def decode_kernel_bytes(*, B: int, Hq: int, Hkv: int, hd: int, elem_bytes: int, ntok_total: int, splits: int,
                        Q: int = 1, sel_entries: int = 0) -> int:
    """Bytes one launch of the decode kernel must move: attended K+V, q, the
    selected page list it reads and the partials it writes."""
    rows = B * Hq * Q
    return ntok_total * 2 * hd * elem_bytes + rows * hd * elem_bytes + 4 * sel_entries + rows * splits * (hd + 2) * 4


def select_decode_bytes(*, B: int, Hq: int, Hkv: int, hd: int, elem_bytes: int, ntok_total: int, splits: int,
                        meta: int, n_cand: int, k_max: int, Q: int = 1) -> int:
    """Bytes the score launch and the select-and-decode launch of one selecting
    step must move: the page summaries, q, the fp32 page scores (written, then
    read), the attended K+V, the page list written (k_max entries and a count
    per problem) and the partials written."""
    rows = B * Hq * Q
    problems = B * Hkv * Q
    scores = problems * n_cand * 4
    return (meta + rows * hd * elem_bytes + 2 * scores + ntok_total * 2 * hd * elem_bytes +
            problems * (k_max + 1) * 4 + rows * splits * (hd + 2) * 4)


def attended_tokens_exact(L: int, P: int, S: int, W: int, pages, Q: int = 1, row: int = None) -> int:
    """Tokens attended by query row `row` (default: the last) given the
    selected logical pages: the sink, the window and the middle part of each
    selected page, each position once, positions <= the row's own."""
    import numpy as np

    row = Q - 1 if row is None else row
    pos = L - Q + row
    se, ws = regions(L, S, W)
    n = min(se, pos + 1) + max(0, min(L, pos + 1) - ws)
    for p in np.unique(np.asarray(pages, dtype=np.int64)):
        a = max(int(p) * P, se)
        z = min((int(p) + 1) * P, ws, pos + 1)
        n += max(0, z - a)
    return n


def grouped_step_bytes(*, B: int, Hq: int, Hkv: int, hd: int, elem_bytes: int, Q: int, n_cand: int, k_max: int,
                       mode: int, union_tokens: int, local_tokens: int, stride: int) -> StepBytes:
    """Algorithmic bytes of one multi-query step decoded by page: the page
    summaries once per (sequence, KV head), q, the per-row page scores
    (written and read back) and page lists, the K+V of the union of the rows'
    selected pages (`union_tokens` middle tokens over all (b, kvh)) and of
    the sink and window (`local_tokens`, each read once per (b, kvh)), the
    partials (`stride` slots per row, written and read) and the output."""
    rows = B * Hq * Q
    problems = B * Hkv * Q
    meta = B * Hkv * n_cand * summary_bytes_per_page(mode, hd, elem_bytes)
    scores = 2 * problems * n_cand * 4 + problems * (k_max + 1) * 4
    kv = (union_tokens + local_tokens) * 2 * hd * elem_bytes
    partials = 2 * rows * stride * (hd + 2) * 4
    out = rows * hd * elem_bytes + rows * 4
    return StepBytes(kv=kv, meta=meta + scores, q=rows * hd * elem_bytes, partials=partials, out=out)

