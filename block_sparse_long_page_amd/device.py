"""Device buffers and a step runner on top of the C ABI.

PyTorch only provides device memory and the stream; every computation is a
call into libsparse_attn.so.  `SparseDecoder.step` runs one decode step:
select (scores + per-KV-head top-k) -> decode (split-K attention) -> combine.
"""
from __future__ import annotations

import contextlib
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import binding as B
from .synth import Cache

_TORCH_ELEM = {B.SA_F32: torch.float32, B.SA_BF16: torch.int16}


def on_stream(stream):
    """Context manager that queues torch's own work (fills, copies) on the
    stream the library calls use: `stream` is None (torch's current stream),
    a raw stream handle or a torch stream."""
    if stream is None:
        return contextlib.nullcontext()
    if isinstance(stream, int):
        stream = torch.cuda.ExternalStream(stream)
    return torch.cuda.stream(stream)


def to_device(arr: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


@dataclass
class DeviceCache:
    B: int
    Hq: int
    Hkv: int
    hd: int
    P: int
    max_pages: int
    num_phys: int
    dtype: int
    k: torch.Tensor
    v: torch.Tensor
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    max_seq_len: int
    # the lengths' value once the queued work has run, when a chunked prefill
    # advanced them itself (None: unknown, so the next chunk sets them)
    known_len: Optional[int] = None

    @classmethod
    def from_host(cls, c: Cache, device="cuda", max_seq_len: Optional[int] = None) -> "DeviceCache":
        msl = int(max_seq_len if max_seq_len is not None else max(1, int(np.max(c.seq_lens))))
        return cls(c.B, c.Hq, c.Hkv, c.hd, c.P, c.max_pages, c.num_phys, c.dtype, to_device(c.k, device),
                   to_device(c.v, device), to_device(c.block_table.astype(np.int32), device),
                   to_device(c.seq_lens.astype(np.int32), device), msl)

    @classmethod
    def empty(cls, B_: int, Hq: int, Hkv: int, hd: int, P: int, tokens: int, dtype: int,
              device="cuda") -> "DeviceCache":
        """A cache of `tokens` token slots per sequence, pages laid out in
        order (sequence b owns physical pages b*n .. b*n+n-1), lengths 0."""
        n = -(-tokens // P)
        k = torch.zeros((B_ * n, Hkv, P, hd), dtype=_TORCH_ELEM[dtype], device=device)
        bt = torch.arange(B_ * n, dtype=torch.int32, device=device).reshape(B_, n)
        return cls(B_, Hq, Hkv, hd, P, n, B_ * n, dtype, k, torch.zeros_like(k), bt,
                   torch.zeros(B_, dtype=torch.int32, device=device), n * P)

    def desc(self, block_table: Optional[torch.Tensor] = None) -> B.sa_kv_desc:
        return B.make_kv_desc(batch=self.B, num_q_heads=self.Hq, num_kv_heads=self.Hkv, head_dim=self.hd,
                               page_size=self.P, max_pages_per_seq=self.max_pages, num_phys_pages=self.num_phys,
                               max_seq_len=self.max_seq_len, dtype=self.dtype, k_cache=self.k, v_cache=self.v,
                               block_table=self.block_table if block_table is None else block_table,
                               seq_lens=self.seq_lens)

    def meta_shape(self, mode: int):
        if mode == B.SA_QUEST:
            return (self.B, self.Hkv, self.max_pages, 2, self.hd)
        return (self.B, self.Hkv, self.max_pages, self.hd)

    def new_meta(self, mode: int) -> torch.Tensor:
        dt = _TORCH_ELEM[self.dtype] if mode == B.SA_QUEST else torch.float32
        return torch.zeros(self.meta_shape(mode), dtype=dt, device=self.k.device)


class SparseDecoder:
    """Buffers and calls of one decode step for a fixed shape."""

    def __init__(self, cache: DeviceCache, *, mode: int, Q: int, sink: int, window: int, budget: int,
                 splits: Optional[int] = None, out_dtype: Optional[int] = None, meta: Optional[torch.Tensor] = None):
        self.c = cache
        self.mode, self.Q, self.sink, self.window, self.budget = mode, Q, sink, window, budget
        self.k_max = budget // cache.P
        self.desc = cache.desc()
        dev = cache.k.device
        self.meta = meta if meta is not None else cache.new_meta(mode)
        self.sel = torch.full((cache.B, cache.Hkv, Q, max(1, self.k_max)), -1, dtype=torch.int32, device=dev)
        self.count = torch.zeros((cache.B, cache.Hkv, Q), dtype=torch.int32, device=dev)
        self.ws_bytes = B.sparse_attn_workspace_bytes(self.desc, Q)
        self.ws = torch.empty(max(1, self.ws_bytes), dtype=torch.uint8, device=dev)
        self.splits = splits or B.sparse_attn_default_splits(self.desc, Q, sink, window, self.k_max)
        rows = cache.B * cache.Hq * Q
        self.rows = rows
        self.part_o = torch.empty((rows, self.splits, cache.hd), dtype=torch.float32, device=dev)
        self.part_ml = torch.empty((rows, self.splits, 2), dtype=torch.float32, device=dev)
        self.out_dtype = cache.dtype if out_dtype is None else out_dtype
        self.out = torch.empty((rows, cache.hd), dtype=_TORCH_ELEM[self.out_dtype], device=dev)
        self.lse = torch.empty((rows,), dtype=torch.float32, device=dev)
        # the merging decode's counters: zero before the first call, and every call leaves them zero
        self.counters = torch.zeros(max(1, B.sparse_attn_merge_counters(self.desc, Q)), dtype=torch.int32,
                                    device=dev)

    def build_meta(self, page_begin: int = 0, page_end: Optional[int] = None, stream=None):
        B.sparse_attn_build_page_meta(self.desc, self.mode, page_begin,
                                      self.c.max_pages if page_end is None else page_end, self.meta, stream)

    def select(self, q: torch.Tensor, window: Optional[int] = None, stream=None):
        B.sparse_attn_select(self.desc, q, self.Q, self.meta, self.mode, self.sink,
                             self.window if window is None else window, self.budget, self.sel, self.count, self.ws,
                             self.ws_bytes, stream)

    def decode(self, q: torch.Tensor, window: Optional[int] = None, dense: bool = False, scale: float = 0.0,
               parts: int = B.SA_PART_ALL, stream=None):
        B.sparse_attn_decode(self.desc, q, self.Q, None if dense else self.sel, None if dense else self.count,
                             self.k_max, self.sink, self.window if window is None else window, parts, scale,
                             self.splits, 0, self.part_o, self.part_ml, stream)

    def select_decode(self, q: torch.Tensor, scale: float = 0.0, stream=None):
        """Selection and decode of a selecting step (sparse_attn_decode_step)."""
        B.sparse_attn_decode_step(self.desc, q, self.Q, self.meta, self.mode, self.sink, self.window, self.budget,
                                  scale, self.splits, self.sel, self.count, self.ws, self.ws_bytes, self.part_o,
                                  self.part_ml, stream)

    def decode_merged(self, q: torch.Tensor, window: Optional[int] = None, scale: float = 0.0, advance: int = 0,
                      stream=None):
        """Decode of the kept pages with the merge in the kernel's own last
        workgroups (sparse_attn_decode_merged): out and lse in one launch; with
        `advance` > 0 every sequence's length then grows by that many tokens."""
        if advance:
            self.c.known_len = None
        B.sparse_attn_decode_merged(self.desc, q, self.Q, self.sel, self.count, self.k_max, self.sink,
                                    self.window if window is None else window, scale, self.splits, self.part_o,
                                    self.part_ml, self.out, self.out_dtype, self.lse, advance, self.counters, stream)

    def select_decode_merged(self, q: torch.Tensor, scale: float = 0.0, advance: int = 0, stream=None):
        """A selecting step whose decode kernel also merges
        (sparse_attn_decode_step_merged): out and lse in two launches."""
        if advance:
            self.c.known_len = None
        B.sparse_attn_decode_step_merged(self.desc, q, self.Q, self.meta, self.mode, self.sink, self.window,
                                         self.budget, scale, self.splits, self.sel, self.count, self.ws, self.ws_bytes,
                                         self.part_o, self.part_ml, self.out, self.out_dtype, self.lse, advance,
                                         stream)

    def fused_step(self, q: torch.Tensor, stream=None):
        self.select_decode(q, stream=stream)
        self.combine(stream=stream)
        return self.out

    def combine(self, stream=None, advance: int = 0):
        """The merge of the split partials; with `advance` > 0 the same launch
        then advances every sequence's length by that many tokens (the step's
        last kernel appending the next token)."""
        if advance:
            self.c.known_len = None
            B.sparse_attn_combine_advance(self.rows, self.c.hd, self.splits, self.part_o, self.part_ml, self.out,
                                          self.out_dtype, self.lse, self.c.seq_lens, self.c.B, advance, stream)
        else:
            B.sparse_attn_combine(self.rows, self.c.hd, self.splits, self.part_o, self.part_ml, self.out,
                                  self.out_dtype, self.lse, stream)

    def step(self, q: torch.Tensor, stream=None):
        self.select(q, stream=stream)
        self.decode(q, stream=stream)
        self.combine(stream=stream)
        return self.out

    # ---- host copies ------------------------------------------------------
    def out_f32(self) -> np.ndarray:
        o = self.out.cpu().numpy()
        if self.out_dtype == B.SA_BF16:
            o = (o.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        return o.reshape(self.c.B, self.c.Hq, self.Q, self.c.hd)

    def lse_f32(self) -> np.ndarray:
        return self.lse.cpu().numpy().reshape(self.c.B, self.c.Hq, self.Q)

    def selection(self):
        cnt = self.count.cpu().numpy()
        sel = self.sel.cpu().numpy()[..., : self.k_max]
        return sel, cnt


class OverlappedStep:
    """One decode step with the selection hidden behind the sink+window work.

    The sink and window do not depend on the selection, so their decode runs
    on a side stream while `sparse_attn_select` runs on the caller's stream;
    then the selected pages' middle tokens are decoded on the caller's stream.
    Both decodes write split partials into disjoint slots of one buffer, and
    one `sparse_attn_combine` merges them.  Streams keep the default priority.
    """

    def __init__(self, dec: SparseDecoder, local_splits: Optional[int] = None, middle_splits: Optional[int] = None):
        self.dec = dec
        c = dec.c
        self.sl = local_splits or max(1, dec.splits * 3 // 8)
        self.sm = middle_splits or max(1, dec.splits - self.sl)
        self.stride = self.sl + self.sm
        dev = c.k.device
        self.part_o = torch.empty((dec.rows, self.stride, c.hd), dtype=torch.float32, device=dev)
        self.part_ml = torch.empty((dec.rows, self.stride, 2), dtype=torch.float32, device=dev)
        self.side = torch.cuda.Stream(device=dev)
        self.fork = torch.cuda.Event()
        self.join = torch.cuda.Event()

    def decode_middle(self, q, desc, window):
        d = self.dec
        B.sparse_attn_decode(desc, q, d.Q, d.sel, d.count, d.k_max, d.sink, window, B.SA_PART_MIDDLE, 0.0,
                             self.sm, self.stride, self.part_o[:, self.sl:], self.part_ml[:, self.sl:])

    def step(self, q: torch.Tensor, desc=None, meta=None, window: Optional[int] = None, middle_events=None):
        d = self.dec
        desc = d.desc if desc is None else desc
        meta = d.meta if meta is None else meta
        window = d.window if window is None else window
        main = torch.cuda.current_stream()
        self.fork.record(main)
        self.side.wait_event(self.fork)
        with torch.cuda.stream(self.side):
            B.sparse_attn_decode(desc, q, d.Q, None, None, 0, d.sink, window, B.SA_PART_LOCAL, 0.0, self.sl,
                                 self.stride, self.part_o, self.part_ml, self.side)
        self.join.record(self.side)
        B.sparse_attn_select(desc, q, d.Q, meta, d.mode, d.sink, window, d.budget, d.sel, d.count, d.ws,
                             d.ws_bytes)
        if middle_events is not None:
            middle_events[0].record(main)
        self.decode_middle(q, desc, window)
        if middle_events is not None:
            middle_events[1].record(main)
        main.wait_event(self.join)
        B.sparse_attn_combine(d.rows, d.c.hd, self.stride, self.part_o, self.part_ml, d.out, d.out_dtype, d.lse)
        return d.out


class GroupedStep:
    """Multi-query decode grouped by page (sparse_attn_decode_grouped) on a
    SparseDecoder's page lists, merged into that decoder's output: every
    selected page is read once per (sequence, KV head) for all the rows that
    chose it."""

    def __init__(self, dec: SparseDecoder, token_splits: Optional[int] = None,
                 local_splits: Optional[int] = None):
        c = dec.c
        self.dec = dec
        # one workgroup per page up to 4096-token pages (measured best at 2048); sink + window
        # splits of about 512 tokens
        self.ts = token_splits or max(1, min(4, c.P // 4096))
        self.ls = local_splits or max(1, min(16, (dec.sink + dec.window + 511) // 512))
        self.stride = dec.k_max * self.ts + self.ls
        self.ws_bytes = B.sparse_attn_grouped_workspace_bytes(dec.desc)
        dev = c.k.device
        self.ws = torch.empty(max(1, self.ws_bytes), dtype=torch.uint8, device=dev)
        self.part_o = torch.empty((dec.rows, self.stride, c.hd), dtype=torch.float32, device=dev)
        self.part_ml = torch.empty((dec.rows, self.stride, 2), dtype=torch.float32, device=dev)

    def decode(self, q: torch.Tensor, window: Optional[int] = None, scale: float = 0.0, stream=None):
        d = self.dec
        B.sparse_attn_decode_grouped(d.desc, q, d.Q, d.sel, d.count, d.k_max, d.sink,
                                     d.window if window is None else window, scale, self.ts, self.ls, self.part_o,
                                     self.part_ml, self.ws, self.ws_bytes, stream)

    def combine(self, stream=None):
        d = self.dec
        B.sparse_attn_combine(d.rows, d.c.hd, self.stride, self.part_o, self.part_ml, d.out, d.out_dtype, d.lse,
                              stream)

    def step(self, q: torch.Tensor, stream=None):
        self.dec.select(q, stream=stream)
        self.decode(q, stream=stream)
        self.combine(stream=stream)
        return self.dec.out



class BlockIndex:
    """A semantic block index of a DeviceCache (sparse_attn_build_block_index)
    and the decode against it: block choice under a token budget
    (sparse_attn_select_blocks), the grouped decode of the chosen blocks plus
    the window of recent tokens (sparse_attn_decode_blocks) and the combine.

    The index covers positions [0, num_tokens); num_blocks defaults to one
    block per 2048 tokens (the semantic-blocks page's average block)."""

    def __init__(self, cache: DeviceCache, num_tokens: int, num_blocks: Optional[int] = None, Q: int = 1,
                 window: int = 64, budget: int = 0, k_max: Optional[int] = None,
                 token_splits: int = 1, local_splits: int = 1, out_dtype: Optional[int] = None):
        c = cache
        self.c, self.N, self.Q, self.window, self.budget = c, num_tokens, Q, window, budget
        self.C = num_blocks or max(1, -(-num_tokens // 2048))
        self.k_max = k_max or self.C
        self.ts, self.ls = token_splits, local_splits
        dev = c.k.device
        self.offsets = torch.zeros((c.B, c.Hkv, self.C + 1), dtype=torch.int32, device=dev)
        self.positions = torch.zeros((c.B, c.Hkv, self.N), dtype=torch.int32, device=dev)
        self.centres = torch.zeros((c.B, c.Hkv, self.C, c.hd), dtype=torch.float32, device=dev)
        self.k_blocks = torch.zeros((c.B, c.Hkv, self.N, c.hd), dtype=c.k.dtype, device=dev)
        self.v_blocks = torch.zeros_like(self.k_blocks)
        self.assignment = torch.zeros((c.B, c.Hkv, self.N), dtype=torch.int32, device=dev)
        self.desc = c.desc()
        self.index = B.make_block_index(num_tokens=self.N, num_blocks=self.C, offsets=self.offsets,
                                        positions=self.positions, centres=self.centres, k_blocks=self.k_blocks,
                                        v_blocks=self.v_blocks)
        self.build_ws_bytes = B.sparse_attn_index_workspace_bytes(self.desc, self.N, self.C)
        self.build_ws = torch.empty(max(1, self.build_ws_bytes), dtype=torch.uint8, device=dev)
        self.rows = c.B * c.Hq * Q
        self.sel = torch.full((c.B, c.Hkv, Q, self.k_max), -1, dtype=torch.int32, device=dev)
        self.count = torch.zeros((c.B, c.Hkv, Q), dtype=torch.int32, device=dev)
        self.stride = self.k_max * self.ts + self.ls
        self.ws_bytes = B.sparse_attn_blocks_workspace_bytes(self.desc, self.index)
        self.ws = torch.empty(max(1, self.ws_bytes), dtype=torch.uint8, device=dev)
        self.part_o = torch.empty((self.rows, self.stride, c.hd), dtype=torch.float32, device=dev)
        self.part_ml = torch.empty((self.rows, self.stride, 2), dtype=torch.float32, device=dev)
        self.out_dtype = c.dtype if out_dtype is None else out_dtype
        self.out = torch.empty((self.rows, c.hd), dtype=_TORCH_ELEM[self.out_dtype], device=dev)
        self.lse = torch.empty((self.rows,), dtype=torch.float32, device=dev)

    def build(self, iterations: int = 8, stream=None):
        B.sparse_attn_build_block_index(self.desc, iterations, self.index, self.assignment, self.build_ws,
                                        self.build_ws_bytes, stream)

    def select(self, q: torch.Tensor, stream=None):
        B.sparse_attn_select_blocks(self.desc, self.index, q, self.Q, self.budget, self.k_max, self.sel, self.count,
                                    stream)

    def decode(self, q: torch.Tensor, scale: float = 0.0, stream=None):
        B.sparse_attn_decode_blocks(self.desc, self.index, q, self.Q, self.sel, self.count, self.k_max, self.window,
                                    scale, self.ts, self.ls, self.part_o, self.part_ml, self.ws, self.ws_bytes,
                                    stream)

    def combine(self, stream=None):
        B.sparse_attn_combine(self.rows, self.c.hd, self.stride, self.part_o, self.part_ml, self.out, self.out_dtype,
                              self.lse, stream)

    def step(self, q: torch.Tensor, stream=None):
        self.select(q, stream=stream)
        self.decode(q, stream=stream)
        self.combine(stream=stream)
        return self.out

    def out_f32(self) -> np.ndarray:
        o = self.out.cpu().numpy()
        if self.out_dtype == B.SA_BF16:
            o = (o.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        return o.reshape(self.c.B, self.c.Hq, self.Q, self.c.hd)

    def lse_f32(self) -> np.ndarray:
        return self.lse.cpu().numpy().reshape(self.c.B, self.c.Hq, self.Q)


class ChunkedPrefill:
    """Sparse prefill of a prompt over one block index of the whole prompt
    (a built BlockIndex with num_tokens = the prompt length): the Q rows at
    [c0, c0 + Q) see the index only before their window [c0 + Q - window,
    c0 + Q), choose at most k_max blocks under the token budget, read each
    chosen block once for all the chunk's rows (split into token_splits
    chunks) plus the window causally, and combine.  The cache's lengths are
    set to c0 + Q for the chunk.

    fused=True: one call, sparse_attn_prefill_chunk (three launches: the
    front, the grouped decode of the blocks and the window's pages, the
    combine); fused=False: sparse_attn_blocks_visible,
    sparse_attn_select_blocks, sparse_attn_decode_blocks (the window by the
    per-row decode) and sparse_attn_combine_advance.  per_call > 1 (fused):
    chunks() runs up to that many consecutive chunks in one
    sparse_attn_prefill_chunks call (the same results as one call each)."""

    def __init__(self, ix: "BlockIndex", Q: int, window: int, k_max: Optional[int] = None, token_splits: int = 1,
                 local_splits: int = 1, out_dtype: Optional[int] = None, fused: bool = True, per_call: int = 1):
        c = ix.c
        self.ix, self.c, self.Q, self.window, self.fused = ix, c, Q, window, fused
        self.per_call = per_call if fused else 1
        self.k_max = k_max or ix.C
        self.ts, self.ls = token_splits, local_splits
        dev = c.k.device
        n = self.per_call
        # visible ends: [B][Hkv][C], or [per_call][B][Hkv][C] per chunk of a call
        self.ends = torch.zeros(((n,) if n > 1 else ()) + (c.B, c.Hkv, ix.C), dtype=torch.int32, device=dev)
        self.index = B.make_block_index(num_tokens=ix.N, num_blocks=ix.C, offsets=ix.offsets,
                                        positions=ix.positions, centres=ix.centres, k_blocks=ix.k_blocks,
                                        v_blocks=ix.v_blocks, visible_end=None if fused else self.ends)
        self.desc = c.desc()
        self.rows = c.B * c.Hq * Q
        self.sel = torch.full((c.B, c.Hkv, n * Q, self.k_max), -1, dtype=torch.int32, device=dev)
        self.count = torch.zeros((c.B, c.Hkv, n * Q), dtype=torch.int32, device=dev)
        self.last_n = 1  # chunks of the last call
        if fused:
            self.stride = B.sparse_attn_prefill_num_splits(self.desc, window, self.k_max, self.ts)
            if self.stride < 0:
                raise B.SparseAttnError(-self.stride, "sparse_attn_prefill_num_splits")
            self.ws_bytes = B.sparse_attn_prefill_chunks_workspace_bytes(self.desc, self.index, n)
        else:
            self.stride = self.k_max * self.ts + self.ls
            self.ws_bytes = B.sparse_attn_blocks_workspace_bytes(self.desc, self.index)
        self.ws = torch.empty(max(1, self.ws_bytes), dtype=torch.uint8, device=dev)
        self.part_o = torch.empty((n * self.rows, self.stride, c.hd), dtype=torch.float32, device=dev)
        self.part_ml = torch.empty((n * self.rows, self.stride, 2), dtype=torch.float32, device=dev)
        self.out_dtype = c.dtype if out_dtype is None else out_dtype
        self.out = torch.empty((n * self.rows, c.hd), dtype=_TORCH_ELEM[self.out_dtype], device=dev)
        self.lse = torch.empty((n * self.rows,), dtype=torch.float32, device=dev)

    def chunk(self, q: torch.Tensor, c0: int, budget: int, stream=None, advance: Optional[int] = None):
        """The rows [c0, c0 + Q) of the prompt.  The sequences' length must
        read c0 + Q: it is set here unless the previous chunk was the one just
        before, whose combine advanced it by Q.  advance=0 (fused) leaves the
        lengths at c0 + Q (the same rows again, e.g. a decode step's chunk)."""
        if self.c.known_len != c0 + self.Q:
            with on_stream(stream):
                self.c.seq_lens.fill_(c0 + self.Q)
        adv = self.Q if advance is None else advance
        if self.fused:
            B.sparse_attn_prefill_chunk(self.desc, self.index, q, self.Q, self.window, budget, self.k_max, 0.0,
                                        self.ts, self.ends, self.sel, self.count, self.part_o, self.part_ml,
                                        self.out, self.out_dtype, self.lse, adv, self.ws, self.ws_bytes, stream)
            self.c.known_len = c0 + self.Q + adv
            self.last_n = 1
            return self.out
        else:
            B.sparse_attn_blocks_visible(self.desc, self.index, self.window, self.ends, stream)
            B.sparse_attn_select_blocks(self.desc, self.index, q, self.Q, budget, self.k_max, self.sel, self.count,
                                        stream)
            B.sparse_attn_decode_blocks(self.desc, self.index, q, self.Q, self.sel, self.count, self.k_max,
                                        self.window, 0.0, self.ts, self.ls, self.part_o, self.part_ml, self.ws,
                                        self.ws_bytes, stream)
            # the next chunk's rows are appended in the same launch
            B.sparse_attn_combine_advance(self.rows, self.c.hd, self.stride, self.part_o, self.part_ml, self.out,
                                          self.out_dtype, self.lse, self.c.seq_lens, self.c.B, self.Q, stream)
        self.c.known_len = c0 + 2 * self.Q  # what the lengths read once the queued work has run
        self.last_n = 1
        return self.out

    def chunks(self, q: torch.Tensor, c0: int, budgets, stream=None):
        """len(budgets) <= per_call consecutive chunks from row c0 in one call:
        q is [B][Hq][n * Q][hd] (chunk j's rows at j*Q), budgets[j] chunk j's
        token budget.  Outputs and lengths as n chunk() calls leave them, with
        the rows of every chunk: out, lse, sel and count hold the call's
        [..][n * Q][..] layout from their first element (out_f32, lse_f32)."""
        n = len(budgets)
        assert self.fused and 1 <= n <= self.per_call
        if self.c.known_len != c0 + self.Q:
            with on_stream(stream):
                self.c.seq_lens.fill_(c0 + self.Q)
        B.sparse_attn_prefill_chunks(self.desc, self.index, q, self.Q, n, self.window, budgets, self.k_max, 0.0,
                                     self.ts, self.ends, self.sel, self.count, self.part_o, self.part_ml, self.out,
                                     self.out_dtype, self.lse, n * self.Q, self.ws, self.ws_bytes, stream)
        self.c.known_len = c0 + (n + 1) * self.Q
        self.last_n = n
        return self.out

    def out_f32(self) -> np.ndarray:
        n = self.last_n
        o = self.out[: n * self.rows].cpu().numpy()
        if self.out_dtype == B.SA_BF16:
            o = (o.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        return o.reshape(self.c.B, self.c.Hq, n * self.Q, self.c.hd)

    def lse_f32(self) -> np.ndarray:
        n = self.last_n
        return self.lse[: n * self.rows].cpu().numpy().reshape(self.c.B, self.c.Hq, n * self.Q)


class KeyDiffEviction:
    """KeyDiff eviction of a DeviceCache to a token budget: the kept tokens of
    every (sequence, KV head) (sparse_attn_keydiff_select) and their K and V
    rows copied, in order, into `dst` (sparse_attn_keydiff_compact), whose
    lengths are then set to the kept counts.

    With `sums=True` the copy also writes the key sums of every 64 slots it
    fills (sparse_attn_keydiff_compact_sums, into `slot_sums`), and
    select(carried=...) takes such sums for the cache's first positions
    (sparse_attn_keydiff_select_carried): the carried eviction of a cache that
    an earlier eviction's copy filled."""

    def __init__(self, src: DeviceCache, dst: DeviceCache, budget: int, sink: int, sums: bool = False):
        self.src, self.dst, self.budget, self.sink = src, dst, budget, sink
        dev = src.k.device
        self.kept = torch.full((src.B, src.Hkv, budget), -1, dtype=torch.int32, device=dev)
        self.count = torch.zeros((src.B, src.Hkv), dtype=torch.int32, device=dev)
        self.src_desc, self.dst_desc = src.desc(), dst.desc()
        self.ws_bytes = B.sparse_attn_keydiff_workspace_bytes(self.src_desc, sink, budget)
        self.ws = torch.empty(max(1, self.ws_bytes), dtype=torch.uint8, device=dev)
        self.slot_groups = B.sparse_attn_keydiff_slot_groups(budget)
        self.slot_sums = (torch.zeros((src.B, src.Hkv, self.slot_groups, src.hd), dtype=torch.float32, device=dev)
                          if sums else None)

    def select(self, stream=None, carried=None):
        """carried: (slot_sums, slot_groups, carried_count) of the copy that
        filled this eviction's source cache, or None."""
        if carried is None:
            B.sparse_attn_keydiff_select(self.src_desc, self.sink, self.budget, self.kept, self.count, self.ws,
                                         self.ws_bytes, stream)
        else:
            sums, groups, ccount = carried
            B.sparse_attn_keydiff_select_carried(self.src_desc, self.sink, self.budget, sums, groups, ccount,
                                                 self.kept, self.count, self.ws, self.ws_bytes, stream)

    def carried(self):
        """What the next eviction of `dst` carries from this one's copy."""
        assert self.slot_sums is not None
        return self.slot_sums, self.slot_groups, self.count

    def compact(self, stream=None):
        if self.slot_sums is None:
            B.sparse_attn_keydiff_compact(self.src_desc, self.kept, self.count, self.budget, self.dst_desc, stream)
        else:
            B.sparse_attn_keydiff_compact_sums(self.src_desc, self.kept, self.count, self.budget, self.dst_desc,
                                               self.slot_sums, stream)
        # every KV head keeps min(L, budget) tokens: the first head's count is the sequence's
        with on_stream(stream):
            self.dst.seq_lens.copy_(self.count[:, 0])

    def evict(self, stream=None):
        self.select(stream)
        self.compact(stream)

    def kept_positions(self):
        """[b][kvh] -> numpy array of the kept positions."""
        kept, cnt = self.kept.cpu().numpy(), self.count.cpu().numpy()
        return [[kept[b, h, : cnt[b, h]] for h in range(kept.shape[1])] for b in range(kept.shape[0])]

