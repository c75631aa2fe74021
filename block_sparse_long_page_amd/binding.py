"""Thin ctypes binding of libsparse_attn.so (include/sparse_attn.h).

The functions keep the C names and only marshal arguments: tensors become
device pointers, the stream defaults to torch's current stream, and a
non-zero status raises SparseAttnError.  Every step of the path runs in the
library's HIP kernels; there is no fallback.  If the library has not been
built, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
# SPARSE_ATTN_LIB selects another build of the same library (development sweeps)
LIB_PATH = os.environ.get("SPARSE_ATTN_LIB") or os.path.join(PKG, "libsparse_attn.so")
HEADER = os.path.join(PKG, os.pardir, "include", "sparse_attn.h")

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_HIP, SA_ERR_SCRATCH = 0, 1, 2, 3, 4
SA_F32, SA_BF16 = 0, 1
SA_QUEST, SA_MEAN, SA_CENTROID, SA_COMPRESSED = 0, 1, 2, 3
SA_PART_LOCAL, SA_PART_MIDDLE, SA_PART_ALL = 1, 2, 3
SA_STEP_SEPARATE, SA_STEP_FUSED = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                      "(python -m block_sparse_long_page_amd._build)")

# The library and PyTorch both need libamdhip64.so.7, and the first copy
# loaded serves the whole process: load PyTorch's (which allocates the
# tensors this binding passes) before the library, so one HIP runtime backs
# both, whatever module imported this one first.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.sparse_attn_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


class sa_kv_desc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
        ("num_phys_pages", ctypes.c_int32), ("max_seq_len", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
    ]


class sa_block_index(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32), ("num_blocks", ctypes.c_int32), ("offsets", ctypes.c_void_p),
        ("positions", ctypes.c_void_p), ("centres", ctypes.c_void_p), ("k_blocks", ctypes.c_void_p),
        ("v_blocks", ctypes.c_void_p), ("visible_end", ctypes.c_void_p),
    ]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_DESC = ctypes.POINTER(sa_kv_desc)
_IDX = ctypes.POINTER(sa_block_index)
_SIGS = {
    "sparse_attn_build_page_meta": (ctypes.c_int, [_DESC, _I, _I, _I, _P, _P]),
    "sparse_attn_select": (ctypes.c_int, [_DESC, _P, _I, _P, _I, _I, _I, _I, _P, _P, _P, ctypes.c_size_t, _P]),
    "sparse_attn_workspace_bytes": (ctypes.c_size_t, [_DESC, _I]),
    "sparse_attn_decode": (ctypes.c_int, [_DESC, _P, _I, _P, _P, _I, _I, _I, _I, ctypes.c_float, _I, _I, _P, _P, _P]),
    "sparse_attn_decode_step": (ctypes.c_int, [_DESC, _P, _I, _P, _I, _I, _I, _I, ctypes.c_float, _I, _P, _P, _P,
                                               ctypes.c_size_t, _P, _P, _P]),
    "sparse_attn_default_splits": (ctypes.c_int32, [_DESC, _I, _I, _I, _I]),
    "sparse_attn_step_path": (ctypes.c_int32, [_DESC, _I, _I, _I, _I, _P]),
    "sparse_attn_combine": (ctypes.c_int, [_I, _I, _I, _P, _P, _P, _I, _P, _P]),
    "sparse_attn_combine_advance": (ctypes.c_int, [_I, _I, _I, _P, _P, _P, _I, _P, _P, _I, _I, _P]),
    "sparse_attn_decode_step_static": (ctypes.c_int, [_DESC, _P, _I, _P, _I, _I, _I, _I, ctypes.c_float, _I, _P, _P,
                                                      _P, _I, _P, _P]),
    "sparse_attn_decode_grouped": (ctypes.c_int, [_DESC, _P, _I, _P, _P, _I, _I, _I, ctypes.c_float, _I, _I, _P, _P,
                                                  _P, ctypes.c_size_t, _P]),
    "sparse_attn_grouped_workspace_bytes": (ctypes.c_size_t, [_DESC]),
    "sparse_attn_index_workspace_bytes": (ctypes.c_size_t, [_DESC, _I, _I]),
    "sparse_attn_build_block_index": (ctypes.c_int, [_DESC, _I, _IDX, _P, _P, ctypes.c_size_t, _P]),
    "sparse_attn_select_blocks": (ctypes.c_int, [_DESC, _IDX, _P, _I, _I, _I, _P, _P, _P]),
    "sparse_attn_blocks_workspace_bytes": (ctypes.c_size_t, [_DESC, _IDX]),
    "sparse_attn_blocks_visible": (ctypes.c_int, [_DESC, _IDX, _I, _P, _P]),
    "sparse_attn_decode_blocks": (ctypes.c_int, [_DESC, _IDX, _P, _I, _P, _P, _I, _I, ctypes.c_float, _I, _I, _P, _P,
                                                 _P, ctypes.c_size_t, _P]),
    "sparse_attn_merge_counters": (ctypes.c_int32, [_DESC, _I]),
    "sparse_attn_decode_merged": (ctypes.c_int, [_DESC, _P, _I, _P, _P, _I, _I, _I, ctypes.c_float, _I, _P, _P, _P,
                                                 _I, _P, _I, _P, _P]),
    "sparse_attn_decode_step_merged": (ctypes.c_int, [_DESC, _P, _I, _P, _I, _I, _I, _I, ctypes.c_float, _I, _P, _P,
                                                      _P, ctypes.c_size_t, _P, _P, _P, _I, _P, _I, _P]),
    "sparse_attn_prefill_chunk": (ctypes.c_int, [_DESC, _IDX, _P, _I, _I, _I, _I, ctypes.c_float, _I, _P, _P, _P,
                                                 _P, _P, _P, _I, _P, _I, _P, ctypes.c_size_t, _P]),
    "sparse_attn_prefill_chunks": (ctypes.c_int, [_DESC, _IDX, _P, _I, _I, _I, _P, _I, ctypes.c_float, _I, _P, _P,
                                                  _P, _P, _P, _P, _I, _P, _I, _P, ctypes.c_size_t, _P]),
    "sparse_attn_prefill_num_splits": (ctypes.c_int32, [_DESC, _I, _I, _I]),
    "sparse_attn_prefill_workspace_bytes": (ctypes.c_size_t, [_DESC, _IDX]),
    "sparse_attn_prefill_chunks_workspace_bytes": (ctypes.c_size_t, [_DESC, _IDX, _I]),
    "sparse_attn_keydiff_workspace_bytes": (ctypes.c_size_t, [_DESC, _I, _I]),
    "sparse_attn_keydiff_select": (ctypes.c_int, [_DESC, _I, _I, _P, _P, _P, ctypes.c_size_t, _P]),
    "sparse_attn_keydiff_compact": (ctypes.c_int, [_DESC, _P, _P, _I, _DESC, _P]),
    "sparse_attn_keydiff_compact_sums": (ctypes.c_int, [_DESC, _P, _P, _I, _DESC, _P, _P]),
    "sparse_attn_keydiff_select_carried": (ctypes.c_int, [_DESC, _I, _I, _P, _I, _P, _P, _P, _P, ctypes.c_size_t,
                                                          _P]),
    "sparse_attn_keydiff_slot_groups": (ctypes.c_int32, [_I]),
    "sparse_attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def header_symbols() -> list:
    """Function names the public header declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+[\s\*]+(sparse_attn_\w+)\s*\(", text, re.M)))


def library():
    return _lib


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str):
    if rc != SA_OK:
        raise SparseAttnError(rc, where)


def make_kv_desc(*, batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages_per_seq, num_phys_pages,
                 max_seq_len, dtype, k_cache, v_cache, block_table, seq_lens) -> sa_kv_desc:
    return sa_kv_desc(batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages_per_seq, num_phys_pages,
                      max_seq_len, dtype, _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens))


def sparse_attn_build_page_meta(kv: sa_kv_desc, score_mode: int, page_begin: int, page_end: int, meta,
                                stream=None) -> None:
    _check(_lib.sparse_attn_build_page_meta(ctypes.byref(kv), score_mode, page_begin, page_end, _ptr(meta),
                                            _stream(stream)), "sparse_attn_build_page_meta")


def sparse_attn_workspace_bytes(kv: sa_kv_desc, num_q_rows: int) -> int:
    return int(_lib.sparse_attn_workspace_bytes(ctypes.byref(kv), num_q_rows))


def sparse_attn_select(kv: sa_kv_desc, q, num_q_rows: int, meta, score_mode: int, sink_len: int, window_len: int,
                       token_budget: int, sel_pages, sel_count, workspace, workspace_bytes: int,
                       stream=None) -> None:
    _check(_lib.sparse_attn_select(ctypes.byref(kv), _ptr(q), num_q_rows, _ptr(meta), score_mode, sink_len,
                                   window_len, token_budget, _ptr(sel_pages), _ptr(sel_count), _ptr(workspace),
                                   workspace_bytes, _stream(stream)), "sparse_attn_select")


def sparse_attn_step_path(kv: sa_kv_desc, sink_len: int, window_len: int, token_budget: int, num_splits: int,
                          workspace) -> int:
    return int(_lib.sparse_attn_step_path(ctypes.byref(kv), sink_len, window_len, token_budget, num_splits,
                                          _ptr(workspace)))


def sparse_attn_default_splits(kv: sa_kv_desc, num_q_rows: int, sink_len: int, window_len: int, k_max: int) -> int:
    return int(_lib.sparse_attn_default_splits(ctypes.byref(kv), num_q_rows, sink_len, window_len, k_max))


def sparse_attn_decode(kv: sa_kv_desc, q, num_q_rows: int, sel_pages, sel_count, k_max: int, sink_len: int,
                       window_len: int, parts: int, softmax_scale: float, num_splits: int, split_stride: int,
                       part_o, part_ml, stream=None) -> None:
    _check(_lib.sparse_attn_decode(ctypes.byref(kv), _ptr(q), num_q_rows, _ptr(sel_pages), _ptr(sel_count), k_max,
                                   sink_len, window_len, parts, softmax_scale, num_splits, split_stride,
                                   _ptr(part_o), _ptr(part_ml), _stream(stream)), "sparse_attn_decode")


def sparse_attn_decode_step(kv: sa_kv_desc, q, num_q_rows: int, meta, score_mode: int, sink_len: int,
                            window_len: int, token_budget: int, softmax_scale: float, num_splits: int, sel_pages,
                            sel_count, workspace, workspace_bytes: int, part_o, part_ml, stream=None) -> None:
    _check(_lib.sparse_attn_decode_step(ctypes.byref(kv), _ptr(q), num_q_rows, _ptr(meta), score_mode, sink_len,
                                        window_len, token_budget, softmax_scale, num_splits, _ptr(sel_pages),
                                        _ptr(sel_count), _ptr(workspace), workspace_bytes, _ptr(part_o),
                                        _ptr(part_ml), _stream(stream)), "sparse_attn_decode_step")


def sparse_attn_decode_step_static(kv: sa_kv_desc, q, num_q_rows: int, meta, score_mode: int, sink_len: int,
                                   window_len: int, token_budget: int, softmax_scale: float, num_splits: int,
                                   sel_pages, sel_count, out, out_dtype: int, lse=None, stream=None) -> None:
    _check(_lib.sparse_attn_decode_step_static(ctypes.byref(kv), _ptr(q), num_q_rows, _ptr(meta), score_mode,
                                               sink_len, window_len, token_budget, softmax_scale, num_splits,
                                               _ptr(sel_pages), _ptr(sel_count), _ptr(out), out_dtype, _ptr(lse),
                                               _stream(stream)), "sparse_attn_decode_step_static")


def sparse_attn_combine(num_rows: int, head_dim: int, num_splits: int, part_o, part_ml, out, out_dtype: int,
                        lse=None, stream=None) -> None:
    _check(_lib.sparse_attn_combine(num_rows, head_dim, num_splits, _ptr(part_o), _ptr(part_ml), _ptr(out),
                                    out_dtype, _ptr(lse), _stream(stream)), "sparse_attn_combine")


def sparse_attn_combine_advance(num_rows: int, head_dim: int, num_splits: int, part_o, part_ml, out, out_dtype: int,
                                lse, seq_lens, batch: int, advance: int, stream=None) -> None:
    _check(_lib.sparse_attn_combine_advance(num_rows, head_dim, num_splits, _ptr(part_o), _ptr(part_ml), _ptr(out),
                                            out_dtype, _ptr(lse), _ptr(seq_lens), batch, advance, _stream(stream)),
           "sparse_attn_combine_advance")


def sparse_attn_decode_grouped(kv: sa_kv_desc, q, num_q_rows: int, sel_pages, sel_count, k_max: int, sink_len: int,
                               window_len: int, softmax_scale: float, token_splits: int, local_splits: int, part_o,
                               part_ml, workspace, workspace_bytes: int, stream=None) -> None:
    _check(_lib.sparse_attn_decode_grouped(ctypes.byref(kv), _ptr(q), num_q_rows, _ptr(sel_pages), _ptr(sel_count),
                                           k_max, sink_len, window_len, softmax_scale, token_splits, local_splits,
                                           _ptr(part_o), _ptr(part_ml), _ptr(workspace), workspace_bytes,
                                           _stream(stream)), "sparse_attn_decode_grouped")


def sparse_attn_grouped_workspace_bytes(kv: sa_kv_desc) -> int:
    return int(_lib.sparse_attn_grouped_workspace_bytes(ctypes.byref(kv)))


def make_block_index(*, num_tokens, num_blocks, offsets, positions, centres, k_blocks, v_blocks,
                     visible_end=None) -> sa_block_index:
    return sa_block_index(num_tokens, num_blocks, _ptr(offsets), _ptr(positions), _ptr(centres), _ptr(k_blocks),
                          _ptr(v_blocks), _ptr(visible_end))


def sparse_attn_index_workspace_bytes(kv: sa_kv_desc, num_tokens: int, num_blocks: int) -> int:
    return int(_lib.sparse_attn_index_workspace_bytes(ctypes.byref(kv), num_tokens, num_blocks))


def sparse_attn_build_block_index(kv: sa_kv_desc, iterations: int, index: sa_block_index, assignment, workspace,
                                  workspace_bytes: int, stream=None) -> None:
    _check(_lib.sparse_attn_build_block_index(ctypes.byref(kv), iterations, ctypes.byref(index), _ptr(assignment),
                                              _ptr(workspace), workspace_bytes, _stream(stream)),
           "sparse_attn_build_block_index")


def sparse_attn_select_blocks(kv: sa_kv_desc, index: sa_block_index, q, num_q_rows: int, token_budget: int,
                              k_max: int, sel_blocks, sel_count, stream=None) -> None:
    _check(_lib.sparse_attn_select_blocks(ctypes.byref(kv), ctypes.byref(index), _ptr(q), num_q_rows, token_budget,
                                          k_max, _ptr(sel_blocks), _ptr(sel_count), _stream(stream)),
           "sparse_attn_select_blocks")


def sparse_attn_keydiff_workspace_bytes(kv: sa_kv_desc, sink_len: int, budget: int) -> int:
    return int(_lib.sparse_attn_keydiff_workspace_bytes(ctypes.byref(kv), sink_len, budget))


def sparse_attn_keydiff_select(kv: sa_kv_desc, sink_len: int, budget: int, kept, kept_count, workspace,
                               workspace_bytes: int, stream=None) -> None:
    _check(_lib.sparse_attn_keydiff_select(ctypes.byref(kv), sink_len, budget, _ptr(kept), _ptr(kept_count),
                                           _ptr(workspace), workspace_bytes, _stream(stream)),
           "sparse_attn_keydiff_select")


def sparse_attn_keydiff_compact(src: sa_kv_desc, kept, kept_count, budget: int, dst: sa_kv_desc,
                                stream=None) -> None:
    _check(_lib.sparse_attn_keydiff_compact(ctypes.byref(src), _ptr(kept), _ptr(kept_count), budget,
                                            ctypes.byref(dst), _stream(stream)), "sparse_attn_keydiff_compact")


def sparse_attn_keydiff_compact_sums(src: sa_kv_desc, kept, kept_count, budget: int, dst: sa_kv_desc, slot_sums,
                                     stream=None) -> None:
    _check(_lib.sparse_attn_keydiff_compact_sums(ctypes.byref(src), _ptr(kept), _ptr(kept_count), budget,
                                                 ctypes.byref(dst), _ptr(slot_sums), _stream(stream)),
           "sparse_attn_keydiff_compact_sums")


def sparse_attn_keydiff_select_carried(kv: sa_kv_desc, sink_len: int, budget: int, slot_sums, slot_groups: int,
                                       carried_count, kept, kept_count, workspace, workspace_bytes: int,
                                       stream=None) -> None:
    _check(_lib.sparse_attn_keydiff_select_carried(ctypes.byref(kv), sink_len, budget, _ptr(slot_sums), slot_groups,
                                                   _ptr(carried_count), _ptr(kept), _ptr(kept_count),
                                                   _ptr(workspace), workspace_bytes, _stream(stream)),
           "sparse_attn_keydiff_select_carried")


def sparse_attn_keydiff_slot_groups(budget: int) -> int:
    return int(_lib.sparse_attn_keydiff_slot_groups(budget))


def sparse_attn_blocks_visible(kv: sa_kv_desc, index: sa_block_index, window_len: int, visible_end,
                               stream=None) -> None:
    _check(_lib.sparse_attn_blocks_visible(ctypes.byref(kv), ctypes.byref(index), window_len, _ptr(visible_end),
                                           _stream(stream)), "sparse_attn_blocks_visible")


def sparse_attn_blocks_workspace_bytes(kv: sa_kv_desc, index: sa_block_index) -> int:
    return int(_lib.sparse_attn_blocks_workspace_bytes(ctypes.byref(kv), ctypes.byref(index)))


def sparse_attn_decode_blocks(kv: sa_kv_desc, index: sa_block_index, q, num_q_rows: int, sel_blocks, sel_count,
                              k_max: int, window_len: int, softmax_scale: float, token_splits: int, local_splits: int,
                              part_o, part_ml, workspace, workspace_bytes: int, stream=None) -> None:
    _check(_lib.sparse_attn_decode_blocks(ctypes.byref(kv), ctypes.byref(index), _ptr(q), num_q_rows,
                                          _ptr(sel_blocks), _ptr(sel_count), k_max, window_len, softmax_scale,
                                          token_splits, local_splits, _ptr(part_o), _ptr(part_ml), _ptr(workspace),
                                          workspace_bytes, _stream(stream)), "sparse_attn_decode_blocks")


def sparse_attn_merge_counters(kv: sa_kv_desc, num_q_rows: int) -> int:
    return int(_lib.sparse_attn_merge_counters(ctypes.byref(kv), num_q_rows))


def sparse_attn_decode_merged(kv: sa_kv_desc, q, num_q_rows: int, sel_pages, sel_count, k_max: int, sink_len: int,
                              window_len: int, softmax_scale: float, num_splits: int, part_o, part_ml, out,
                              out_dtype: int, lse, advance: int, counters, stream=None) -> None:
    _check(_lib.sparse_attn_decode_merged(ctypes.byref(kv), _ptr(q), num_q_rows, _ptr(sel_pages), _ptr(sel_count),
                                          k_max, sink_len, window_len, softmax_scale, num_splits, _ptr(part_o),
                                          _ptr(part_ml), _ptr(out), out_dtype, _ptr(lse), advance, _ptr(counters),
                                          _stream(stream)), "sparse_attn_decode_merged")


def sparse_attn_decode_step_merged(kv: sa_kv_desc, q, num_q_rows: int, meta, score_mode: int, sink_len: int,
                                   window_len: int, token_budget: int, softmax_scale: float, num_splits: int,
                                   sel_pages, sel_count, workspace, workspace_bytes: int, part_o, part_ml, out,
                                   out_dtype: int, lse, advance: int, stream=None) -> None:
    _check(_lib.sparse_attn_decode_step_merged(ctypes.byref(kv), _ptr(q), num_q_rows, _ptr(meta), score_mode,
                                               sink_len, window_len, token_budget, softmax_scale, num_splits,
                                               _ptr(sel_pages), _ptr(sel_count), _ptr(workspace), workspace_bytes,
                                               _ptr(part_o), _ptr(part_ml), _ptr(out), out_dtype, _ptr(lse), advance,
                                               _stream(stream)), "sparse_attn_decode_step_merged")


def sparse_attn_prefill_num_splits(kv: sa_kv_desc, window_len: int, k_max: int, token_splits: int) -> int:
    return int(_lib.sparse_attn_prefill_num_splits(ctypes.byref(kv), window_len, k_max, token_splits))


def sparse_attn_prefill_workspace_bytes(kv: sa_kv_desc, index: sa_block_index) -> int:
    return int(_lib.sparse_attn_prefill_workspace_bytes(ctypes.byref(kv), ctypes.byref(index)))


def sparse_attn_prefill_chunk(kv: sa_kv_desc, index: sa_block_index, q, num_q_rows: int, window_len: int,
                              token_budget: int, k_max: int, softmax_scale: float, token_splits: int, visible_end,
                              sel_blocks, sel_count, part_o, part_ml, out, out_dtype: int, lse, advance: int,
                              workspace, workspace_bytes: int, stream=None) -> None:
    _check(_lib.sparse_attn_prefill_chunk(ctypes.byref(kv), ctypes.byref(index), _ptr(q), num_q_rows, window_len,
                                          token_budget, k_max, softmax_scale, token_splits, _ptr(visible_end),
                                          _ptr(sel_blocks), _ptr(sel_count), _ptr(part_o), _ptr(part_ml), _ptr(out),
                                          out_dtype, _ptr(lse), advance, _ptr(workspace), workspace_bytes,
                                          _stream(stream)), "sparse_attn_prefill_chunk")


def sparse_attn_prefill_chunks_workspace_bytes(kv: sa_kv_desc, index: sa_block_index, num_chunks: int) -> int:
    return int(_lib.sparse_attn_prefill_chunks_workspace_bytes(ctypes.byref(kv), ctypes.byref(index), num_chunks))


def sparse_attn_prefill_chunks(kv: sa_kv_desc, index: sa_block_index, q, num_q_rows: int, num_chunks: int,
                               window_len: int, token_budgets, k_max: int, softmax_scale: float, token_splits: int,
                               visible_end, sel_blocks, sel_count, part_o, part_ml, out, out_dtype: int, lse,
                               advance: int, workspace, workspace_bytes: int, stream=None) -> None:
    """token_budgets: a sequence of num_chunks ints (passed as a host array)."""
    budgets = (ctypes.c_int32 * max(1, len(token_budgets)))(*[int(x) for x in token_budgets])
    _check(_lib.sparse_attn_prefill_chunks(ctypes.byref(kv), ctypes.byref(index), _ptr(q), num_q_rows, num_chunks,
                                           window_len, ctypes.addressof(budgets), k_max, softmax_scale,
                                           token_splits, _ptr(visible_end), _ptr(sel_blocks), _ptr(sel_count),
                                           _ptr(part_o), _ptr(part_ml), _ptr(out), out_dtype, _ptr(lse), advance,
                                           _ptr(workspace), workspace_bytes, _stream(stream)),
           "sparse_attn_prefill_chunks")


def sparse_attn_status_string(status: int) -> str:
    return _lib.sparse_attn_status_string(status).decode()
