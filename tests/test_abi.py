"""The C ABI on the host: the library loads, exports every function the
header declares, and rejects every bad argument with its status code before
any HIP call (so these run without a GPU and queue nothing)."""
import ctypes

import pytest

B = pytest.importorskip("block_sparse_long_page_amd.binding")

DEV = 0x1000  # a fake device address: never dereferenced, every call below fails validation


def _desc(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, max_pages_per_seq=8,
                num_phys_pages=16, max_seq_len=128, dtype=B.SA_BF16, k_cache=DEV, v_cache=DEV,
                block_table=DEV, seq_lens=DEV)
    base.update(kw)
    return B.make_kv_desc(**base)


def test_exports_every_header_function():
    names = B.header_symbols()
    assert set(names) == {
        "sparse_attn_build_page_meta", "sparse_attn_select", "sparse_attn_workspace_bytes", "sparse_attn_decode",
        "sparse_attn_decode_step", "sparse_attn_default_splits", "sparse_attn_combine", "sparse_attn_status_string",
        "sparse_attn_decode_grouped", "sparse_attn_grouped_workspace_bytes", "sparse_attn_index_workspace_bytes",
        "sparse_attn_build_block_index", "sparse_attn_select_blocks", "sparse_attn_blocks_workspace_bytes",
        "sparse_attn_decode_blocks", "sparse_attn_blocks_visible", "sparse_attn_keydiff_workspace_bytes",
        "sparse_attn_keydiff_select", "sparse_attn_keydiff_compact", "sparse_attn_step_path",
        "sparse_attn_decode_step_static", "sparse_attn_combine_advance", "sparse_attn_prefill_chunk",
        "sparse_attn_prefill_num_splits", "sparse_attn_prefill_workspace_bytes", "sparse_attn_decode_merged",
        "sparse_attn_decode_step_merged", "sparse_attn_merge_counters", "sparse_attn_keydiff_compact_sums",
        "sparse_attn_keydiff_select_carried", "sparse_attn_keydiff_slot_groups", "sparse_attn_prefill_chunks",
        "sparse_attn_prefill_chunks_workspace_bytes"}
    lib = B.library()
    for n in names:
        assert getattr(lib, n) is not None


def test_status_strings():
    assert B.sparse_attn_status_string(0) == "ok"
    assert "invalid" in B.sparse_attn_status_string(1)
    assert "unsupported" in B.sparse_attn_status_string(2)
    assert "HIP" in B.sparse_attn_status_string(3)
    assert B.sparse_attn_status_string(99) == "unknown status"


BAD_DESCS = [
    (dict(batch=0), B.SA_ERR_INVALID_ARG),
    (dict(num_kv_heads=0), B.SA_ERR_INVALID_ARG),
    (dict(num_q_heads=7), B.SA_ERR_INVALID_ARG),  # not a multiple of the KV heads
    (dict(num_q_heads=6), B.SA_ERR_UNSUPPORTED),  # GQA ratio 3
    (dict(num_q_heads=64), B.SA_ERR_UNSUPPORTED),  # GQA ratio 32
    (dict(head_dim=96), B.SA_ERR_UNSUPPORTED),
    (dict(dtype=5), B.SA_ERR_UNSUPPORTED),
    (dict(page_size=0), B.SA_ERR_INVALID_ARG),
    (dict(page_size=32768, max_pages_per_seq=1, max_seq_len=1), B.SA_ERR_UNSUPPORTED),
    (dict(max_seq_len=129), B.SA_ERR_INVALID_ARG),  # more than max_pages * page_size
    (dict(max_seq_len=0), B.SA_ERR_INVALID_ARG),
    (dict(num_phys_pages=0), B.SA_ERR_INVALID_ARG),
    (dict(k_cache=None), B.SA_ERR_INVALID_ARG),
    (dict(v_cache=None), B.SA_ERR_INVALID_ARG),
    (dict(block_table=None), B.SA_ERR_INVALID_ARG),
    (dict(seq_lens=None), B.SA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("bad,code", BAD_DESCS)
def test_descriptor_checks(bad, code):
    lib = B.library()
    d = _desc(**bad)
    assert lib.sparse_attn_build_page_meta(ctypes.byref(d), 0, 0, 8, DEV, None) == code
    assert lib.sparse_attn_select(ctypes.byref(d), DEV, 1, DEV, 0, 16, 16, 32, DEV, DEV, DEV, 1 << 20, None) == code
    assert lib.sparse_attn_decode(ctypes.byref(d), DEV, 1, DEV, DEV, 2, 16, 16, 3, 0.0, 4, 0, DEV, DEV, None) == code


def test_null_descriptor():
    lib = B.library()
    assert lib.sparse_attn_build_page_meta(None, 0, 0, 1, DEV, None) == B.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_select(None, DEV, 1, DEV, 0, 0, 1, 0, DEV, DEV, DEV, 0, None) == B.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_decode(None, DEV, 1, None, None, 0, 0, 1, 3, 0.0, 1, 0, DEV, DEV, None) == B.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_workspace_bytes(None, 1) == 0


def test_page_meta_checks():
    lib = B.library()
    d = _desc()
    assert lib.sparse_attn_build_page_meta(ctypes.byref(d), 0, 0, 8, None, None) == B.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_build_page_meta(ctypes.byref(d), 0, -1, 8, DEV, None) == B.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_build_page_meta(ctypes.byref(d), 0, 5, 4, DEV, None) == B.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_build_page_meta(ctypes.byref(d), 4, 0, 8, DEV, None) == B.SA_ERR_UNSUPPORTED
    # an empty range is a valid no-op that queues nothing
    assert lib.sparse_attn_build_page_meta(ctypes.byref(d), 0, 4, 4, DEV, None) == B.SA_OK
    assert lib.sparse_attn_build_page_meta(ctypes.byref(d), 0, 8, 100, DEV, None) == B.SA_OK


def test_select_checks():
    lib = B.library()
    d = _desc()
    ws = lib.sparse_attn_workspace_bytes(ctypes.byref(d), 1)
    # fp32 scores [B][Hkv][Q][max_pages], then a 256-byte status area of the selecting step, then the
    # merge's counters (one per (sequence, KV head, row), one per sequence), each 256-byte aligned
    assert ws == ((4 * 2 * 2 * 1 * 8 + 255) // 256) * 256 + 256 + 256

    def sel(**kw):
        a = dict(q=DEV, rows=1, meta=DEV, mode=0, S=16, W=16, budget=32, sel=DEV, cnt=DEV, ws=DEV, wsb=ws)
        a.update(kw)
        return lib.sparse_attn_select(ctypes.byref(d), a["q"], a["rows"], a["meta"], a["mode"], a["S"], a["W"],
                                      a["budget"], a["sel"], a["cnt"], a["ws"], a["wsb"], None)

    assert sel(q=None) == B.SA_ERR_INVALID_ARG
    assert sel(meta=None) == B.SA_ERR_INVALID_ARG
    assert sel(cnt=None) == B.SA_ERR_INVALID_ARG
    assert sel(sel=None) == B.SA_ERR_INVALID_ARG  # k_max = 2 needs an output
    assert sel(rows=0) == B.SA_ERR_INVALID_ARG
    assert sel(rows=129) == B.SA_ERR_INVALID_ARG  # more rows than tokens
    assert sel(S=-1) == B.SA_ERR_INVALID_ARG
    assert sel(W=0) == B.SA_ERR_INVALID_ARG  # the current token must be attended
    assert sel(budget=-1) == B.SA_ERR_INVALID_ARG
    assert sel(ws=None) == B.SA_ERR_INVALID_ARG
    assert sel(wsb=4 * 2 * 2 * 1 * 8 - 1) == B.SA_ERR_INVALID_ARG  # the scores alone do not fit
    assert sel(mode=7) == B.SA_ERR_UNSUPPORTED


def test_decode_checks():
    lib = B.library()
    d = _desc()

    def dec(**kw):
        a = dict(q=DEV, rows=1, sel=DEV, cnt=DEV, kmax=2, S=16, W=16, parts=3, scale=0.0, splits=4, stride=0,
                 po=DEV, pml=DEV)
        a.update(kw)
        return lib.sparse_attn_decode(ctypes.byref(d), a["q"], a["rows"], a["sel"], a["cnt"], a["kmax"], a["S"],
                                      a["W"], a["parts"], a["scale"], a["splits"], a["stride"], a["po"], a["pml"],
                                      None)

    assert dec(q=None) == B.SA_ERR_INVALID_ARG
    assert dec(po=None) == B.SA_ERR_INVALID_ARG
    assert dec(pml=None) == B.SA_ERR_INVALID_ARG
    assert dec(cnt=None) == B.SA_ERR_INVALID_ARG  # a page list needs its counts
    assert dec(rows=0) == B.SA_ERR_INVALID_ARG
    assert dec(S=-1) == B.SA_ERR_INVALID_ARG
    assert dec(W=0) == B.SA_ERR_INVALID_ARG
    assert dec(kmax=-1) == B.SA_ERR_INVALID_ARG
    assert dec(splits=0) == B.SA_ERR_INVALID_ARG
    assert dec(splits=1025) == B.SA_ERR_INVALID_ARG
    assert dec(scale=float("nan")) == B.SA_ERR_INVALID_ARG
    assert dec(scale=float("inf")) == B.SA_ERR_INVALID_ARG
    assert dec(parts=0) == B.SA_ERR_INVALID_ARG
    assert dec(parts=4) == B.SA_ERR_INVALID_ARG
    assert dec(stride=3) == B.SA_ERR_INVALID_ARG  # fewer slots than splits
    assert dec(stride=1025) == B.SA_ERR_INVALID_ARG


def test_decode_step_checks():
    lib = B.library()
    d = _desc()
    ws = lib.sparse_attn_workspace_bytes(ctypes.byref(d), 1)

    def step(**kw):
        a = dict(q=DEV, rows=1, meta=DEV, mode=0, S=16, W=16, budget=32, scale=0.0, splits=4, sel=DEV, cnt=DEV,
                 ws=DEV, wsb=ws, po=DEV, pml=DEV)
        a.update(kw)
        return lib.sparse_attn_decode_step(ctypes.byref(d), a["q"], a["rows"], a["meta"], a["mode"], a["S"], a["W"],
                                           a["budget"], a["scale"], a["splits"], a["sel"], a["cnt"], a["ws"],
                                           a["wsb"], a["po"], a["pml"], None)

    assert step(q=None) == B.SA_ERR_INVALID_ARG
    assert step(meta=None) == B.SA_ERR_INVALID_ARG
    assert step(cnt=None) == B.SA_ERR_INVALID_ARG
    assert step(sel=None) == B.SA_ERR_INVALID_ARG
    assert step(po=None) == B.SA_ERR_INVALID_ARG
    assert step(pml=None) == B.SA_ERR_INVALID_ARG
    assert step(rows=0) == B.SA_ERR_INVALID_ARG
    assert step(S=-1) == B.SA_ERR_INVALID_ARG
    assert step(W=0) == B.SA_ERR_INVALID_ARG
    assert step(budget=-1) == B.SA_ERR_INVALID_ARG
    assert step(splits=0) == B.SA_ERR_INVALID_ARG
    assert step(splits=1025) == B.SA_ERR_INVALID_ARG
    assert step(scale=float("nan")) == B.SA_ERR_INVALID_ARG
    assert step(ws=None) == B.SA_ERR_INVALID_ARG
    assert step(wsb=ws - 1) == B.SA_ERR_INVALID_ARG
    assert step(mode=7) == B.SA_ERR_UNSUPPORTED
    for bad, code in BAD_DESCS:
        dd = _desc(**bad)
        assert lib.sparse_attn_decode_step(ctypes.byref(dd), DEV, 1, DEV, 0, 16, 16, 32, 0.0, 4, DEV, DEV, DEV, ws,
                                           DEV, DEV, None) == code


def test_decode_grouped_checks():
    lib = B.library()
    d = _desc()
    ws = lib.sparse_attn_grouped_workspace_bytes(ctypes.byref(d))
    # counts, page records (16 bytes), slots; each region 256-byte aligned
    assert ws == 256 + ((2 * 2 * 8 * 16 + 255) // 256) * 256 + ((2 * 2 * 8 * 128 * 2 + 255) // 256) * 256
    assert lib.sparse_attn_grouped_workspace_bytes(None) == 0

    def grouped(**kw):
        a = dict(q=DEV, rows=4, sel=DEV, cnt=DEV, kmax=4, S=16, W=16, scale=0.0, ts=2, ls=1, po=DEV, pml=DEV,
                 ws=DEV, wsb=ws)
        a.update(kw)
        return lib.sparse_attn_decode_grouped(ctypes.byref(a.get("desc", d)), a["q"], a["rows"], a["sel"], a["cnt"],
                                              a["kmax"], a["S"], a["W"], a["scale"], a["ts"], a["ls"], a["po"],
                                              a["pml"], a["ws"], a["wsb"], None)

    assert grouped(q=None) == B.SA_ERR_INVALID_ARG
    assert grouped(po=None) == B.SA_ERR_INVALID_ARG
    assert grouped(pml=None) == B.SA_ERR_INVALID_ARG
    assert grouped(sel=None) == B.SA_ERR_INVALID_ARG
    assert grouped(cnt=None) == B.SA_ERR_INVALID_ARG
    assert grouped(rows=0) == B.SA_ERR_INVALID_ARG
    assert grouped(rows=129) == B.SA_ERR_INVALID_ARG  # more rows than the cache holds tokens
    assert grouped(S=-1) == B.SA_ERR_INVALID_ARG
    assert grouped(W=0) == B.SA_ERR_INVALID_ARG
    assert grouped(kmax=-1) == B.SA_ERR_INVALID_ARG
    assert grouped(ts=0) == B.SA_ERR_INVALID_ARG
    assert grouped(ts=65) == B.SA_ERR_INVALID_ARG
    assert grouped(ls=0) == B.SA_ERR_INVALID_ARG
    assert grouped(kmax=600, ts=2) == B.SA_ERR_INVALID_ARG  # more than 1024 slots per row
    assert grouped(scale=float("nan")) == B.SA_ERR_INVALID_ARG
    assert grouped(ws=None) == B.SA_ERR_INVALID_ARG
    assert grouped(wsb=ws - 1) == B.SA_ERR_INVALID_ARG
    assert grouped(ws=DEV + 16) == B.SA_ERR_INVALID_ARG  # not 256-byte aligned
    big = _desc(max_seq_len=256, max_pages_per_seq=16, num_phys_pages=32)
    wsb = lib.sparse_attn_grouped_workspace_bytes(ctypes.byref(big))
    assert grouped(desc=big, rows=129, wsb=wsb) == B.SA_ERR_UNSUPPORTED  # one mask bit per row, two 64-bit words
    assert grouped(desc=_desc(dtype=B.SA_F32)) == B.SA_ERR_UNSUPPORTED
    for bad, code in BAD_DESCS:
        assert grouped(desc=_desc(**bad)) == code


def test_merged_decode_checks():
    """The decode and selecting step that merge in their own last workgroup:
    every argument is checked before any HIP call."""
    lib = B.library()
    d = _desc()
    assert lib.sparse_attn_merge_counters(ctypes.byref(d), 3) == 2 * 2 * 3 + 2
    assert lib.sparse_attn_merge_counters(None, 1) == -B.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_merge_counters(ctypes.byref(d), 0) == -B.SA_ERR_INVALID_ARG

    def dec(**kw):
        a = dict(desc=d, q=DEV, rows=1, sel=DEV, cnt=DEV, kmax=2, S=16, W=16, scale=0.0, splits=4, po=DEV, pml=DEV,
                 out=DEV, odt=B.SA_BF16, lse=None, adv=0, ctr=DEV)
        a.update(kw)
        return lib.sparse_attn_decode_merged(ctypes.byref(a["desc"]), a["q"], a["rows"], a["sel"], a["cnt"],
                                             a["kmax"], a["S"], a["W"], a["scale"], a["splits"], a["po"], a["pml"],
                                             a["out"], a["odt"], a["lse"], a["adv"], a["ctr"], None)

    for f in ("q", "po", "pml", "out", "ctr"):
        assert dec(**{f: None}) == B.SA_ERR_INVALID_ARG
    assert dec(cnt=None) == B.SA_ERR_INVALID_ARG  # a page list needs its counts
    assert dec(rows=0) == B.SA_ERR_INVALID_ARG
    assert dec(S=-1) == B.SA_ERR_INVALID_ARG
    assert dec(W=0) == B.SA_ERR_INVALID_ARG
    assert dec(adv=-1) == B.SA_ERR_INVALID_ARG
    assert dec(splits=0) == B.SA_ERR_INVALID_ARG
    assert dec(splits=65) == B.SA_ERR_INVALID_ARG  # the last workgroup merges at most 64 splits
    assert dec(scale=float("nan")) == B.SA_ERR_INVALID_ARG
    assert dec(desc=_desc(dtype=B.SA_F32)) == B.SA_ERR_UNSUPPORTED
    assert dec(odt=7) == B.SA_ERR_UNSUPPORTED
    for bad, code in BAD_DESCS:
        assert dec(desc=_desc(**bad)) == code
    ws = lib.sparse_attn_workspace_bytes(ctypes.byref(d), 1)

    def step(**kw):
        a = dict(desc=d, q=DEV, rows=1, meta=DEV, mode=0, S=16, W=16, budget=32, scale=0.0, splits=4, sel=DEV,
                 cnt=DEV, ws=DEV, wsb=ws, po=DEV, pml=DEV, out=DEV, odt=B.SA_BF16, lse=None, adv=0)
        a.update(kw)
        return lib.sparse_attn_decode_step_merged(ctypes.byref(a["desc"]), a["q"], a["rows"], a["meta"], a["mode"],
                                                  a["S"], a["W"], a["budget"], a["scale"], a["splits"], a["sel"],
                                                  a["cnt"], a["ws"], a["wsb"], a["po"], a["pml"], a["out"], a["odt"],
                                                  a["lse"], a["adv"], None)

    for f in ("q", "meta", "po", "pml", "out", "ws", "cnt"):
        assert step(**{f: None}) == B.SA_ERR_INVALID_ARG
    assert step(wsb=ws - 1) == B.SA_ERR_INVALID_ARG
    assert step(adv=-1) == B.SA_ERR_INVALID_ARG
    assert step(splits=65) == B.SA_ERR_INVALID_ARG
    assert step(mode=9) == B.SA_ERR_UNSUPPORTED
    assert step(desc=_desc(dtype=B.SA_F32)) == B.SA_ERR_UNSUPPORTED
    assert step(odt=7) == B.SA_ERR_UNSUPPORTED


def test_combine_checks():
    lib = B.library()

    def comb(**kw):
        a = dict(rows=4, hd=128, splits=2, po=DEV, pml=DEV, out=DEV, odt=1, lse=None)
        a.update(kw)
        return lib.sparse_attn_combine(a["rows"], a["hd"], a["splits"], a["po"], a["pml"], a["out"], a["odt"],
                                       a["lse"], None)

    assert comb(rows=0) == B.SA_ERR_INVALID_ARG
    assert comb(po=None) == B.SA_ERR_INVALID_ARG
    assert comb(pml=None) == B.SA_ERR_INVALID_ARG
    assert comb(out=None) == B.SA_ERR_INVALID_ARG
    assert comb(splits=0) == B.SA_ERR_INVALID_ARG
    assert comb(splits=2000) == B.SA_ERR_INVALID_ARG
    assert comb(hd=96) == B.SA_ERR_UNSUPPORTED
    assert comb(odt=3) == B.SA_ERR_UNSUPPORTED

    def adv(**kw):
        a = dict(rows=4, hd=128, splits=2, po=DEV, pml=DEV, out=DEV, odt=1, lse=None, lens=DEV, batch=2, advance=1)
        a.update(kw)
        return lib.sparse_attn_combine_advance(a["rows"], a["hd"], a["splits"], a["po"], a["pml"], a["out"],
                                               a["odt"], a["lse"], a["lens"], a["batch"], a["advance"], None)

    assert adv(lens=None) == B.SA_ERR_INVALID_ARG
    assert adv(batch=0) == B.SA_ERR_INVALID_ARG
    assert adv(advance=-1) == B.SA_ERR_INVALID_ARG
    assert adv(rows=0) == B.SA_ERR_INVALID_ARG
    assert adv(splits=0) == B.SA_ERR_INVALID_ARG
    assert adv(hd=96) == B.SA_ERR_UNSUPPORTED


def test_default_splits_fill_the_gpu():
    lib = B.library()
    # the headline layer: 4 sequences x 8 KV heads, 12544 attended tokens each
    d = _desc(batch=4, num_q_heads=64, num_kv_heads=8, page_size=64, max_pages_per_seq=2048,
              num_phys_pages=8192, max_seq_len=131072)
    s = lib.sparse_attn_default_splits(ctypes.byref(d), 1, 256, 4096, 128)
    assert 8 <= s <= 64  # about one round of workgroups over the CUs
    tiny = _desc(batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64, max_pages_per_seq=128, max_seq_len=2048)
    assert lib.sparse_attn_default_splits(ctypes.byref(tiny), 1, 16, 64, 8) >= 1


def _fastdiv(d):
    """The host's magic pair for n / d (mirrors make_fastdiv)."""
    s = 0
    while (1 << s) < d:
        s += 1
    magic = ((1 << 32) * ((1 << s) - d)) // d + 1
    return magic & 0xFFFFFFFF, s


@pytest.mark.parametrize("d", [1, 2, 3, 5, 7, 16, 24, 32, 48, 64, 100, 2047, 2048, 4095, 16384])
def test_fast_division_is_exact_below_2_31(d):
    import numpy as np

    magic, s = _fastdiv(d)
    rng = np.random.default_rng(d)
    n = np.concatenate([np.arange(0, 5000), rng.integers(0, 2**31, 20000), [2**31 - 1, 2**31 - 2]]).astype(np.uint64)
    hi = (n * np.uint64(magic)) >> np.uint64(32)
    q = ((hi + n) & np.uint64(0xFFFFFFFF)) >> np.uint64(s)
    assert ((hi + n) < np.uint64(1 << 32)).all()
    np.testing.assert_array_equal(q, n // np.uint64(d))


def _index(**kw):
    base = dict(num_tokens=100, num_blocks=4, offsets=DEV, positions=DEV, centres=DEV, k_blocks=DEV, v_blocks=DEV)
    base.update(kw)
    return B.make_block_index(**base)


def test_block_index_checks():
    lib = B.library()
    d = _desc()
    ix = _index()
    ws = lib.sparse_attn_index_workspace_bytes(ctypes.byref(d), 100, 4)
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    nbk, N, C, hd = 4, 100, 4, 128
    nseg = (N + 127) // 128 + C
    # 1/|k|, bf16 centres, assignment, chunk counts, segment bases, segment blocks, segment sums
    assert ws == (up(nbk * N * 4) + up(nbk * C * hd * 2) + up(nbk * N * 4) + up(nbk * 1 * C * 4)
                  + up(nbk * (C + 1) * 4) + up(nbk * nseg * 4) + up(nbk * nseg * hd * 4))
    assert lib.sparse_attn_index_workspace_bytes(None, 100, 4) == 0
    assert lib.sparse_attn_index_workspace_bytes(ctypes.byref(d), 0, 4) == 0

    def build(**kw):
        a = dict(desc=d, it=4, ix=ix, assign=None, ws=DEV, wsb=ws)
        a.update(kw)
        ixp = ctypes.byref(a["ix"]) if a["ix"] is not None else None
        return lib.sparse_attn_build_block_index(ctypes.byref(a["desc"]), a["it"], ixp, a["assign"], a["ws"],
                                                 a["wsb"], None)

    assert build(ix=None) == B.SA_ERR_INVALID_ARG
    for f in ("offsets", "positions", "centres", "k_blocks", "v_blocks"):
        assert build(ix=_index(**{f: None})) == B.SA_ERR_INVALID_ARG
    assert build(ix=_index(k_blocks=DEV + 8)) == B.SA_ERR_INVALID_ARG  # rows are written 16 bytes at a time
    assert build(ix=_index(num_tokens=0)) == B.SA_ERR_INVALID_ARG
    assert build(ix=_index(num_tokens=129)) == B.SA_ERR_INVALID_ARG  # beyond max_seq_len
    assert build(ix=_index(num_blocks=0)) == B.SA_ERR_INVALID_ARG
    assert build(ix=_index(num_blocks=101)) == B.SA_ERR_INVALID_ARG  # more blocks than tokens
    assert build(it=-1) == B.SA_ERR_INVALID_ARG
    assert build(it=65) == B.SA_ERR_INVALID_ARG
    assert build(ws=None) == B.SA_ERR_INVALID_ARG
    assert build(wsb=ws - 1) == B.SA_ERR_INVALID_ARG
    assert build(ws=DEV + 16) == B.SA_ERR_INVALID_ARG
    assert build(desc=_desc(dtype=B.SA_F32)) == B.SA_ERR_UNSUPPORTED
    big = _desc(max_seq_len=8192, max_pages_per_seq=512, num_phys_pages=1024)
    assert build(desc=big, ix=_index(num_tokens=8192, num_blocks=4097)) == B.SA_ERR_UNSUPPORTED
    for bad, code in BAD_DESCS:
        assert build(desc=_desc(**bad)) == code

    def select(**kw):
        a = dict(q=DEV, rows=2, budget=64, kmax=2, sel=DEV, cnt=DEV)
        a.update(kw)
        return lib.sparse_attn_select_blocks(ctypes.byref(d), ctypes.byref(ix), a["q"], a["rows"], a["budget"],
                                             a["kmax"], a["sel"], a["cnt"], None)

    assert select(q=None) == B.SA_ERR_INVALID_ARG
    assert select(sel=None) == B.SA_ERR_INVALID_ARG
    assert select(cnt=None) == B.SA_ERR_INVALID_ARG
    assert select(rows=0) == B.SA_ERR_INVALID_ARG
    assert select(budget=-1) == B.SA_ERR_INVALID_ARG
    assert select(kmax=0) == B.SA_ERR_INVALID_ARG
    assert select(kmax=5) == B.SA_ERR_INVALID_ARG  # more than the index's blocks

    wsd = lib.sparse_attn_blocks_workspace_bytes(ctypes.byref(d), ctypes.byref(ix))
    assert wsd == 256 + up(nbk * C * 16) + up(nbk * C * 128 * 2)

    def decode(**kw):
        a = dict(q=DEV, rows=2, sel=DEV, cnt=DEV, kmax=2, W=4, scale=0.0, ts=1, ls=1, po=DEV, pml=DEV, ws=DEV, wsb=wsd)
        a.update(kw)
        return lib.sparse_attn_decode_blocks(ctypes.byref(d), ctypes.byref(ix), a["q"], a["rows"], a["sel"],
                                             a["cnt"], a["kmax"], a["W"], a["scale"], a["ts"], a["ls"], a["po"],
                                             a["pml"], a["ws"], a["wsb"], None)

    assert decode(W=1) == B.SA_ERR_INVALID_ARG  # the window must hold the rows
    assert decode(kmax=5) == B.SA_ERR_INVALID_ARG
    assert decode(sel=None) == B.SA_ERR_INVALID_ARG
    assert decode(ws=None) == B.SA_ERR_INVALID_ARG
    assert decode(wsb=wsd - 1) == B.SA_ERR_INVALID_ARG
    assert decode(ts=0) == B.SA_ERR_INVALID_ARG
    assert decode(po=None) == B.SA_ERR_INVALID_ARG
    assert decode(rows=129, W=129) != B.SA_OK  # past the row limit (and the 128-token cache)


def test_prefill_chunk_checks():
    lib = B.library()
    d = _desc()
    ix = _index()
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    nbk, C = 4, 4
    wsp = lib.sparse_attn_prefill_workspace_bytes(ctypes.byref(d), ctypes.byref(ix))
    # slot table, rows of each group of 8 per block, item counters
    assert wsp == up(nbk * C * 128 * 2) + up(nbk * C * 16) + up(nbk * 4)
    assert lib.sparse_attn_prefill_workspace_bytes(None, ctypes.byref(ix)) == 0
    # slots per row: (k_max + window pages) * token chunks; the window [L - W, L)
    # touches at most (W - 1) // P + 2 pages
    assert lib.sparse_attn_prefill_num_splits(ctypes.byref(d), 16, 2, 3) == (2 + 2) * 3
    assert lib.sparse_attn_prefill_num_splits(ctypes.byref(d), 17, 2, 1) == 2 + 3
    assert lib.sparse_attn_prefill_num_splits(ctypes.byref(d), 1, 1, 1) == 1 + 2
    assert lib.sparse_attn_prefill_num_splits(ctypes.byref(d), 0, 2, 1) == -B.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_prefill_num_splits(ctypes.byref(d), 16, 0, 1) == -B.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_prefill_num_splits(ctypes.byref(d), 16, 2, 65) == -B.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_prefill_num_splits(ctypes.byref(d), 16, 600, 2) == -B.SA_ERR_UNSUPPORTED  # > 1024
    assert lib.sparse_attn_prefill_num_splits(None, 16, 2, 1) == -B.SA_ERR_INVALID_ARG

    def chunk(**kw):
        a = dict(desc=d, ix=ix, q=DEV, rows=2, W=4, budget=64, kmax=2, scale=0.0, ts=1, ends=DEV, sel=DEV, cnt=DEV,
                 po=DEV, pml=DEV, out=DEV, odt=B.SA_BF16, lse=None, adv=0, ws=DEV, wsb=wsp)
        a.update(kw)
        ixp = ctypes.byref(a["ix"]) if a["ix"] is not None else None
        return lib.sparse_attn_prefill_chunk(ctypes.byref(a["desc"]), ixp, a["q"], a["rows"], a["W"], a["budget"],
                                             a["kmax"], a["scale"], a["ts"], a["ends"], a["sel"], a["cnt"], a["po"],
                                             a["pml"], a["out"], a["odt"], a["lse"], a["adv"], a["ws"], a["wsb"],
                                             None)

    assert chunk(ix=None) == B.SA_ERR_INVALID_ARG
    for f in ("q", "ends", "sel", "cnt", "po", "pml", "out"):
        assert chunk(**{f: None}) == B.SA_ERR_INVALID_ARG
    assert chunk(rows=0) == B.SA_ERR_INVALID_ARG
    assert chunk(W=1) == B.SA_ERR_INVALID_ARG  # the window must hold the rows
    assert chunk(budget=-1) == B.SA_ERR_INVALID_ARG
    assert chunk(adv=-1) == B.SA_ERR_INVALID_ARG
    assert chunk(kmax=0) == B.SA_ERR_INVALID_ARG
    assert chunk(kmax=5) == B.SA_ERR_INVALID_ARG  # more than the index's blocks
    assert chunk(ts=0) == B.SA_ERR_INVALID_ARG
    assert chunk(ts=65) == B.SA_ERR_INVALID_ARG
    assert chunk(scale=float("nan")) == B.SA_ERR_INVALID_ARG
    assert chunk(scale=float("inf")) == B.SA_ERR_INVALID_ARG
    assert chunk(ws=None) == B.SA_ERR_INVALID_ARG
    assert chunk(wsb=wsp - 1) == B.SA_ERR_INVALID_ARG
    assert chunk(ws=DEV + 16) == B.SA_ERR_INVALID_ARG
    assert chunk(odt=7) == B.SA_ERR_UNSUPPORTED
    assert chunk(desc=_desc(dtype=B.SA_F32)) == B.SA_ERR_UNSUPPORTED
    assert chunk(rows=129, W=129) != B.SA_OK  # past the row limit (and the 128-token cache)
    big = _desc(max_seq_len=8192, max_pages_per_seq=512, num_phys_pages=1024)
    assert chunk(desc=big, ix=_index(num_tokens=8192, num_blocks=513), kmax=1) == B.SA_ERR_UNSUPPORTED
    assert chunk(desc=big, ix=_index(num_tokens=8192, num_blocks=600), kmax=600, ts=2) == B.SA_ERR_UNSUPPORTED
    for bad, code in BAD_DESCS:
        assert chunk(desc=_desc(**bad)) == code

    # several chunks per call: one slot table, row-count table and counter per chunk
    for n in (1, 3, 16):
        assert lib.sparse_attn_prefill_chunks_workspace_bytes(ctypes.byref(d), ctypes.byref(ix), n) == \
            up(n * nbk * C * 128 * 2) + up(n * nbk * C * 16) + up(n * nbk * 4)
    assert lib.sparse_attn_prefill_chunks_workspace_bytes(ctypes.byref(d), ctypes.byref(ix), 0) == 0
    assert lib.sparse_attn_prefill_chunks_workspace_bytes(ctypes.byref(d), ctypes.byref(ix), 17) == 0
    assert lib.sparse_attn_prefill_chunks_workspace_bytes(None, ctypes.byref(ix), 2) == 0
    ws3 = lib.sparse_attn_prefill_chunks_workspace_bytes(ctypes.byref(d), ctypes.byref(ix), 3)

    def chunks(**kw):
        a = dict(desc=d, ix=ix, q=DEV, rows=2, n=3, W=4, budgets=[64, 64, 64], kmax=2, scale=0.0, ts=1, ends=DEV,
                 sel=DEV, cnt=DEV, po=DEV, pml=DEV, out=DEV, odt=B.SA_BF16, lse=None, adv=0, ws=DEV, wsb=ws3)
        a.update(kw)
        bud = None if a["budgets"] is None else (ctypes.c_int32 * len(a["budgets"]))(*a["budgets"])
        ixp = ctypes.byref(a["ix"]) if a["ix"] is not None else None
        return lib.sparse_attn_prefill_chunks(ctypes.byref(a["desc"]), ixp, a["q"], a["rows"], a["n"], a["W"],
                                              None if bud is None else ctypes.addressof(bud), a["kmax"], a["scale"],
                                              a["ts"], a["ends"], a["sel"], a["cnt"], a["po"], a["pml"], a["out"],
                                              a["odt"], a["lse"], a["adv"], a["ws"], a["wsb"], None)

    assert chunks(budgets=None) == B.SA_ERR_INVALID_ARG
    assert chunks(budgets=[64, -1, 64]) == B.SA_ERR_INVALID_ARG
    assert chunks(n=0) == B.SA_ERR_INVALID_ARG
    assert chunks(n=17, budgets=[1] * 17) == B.SA_ERR_INVALID_ARG
    assert chunks(wsb=ws3 - 1) == B.SA_ERR_INVALID_ARG  # three chunks' tables
    assert chunks(rows=64, n=3, W=64) == B.SA_ERR_INVALID_ARG  # 192 rows past the 128-token cache
    for f in ("q", "ends", "sel", "cnt", "po", "pml", "out"):
        assert chunks(**{f: None}) == B.SA_ERR_INVALID_ARG
    for bad, code in BAD_DESCS:
        assert chunks(desc=_desc(**bad)) == code


def test_keydiff_checks():
    lib = B.library()
    d = _desc()
    ws = lib.sparse_attn_keydiff_workspace_bytes(ctypes.byref(d), 4, 64)
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # chunk key sums (one chunk), then the distances
    assert ws == up(2 * 2 * 1 * 128 * 4) + up(2 * 2 * 128 * 4)
    assert lib.sparse_attn_keydiff_workspace_bytes(None, 4, 64) == 0
    assert lib.sparse_attn_keydiff_workspace_bytes(ctypes.byref(d), -1, 64) == 0
    assert lib.sparse_attn_keydiff_workspace_bytes(ctypes.byref(d), 4, 0) == 0

    def sel(**kw):
        a = dict(desc=d, sink=4, budget=64, kept=DEV, cnt=DEV, ws=DEV, wsb=ws)
        a.update(kw)
        return lib.sparse_attn_keydiff_select(ctypes.byref(a["desc"]), a["sink"], a["budget"], a["kept"], a["cnt"],
                                              a["ws"], a["wsb"], None)

    assert sel(kept=None) == B.SA_ERR_INVALID_ARG
    assert sel(cnt=None) == B.SA_ERR_INVALID_ARG
    assert sel(ws=None) == B.SA_ERR_INVALID_ARG
    assert sel(wsb=ws - 1) == B.SA_ERR_INVALID_ARG
    assert sel(ws=DEV + 8) == B.SA_ERR_INVALID_ARG  # read as 16-byte vectors
    assert sel(sink=-1) == B.SA_ERR_INVALID_ARG
    assert sel(budget=0) == B.SA_ERR_INVALID_ARG
    assert sel(budget=3) == B.SA_ERR_INVALID_ARG  # below the sink
    # past 12288 candidates: chunks of 8192 and a merge of their picks
    big = _desc(max_seq_len=16384, max_pages_per_seq=1024, num_phys_pages=2048)
    wsb = lib.sparse_attn_keydiff_workspace_bytes(ctypes.byref(big), 4, 14336)
    base = lib.sparse_attn_keydiff_workspace_bytes(ctypes.byref(big), 4, 16384)  # nothing evicted: one workgroup
    assert wsb == base + 2 * up(2 * 2 * 2 * 8192 * 4)  # two chunks' picks, keys and indices
    assert sel(desc=big, wsb=wsb - 1, budget=14336, sink=4) == B.SA_ERR_INVALID_ARG
    # 2 chunks x 8192 picks (16380 candidates, 14332 evicted) do not fit the merge
    wsb2 = lib.sparse_attn_keydiff_workspace_bytes(ctypes.byref(big), 4, 2048)
    assert sel(desc=big, wsb=wsb2, budget=2048, sink=4) == B.SA_ERR_UNSUPPORTED
    huge = _desc(batch=1, num_kv_heads=1, num_q_heads=1, max_seq_len=17 * 8192 + 8, max_pages_per_seq=17 * 512 + 1,
                 num_phys_pages=17 * 512 + 1)
    wsh = lib.sparse_attn_keydiff_workspace_bytes(ctypes.byref(huge), 4, 17 * 8192 + 4)
    assert sel(desc=huge, wsb=wsh, budget=17 * 8192 + 4, sink=4) == B.SA_ERR_UNSUPPORTED  # 17 chunks
    for bad, code in BAD_DESCS:
        assert sel(desc=_desc(**bad)) == code

    def comp(**kw):
        a = dict(src=d, dst=_desc(max_pages_per_seq=4, num_phys_pages=8, max_seq_len=64), kept=DEV, cnt=DEV,
                 budget=64)
        a.update(kw)
        return lib.sparse_attn_keydiff_compact(ctypes.byref(a["src"]), a["kept"], a["cnt"], a["budget"],
                                               ctypes.byref(a["dst"]), None)

    def sel_c(**kw):
        a = dict(desc=d, sink=4, budget=64, sums=DEV, groups=1, ccount=DEV, kept=DEV, cnt=DEV, ws=DEV, wsb=ws)
        a.update(kw)
        return lib.sparse_attn_keydiff_select_carried(ctypes.byref(a["desc"]), a["sink"], a["budget"], a["sums"],
                                                      a["groups"], a["ccount"], a["kept"], a["cnt"], a["ws"],
                                                      a["wsb"], None)

    assert sel_c(sums=None) == B.SA_ERR_INVALID_ARG
    assert sel_c(ccount=None) == B.SA_ERR_INVALID_ARG
    assert sel_c(groups=0) == B.SA_ERR_INVALID_ARG
    assert sel_c(kept=None) == B.SA_ERR_INVALID_ARG
    assert sel_c(wsb=ws - 1) == B.SA_ERR_INVALID_ARG
    assert sel_c(budget=3) == B.SA_ERR_INVALID_ARG
    for bad, code in BAD_DESCS:
        assert sel_c(desc=_desc(**bad)) == code
    assert lib.sparse_attn_keydiff_slot_groups(64) == 1
    assert lib.sparse_attn_keydiff_slot_groups(65) == 2
    assert lib.sparse_attn_keydiff_slot_groups(8192) == 128
    assert lib.sparse_attn_keydiff_slot_groups(0) == -B.SA_ERR_INVALID_ARG

    def comp_s(**kw):
        a = dict(src=d, dst=_desc(max_pages_per_seq=4, num_phys_pages=8, max_seq_len=64), kept=DEV, cnt=DEV,
                 budget=64, sums=DEV)
        a.update(kw)
        return lib.sparse_attn_keydiff_compact_sums(ctypes.byref(a["src"]), a["kept"], a["cnt"], a["budget"],
                                                    ctypes.byref(a["dst"]), a["sums"], None)

    assert comp_s(sums=None) == B.SA_ERR_INVALID_ARG
    assert comp_s(kept=None) == B.SA_ERR_INVALID_ARG
    assert comp_s(budget=65) == B.SA_ERR_INVALID_ARG

    assert comp(kept=None) == B.SA_ERR_INVALID_ARG
    assert comp(cnt=None) == B.SA_ERR_INVALID_ARG
    assert comp(budget=0) == B.SA_ERR_INVALID_ARG
    assert comp(budget=65) == B.SA_ERR_INVALID_ARG  # beyond the destination's 64 slots
    assert comp(dst=_desc(max_pages_per_seq=4, num_phys_pages=8, max_seq_len=64, head_dim=64)) == B.SA_ERR_INVALID_ARG
    assert comp(dst=_desc(max_pages_per_seq=4, num_phys_pages=8, max_seq_len=64, dtype=B.SA_F32)) == \
        B.SA_ERR_INVALID_ARG
    assert comp(dst=_desc(max_pages_per_seq=4, num_phys_pages=8, max_seq_len=64, batch=3)) == B.SA_ERR_INVALID_ARG
    assert comp(dst=_desc(max_pages_per_seq=4, num_phys_pages=8, max_seq_len=64, num_kv_heads=4)) == \
        B.SA_ERR_INVALID_ARG
    for bad, code in BAD_DESCS:
        assert comp(src=_desc(**bad)) == code
        assert comp(dst=_desc(**bad)) == code


def test_blocks_visible_checks():
    lib = B.library()

    def vis(**kw):
        a = dict(desc=_desc(), ix=_index(), W=8, out=DEV)
        a.update(kw)
        ixp = ctypes.byref(a["ix"]) if a["ix"] is not None else None
        return lib.sparse_attn_blocks_visible(ctypes.byref(a["desc"]), ixp, a["W"], a["out"], None)

    assert vis(out=None) == B.SA_ERR_INVALID_ARG
    assert vis(W=-1) == B.SA_ERR_INVALID_ARG
    assert vis(ix=None) == B.SA_ERR_INVALID_ARG
    assert vis(ix=_index(positions=None)) == B.SA_ERR_INVALID_ARG
    assert vis(ix=_index(num_blocks=0)) == B.SA_ERR_INVALID_ARG
    for bad, code in BAD_DESCS:
        assert vis(desc=_desc(**bad)) == code



def test_launches_past_the_dispatch_limit_are_refused():
    """A launch whose grid would exceed 2^32 work-items is refused on the
    host (SA_ERR_UNSUPPORTED), before anything is queued."""
    lib = B.library()
    # decode: 1024 * 8 * 1 * 1024 workgroups of 512 work-items = 2^32
    d = _desc(batch=1024, num_q_heads=8, num_kv_heads=8)
    assert lib.sparse_attn_decode(ctypes.byref(d), DEV, 1, DEV, DEV, 2, 16, 16, 3, 0.0, 1024, 0, DEV, DEV,
                                  None) == B.SA_ERR_UNSUPPORTED
    ws = lib.sparse_attn_workspace_bytes(ctypes.byref(d), 1)
    assert lib.sparse_attn_decode_step(ctypes.byref(d), DEV, 1, DEV, 0, 16, 16, 32, 0.0, 1024, DEV, DEV, DEV, ws,
                                       DEV, DEV, None) == B.SA_ERR_UNSUPPORTED
    # grouped: union of min(4096 pages, 128 rows * 8) = 1024 pages x 64 token chunks x 128 (b, kvh) x 512
    g = _desc(batch=64, num_q_heads=8, num_kv_heads=2, max_pages_per_seq=4096, num_phys_pages=4096,
              max_seq_len=4096 * 16)
    gws = lib.sparse_attn_grouped_workspace_bytes(ctypes.byref(g))
    assert lib.sparse_attn_decode_grouped(ctypes.byref(g), DEV, 128, DEV, DEV, 8, 16, 128, 0.0, 64, 1, DEV, DEV,
                                          DEV, gws, None) == B.SA_ERR_UNSUPPORTED
    # and the per-row decode of the sink and window: 64 * 2 * 128 rows x 1024 local splits of 512 = 2^33
    assert lib.sparse_attn_decode_grouped(ctypes.byref(g), DEV, 128, DEV, DEV, 0, 16, 128, 0.0, 1, 1024, DEV, DEV,
                                          DEV, gws, None) == B.SA_ERR_UNSUPPORTED
    # combine: one 64-lane wave per row
    assert lib.sparse_attn_combine(1 << 26, 128, 2, DEV, DEV, DEV, 1, None, None) == B.SA_ERR_UNSUPPORTED


def test_step_path_reports_the_kernels_decode_step_queues():
    lib = B.library()
    d = _desc(max_pages_per_seq=8)
    ws = 0x10000  # 16-byte aligned
    assert B.sparse_attn_step_path(d, 16, 16, 32, 4, ws) == B.SA_STEP_FUSED
    assert B.sparse_attn_step_path(d, 16, 16, 32, 4, ws + 4) == B.SA_STEP_SEPARATE  # misaligned workspace
    assert B.sparse_attn_step_path(_desc(dtype=B.SA_F32), 16, 16, 32, 4, ws) == B.SA_STEP_SEPARATE
    assert B.sparse_attn_step_path(d, 16, 16, 0, 4, ws) == B.SA_STEP_SEPARATE  # no pages to select
    assert B.sparse_attn_step_path(_desc(max_pages_per_seq=10, max_seq_len=160), 16, 16, 32, 4,
                                   ws) == B.SA_STEP_SEPARATE  # rows not a multiple of 4 entries
    # a sink + window + budget that one workgroup of the fused kernel cannot hold at one split
    assert B.sparse_attn_step_path(d, 4000, 16, 32, 1, ws) == B.SA_STEP_SEPARATE
    assert B.sparse_attn_step_path(_desc(batch=0), 16, 16, 32, 4, ws) == -B.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_step_path(None, 16, 16, 32, 4, ws) == -B.SA_ERR_INVALID_ARG


def test_static_step_checks():
    """The entry point without caller buffers checks everything, and the
    size of its static scratch, before any HIP call."""
    lib = B.library()
    d = _desc()

    def st(desc=None, **kw):
        a = dict(q=DEV, rows=1, meta=DEV, mode=0, S=16, W=16, budget=32, scale=0.0, splits=4, sel=DEV, cnt=DEV,
                 out=DEV, odt=1, lse=None)
        a.update(kw)
        return lib.sparse_attn_decode_step_static(ctypes.byref(desc or d), a["q"], a["rows"], a["meta"], a["mode"],
                                                  a["S"], a["W"], a["budget"], a["scale"], a["splits"], a["sel"],
                                                  a["cnt"], a["out"], a["odt"], a["lse"], None)

    assert st(q=None) == B.SA_ERR_INVALID_ARG
    assert st(meta=None) == B.SA_ERR_INVALID_ARG
    assert st(out=None) == B.SA_ERR_INVALID_ARG
    assert st(sel=None) == B.SA_ERR_INVALID_ARG
    assert st(cnt=None) == B.SA_ERR_INVALID_ARG
    assert st(rows=0) == B.SA_ERR_INVALID_ARG
    assert st(W=0) == B.SA_ERR_INVALID_ARG
    assert st(splits=0) == B.SA_ERR_INVALID_ARG
    assert st(odt=5) == B.SA_ERR_UNSUPPORTED
    assert st(mode=9) == B.SA_ERR_UNSUPPORTED
    # 64 sequences x 64 q heads x 64 splits of (128 + 2) floats: 136 MB of partials
    big = _desc(batch=64, num_q_heads=64, num_kv_heads=8)
    assert st(desc=big, splits=64) == B.SA_ERR_SCRATCH
    assert "static scratch" in B.sparse_attn_status_string(B.SA_ERR_SCRATCH)
    for bad, code in BAD_DESCS:
        assert st(desc=_desc(**bad)) == code


def test_selection_past_one_workgroup_sizes_and_limits():
    """Past 12288 candidate pages per sequence the selection runs per chunk of
    8192 and merges the winners: the workspace holds every chunk's winners,
    and shapes whose winners would not fit the merge are refused."""
    lib = B.library()
    d = _desc(batch=1, num_q_heads=8, num_kv_heads=1, page_size=64, max_pages_per_seq=16384,
              num_phys_pages=16384, max_seq_len=16384 * 64)
    ws = lib.sparse_attn_workspace_bytes(ctypes.byref(d), 1)
    scores = 4 * 16384
    part = 4 * 2 * 8192  # two chunks of 8192 winners, keys and indices
    assert ws >= scores + 2 * part
    sel = lambda budget, wsb=ws: lib.sparse_attn_select(ctypes.byref(d), DEV, 1, DEV, 0, 256, 4096, budget, DEV,
                                                       DEV, DEV, wsb, None)
    assert sel(64 * 6145) == B.SA_ERR_UNSUPPORTED  # 2 chunks x 6145 winners > 12288
    assert sel(64 * 1024, wsb=scores + part) == B.SA_ERR_INVALID_ARG  # no room for the winners
    big = _desc(batch=1, num_q_heads=8, num_kv_heads=1, page_size=1, max_pages_per_seq=65 * 8192,
                num_phys_pages=65 * 8192, max_seq_len=65 * 8192)
    wsb = lib.sparse_attn_workspace_bytes(ctypes.byref(big), 1)
    assert lib.sparse_attn_select(ctypes.byref(big), DEV, 1, DEV, 0, 0, 16, 8, DEV, DEV, DEV, wsb,
                                  None) == B.SA_ERR_UNSUPPORTED  # more than 64 chunks
    # the step refuses the same shapes before any launch
    assert lib.sparse_attn_decode_step(ctypes.byref(d), DEV, 1, DEV, 0, 256, 4096, 64 * 6145, 0.0, 8, DEV, DEV, DEV,
                                       ws, DEV, DEV, None) == B.SA_ERR_UNSUPPORTED
