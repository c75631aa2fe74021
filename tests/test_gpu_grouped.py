"""Parity of the multi-query decode grouped by page (sparse_attn_decode_grouped)
with the fp64 oracle on the GPU's own per-row selection, against the per-row
decode of the same selection, and its determinism.  Shapes cover every GQA
group size, both head dims, pages of 16 to 2048 tokens, 5 to 128 query rows,
windows shorter than the row count (causal masking of middle tokens), two
passes over the query columns (G = 8 with 64 rows), rows whose lists are
shorter than k_max, several token and sink/window split counts, and
pages whose chunks end at the edges of the 64-token stages."""
import numpy as np
import pytest

import oracle
from block_sparse_long_page_amd import synth
from parity import check_lse, check_output

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from block_sparse_long_page_amd.device import DeviceCache, GroupedStep, SparseDecoder, to_device  # noqa: E402

CASES = {
    "g4-p64-q16": dict(B=2, Hq=8, Hkv=2, hd=128, P=64, seq_lens=[3000, 1777], sink=32, window=64, budget=512, Q=16),
    "g8-p32-q5-causal": dict(B=2, Hq=16, Hkv=2, hd=128, P=32, seq_lens=[1500, 700], sink=16, window=3, budget=256,
                             Q=5),
    "g1-hd64-p16-q64": dict(B=2, Hq=2, Hkv=2, hd=64, P=16, seq_lens=[2048, 999], sink=16, window=64, budget=256,
                            Q=64),
    "g16-p128-q7": dict(B=1, Hq=16, Hkv=1, hd=128, P=128, seq_lens=[5000], sink=0, window=100, budget=1024, Q=7),
    "g8-p64-q64-two-passes": dict(B=2, Hq=16, Hkv=2, hd=128, P=64, seq_lens=[4096, 2500], sink=64, window=64,
                                  budget=512, Q=64),
    "g2-hd64-p16-short": dict(B=3, Hq=4, Hkv=2, hd=64, P=16, seq_lens=[200, 40, 777], sink=8, window=16,
                              budget=1024, Q=9),
    "g4-p2048-q64-blocks": dict(B=1, Hq=8, Hkv=2, hd=128, P=2048, seq_lens=[16384 + 64], sink=0, window=64,
                                budget=4096, Q=64),
    # more than 64 rows: the second word of the row masks and of the slot table
    "g4-p64-q128": dict(B=2, Hq=8, Hkv=2, hd=128, P=64, seq_lens=[4000, 3333], sink=32, window=128, budget=512,
                        Q=128),
    "g8-hd64-p32-q100-causal": dict(B=1, Hq=8, Hkv=1, hd=64, P=32, seq_lens=[2500], sink=16, window=50, budget=320,
                                    Q=100),
}


def _problem(name, mode="quest", seed=0):
    return synth.random_problem(**CASES[name], mode=mode, dtype="bf16", seed=2000 + seed, shuffle=True,
                                spare_pages=3, clusters=6)


def _setup(pr, ts=None, ls=None):
    dc = DeviceCache.from_host(pr.cache)
    dec = SparseDecoder(dc, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget)
    q = to_device(pr.q)
    dec.build_meta()
    dec.select(q)
    return dc, dec, GroupedStep(dec, token_splits=ts, local_splits=ls), q


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("splits", [(None, None), (1, 1), (3, 2)])
def test_grouped_matches_oracle_and_per_row(name, splits):
    mode = "centroid" if "blocks" in name else "quest"
    pr = _problem(name, mode)
    dc, dec, gs, q = _setup(pr, *splits)
    gs.decode(q)
    gs.combine()
    torch.cuda.synchronize()
    sel, cnt = dec.selection()
    ref = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget,
                     sel=sel, cnt=cnt)
    out_g, lse_g = dec.out_f32(), dec.lse_f32()
    check_output(out_g, ref.out, pr.cache.dtype, name + " grouped")
    check_lse(lse_g, ref.lse, name + " grouped")
    # bitwise repeatable
    o1, l1 = dec.out.clone(), dec.lse.clone()
    gs.decode(q)
    gs.combine()
    torch.cuda.synchronize()
    assert torch.equal(dec.out, o1) and torch.equal(dec.lse, l1)
    # the per-row decode of the same lists attends the same tokens
    dec.decode(q)
    dec.combine()
    torch.cuda.synchronize()
    check_output(out_g, dec.out_f32(), pr.cache.dtype, name + " grouped vs per-row")
    np.testing.assert_allclose(lse_g, dec.lse_f32(), rtol=0, atol=2e-3)


# (page size, length, budget, token splits, head dim): a page's chunk of
# tokens at 1, 63 and 65 tokens and at 192, 193 and 200 (three stages of 64
# in flight, one past them, and a ragged fourth), pages that are no power of two
@pytest.mark.parametrize("P,L,budget,ts,hd", [
    (1, 600, 64, 1, 128), (63, 3000, 630, 1, 128), (65, 3000, 650, 1, 64), (192, 5000, 1920, 1, 128),
    (193, 5000, 1930, 1, 64), (400, 6000, 2000, 2, 128)])
def test_grouped_at_stage_edges(P, L, budget, ts, hd):
    pr = synth.random_problem(B=2, Hq=8, Hkv=2, hd=hd, P=P, seq_lens=[L, L - 77], sink=5, window=70, budget=budget,
                              Q=8, mode="quest", dtype="bf16", seed=P + L + hd, shuffle=True, spare_pages=3,
                              clusters=6)
    dc, dec, gs, q = _setup(pr, ts, 1)
    gs.decode(q)
    gs.combine()
    torch.cuda.synchronize()
    sel, cnt = dec.selection()
    ref = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget,
                     sel=sel, cnt=cnt)
    what = f"P={P} L={L} budget={budget} ts={ts} hd={hd}"
    check_output(dec.out_f32(), ref.out, pr.cache.dtype, what)
    check_lse(dec.lse_f32(), ref.lse, what)


def test_grouped_shares_pages_between_rows():
    """Rows with the same query choose the same pages: the union is one
    row's list and every row's output is identical to that row's."""
    pr = _problem("g4-p64-q16")
    pr.q[:] = pr.q[:, :, :1, :]  # every row carries row 0's query
    dc, dec, gs, q = _setup(pr)
    gs.decode(q)
    gs.combine()
    torch.cuda.synchronize()
    sel, cnt = dec.selection()
    assert (sel == sel[:, :, :1, :]).all() and (cnt == cnt[:, :, :1]).all()
    ref = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget,
                     sel=sel, cnt=cnt)
    check_output(dec.out_f32(), ref.out, pr.cache.dtype, "shared")
    check_lse(dec.lse_f32(), ref.lse, "shared")


def test_grouped_without_pages_is_the_sink_and_window():
    """k_max = 0 (no budget): the grouped call attends sink + window only."""
    kw = dict(CASES["g4-p64-q16"])
    kw["budget"] = 0
    pr = synth.random_problem(**kw, mode="quest", dtype="bf16", seed=7, shuffle=True)
    dc, dec, gs, q = _setup(pr)
    gs.decode(q)
    gs.combine()
    torch.cuda.synchronize()
    sel, cnt = dec.selection()
    ref = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=0,
                     sel=sel, cnt=cnt)
    check_output(dec.out_f32(), ref.out, pr.cache.dtype, "no pages")


def test_grouped_ignores_bad_list_entries():
    """Entries outside the candidate pages, or not above the entry before
    them (a repeated page among them), are not attended by the grouped
    decode: its output equals the oracle over the lists with those entries
    removed, and no slot is left unwritten (finite outputs)."""
    pr = _problem("g4-p64-q16", seed=5)
    dc, dec, gs, q = _setup(pr)
    torch.cuda.synchronize()
    sel, cnt = dec.selection()
    sel, cnt = sel.copy(), cnt.copy()
    c = pr.cache
    k_max = sel.shape[-1]
    for b in range(c.B):
        L = int(c.seq_lens[b])
        se = min(pr.sink, L)
        ws = max(se, L - pr.window)
        phi = (ws - 1) // c.P
        for kvh in range(c.Hkv):
            assert (cnt[b, kvh, :4] >= 4).all()
            sel[b, kvh, 0, 1] = phi + 1 + kvh          # past the candidates (a window page or beyond)
            sel[b, kvh, 1, 2] = sel[b, kvh, 1, 1]      # a repeated page
            sel[b, kvh, 2, 3] = -7                     # negative
            sel[b, kvh, 3, cnt[b, kvh, 3] - 1] = sel[b, kvh, 3, 0]  # below its predecessor
    full = dec.sel.cpu().numpy()
    full[..., :k_max] = sel
    dec.sel.copy_(torch.from_numpy(full))
    gs.decode(q)
    gs.combine()
    torch.cuda.synchronize()
    clean_sel = np.full_like(sel, -1)
    clean_cnt = np.zeros_like(cnt)
    for b in range(c.B):
        L = int(c.seq_lens[b])
        se = min(pr.sink, L)
        ws = max(se, L - pr.window)
        plo, phi = se // c.P, (ws - 1) // c.P
        for kvh in range(c.Hkv):
            for i in range(pr.Q):
                row = sel[b, kvh, i, :cnt[b, kvh, i]]
                keep = [int(p) for j, p in enumerate(row) if plo <= p <= phi and (j == 0 or p > row[j - 1])]
                clean_sel[b, kvh, i, :len(keep)] = keep
                clean_cnt[b, kvh, i] = len(keep)
    assert (clean_cnt < cnt).sum() == 4 * c.B * c.Hkv
    ref = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget,
                     sel=clean_sel[..., :k_max], cnt=clean_cnt)
    check_output(dec.out_f32(), ref.out, c.dtype, "bad entries")
    check_lse(dec.lse_f32(), ref.lse, "bad entries")
