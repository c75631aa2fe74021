"""Parity of each HIP kernel with the fp64 oracle on small shapes that still
span several tiles and ragged tails: summaries, selection (band rule),
split-K decode + combine on the GPU's own selection, the dense path, split
invariance, determinism, incremental summaries and degenerate cases."""
import numpy as np
import pytest

import oracle
from block_sparse_long_page_amd import synth
from helpers import dense_keys_values, query
from parity import check_lse, check_output, check_selection

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from block_sparse_long_page_amd import binding as B  # noqa: E402
from block_sparse_long_page_amd.device import DeviceCache, SparseDecoder, to_device  # noqa: E402

CASES = {
    "bf16-hd128-g8-p64": dict(B=2, Hq=16, Hkv=2, hd=128, P=64, seq_lens=[3000, 1777], sink=64, window=256,
                              budget=512, dtype="bf16"),
    "bf16-hd128-g4-p16": dict(B=3, Hq=8, Hkv=2, hd=128, P=16, seq_lens=[2048, 999, 40], sink=32, window=100,
                              budget=256, dtype="bf16"),
    "f32-hd64-g4-p16": dict(B=1, Hq=4, Hkv=1, hd=64, P=16, seq_lens=[2048], sink=16, window=64, budget=128,
                            dtype="f32"),
    "bf16-hd64-g1-p7": dict(B=2, Hq=2, Hkv=2, hd=64, P=7, seq_lens=[700, 333], sink=5, window=30, budget=70,
                            dtype="bf16"),
    "bf16-hd128-g16-p32": dict(B=1, Hq=16, Hkv=1, hd=128, P=32, seq_lens=[4100], sink=0, window=33, budget=640,
                               dtype="bf16"),
    "f32-hd128-g2-p1": dict(B=2, Hq=4, Hkv=2, hd=128, P=1, seq_lens=[300, 129], sink=3, window=7, budget=40,
                            dtype="f32"),
    "bf16-hd128-g8-q5": dict(B=2, Hq=16, Hkv=2, hd=128, P=32, seq_lens=[1500, 700], sink=16, window=3, budget=256,
                             dtype="bf16", Q=5),
}
MODES = ["quest", "mean", "centroid", "compressed"]


def _problem(name, mode, seed=0, **over):
    kw = dict(CASES[name])
    kw.update(over)
    return synth.random_problem(**kw, mode=mode, seed=1000 + seed, shuffle=True, spare_pages=5, clusters=8)


def _run(pr, splits=None, dense=False):
    dc = DeviceCache.from_host(pr.cache)
    dec = SparseDecoder(dc, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget, splits=splits)
    q = to_device(pr.q)
    dec.build_meta()
    if not dense:
        dec.select(q)
    dec.decode(q, dense=dense)
    dec.combine()
    torch.cuda.synchronize()
    return dc, dec


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("mode", MODES)
def test_page_summaries(name, mode):
    pr = _problem(name, mode)
    dc = DeviceCache.from_host(pr.cache)
    meta = dc.new_meta(pr.mode)
    B.sparse_attn_build_page_meta(dc.desc(), pr.mode, 0, dc.max_pages, meta)
    torch.cuda.synchronize()
    got = meta.cpu().numpy()
    c = pr.cache
    if pr.mode == oracle.QUEST:
        got = synth.to_f32(got.view(np.uint16), c.dtype) if c.dtype == 1 else got
    for b in range(c.B):
        L = int(c.seq_lens[b])
        n_pages = -(-L // c.P)
        assert (got[b, :, n_pages:] == 0).all()  # pages past the sequence are never written
        for p in range(n_pages):
            for kvh in range(c.Hkv):
                ref, n = oracle.page_summary(c, pr.mode, b, kvh, p)
                g = got[b, kvh, p].reshape(-1).astype(np.float64)
                if pr.mode == oracle.QUEST:
                    np.testing.assert_array_equal(g, ref)  # min/max are exact
                else:
                    K = dense_keys_values(c, b, kvh)[0][p * c.P:p * c.P + n]
                    scale = np.abs(K).mean(0) if pr.mode in (oracle.MEAN, oracle.COMPRESSED) else 1.0
                    assert np.all(np.abs(g - ref) <= 2e-6 * (scale + 1e-30) + 1e-7 * (pr.mode == oracle.CENTROID))


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("mode", MODES)
def test_selection_and_output(name, mode):
    pr = _problem(name, mode)
    dc, dec = _run(pr)
    sel, cnt = dec.selection()
    r = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget,
                   want_scores=True)
    check_selection(sel, cnt, r.scores, pr.k_pages)
    ref = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget,
                     sel=sel, cnt=cnt)
    check_output(dec.out_f32(), ref.out, pr.cache.dtype, name)
    check_lse(dec.lse_f32(), ref.lse, name)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("splits", [None, 1, 5])
def test_select_decode_step(name, mode, splits):
    """sparse_attn_decode_step: the same page lists as sparse_attn_select, the
    oracle's attention over them, and bitwise-repeatable results."""
    pr = _problem(name, mode, seed=7)
    dc, dec = _run(pr, splits=splits)
    sel_ref, cnt_ref = dec.selection()
    q = to_device(pr.q)
    dec.sel.fill_(-7)
    dec.count.fill_(-7)
    dec.fused_step(q)
    torch.cuda.synchronize()
    sel, cnt = dec.selection()
    np.testing.assert_array_equal(cnt, cnt_ref)
    np.testing.assert_array_equal(sel, sel_ref)
    full = dec.sel.cpu().numpy()
    for idx in np.ndindex(cnt.shape):
        assert (full[idx][cnt[idx]:] == -1).all()
    ref = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget,
                     sel=sel, cnt=cnt)
    check_output(dec.out_f32(), ref.out, pr.cache.dtype, name)
    check_lse(dec.lse_f32(), ref.lse, name)
    out1, lse1 = dec.out.clone(), dec.lse.clone()
    dec.fused_step(q)
    torch.cuda.synchronize()
    assert torch.equal(dec.out, out1) and torch.equal(dec.lse, lse1)


# (sink, window, budget, splits, length), 16-token pages: the select-and-decode
# workgroup's sink-and-window share at 1, 15, 16 and 128 tokens and at about
# three tiles per streaming wave, its middle share at one tile, one tile per
# wave and the most one workgroup takes (2048 tokens, 16 tiles per wave), a
# first selected page cut by the sink, and a sequence with fewer candidate
# pages than the budget (nothing ranked)
@pytest.mark.parametrize("S,W,budget,splits,L", [
    (0, 1, 16, 1, 600), (7, 8, 128, 1, 1000), (1, 14, 2016, 1, 4000), (64, 337, 1600, 1, 5000),
    (3, 1000, 1008, 3, 6000), (16, 112, 1888, 2, 3000), (4, 32, 1984, 1, 300)])
@pytest.mark.parametrize("hd", [128, 64])
def test_select_decode_at_tile_edges(S, W, budget, splits, L, hd):
    # the select-and-decode kernel runs when every workgroup's table fits in
    # 2048 entries (its share of the sink and window rounded up to 16, plus
    # its share of the pages) and the block-table rows are 16-byte vectors
    assert splits >= -(-(S + W + budget) // 2031)
    pr = synth.random_problem(B=2, Hq=8, Hkv=2, hd=hd, P=16, seq_lens=[L, L - 17], sink=S, window=W, budget=budget,
                              dtype="bf16", seed=L + S + W + hd, shuffle=True, spare_pages=3, clusters=8,
                              max_pages=-(-L // 64) * 4)
    dc, dec = _run(pr, splits=splits)
    sel_ref, cnt_ref = dec.selection()
    q = to_device(pr.q)
    dec.sel.fill_(-7)
    dec.count.fill_(-7)
    dec.fused_step(q)
    torch.cuda.synchronize()
    sel, cnt = dec.selection()
    np.testing.assert_array_equal(cnt, cnt_ref)
    np.testing.assert_array_equal(sel, sel_ref)
    ref = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=1, sink=S, window=W, budget=budget, sel=sel, cnt=cnt)
    what = f"S={S} W={W} budget={budget} splits={splits} L={L} hd={hd}"
    check_output(dec.out_f32(), ref.out, pr.cache.dtype, what)
    check_lse(dec.lse_f32(), ref.lse, what)


@pytest.mark.parametrize("pattern", ["all-equal", "two-values", "two-values-wide", "small-tie-band"])
@pytest.mark.parametrize("fused", [False, True])
def test_tied_scores_take_the_lower_pages(pattern, fused):
    """Exact ties in the page scores (pages whose tokens all hold one key
    vector) go to the lower logical page, as in the oracle: every key equal;
    a boundary of ~n/2 equal keys (the multi-pass select), about 120 and,
    over 2000 pages, about 1000; and a boundary of a few dozen equal keys
    (ranked directly)."""
    lens = [16384, 3000] if pattern == "two-values-wide" else [2048, 1500]
    pr = synth.random_problem(B=2, Hq=16, Hkv=2, hd=128, P=8, seq_lens=lens, sink=32, window=64,
                              budget=30 * 8, mode="quest", seed=11, shuffle=True)
    c = pr.cache
    rng = np.random.default_rng(3)
    vecs = synth.store(rng.standard_normal((3, c.Hkv, c.hd)).astype(np.float32), c.dtype)
    for b in range(c.B):
        n_pages = -(-int(c.seq_lens[b]) // c.P)
        for p in range(n_pages):
            if pattern == "all-equal":
                w = 0
            elif pattern in ("two-values", "two-values-wide"):
                w = p % 2
            else:  # 10 pages of one value, 40 of a second, the rest a third
                w = 0 if p % 50 < 10 else 1 if p % 50 < 50 and p < 50 else 2
            c.k[c.block_table[b, p]] = vecs[w][:, None, :]
    dc = DeviceCache.from_host(c)
    dec = SparseDecoder(dc, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget)
    q = to_device(pr.q)
    dec.build_meta()
    if fused:
        dec.fused_step(q)
    else:
        dec.step(q)
    torch.cuda.synchronize()
    sel, cnt = dec.selection()
    r = oracle.run(c, pr.q, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget, want_scores=True)
    np.testing.assert_array_equal(cnt, r.cnt)
    np.testing.assert_array_equal(sel, r.sel)  # exact ties: the same (lowest) pages
    ref = oracle.run(c, pr.q, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget, sel=sel,
                     cnt=cnt)
    check_output(dec.out_f32(), ref.out, c.dtype, pattern)


def test_select_decode_at_the_candidate_limit():
    """8448 pages per sequence (the most the select-and-decode kernel stages
    in its local memory; 33792 tokens of 4-token pages): the fused step keeps
    the oracle's page lists and attention, and so does the sequence next to
    it that is a few pages short of the limit."""
    pr = synth.random_problem(B=2, Hq=8, Hkv=2, hd=128, P=4, seq_lens=[33792, 33781], sink=16, window=64,
                              budget=4 * 700, mode="quest", dtype="bf16", seed=31, shuffle=True, clusters=8)
    assert pr.cache.max_pages == 8448
    dc = DeviceCache.from_host(pr.cache)
    dec = SparseDecoder(dc, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget)
    q = to_device(pr.q)
    dec.build_meta()
    dec.fused_step(q)
    torch.cuda.synchronize()
    sel, cnt = dec.selection()
    r = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget,
                   want_scores=True)
    check_selection(sel, cnt, r.scores, pr.k_pages)
    ref = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget, sel=sel,
                     cnt=cnt)
    check_output(dec.out_f32(), ref.out, pr.cache.dtype, "candidate limit")
    check_lse(dec.lse_f32(), ref.lse, "candidate limit")


@pytest.mark.parametrize("name", ["bf16-hd128-g8-p64", "f32-hd64-g4-p16", "bf16-hd128-g16-p32", "bf16-hd128-g8-q5",
                                  "bf16-hd64-g1-p7"])
@pytest.mark.parametrize("mode", MODES)
def test_group_scores_are_fp32_accurate(name, mode):
    """The group scores sparse_attn_select leaves in its workspace agree with
    the oracle's fp64 scores to fp32 rounding: within SCORE_REL of
    max_h |q_h|_1 * max(max |k|, 1) (every summary element is at most
    max |k| in size, a centroid's at most 1), for every candidate page."""
    SCORE_REL = 3e-6
    pr = _problem(name, mode, seed=5)
    c = pr.cache
    dc = DeviceCache.from_host(c)
    dec = SparseDecoder(dc, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget)
    q = to_device(pr.q)
    dec.build_meta()
    dec.select(q)
    torch.cuda.synchronize()
    n = c.B * c.Hkv * pr.Q * c.max_pages
    got = dec.ws[: 4 * n].view(torch.float32).reshape(c.B, c.Hkv, pr.Q, c.max_pages).cpu().numpy()
    r = oracle.run(c, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget,
                   want_scores=True)
    G = c.Hq // c.Hkv
    worst = 0.0
    for b in range(c.B):
        for kvh in range(c.Hkv):
            kmax = max(float(np.abs(dense_keys_values(c, b, kvh)[0]).max()), 1.0)
            for i in range(pr.Q):
                ref = r.scores[b, kvh, i]
                cand = ~np.isnan(ref)
                qn = max(np.abs(query(pr, b, kvh * G + h, i)).sum() for h in range(G))
                err = np.abs(got[b, kvh, i][cand].astype(np.float64) - ref[cand]) / (qn * kmax)
                worst = max(worst, float(err.max()) if err.size else 0.0)
    print(f"{name} {mode}: worst score error {worst:.2e} of |q|_1 max|k|")
    assert worst <= SCORE_REL


@pytest.mark.parametrize("name", list(CASES))
def test_dense_path(name):
    pr = _problem(name, "quest")
    dc, dec = _run(pr, dense=True)
    ref = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=10**9)
    check_output(dec.out_f32(), ref.out, pr.cache.dtype, name)
    check_lse(dec.lse_f32(), ref.lse, name)


# (lengths of the two sequences, splits): with one split a workgroup's row
# table holds every token, so these put its last round of 128 rows (8 waves
# of 16) at 1, 127, 128 and 129 rows, the rounds' count at each residue of the
# three in flight, and the 2048-row chunks of the table one past and one short
@pytest.mark.parametrize("lens,splits", [
    ([1, 127], 1), ([128, 129], 1), ([255, 256], 1), ([383, 384], 1), ([385, 511], 1), ([640, 767], 1),
    ([2047, 2048], 1), ([2049, 2433], 1), ([4481, 6145], 1), ([6145, 385], 3), ([769, 3], 5)])
@pytest.mark.parametrize("hd", [128, 64])
def test_dense_decode_at_round_edges(lens, splits, hd):
    pr = synth.random_problem(B=2, Hq=8, Hkv=2, hd=hd, P=16, seq_lens=lens, sink=4, window=32, budget=64,
                              dtype="bf16", seed=sum(lens) + hd, shuffle=True, spare_pages=3)
    dc, dec = _run(pr, splits=splits, dense=True)
    ref = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=10**9)
    what = f"lens={lens} splits={splits} hd={hd}"
    check_output(dec.out_f32(), ref.out, pr.cache.dtype, what)
    check_lse(dec.lse_f32(), ref.lse, what)


@pytest.mark.parametrize("name", ["bf16-hd128-g8-p64", "f32-hd64-g4-p16", "bf16-hd64-g1-p7"])
def test_split_count_invariance_and_determinism(name):
    pr = _problem(name, "quest", seed=3)
    ref = None
    for splits in (1, 2, 3, 17, 64):
        dc, dec = _run(pr, splits=splits)
        out = dec.out_f32()
        sel, cnt = dec.selection()
        if ref is None:
            ref = out
            o_ref = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window,
                               budget=pr.budget, sel=sel, cnt=cnt)
        check_output(out, o_ref.out, pr.cache.dtype, f"{name} splits={splits}")
        dc2, dec2 = _run(pr, splits=splits)
        assert torch.equal(dec.out, dec2.out) and torch.equal(dec.lse, dec2.lse)  # bitwise reproducible
        assert torch.equal(dec.sel, dec2.sel)


def test_combine_matches_oracle_merge():
    rng = np.random.default_rng(5)
    rows, hd, splits = 37, 128, 9
    po = rng.standard_normal((rows, splits, hd)).astype(np.float32)
    ml = np.stack([rng.normal(0, 4, (rows, splits)), rng.uniform(0.5, 50, (rows, splits))], -1).astype(np.float32)
    ml[3, :, 0] = -np.inf  # a row with every part empty
    ml[3, :, 1] = 0
    ml[5, 2:7, 0] = -np.inf  # some empty parts
    ml[5, 2:7, 1] = 0
    clean = po.copy()
    po[3, :, :] = np.nan  # whatever an empty part's o holds is left out
    po[5, 2:7, ::2] = np.inf
    po[5, 2:7, 1::2] = np.nan
    clean[3], clean[5, 2:7] = 0, 0
    out = torch.empty((rows, hd), dtype=torch.float32, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    B.sparse_attn_combine(rows, hd, splits, to_device(po), to_device(ml), out, B.SA_F32, lse)
    torch.cuda.synchronize()
    got, gl = out.cpu().numpy(), lse.cpu().numpy()
    for r in range(rows):
        if r == 3:
            assert (got[r] == 0).all() and gl[r] == -np.inf
            continue
        ref, rl = oracle.merge(clean[r], ml[r, :, 0], ml[r, :, 1])
        np.testing.assert_allclose(got[r], ref, atol=2e-6, rtol=1e-5)
        assert abs(gl[r] - rl) < 1e-5 * max(1, abs(rl))


@pytest.mark.parametrize("mode", ["quest", "compressed"])
def test_incremental_summary_of_an_appended_page(mode):
    """An append changes the last page's summary and, for compressed keys,
    the one before it (its block reaches into the last page): rebuilding
    just those gives the full rebuild bit for bit."""
    pr = synth.random_problem(B=2, Hq=8, Hkv=2, hd=128, P=32, seq_lens=[1000, 1000], sink=16, window=64,
                              budget=256, dtype="bf16", seed=9, max_pages=40, mode=mode)
    c = pr.cache
    m = pr.mode
    reach = 1 if m == oracle.COMPRESSED else 0
    dc = DeviceCache.from_host(c, max_seq_len=40 * 32)
    meta = dc.new_meta(m)
    d = dc.desc()
    B.sparse_attn_build_page_meta(d, m, 0, dc.max_pages, meta)
    for L in (1001, 1023, 1024, 1025):  # append tokens one page-piece at a time
        dc.seq_lens.fill_(L)
        c.seq_lens[:] = L
        last = (L - 1) // 32
        if c.block_table[0, last] < 0:  # grow the table: give the new page a physical home
            for b in range(c.B):
                c.block_table[b, last] = b * c.max_pages + last
            dc.block_table.copy_(to_device(c.block_table))
        B.sparse_attn_build_page_meta(d, m, max(0, last - reach), last + 1, meta)
    full = dc.new_meta(m)
    B.sparse_attn_build_page_meta(d, m, 0, dc.max_pages, full)
    torch.cuda.synchronize()
    assert torch.equal(meta, full)


def test_summaries_refreshed_at_selection_match_per_token_folding():
    """The refresh schedule of the hybrid decode loop, two ways over 70 steps
    of one appended token each (selection every 32 steps, the window grown
    by the steps since): folding each token into the last page's summary as
    it arrives, and summarising the pages appended since the last selection
    right before the next one.  Summaries are read only when selecting, so
    the summaries at every selection and every step's output are identical."""
    L0, T, R, W = 4000, 70, 32, 64
    pr = synth.random_problem(B=2, Hq=8, Hkv=2, hd=128, P=32, seq_lens=[L0 + T, L0 + T], sink=16, window=W,
                              budget=32 * 16, dtype="bf16", seed=21, shuffle=True, clusters=8)
    c = pr.cache
    c.seq_lens[:] = L0
    dc = DeviceCache.from_host(c, max_seq_len=L0 + T)
    eager = SparseDecoder(dc, mode=pr.mode, Q=1, sink=pr.sink, window=W, budget=pr.budget)
    lazy = SparseDecoder(dc, mode=pr.mode, Q=1, sink=pr.sink, window=W, budget=pr.budget)
    eager.build_meta()
    lazy.build_meta()
    rng = np.random.default_rng(5)
    t_ref = 0
    for t in range(T):
        L = L0 + t
        if t > 0:
            dc.seq_lens.fill_(L)
            eager.build_meta((L - 1) // dc.P, (L - 1) // dc.P + 1)
        q = to_device(synth.store(rng.standard_normal((c.B, c.Hq, 1, c.hd)).astype(np.float32), c.dtype))
        outs = []
        for dec in (eager, lazy):
            if t % R == 0:
                if dec is lazy and t > 0:
                    dec.build_meta((L0 + t_ref - 1) // dc.P, (L - 1) // dc.P + 1)
                dec.select_decode(q)
            else:
                dec.decode(q, window=W + (t - t_ref))
            dec.combine()
            outs.append(dec.out.clone())
        if t % R == 0:
            t_ref = t
            torch.cuda.synchronize()
            assert torch.equal(eager.meta, lazy.meta), t
            assert torch.equal(eager.sel, lazy.sel) and torch.equal(eager.count, lazy.count), t
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), t


@pytest.mark.parametrize("L,S,W,budget,Q", [
    (1, 0, 1, 0, 1),  # a single token
    (5, 2, 1, 64, 5),  # every position is a query row
    (100, 200, 8, 64, 1),  # the sink covers the sequence
    (100, 8, 500, 64, 2),  # the window covers the sequence
    (200, 60, 60, 32, 1),  # sink + window covers almost everything
    (1000, 16, 16, 10**6, 1),  # budget covers every candidate
    (1000, 16, 16, 0, 3),  # no selected pages: sink + window only
])
def test_degenerate_shapes(L, S, W, budget, Q):
    pr = synth.random_problem(B=2, Hq=8, Hkv=2, hd=128, P=16, seq_lens=[L, max(Q, L // 2)], sink=S, window=W,
                              budget=budget, dtype="bf16", Q=Q, seed=L + S + W, shuffle=True)
    dc, dec = _run(pr)
    sel, cnt = dec.selection()
    r = oracle.run(pr.cache, pr.q, mode=0, Q=Q, sink=S, window=W, budget=budget, want_scores=True)
    check_selection(sel, cnt, r.scores, pr.k_pages)
    ref = oracle.run(pr.cache, pr.q, mode=0, Q=Q, sink=S, window=W, budget=budget, sel=sel, cnt=cnt)
    check_output(dec.out_f32(), ref.out, 1, "degenerate")


def test_empty_sequence_gives_zero_output():
    pr = synth.random_problem(B=2, Hq=4, Hkv=1, hd=64, P=16, seq_lens=[64, 64], sink=4, window=8, budget=32,
                              dtype="f32", seed=3)
    dc = DeviceCache.from_host(pr.cache)
    dc.seq_lens[1] = 0
    dec = SparseDecoder(dc, mode=0, Q=1, sink=4, window=8, budget=32, splits=4)
    q = to_device(pr.q)
    dec.build_meta()
    dec.step(q)
    torch.cuda.synchronize()
    out, lse = dec.out_f32(), dec.lse_f32()
    assert (out[1] == 0).all() and (lse[1] == -np.inf).all()
    assert (dec.count.cpu().numpy()[1] == 0).all()
    pr.cache.seq_lens[1] = 1  # the oracle needs a token; compare only sequence 0
    ref = oracle.run(pr.cache, pr.q, mode=0, Q=1, sink=4, window=8, budget=32,
                     sel=dec.selection()[0], cnt=dec.selection()[1])
    check_output(out[0], ref.out[0], 0)


@pytest.mark.parametrize("name", ["bf16-hd128-g8-p64", "bf16-hd128-g4-p16", "f32-hd64-g4-p16", "bf16-hd128-g8-q5"])
@pytest.mark.parametrize("splits", [(1, 1), (3, 5), (7, 2)])
def test_overlapped_sink_window_and_middle_decodes(name, splits):
    from block_sparse_long_page_amd.device import OverlappedStep

    pr = _problem(name, "quest", seed=4)
    dc = DeviceCache.from_host(pr.cache)
    dec = SparseDecoder(dc, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget)
    q = to_device(pr.q)
    dec.build_meta()
    ov = OverlappedStep(dec, local_splits=splits[0], middle_splits=splits[1])
    ov.step(q)
    torch.cuda.synchronize()
    out_ov, lse_ov = dec.out_f32(), dec.lse_f32()
    sel, cnt = dec.selection()
    ref = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget,
                     sel=sel, cnt=cnt)
    check_output(out_ov, ref.out, pr.cache.dtype, f"{name} overlapped")
    check_lse(lse_ov, ref.lse, f"{name} overlapped")
    dec.step(q)  # one call over the whole set
    torch.cuda.synchronize()
    np.testing.assert_allclose(out_ov, dec.out_f32(), atol=TOL_SPLIT[pr.cache.dtype], rtol=0)


TOL_SPLIT = {0: 2e-6, 1: 1e-2}  # fp32 rounding only; bf16: outputs are rounded to bf16


def test_select_decode_wait_bound_is_reported(monkeypatch):
    """The select-and-decode kernel's wait for its page list is bounded.  With
    the bound lowered to one round from the host (every wave still leaves its
    loop and the kernel ends normally), the workgroups that could not finish
    their share write NaN partials: the combined rows are NaN, never a silently
    wrong value, and a synchronised call reports SA_ERR_HIP.  The next call at
    the normal bound finds the status word cleared and matches the oracle."""
    pr = synth.random_problem(B=1, Hq=8, Hkv=1, hd=128, P=64, seq_lens=[16384], sink=64, window=1024,
                              budget=2048, mode="quest", dtype="bf16", seed=5, shuffle=True)
    dc = DeviceCache.from_host(pr.cache)
    dec = SparseDecoder(dc, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget, splits=2)
    q = to_device(pr.q)
    dec.build_meta()
    assert B.sparse_attn_step_path(dec.desc, pr.sink, pr.window, pr.budget, dec.splits, dec.ws) == B.SA_STEP_FUSED
    torch.cuda.synchronize()
    monkeypatch.setenv("SPARSE_ATTN_SPIN_LIMIT", "1")
    monkeypatch.setenv("SPARSE_ATTN_SYNC", "1")
    with pytest.raises(B.SparseAttnError) as err:
        dec.select_decode(q)
    assert err.value.status == B.SA_ERR_HIP
    dec.combine()
    torch.cuda.synchronize()
    assert np.isnan(dec.out_f32()).all() and np.isnan(dec.lse_f32()).all()
    monkeypatch.delenv("SPARSE_ATTN_SPIN_LIMIT")
    dec.fused_step(q)  # still synchronised: the status word must read clear
    torch.cuda.synchronize()
    sel, cnt = dec.selection()
    ref = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget,
                     sel=sel, cnt=cnt)
    check_output(dec.out_f32(), ref.out, pr.cache.dtype, "after the bound")


@pytest.mark.parametrize("pattern", ["random", "all-equal"])
def test_selection_over_chunks_of_candidates(pattern):
    """More candidate pages than one workgroup ranks (20000 and 12500 pages of
    4 tokens): each chunk of 8192 candidates keeps its best and a merge ranks
    them.  The pages match the oracle within the band, and with every key
    equal (exact ties across the chunk boundaries) they are exactly the
    lowest candidates, as in the oracle."""
    pr = synth.random_problem(B=2, Hq=8, Hkv=2, hd=64, P=4, seq_lens=[80000, 50000], sink=16, window=64,
                              budget=4 * 900, mode="quest", dtype="bf16", seed=17, shuffle=True, clusters=8)
    c = pr.cache
    if pattern == "all-equal":
        vec = synth.store(np.random.default_rng(5).standard_normal((c.Hkv, c.hd)).astype(np.float32), c.dtype)
        c.k[:] = vec[None, :, None, :]
    assert c.max_pages == 20000
    dc = DeviceCache.from_host(c)
    dec = SparseDecoder(dc, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget)
    assert B.sparse_attn_step_path(dec.desc, pr.sink, pr.window, pr.budget, dec.splits, dec.ws) == B.SA_STEP_SEPARATE
    q = to_device(pr.q)
    dec.build_meta()
    dec.fused_step(q)
    torch.cuda.synchronize()
    sel, cnt = dec.selection()
    r = oracle.run(c, pr.q, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget, want_scores=True)
    if pattern == "all-equal":
        np.testing.assert_array_equal(cnt, r.cnt)
        np.testing.assert_array_equal(sel, r.sel)
    else:
        check_selection(sel, cnt, r.scores, pr.k_pages)
    ref = oracle.run(c, pr.q, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget, sel=sel,
                     cnt=cnt)
    check_output(dec.out_f32(), ref.out, c.dtype, pattern)
    check_lse(dec.lse_f32(), ref.lse, pattern)


@pytest.mark.parametrize("pattern", ["clustered", "random", "few-values"])
def test_block_topk_is_exact_on_the_gpu_scores(pattern):
    """The separate selection's top-k (k_topk) against the exact top-k of the
    fp32 scores the score kernel left in the workspace (larger first, ties to
    the lower page; -0 ranks as +0): no band, every page must match.
    'clustered' draws every key near one vector, so the scores crowd into a
    few radix buckets and the boundary bucket is refined over further digits;
    'few-values' leaves more than 64 equal scores at the boundary."""
    pr = synth.random_problem(B=2, Hq=16, Hkv=2, hd=128, P=8, seq_lens=[16384, 9000], sink=32, window=64,
                              budget=300 * 8, mode="quest", seed=23, shuffle=True)
    c = pr.cache
    rng = np.random.default_rng(7)
    base = rng.standard_normal((c.Hkv, c.hd)).astype(np.float32)
    if pattern == "clustered":
        k = base[None, :, None, :] + 0.02 * rng.standard_normal(c.k.shape).astype(np.float32)
        c.k[:] = synth.store(k, c.dtype)
    elif pattern == "few-values":
        vecs = synth.store(rng.standard_normal((5, c.Hkv, c.hd)).astype(np.float32), c.dtype)
        for b in range(c.B):
            for p in range(-(-int(c.seq_lens[b]) // c.P)):
                c.k[c.block_table[b, p]] = vecs[(p * 7) % 5][:, None, :]
    dc = DeviceCache.from_host(c)
    dec = SparseDecoder(dc, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget)
    q = to_device(pr.q)
    dec.build_meta()
    dec.select(q)
    torch.cuda.synchronize()
    sel, cnt = dec.selection()
    scores = dec.ws[: c.B * c.Hkv * c.max_pages * 4].view(torch.float32).cpu().numpy()
    scores = scores.reshape(c.B, c.Hkv, c.max_pages)
    kp = pr.budget // c.P
    for b in range(c.B):
        L = int(c.seq_lens[b])
        se = min(pr.sink, L)
        ws = max(se, L - pr.window)
        plo = se // c.P
        ncand = (ws - 1) // c.P - plo + 1 if ws > se else 0
        k = min(kp, ncand)
        for h in range(c.Hkv):
            s = scores[b, h, plo:plo + ncand].astype(np.float32) + np.float32(0.0)  # -0 -> +0
            order = np.lexsort((np.arange(ncand), -s.astype(np.float64)))
            want = np.sort(order[:k]) + plo
            assert cnt[b, h, 0] == k
            np.testing.assert_array_equal(sel[b, h, 0, :k], want, err_msg=f"{pattern} b{b} h{h}")
