"""Chunked sparse prefill on the GPU over one index of the whole prompt, by
sparse_attn_prefill_chunk (one call: front, grouped decode of the blocks and
the window's pages, combine) and by the separate calls
(sparse_attn_blocks_visible, sparse_attn_select_blocks,
sparse_attn_decode_blocks), against the fp64 oracle of oracle/semantic.py, on
the GPU's own index: the visible part of every block exactly, the block choice exactly
where no two block scores are within 1e-4 relative of each other at the
budget's edge and elsewhere a valid greedy choice for an order consistent
within that band (tests/parity.py::check_block_choice, such rows counted and
bounded), and the outputs against the oracle's attention over the GPU's
blocks (their visible rows) and the chunk's window.  With every block chosen
each row must be dense causal attention over its prefix, chunk after chunk
over the whole prompt."""
import numpy as np
import pytest

from oracle import semantic as sem
from block_sparse_long_page_amd import configs, synth
from block_sparse_long_page_amd.synth import to_f32
from helpers import dense_keys_values, masked_attention
from parity import check_block_choice, check_lse, check_output

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from block_sparse_long_page_amd.device import BlockIndex, ChunkedPrefill, DeviceCache, to_device  # noqa: E402

CASES = {
    # (G, head_dim, blocks of 64 tokens (128 for chunks of more than 64 rows), chunk rows, window, index blocks)
    "g4-hd128": (4, 128, 16, 16, 48, 12),
    "g2-hd64-ragged": (2, 64, 12, 24, 30, 9),
    "g8-hd128-chunk64": (8, 128, 20, 64, 64, 16),
    "g4-hd128-chunk128": (4, 128, 20, 128, 128, 16),
    # the front's other lane layouts: two lanes per block (17..32 blocks), one
    # lane per block over two rounds (more than 64), a window wider than the chunk
    "g4-hd128-c24-wide-window": (4, 128, 30, 32, 40, 24),
    "g1-hd128-c70": (1, 128, 40, 16, 16, 70),
}


def _setup(name, seed=0, ts=1, k_max=None, fused=True):
    G, hd, nblk, T, W, C = CASES[name]
    bt = 64 if T <= 64 else 128  # the generator appends the last chunk as one page
    wl = configs.SEMANTIC_512K.scaled(batch=2, num_q_heads=2 * G, num_kv_heads=2, head_dim=hd,
                                      context=nblk * bt + 5, page_size=bt, window=T, budget=4 * bt, q_rows=T)
    pr = synth.semantic_problem(wl, seed=seed, blocks=nblk, block_tokens=bt, scatter=True)
    c = pr.cache
    L = int(c.seq_lens[0])
    rng = np.random.default_rng(seed)
    q_all = synth.store(rng.standard_normal((c.B, c.Hq, L, c.hd)).astype(np.float32) * 0.3, c.dtype)
    dc = DeviceCache.from_host(c)
    ix = BlockIndex(dc, L, C, Q=T, window=W, budget=0, k_max=C)
    ix.build(iterations=3)
    torch.cuda.synchronize()
    pf = ChunkedPrefill(ix, T, W, k_max=k_max, token_splits=ts, fused=fused)
    return pr, c, dc, ix, pf, q_all, L, T, W, C


def _qchunk(q_all, c0, T):
    return to_device(np.ascontiguousarray(q_all[:, :, c0:c0 + T]))


def _qgroup(q_all, c, b, kvh, pos):
    G = c.Hq // c.Hkv
    return np.stack([to_f32(q_all[b, kvh * G + h, pos], c.dtype).astype(np.float64) for h in range(G)])


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name,ts,k_max", [(n, 1, None) for n in CASES] + [("g4-hd128", 3, None),
                                                                          ("g8-hd128-chunk64", 2, 3),
                                                                          ("g4-hd128-c24-wide-window", 2, 5)])
def test_prefill_chunks_match_the_oracle(name, ts, k_max, fused):
    pr, c, dc, ix, pf, q_all, L, T, W, C = _setup(name, seed=1, ts=ts, k_max=k_max, fused=fused)
    G = c.Hq // c.Hkv
    perm_all, off_all = ix.positions.cpu().numpy(), ix.offsets.cpu().numpy()
    mu_all = ix.centres.cpu().numpy().astype(np.float64)
    # the first chunk sees no index, the next ones a growing part, the last all but its window
    starts = sorted({0, T, (L - T) // 3, (L - T) // 2, L - T})
    ties = rows = 0
    for c0 in starts:
        budget = max(1, (c0 + T) // 16)
        pf.chunk(_qchunk(q_all, c0, T), c0, budget)
        torch.cuda.synchronize()
        ends = pf.ends.cpu().numpy()
        sel, cnt = pf.sel.cpu().numpy(), pf.count.cpu().numpy()
        out, lse = pf.out_f32(), pf.lse_f32()
        bound = c0 + T - W
        for b in range(c.B):
            for kvh in range(c.Hkv):
                K, V = dense_keys_values(c, b, kvh)
                perm, off, mu = perm_all[b, kvh], off_all[b, kvh], mu_all[b, kvh]
                vis = sem.visible_sizes(perm, off, bound)
                np.testing.assert_array_equal(ends[b, kvh] - off[:-1], vis)
                for i in range(T):
                    pos = c0 + i
                    qg = _qgroup(q_all, c, b, kvh, pos)
                    s = sem.block_scores(qg, mu)
                    got = sel[b, kvh, i, :cnt[b, kvh, i]]
                    assert (sel[b, kvh, i, cnt[b, kvh, i]:] == -1).all()
                    ties += check_block_choice(got, s, vis, budget, pf.k_max)
                    rows += 1
                    toks = np.concatenate([perm[off[x]:off[x] + vis[x]] for x in got] +
                                          [np.arange(max(0, bound), pos + 1)]).astype(np.int64)
                    for h in range(G):
                        o, l_ = sem.attend(qg[h], K[toks], V[toks], 1.0 / np.sqrt(c.hd))
                        check_output(out[b, kvh * G + h, i][None], o[None], c.dtype, f"{name} c0={c0}")
                        check_lse(lse[b, kvh * G + h, i][None], np.array([l_]), f"{name} c0={c0}")
    print(f"{name}: {ties} of {rows} rows with a near tie at the edge")
    assert ties <= max(2, rows // 10)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name,ts", [("g4-hd128", 1), ("g2-hd64-ragged", 4), ("g4-hd128-c24-wide-window", 3)])
def test_prefill_with_every_block_is_dense_causal(name, ts, fused):
    """Every chunk of the prompt with an unlimited budget: each row attends
    its whole prefix exactly once (visible block parts + window), whatever
    the token chunks per block."""
    pr, c, dc, ix, pf, q_all, L, T, W, C = _setup(name, seed=2, ts=ts, fused=fused)
    G = c.Hq // c.Hkv
    keys = [[dense_keys_values(c, b, kvh) for kvh in range(c.Hkv)] for b in range(c.B)]
    for c0 in range(0, L - T + 1, T):
        pf.chunk(_qchunk(q_all, c0, T), c0, 10**9)
        torch.cuda.synchronize()
        out, lse = pf.out_f32(), pf.lse_f32()
        ref_o = np.zeros(out.shape)
        ref_l = np.zeros(lse.shape)
        for b in range(c.B):
            for kvh in range(c.Hkv):
                K, V = keys[b][kvh]
                for i in range(T):
                    pos = c0 + i
                    qg = _qgroup(q_all, c, b, kvh, pos)
                    for h in range(G):
                        ref_o[b, kvh * G + h, i], ref_l[b, kvh * G + h, i] = masked_attention(
                            qg[h], K, V, np.arange(L) <= pos, 1.0 / np.sqrt(c.hd))
        check_output(out, ref_o, c.dtype, f"{name} c0={c0}")
        check_lse(lse, ref_l, f"{name} c0={c0}")


@pytest.mark.parametrize("name,ts", [("g4-hd128-chunk128", 3), ("g1-hd128-c70", 2)])
def test_fused_prefill_writes_every_partial_slot(name, ts):
    """Partials filled with NaN before each chunk: every slot the merge reads
    is written by the call (unused list entries and window chunks a row does
    not see included), so every output is finite and equals the separate
    calls' to rounding."""
    pr, c, dc, ix, pf, q_all, L, T, W, C = _setup(name, seed=3, ts=ts, k_max=4)
    ref = ChunkedPrefill(ix, T, W, k_max=4, token_splits=ts, fused=False)
    for c0 in (0, (L - T) // 2, L - T):
        budget = max(1, (c0 + T) // 16)
        qd = _qchunk(q_all, c0, T)
        pf.part_o.fill_(float("nan"))
        pf.part_ml.fill_(float("nan"))
        pf.chunk(qd, c0, budget)
        torch.cuda.synchronize()
        out, lse = pf.out_f32(), pf.lse_f32()
        assert np.isfinite(out).all() and np.isfinite(lse).all(), f"{name} c0={c0}"
        ref.chunk(qd, c0, budget)
        torch.cuda.synchronize()
        same = (pf.sel.cpu().numpy() == ref.sel.cpu().numpy()).all(axis=-1)
        assert same.mean() > 0.9, f"{name} c0={c0}: lists differ beyond near ties"
        np.testing.assert_array_equal(pf.ends.cpu().numpy(), ref.ends.cpu().numpy())
        o1, o2 = out.reshape(c.B, c.Hkv, -1, T, c.hd), ref.out_f32().reshape(c.B, c.Hkv, -1, T, c.hd)
        for b in range(c.B):
            for kvh in range(c.Hkv):
                for i in range(T):
                    if same[b, kvh, i]:
                        check_output(o1[b, kvh, :, i], o2[b, kvh, :, i].astype(np.float64), c.dtype,
                                     f"{name} c0={c0} row {i}")


def test_fused_prefill_is_bitwise_reproducible():
    pr, c, dc, ix, pf, q_all, L, T, W, C = _setup("g4-hd128", seed=4, ts=3)
    c0 = (L - T) // 2
    qd = _qchunk(q_all, c0, T)
    outs = []
    for _ in range(2):
        pf.chunk(qd, c0, max(1, (c0 + T) // 16))
        torch.cuda.synchronize()
        outs.append((pf.out.clone(), pf.lse.clone(), pf.sel.clone()))
    for x, y in zip(outs[0], outs[1]):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name,ts,per_call", [("g4-hd128", 3, 3), ("g8-hd128-chunk64", 2, 4),
                                              ("g1-hd128-c70", 2, 2), ("g2-hd64-ragged", 1, 5)])
def test_several_chunks_per_call_equal_one_call_each(name, ts, per_call):
    """sparse_attn_prefill_chunks over consecutive chunks (the last call of
    the prompt with fewer) gives, bit for bit, the outputs, lse, lists,
    counts and visible ends of one sparse_attn_prefill_chunk call per chunk,
    and leaves the lengths where those calls do."""
    pr, c, dc, ix, one, q_all, L, T, W, C = _setup(name, seed=6, ts=ts, k_max=4)
    many = ChunkedPrefill(ix, T, W, k_max=4, token_splits=ts, per_call=per_call)
    starts = list(range(0, L - T + 1, T))
    for g0 in range(0, len(starts), per_call):
        group = starts[g0:g0 + per_call]
        budgets = [max(1, (c0 + T) // 16) for c0 in group]
        n = len(group)
        qd = to_device(np.ascontiguousarray(q_all[:, :, group[0]:group[-1] + T]))
        many.part_o.fill_(float("nan"))
        many.part_ml.fill_(float("nan"))
        many.chunks(qd, group[0], budgets)
        torch.cuda.synchronize()
        lens_many = dc.seq_lens.clone()
        out_m = many.out[: n * one.rows].view(c.B, c.Hq, n, T, c.hd)
        lse_m = many.lse[: n * one.rows].view(c.B, c.Hq, n, T)
        # a call of n chunks lays its lists out as [B][Hkv][n * T][...] from the buffers' start
        km = many.sel.shape[-1]
        sel_m = many.sel.view(-1)[: c.B * c.Hkv * n * T * km].view(c.B, c.Hkv, n, T, km)
        cnt_m = many.count.view(-1)[: c.B * c.Hkv * n * T].view(c.B, c.Hkv, n, T)
        ends_m = many.ends.view(-1, c.B, c.Hkv, C)[:n]
        for jc, c0 in enumerate(group):
            one.chunk(_qchunk(q_all, c0, T), c0, budgets[jc])
            torch.cuda.synchronize()
            ctx = f"{name} chunk at {c0} ({jc} of {n})"
            assert torch.equal(out_m[:, :, jc], one.out.view(c.B, c.Hq, T, c.hd)), ctx
            assert torch.equal(lse_m[:, :, jc], one.lse.view(c.B, c.Hq, T)), ctx
            assert torch.equal(sel_m[:, :, jc], one.sel), ctx
            assert torch.equal(cnt_m[:, :, jc], one.count), ctx
            assert torch.equal(ends_m[jc], one.ends), ctx
        assert torch.equal(dc.seq_lens, lens_many)  # both left the lengths at the next chunk's
