"""Chunked sparse prefill on the GPU (sparse_attn_blocks_visible with
sparse_attn_select_blocks and sparse_attn_decode_blocks over one index of the
whole prompt) against the fp64 oracle of oracle/semantic.py, on the GPU's own
index: the visible part of every block exactly, the block choice exactly
where no two block scores are within 1e-4 relative of each other at the
budget's edge, and the outputs against the oracle's attention over the GPU's
blocks (their visible rows) and the chunk's window.  With every block chosen
each row must be dense causal attention over its prefix, chunk after chunk
over the whole prompt."""
import numpy as np
import pytest

from oracle import semantic as sem
from block_sparse_long_page_amd import configs, synth
from block_sparse_long_page_amd.synth import to_f32
from helpers import dense_keys_values, masked_attention
from parity import check_lse, check_output

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
}


def _setup(name, seed=0, ts=1, k_max=None):
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
    return pr, c, dc, ix, ChunkedPrefill(ix, T, W, k_max=k_max, token_splits=ts), q_all, L, T, W, C


def _qchunk(q_all, c0, T):
    return to_device(np.ascontiguousarray(q_all[:, :, c0:c0 + T]))


def _qgroup(q_all, c, b, kvh, pos):
    G = c.Hq // c.Hkv
    return np.stack([to_f32(q_all[b, kvh * G + h, pos], c.dtype).astype(np.float64) for h in range(G)])


@pytest.mark.parametrize("name,ts,k_max", [(n, 1, None) for n in CASES] + [("g4-hd128", 3, None),
                                                                          ("g8-hd128-chunk64", 2, 3)])
def test_prefill_chunks_match_the_oracle(name, ts, k_max):
    pr, c, dc, ix, pf, q_all, L, T, W, C = _setup(name, seed=1, ts=ts, k_max=k_max)
    G = c.Hq // c.Hkv
    perm_all, off_all = ix.positions.cpu().numpy(), ix.offsets.cpu().numpy()
    mu_all = ix.centres.cpu().numpy().astype(np.float64)
    # the first chunk sees no index, the next ones a growing part, the last all but its window
    starts = sorted({0, T, (L - T) // 3, (L - T) // 2, L - T})
    exact = 0
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
                    want = sem.select_blocks(s, vis, budget, pf.k_max)
                    got = sel[b, kvh, i, :cnt[b, kvh, i]]
                    assert np.all(np.diff(got) > 0) and np.all(vis[got] > 0)
                    order = sorted((x for x in range(C) if vis[x] > 0), key=lambda x: (-s[x], x))
                    n = len(want)
                    edge = s[order[max(0, n - 1):n + 2]] if order else np.zeros(0)
                    tau = 1e-4 * max(1e-30, np.abs(s).max())
                    if len(edge) < 2 or np.min(-np.diff(edge)) > tau:
                        np.testing.assert_array_equal(got, want)
                        exact += 1
                    toks = np.concatenate([perm[off[x]:off[x] + vis[x]] for x in got] +
                                          [np.arange(max(0, bound), pos + 1)]).astype(np.int64)
                    for h in range(G):
                        o, l_ = sem.attend(qg[h], K[toks], V[toks], 1.0 / np.sqrt(c.hd))
                        check_output(out[b, kvh * G + h, i][None], o[None], c.dtype, f"{name} c0={c0}")
                        check_lse(lse[b, kvh * G + h, i][None], np.array([l_]), f"{name} c0={c0}")
    assert exact > 0


@pytest.mark.parametrize("name,ts", [("g4-hd128", 1), ("g2-hd64-ragged", 4)])
def test_prefill_with_every_block_is_dense_causal(name, ts):
    """Every chunk of the prompt with an unlimited budget: each row attends
    its whole prefix exactly once (visible block parts + window), whatever
    the token chunks per block."""
    pr, c, dc, ix, pf, q_all, L, T, W, C = _setup(name, seed=2, ts=ts)
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
