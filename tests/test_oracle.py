"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test pins one step of the oracle to something other than itself:
  * budget >= context reduces to dense causal attention (textbook softmax,
    written independently in tests/helpers.py);
  * budget 0 reduces to StreamingLLM sink + window, and S = 0 to a pure
    sliding window;
  * the Quest score is an upper bound on max_t q.k_t over the page, exactly in
    fp64 with the same summation order, and attains it on one-token pages;
  * summaries obey their defining invariants (bounds attained, linearity of
    the mean, unit-norm and scale-invariant centroids), ignoring tokens past
    the sequence end;
  * selection + token set + attention match brute-force enumeration of all
    k-subsets on micro cases, planted exact ties included;
  * the log-sum-exp merge of any partition equals attention over the union;
  * planted needle pages are selected (the course module's needle probe).
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from block_sparse_long_page_amd import configs, synth
from helpers import dense_keys_values, masked_attention, query, seq_dot

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")

SMALL = [
    dict(B=2, Hq=4, Hkv=2, hd=16, P=8, seq_lens=[100, 61], sink=8, window=16, dtype="bf16", Q=2),
    dict(B=1, Hq=8, Hkv=1, hd=32, P=16, seq_lens=[257], sink=4, window=20, dtype="f32", Q=1),
    dict(B=3, Hq=2, Hkv=2, hd=8, P=4, seq_lens=[5, 40, 33], sink=2, window=3, dtype="bf16", Q=3),
]


def _allowed(L, S, W, pos, pages=(), P=1):
    t = np.arange(L)
    a = (t < S) | (t >= L - W)
    for p in pages:
        a |= (t // P == p) & (t >= S) & (t < L - W)
    return a & (t <= pos)


def _check_against_mask(pr, r, pages_of=None, tol=1e-12):
    c = pr.cache
    G = c.Hq // c.Hkv
    scale = 1.0 / np.sqrt(c.hd)
    for b in range(c.B):
        L = int(c.seq_lens[b])
        for h in range(c.Hq):
            K, V = dense_keys_values(c, b, h // G)
            for i in range(pr.Q):
                pos = L - pr.Q + i
                pages = pages_of(b, h // G, i) if pages_of else ()
                allowed = _allowed(L, pr.sink, pr.window, pos, pages, c.P)
                ref, lse = masked_attention(query(pr, b, h, i), K, V, allowed, scale)
                np.testing.assert_allclose(r.out[b, h, i], ref, rtol=0, atol=tol)
                assert abs(r.lse[b, h, i] - lse) <= tol * max(1.0, abs(lse))
                assert r.ntok[b, h, i] == allowed.sum()


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("mode", ["quest", "mean", "centroid", "compressed"])
@pytest.mark.parametrize("shuffle", [False, True])
def test_budget_covering_context_is_dense_attention(case, mode, shuffle):
    kw = dict(SMALL[case])
    pr = synth.random_problem(**kw, budget=10**6, mode=mode, seed=11 + case, shuffle=shuffle, spare_pages=3)
    r = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget)
    c = pr.cache
    G = c.Hq // c.Hkv
    for b in range(c.B):
        L = int(c.seq_lens[b])
        for h in range(c.Hq):
            K, V = dense_keys_values(c, b, h // G)
            for i in range(pr.Q):
                pos = L - pr.Q + i
                ref, lse = masked_attention(query(pr, b, h, i), K, V, np.arange(L) <= pos, 1.0 / np.sqrt(c.hd))
                np.testing.assert_allclose(r.out[b, h, i], ref, rtol=0, atol=1e-12)
                assert abs(r.lse[b, h, i] - lse) <= 1e-12 * max(1.0, abs(lse))
                assert r.ntok[b, h, i] == pos + 1


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("sink_zero", [False, True])
def test_zero_budget_is_sink_plus_window(case, sink_zero):
    kw = dict(SMALL[case])
    if sink_zero:
        kw["sink"] = 0
    pr = synth.random_problem(**kw, budget=0, seed=21 + case, shuffle=True)
    r = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=0)
    assert (r.cnt == 0).all()
    _check_against_mask(pr, r)


def test_window_reading_of_the_printed_example():
    g = json.load(open(GOLDEN))["window_example"]
    pos, w = g["position"], g["w"]
    pr = synth.random_problem(B=1, Hq=1, Hkv=1, hd=8, P=16, seq_lens=[pos + 1], sink=0, window=w, budget=0,
                              dtype="f32", seed=5)
    r = oracle.run(pr.cache, pr.q, mode=0, Q=1, sink=0, window=w, budget=0)
    assert r.ntok[0, 0, 0] == w
    K, V = dense_keys_values(pr.cache, 0, 0)
    t = np.arange(pos + 1)
    allowed = (t >= pos - w + 1) & (t <= g["printed_last"])
    ref, _ = masked_attention(query(pr, 0, 0, 0), K, V, allowed, 1 / np.sqrt(8))
    np.testing.assert_allclose(r.out[0, 0, 0], ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quest_score_bounds_every_key_of_the_page(dtype):
    pr = synth.random_problem(B=2, Hq=4, Hkv=2, hd=32, P=8, seq_lens=[203, 97], sink=0, window=1, budget=0,
                              dtype=dtype, seed=7, shuffle=True, clusters=4)
    c = pr.cache
    G = c.Hq // c.Hkv
    for b in range(c.B):
        L = int(c.seq_lens[b])
        for kvh in range(c.Hkv):
            K, _ = dense_keys_values(c, b, kvh)
            for p in range(-(-L // c.P)):
                summ, n = oracle.page_summary(c, oracle.QUEST, b, kvh, p)
                toks = K[p * c.P: p * c.P + n]
                for g in range(G):
                    qh = query(pr, b, kvh * G + g, 0)
                    u = oracle.page_score(oracle.QUEST, summ, qh)
                    best = max(seq_dot(qh, kt) for kt in toks)
                    assert u >= best  # exact: rounding is monotone and the order is the same
                    if n == 1:
                        assert u == best


def test_quest_bound_tight_on_one_token_pages():
    # every page holds one token: the bound is the dot product itself
    pr = synth.random_problem(B=1, Hq=2, Hkv=1, hd=16, P=1, seq_lens=[40], sink=0, window=1, budget=0,
                              dtype="bf16", seed=8)
    K, _ = dense_keys_values(pr.cache, 0, 0)
    for p in range(40):
        summ, n = oracle.page_summary(pr.cache, oracle.QUEST, 0, 0, p)
        assert n == 1
        for h in range(2):
            qh = query(pr, 0, h, 0)
            assert oracle.page_score(oracle.QUEST, summ, qh) == seq_dot(qh, K[p])


def _poisoned(pr):
    """Fill the slots past each sequence's end with huge values: summaries
    must not see them."""
    c = pr.cache
    for b in range(c.B):
        L = int(c.seq_lens[b])
        last = (L - 1) // c.P
        off = L - last * c.P
        if off < c.P:
            phys = c.block_table[b, last]
            c.k[phys, :, off:] = synth.store(np.full((c.Hkv, c.P - off, c.hd), 1e6, np.float32), c.dtype)
    return pr


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_summary_invariants(dtype):
    pr = _poisoned(synth.random_problem(B=2, Hq=2, Hkv=2, hd=16, P=8, seq_lens=[45, 19], sink=0, window=1,
                                        budget=0, dtype=dtype, seed=9, shuffle=True))
    c = pr.cache
    for b in range(c.B):
        L = int(c.seq_lens[b])
        for kvh in range(c.Hkv):
            K, _ = dense_keys_values(c, b, kvh)
            for p in range(-(-L // c.P)):
                toks = K[p * c.P: min(L, (p + 1) * c.P)]
                qm, n = oracle.page_summary(c, oracle.QUEST, b, kvh, p)
                assert n == len(toks)
                mn, mx = qm[: c.hd], qm[c.hd:]
                assert (toks >= mn).all() and (toks <= mx).all()
                assert ((toks == mn).any(axis=0)).all() and ((toks == mx).any(axis=0)).all()
                mu, _ = oracle.page_summary(c, oracle.MEAN, b, kvh, p)
                assert (mu >= mn).all() and (mu <= mx).all()
                qv = query(pr, b, kvh, 0)
                lin = np.mean([seq_dot(qv, t) for t in toks])
                assert abs(oracle.page_score(oracle.MEAN, mu, qv) - lin) <= 1e-12 * (1 + np.abs(qv) @ np.abs(mu) * n)
                cen, _ = oracle.page_summary(c, oracle.CENTROID, b, kvh, p)
                assert abs(np.linalg.norm(cen) - 1.0) < 1e-12


def test_centroid_ignores_key_lengths_and_recovers_a_shared_direction():
    pr = synth.random_problem(B=1, Hq=1, Hkv=1, hd=16, P=8, seq_lens=[24], sink=0, window=1, budget=0,
                              dtype="f32", seed=10)
    c = pr.cache
    before = [oracle.page_summary(c, oracle.CENTROID, 0, 0, p)[0] for p in range(3)]
    rng = np.random.default_rng(0)
    c.k[...] *= np.float32(2.0) ** rng.integers(-3, 4, size=c.k.shape[:3])[..., None].astype(np.float32)
    after = [oracle.page_summary(c, oracle.CENTROID, 0, 0, p)[0] for p in range(3)]
    for a, z in zip(before, after):
        np.testing.assert_allclose(a, z, atol=1e-14, rtol=0)
    d = rng.standard_normal(16).astype(np.float32)
    phys = c.block_table[0, 1]
    c.k[phys, 0] = d[None, :] * np.arange(1, 9, dtype=np.float32)[:, None]
    cen, _ = oracle.page_summary(c, oracle.CENTROID, 0, 0, 1)
    np.testing.assert_allclose(cen, d / np.linalg.norm(d.astype(np.float64)), atol=1e-14)


# ---- brute force on micro cases ---------------------------------------------

def _brute_scores(pr, b, kvh, i, mode):
    """Group score of every candidate page, from dense keys, in the test."""
    c = pr.cache
    G = c.Hq // c.Hkv
    L = int(c.seq_lens[b])
    K, _ = dense_keys_values(c, b, kvh)
    S, W = pr.sink, pr.window
    scores = {}
    for p in range(-(-L // c.P)):
        toks = np.arange(p * c.P, min(L, (p + 1) * c.P))
        if not ((toks >= S) & (toks < L - W)).any():
            continue
        kp = K[toks]
        best = -np.inf
        for g in range(G):
            qh = query(pr, b, kvh * G + g, i)
            if mode == "quest":
                s = seq_dot(np.ones_like(qh), np.maximum(qh * kp.min(0), qh * kp.max(0)))
            elif mode == "mean":
                s = seq_dot(qh, kp.sum(0) / len(kp))
            elif mode == "compressed":  # blocks of two pages with a one-page stride: the two that cover p
                s = -np.inf
                for j in (p - 1, p):
                    if j >= 0:
                        kb = K[j * c.P:min(L, (j + 2) * c.P)]
                        s = max(s, seq_dot(qh, kb.sum(0) / len(kb)))
            else:
                u = (kp / np.linalg.norm(kp, axis=1, keepdims=True)).sum(0)
                s = seq_dot(qh, u / np.linalg.norm(u))
            best = max(best, s)
        scores[p] = best
    return scores


def _brute_topk(scores, k):
    """All k-subsets; the best is the largest score sum, then the smallest
    ascending index tuple."""
    pages = sorted(scores)
    k = min(k, len(pages))
    best_key, best = None, ()
    for sub in itertools.combinations(pages, k):
        key = (-sum(scores[p] for p in sub), sub)
        if best_key is None or key < best_key:
            best_key, best = key, sub
    return list(best)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("mode", ["quest", "mean", "centroid", "compressed"])
def test_selection_and_output_match_brute_force(seed, mode):
    rng = np.random.default_rng(100 + seed)
    P = [4, 8][seed % 2]
    L = int(rng.integers(60, 129)) if P == 8 else int(rng.integers(30, 70))
    G = [1, 2, 4][seed % 3]
    S = int(rng.integers(0, 2 * P))
    W = int(rng.integers(1, 3 * P))
    k = int(rng.integers(1, 5))
    pr = synth.random_problem(B=2, Hq=2 * G, Hkv=2, hd=8, P=P, seq_lens=[L, L - 3], sink=S, window=W,
                              budget=k * P + int(rng.integers(0, P)), mode=mode, dtype="bf16",
                              Q=2, seed=200 + seed, shuffle=True)
    c = pr.cache
    # plant exact ties: copy one page's keys onto two other pages
    n_pages = -(-(L - 3) // P)
    src, d1, d2 = rng.choice(np.arange(1, n_pages - 1), size=3, replace=False)
    for b in range(2):
        for dst in (d1, d2):
            c.k[c.block_table[b, dst]] = c.k[c.block_table[b, src]]
    r = oracle.run(c, pr.q, mode=pr.mode, Q=2, sink=S, window=W, budget=pr.budget, want_scores=True)
    chosen = {}
    for b in range(2):
        for kvh in range(2):
            for i in range(2):
                sc = _brute_scores(pr, b, kvh, i, mode)
                assert len(sc) <= 16
                for p, s in sc.items():
                    assert r.scores[b, kvh, i, p] == pytest.approx(s, rel=1e-12, abs=1e-12)
                want = _brute_topk(sc, pr.budget // P)
                got = list(r.sel[b, kvh, i, : r.cnt[b, kvh, i]])
                assert got == want
                chosen[(b, kvh, i)] = want
    _check_against_mask(pr, r, pages_of=lambda b, kvh, i: chosen[(b, kvh, i)])


def test_topk_ties_go_to_the_lower_page():
    s = np.array([3.0, 5.0, 5.0, 1.0, 5.0, 3.0, 3.0, 0.0])
    cand = np.ones(8, np.uint8)
    cand[4] = 0
    assert list(oracle.topk(s, cand, 2)) == [1, 2]
    assert list(oracle.topk(s, cand, 3)) == [0, 1, 2]
    assert list(oracle.topk(s, cand, 4)) == [0, 1, 2, 5]
    assert list(oracle.topk(s, cand, 20)) == [0, 1, 2, 3, 5, 6, 7]
    assert list(oracle.topk(s, cand, 0)) == []


def test_external_selection_is_attended():
    pr = synth.random_problem(B=1, Hq=4, Hkv=2, hd=16, P=8, seq_lens=[120], sink=8, window=16, budget=24,
                              dtype="bf16", seed=31, shuffle=True)
    sel = np.array([[[[2, 5, 9]], [[1, 3, 12]]]], dtype=np.int32)
    cnt = np.array([[[3], [2]]], dtype=np.int32)
    r = oracle.run(pr.cache, pr.q, mode=0, Q=1, sink=8, window=16, budget=24, sel=sel, cnt=cnt)
    _check_against_mask(pr, r, pages_of=lambda b, kvh, i: list(sel[b, kvh, i, : cnt[b, kvh, i]]))


# ---- partial merging ---------------------------------------------------------

@pytest.mark.parametrize("nparts", [1, 2, 3, 7, 16, 64])
def test_merge_of_any_partition_is_attention_over_the_union(nparts):
    rng = np.random.default_rng(nparts)
    n, hd = 300, 16
    K = rng.standard_normal((n, hd))
    V = rng.standard_normal((n, hd))
    q = rng.standard_normal(hd) * 2
    allowed = rng.random(n) < 0.7
    ref, ref_lse = masked_attention(q, K, V, allowed, 0.25)
    idx = np.flatnonzero(allowed)
    part = rng.integers(0, nparts, size=idx.size)
    o = np.zeros((nparts, hd))
    m = np.full(nparts, -np.inf)
    l = np.zeros(nparts)
    for s in range(nparts):
        sub = idx[part == s]
        if sub.size:
            z = (K[sub] @ q) * 0.25
            m[s] = z.max()
            w = np.exp(z - m[s])
            l[s] = w.sum()
            o[s] = (w @ V[sub]) / l[s]
    perm = rng.permutation(nparts)
    for order in (np.arange(nparts), perm):
        out, lse = oracle.merge(o[order], m[order], l[order])
        np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)
        assert abs(lse - ref_lse) < 1e-12


# ---- needle probes -----------------------------------------------------------

@pytest.mark.parametrize("wl", [configs.TINY, configs.QWEN3_8B], ids=lambda w: w.name)
def test_planted_needle_pages_are_selected(wl):
    pr = synth.workload_problem(wl)
    assert pr.needles
    r = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget)
    for (b, kvh, p) in pr.needles:
        assert p in set(r.sel[b, kvh, 0, : r.cnt[b, kvh, 0]])
    assert (r.cnt == wl.k_pages).all()


def test_compressed_key_is_the_mean_over_two_pages():
    """The compressed key of the block starting at page p is the mean of the
    two pages' keys: the token-weighted average of the two pages' mean
    summaries (pinned above), ragged last page included."""
    pr = synth.random_problem(B=2, Hq=4, Hkv=2, hd=16, P=8, seq_lens=[83, 60], sink=4, window=8, budget=16,
                              dtype="bf16", seed=41, shuffle=True)
    c = pr.cache
    for b in range(2):
        n_pages = -(-int(c.seq_lens[b]) // c.P)
        for kvh in range(2):
            for p in range(n_pages):
                got, n = oracle.page_summary(c, oracle.COMPRESSED, b, kvh, p)
                m0, n0 = oracle.page_summary(c, oracle.MEAN, b, kvh, p)
                m1, n1 = oracle.page_summary(c, oracle.MEAN, b, kvh, p + 1) if p + 1 < n_pages else (0.0, 0)
                assert n == n0 + n1
                np.testing.assert_allclose(got, (n0 * m0 + n1 * np.asarray(m1)) / (n0 + n1), rtol=0, atol=1e-13)


def test_compressed_blocks_pull_in_the_needle_neighbours():
    """A needle page p (every token 3 q + noise) lifts both blocks that hold
    it, so pages p-1, p and p+1 (each covered by one of them) outscore the
    rest; with the mean summaries only page p stands out."""
    rng = np.random.default_rng(9)
    pr = synth.random_problem(B=1, Hq=1, Hkv=1, hd=32, P=16, seq_lens=[40 * 16], sink=0, window=16, budget=3 * 16,
                              dtype="bf16", seed=42, shuffle=True)
    c = pr.cache
    q = synth.to_f32(pr.q[0, 0, 0], c.dtype)
    p = 17
    keys = 3 * q[None, :] + rng.standard_normal((c.P, c.hd)).astype(np.float32)
    c.k[c.block_table[0, p], 0] = synth.store(keys, c.dtype)
    rc = oracle.run(c, pr.q, mode=oracle.COMPRESSED, Q=1, sink=0, window=16, budget=3 * 16)
    np.testing.assert_array_equal(rc.sel[0, 0, 0], [p - 1, p, p + 1])
    rm = oracle.run(c, pr.q, mode=oracle.MEAN, Q=1, sink=0, window=16, budget=16)
    np.testing.assert_array_equal(rm.sel[0, 0, 0], [p])
