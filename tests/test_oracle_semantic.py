"""Pins of the semantic-index oracle (oracle/semantic.py) against what the
semantic-blocks page and the mathematics fix, each independent of the
function it pins:
  * k-means: a key equal to a centre goes to it (Cauchy-Schwarz), and the
    assignment is unchanged by positive rescaling of the keys and by a common
    rotation of keys and centres; a cluster symmetric about a direction has
    that direction as its centre, and an empty cluster keeps its centre; the
    objective never decreases; planted well-separated clusters are
    recovered exactly;
  * the block layout is a stable grouping (a permutation, blocks contiguous
    and in order, positions ascending inside a block);
  * with equal block sizes the greedy token-budget selection is the
    (score desc, index asc) top-k of the C oracle (pinned by brute force in
    test_oracle.py); a budget over every token takes every block, a zero
    budget the best one, and a larger budget never drops a block;
  * attention over every block plus the recent tokens is dense causal
    attention (tests/helpers.py), and on a cache whose clusters are already
    its pages the index reproduces the paged centroid path of the C oracle;
  * a prefill chunk over an index of the whole prompt: with every block
    chosen each row is dense causal attention over its prefix, whatever the
    chunk and window; with an index of the prefix before the window only it
    is the decode path above; visible sizes count positions directly.
"""
import numpy as np
import pytest

import oracle
from oracle import semantic as sem
from block_sparse_long_page_amd import configs, synth
from helpers import dense_keys_values, masked_attention, query


def _clusters(rng, C, n, hd, spread=0.05):
    dirs = rng.standard_normal((C, hd))
    dirs /= np.linalg.norm(dirs, axis=1, keepdims=True)
    labels = np.repeat(np.arange(C), n)
    keys = dirs[labels] + spread * rng.standard_normal((C * n, hd))
    keys *= rng.uniform(0.5, 3.0, size=(C * n, 1))  # lengths do not matter to spherical k-means
    return keys, labels, dirs


def test_key_equal_to_a_centre_goes_to_it():
    rng = np.random.default_rng(0)
    mu = sem.unit_keys(rng.standard_normal((12, 16)))
    a = sem.assign(mu * 3.0, mu)
    np.testing.assert_array_equal(a, np.arange(12))


def test_assignment_ignores_key_length_and_a_common_rotation():
    rng = np.random.default_rng(1)
    u = sem.unit_keys(rng.standard_normal((300, 24)))
    mu = sem.unit_keys(rng.standard_normal((10, 24)))
    a = sem.assign(u, mu)
    np.testing.assert_array_equal(sem.assign(sem.unit_keys(u * rng.uniform(0.1, 9.0, (300, 1))), mu), a)
    rot, _ = np.linalg.qr(rng.standard_normal((24, 24)))
    np.testing.assert_array_equal(sem.assign(u @ rot, mu @ rot), a)


def test_ties_go_to_the_lower_centre():
    mu = np.eye(4)[[0, 1, 1, 2]]  # centres 1 and 2 coincide
    u = np.array([[0.0, 1.0, 0.0, 0.0], [0.6, 0.8, 0.0, 0.0]])
    np.testing.assert_array_equal(sem.assign(u, mu), [1, 1])


def test_symmetric_cluster_centre_and_empty_cluster():
    d = np.array([1.0, 0.0, 0.0])
    u = sem.unit_keys(np.array([[1.0, 0.5, 0.0], [1.0, -0.5, 0.0], [1.0, 0.0, 0.3], [1.0, 0.0, -0.3]]))
    prev = np.array([[0.0, 1.0, 0.0], [0.0, 0.0, 1.0]])
    mu = sem.update(u, np.zeros(4, dtype=np.int32), prev)
    np.testing.assert_allclose(mu[0], d, atol=1e-15)
    np.testing.assert_array_equal(mu[1], prev[1])  # no keys: the previous centre


def test_objective_never_decreases():
    rng = np.random.default_rng(2)
    keys = rng.standard_normal((2000, 32)) + 0.5 * rng.standard_normal((1, 32))
    _, _, hist = sem.spherical_kmeans(keys, 24, 12)
    assert all(b >= a - 1e-9 for a, b in zip(hist, hist[1:])), hist


def test_planted_clusters_are_recovered():
    """Clusters stored one after another: the evenly spaced starts fall one
    per cluster and the planted partition comes back exactly."""
    rng = np.random.default_rng(3)
    C, n = 12, 50
    keys, labels, dirs = _clusters(rng, C, n, 32)
    mu, a, _ = sem.spherical_kmeans(keys, C, 10)
    np.testing.assert_array_equal(a, labels)
    assert np.all(np.sum(mu * dirs, axis=1) > 0.99)


def test_interleaved_clusters_reach_a_fixed_point():
    """Clusters interleaved in position order: the iterations end at a fixed
    point of (assign, update), and no planted cluster is split between two
    blocks unless two starts fell inside it."""
    rng = np.random.default_rng(3)
    C, n = 12, 50
    keys, labels, _ = _clusters(rng, C, n, 32)
    order = rng.permutation(C * n)
    keys, labels = keys[order], labels[order]
    mu, a, _ = sem.spherical_kmeans(keys, C, 10)
    u = sem.unit_keys(keys)
    np.testing.assert_array_equal(sem.assign(u, sem.update(u, a, mu)), a)
    starts = labels[(np.arange(C) * C * n) // C]
    for x in range(C):
        if np.sum(starts == x) <= 1:
            assert len(np.unique(a[labels == x])) == 1


def test_block_layout_is_a_stable_grouping():
    rng = np.random.default_rng(4)
    a = rng.integers(0, 9, size=500).astype(np.int32)
    a[a == 5] = 6  # an empty block
    perm, off = sem.block_layout(a, 9)
    assert sorted(perm.tolist()) == list(range(500))
    assert np.all(np.diff(a[perm]) >= 0)
    for c in range(9):
        rows = perm[off[c]:off[c + 1]]
        assert np.all(a[rows] == c) and np.all(np.diff(rows) > 0)
    assert off[5] == off[6] and off[-1] == 500


@pytest.mark.parametrize("budget", [0, 64, 100, 640, 10**6])
def test_equal_blocks_reduce_to_the_page_topk(budget):
    rng = np.random.default_rng(5)
    C, size = 40, 64
    scores = np.round(rng.standard_normal(C), 1)  # planted exact ties
    got = sem.select_blocks(scores, np.full(C, size), budget, k_max=C)
    k = min(C, max(1, budget // size))
    want = oracle.topk(scores, np.ones(C, dtype=np.uint8), k)
    np.testing.assert_array_equal(got, np.sort(want))


def test_budget_limits_and_monotonicity():
    rng = np.random.default_rng(6)
    C = 30
    scores = rng.standard_normal(C)
    sizes = rng.integers(1, 200, size=C)
    sizes[7] = 0
    assert set(sem.select_blocks(scores, sizes, 10**6, C).tolist()) == set(range(C)) - {7}
    best = max((c for c in range(C) if sizes[c] > 0), key=lambda c: scores[c])
    np.testing.assert_array_equal(sem.select_blocks(scores, sizes, 0, C), [best])
    prev = set()
    for budget in range(0, int(sizes.sum()) + 50, 37):
        cur = set(sem.select_blocks(scores, sizes, budget, C).tolist())
        assert prev <= cur and int(sizes[list(cur)].sum()) <= max(budget, int(sizes[best]))
        prev = cur
    assert len(sem.select_blocks(scores, sizes, 10**6, 5)) == 5


def _tiny_semantic(scatter, seed=0):
    wl = configs.SEMANTIC_512K.scaled(batch=1, num_q_heads=4, num_kv_heads=2, head_dim=32, context=8 * 64 + 4,
                                      page_size=64, window=4, budget=3 * 64, q_rows=4)
    return synth.semantic_problem(wl, seed=seed, blocks=8, block_tokens=64, scatter=scatter)


def _blocked_reference(pr, b, kvh, C, iters, budget, k_max):
    """The oracle's index and attention for every row and head of one
    (sequence, KV head): [(out, lse)] per (head, row), and the blocks."""
    c = pr.cache
    K, V = dense_keys_values(c, b, kvh)
    L = K.shape[0]
    N = L - pr.window
    mu, a, _ = sem.spherical_kmeans(K[:N], C, iters)
    perm, off = sem.block_layout(a, C)
    sizes = np.diff(off)
    G = c.Hq // c.Hkv
    res, chosen = {}, []
    for i in range(pr.Q):
        qg = np.stack([query(pr, b, kvh * G + h, i) for h in range(G)])
        blocks = sem.select_blocks(sem.block_scores(qg, mu), sizes, budget, k_max)
        chosen.append(blocks)
        pos = L - pr.Q + i
        toks = np.concatenate([perm[off[x]:off[x + 1]] for x in blocks] + [np.arange(L - pr.window, pos + 1)])
        for h in range(G):
            res[h, i] = sem.attend(qg[h], K[toks], V[toks], 1.0 / np.sqrt(c.hd))
    return res, chosen, (mu, a, perm, off)


def test_full_budget_is_dense_causal_attention():
    pr = _tiny_semantic(scatter=True)
    c = pr.cache
    K, V = dense_keys_values(c, 0, 1)
    res, _, _ = _blocked_reference(pr, 0, 1, 8, 4, budget=10**6, k_max=8)
    L = K.shape[0]
    G = c.Hq // c.Hkv
    for i in range(pr.Q):
        pos = L - pr.Q + i
        for h in range(G):
            o, lse = masked_attention(query(pr, 0, G + h, i), K, V, np.arange(L) <= pos, 1.0 / np.sqrt(c.hd))
            np.testing.assert_allclose(res[h, i][0], o, atol=1e-12)
            assert abs(res[h, i][1] - lse) < 1e-12


def test_pages_that_are_clusters_give_the_paged_centroid_path():
    pr = _tiny_semantic(scatter=False)
    c = pr.cache
    r = oracle.run(c, pr.q, mode=oracle.CENTROID, Q=pr.Q, sink=0, window=pr.window, budget=pr.budget)
    G = c.Hq // c.Hkv
    for kvh in range(c.Hkv):
        res, chosen, (mu, a, perm, off) = _blocked_reference(pr, 0, kvh, 8, 4, pr.budget, k_max=8)
        np.testing.assert_array_equal(a, np.repeat(np.arange(8), 64))  # block x = page x
        for i in range(pr.Q):
            np.testing.assert_array_equal(chosen[i], r.sel[0, kvh, i, :r.cnt[0, kvh, i]])
            for h in range(G):
                np.testing.assert_allclose(res[h, i][0], r.out[0, kvh * G + h, i], atol=1e-12)
                assert abs(res[h, i][1] - r.lse[0, kvh * G + h, i]) < 1e-12


def _prefill_setup(seed=0):
    pr = _tiny_semantic(scatter=True, seed=seed)
    c = pr.cache
    K, V = dense_keys_values(c, 0, 1)
    L = K.shape[0]
    mu, a, _ = sem.spherical_kmeans(K, 8, 4)  # an index of the whole prompt
    perm, off = sem.block_layout(a, 8)
    G = c.Hq // c.Hkv
    q = np.random.default_rng(seed).standard_normal((L, G, c.hd))
    return c, K, V, L, mu, perm, off, q


def test_visible_sizes_count_positions():
    c, K, V, L, mu, perm, off, q = _prefill_setup()
    for bound in (0, 1, 100, 333, L, L + 5):
        vis = sem.visible_sizes(perm, off, bound)
        for x in range(8):
            assert vis[x] == len([t for t in perm[off[x]:off[x + 1]] if t < bound])
    np.testing.assert_array_equal(sem.visible_sizes(perm, off, L), np.diff(off))


@pytest.mark.parametrize("c0,T,W", [(0, 4, 4), (100, 8, 8), (200, 16, 40), (510, 6, 6)])  # 510 + 6 = L
def test_prefill_with_every_block_is_dense_causal(c0, T, W):
    c, K, V, L, mu, perm, off, q = _prefill_setup()
    res = sem.prefill_chunk(K, V, q[c0:c0 + T], mu, perm, off, c0, W, budget=10**9, k_max=8,
                            scale=1.0 / np.sqrt(c.hd))
    for i, (blocks, heads) in enumerate(res):
        pos = c0 + i
        for h, (o, lse) in enumerate(heads):
            ref_o, ref_l = masked_attention(q[pos, h], K, V, np.arange(L) <= pos, 1.0 / np.sqrt(c.hd))
            np.testing.assert_allclose(o, ref_o, atol=1e-12)
            assert abs(lse - ref_l) < 1e-12


def test_prefill_chunk_over_the_prefix_index_is_the_decode():
    """An index of [0, N) with N at the chunk's window start: every block is
    wholly visible, and the chunk is the decode path over blocks + window."""
    pr = _tiny_semantic(scatter=True, seed=3)
    c = pr.cache
    res, chosen, (mu, a, perm, off) = _blocked_reference(pr, 0, 1, 8, 4, pr.budget, k_max=8)
    K, V = dense_keys_values(c, 0, 1)
    L = K.shape[0]
    G = c.Hq // c.Hkv
    qrows = [np.stack([query(pr, 0, G + h, i) for h in range(G)]) for i in range(pr.Q)]
    got = sem.prefill_chunk(K, V, qrows, mu, perm, off, L - pr.Q, pr.window, pr.budget, 8, 1.0 / np.sqrt(c.hd))
    for i, (blocks, heads) in enumerate(got):
        np.testing.assert_array_equal(blocks, chosen[i])
        for h, (o, lse) in enumerate(heads):
            np.testing.assert_allclose(o, res[h, i][0], atol=1e-12)
            assert abs(lse - res[h, i][1]) < 1e-12

