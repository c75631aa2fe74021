"""Pins of the KeyDiff eviction oracle (oracle/keydiff.py) against what course
module 14 (section 14.4 and exercise 14.2) and the mathematics fix, each
independent of the function it pins:
  * evicting one token, the one-shot rule equals the exercise's rule (drop
    the key closest to the mean of the kept keys, the first on ties), on
    random keys and on a planted exact tie;
  * two clusters of identical keys: the distances are n2/n |a - b| and
    n1/n |a - b| in closed form, so the smaller cluster is kept first (its
    later positions first when not all fit) and the later positions of the
    other fill the rest;
  * the result is unchanged by translating every key by one vector and by
    scaling them (exact on integer keys);
  * the sink is kept even when its keys are the mean itself;
  * the exercise's needle (an outlier key among 1024 noise keys) survives
    every budget above the sink, by both rules;
  * blockwise eviction keeps at most the budget after every block, never
    drops the sink, and with one block is a single eviction.
"""
import numpy as np
import pytest

from oracle import keydiff as kd


@pytest.mark.parametrize("n,sink,seed", [(9, 0, 0), (33, 4, 1), (200, 16, 2), (64, 63, 3), (500, 1, 4)])
def test_one_eviction_is_the_exercise_rule(n, sink, seed):
    rng = np.random.default_rng(seed)
    keys = rng.standard_normal((n, 24))
    np.testing.assert_array_equal(kd.keep(keys, n - 1, sink), kd.evict_one_at_a_time(keys, n - 1, sink))


def test_planted_tie_evicts_the_earlier_position():
    """Two identical keys sitting exactly on the mean are both closest; the
    exercise drops the first, so the later one is kept."""
    rng = np.random.default_rng(5)
    keys = rng.integers(-8, 9, size=(40, 16)).astype(np.float64)
    keys[7] = 0.0
    keys[21] = 0.0
    keys -= keys.mean(axis=0)  # the mean is now exactly 0 = keys 7 and 21
    assert np.all(keys[7] == keys[21])
    ref = kd.evict_one_at_a_time(keys, 39, 2)
    assert 7 not in ref and 21 in ref
    np.testing.assert_array_equal(kd.keep(keys, 39, 2), ref)


@pytest.mark.parametrize("budget", [3, 5, 9, 14])
def test_two_clusters_in_closed_form(budget):
    """n1 = 4 copies of a and n2 = 12 of b after a 2-token sink of b's: the a's
    lie (n2 / n)|a - b| from the mean, the b's (n1 / n)|a - b|."""
    a, b = np.full(8, 3.0), np.full(8, -1.0)
    lab = np.array([1, 1, 0, 1, 1, 0, 1, 1, 1, 0, 1, 1, 1, 0, 1, 1])  # 0 = a
    keys = np.where(lab[:, None] == 0, a, b)
    d = kd.distances(keys)
    n, n1 = len(lab), int(np.sum(lab == 0))
    np.testing.assert_allclose(d[lab == 0], (n - n1) / n * np.linalg.norm(a - b), rtol=1e-15)
    np.testing.assert_allclose(d[lab == 1], n1 / n * np.linalg.norm(a - b), rtol=1e-15)
    sink = 2
    a_pos = [i for i in range(sink, n) if lab[i] == 0]
    b_pos = [i for i in range(sink, n) if lab[i] == 1]
    rest = budget - sink  # equal distances inside a cluster: its later positions first
    take_a = min(rest, len(a_pos))
    want = list(range(sink)) + a_pos[len(a_pos) - take_a:] + b_pos[len(b_pos) - (rest - take_a):]
    np.testing.assert_array_equal(kd.keep(keys, budget, sink), sorted(want))


def test_translation_and_scale_do_not_change_the_kept_set():
    rng = np.random.default_rng(6)
    keys = rng.integers(-20, 21, size=(256, 32)).astype(np.float64)
    ref = kd.keep(keys, 100, 8)
    np.testing.assert_array_equal(kd.keep(keys + rng.integers(-50, 51, size=32), 100, 8), ref)
    np.testing.assert_array_equal(kd.keep(keys * 4.0, 100, 8), ref)


def test_sink_is_kept_even_at_the_mean():
    rng = np.random.default_rng(7)
    keys = rng.standard_normal((100, 16))
    keys -= keys.mean(axis=0)
    keys[:4] = 0.0  # the least distinctive keys of all
    keys -= keys.mean(axis=0)
    kept = kd.keep(keys, 10, 4)
    assert list(kept[:4]) == [0, 1, 2, 3] and len(kept) == 10
    assert 0 not in kd.keep(keys, 10, 0)


def test_budget_covering_the_cache_keeps_everything():
    keys = np.random.default_rng(8).standard_normal((50, 8))
    np.testing.assert_array_equal(kd.keep(keys, 50, 4), np.arange(50))
    np.testing.assert_array_equal(kd.keep(keys, 80, 60), np.arange(50))
    with pytest.raises(ValueError):
        kd.keep(keys, 3, 4)


def test_needle_survives_eviction():
    """Exercise 14.2's toy: 1024 keys N(0, I/D), D = 64, and at position 512 a
    needle key shifted by 3/sqrt(D) along every channel; the needle is the
    most distinctive key, so it is kept at every budget above the sink."""
    rng = np.random.default_rng(0)
    D = 64
    keys = rng.standard_normal((1024, D)) / np.sqrt(D)
    keys[512] = rng.standard_normal(D) / np.sqrt(D) + 3.0 / np.sqrt(D)
    assert int(np.argmax(kd.distances(keys))) == 512
    for budget in (1024, 768, 512, 384, 256, 128, 64, 32, 16, 5):
        assert 512 in kd.keep(keys, budget, 4)
    for budget in (768, 16):
        assert 512 in kd.evict_one_at_a_time(keys, budget, 4)


def test_blockwise_eviction_holds_the_budget():
    rng = np.random.default_rng(9)
    keys = rng.standard_normal((1000, 16))
    states = kd.blockwise(keys, 96, 256, 8)
    assert len(states) == -(-1000 // 96)
    for i, held in enumerate(states):
        assert len(held) == min(256, min(1000, 96 * (i + 1)))
        assert np.all(np.diff(held) > 0) and list(held[:8]) == list(range(8))
    np.testing.assert_array_equal(kd.blockwise(keys, 1000, 256, 8)[0], kd.keep(keys, 256, 8))
