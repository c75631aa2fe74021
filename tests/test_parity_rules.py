"""The comparison rules of tests/parity.py pinned by brute force.

The GPU ranks fp32 scores, so where scores lie within the band tau of each
other its order may differ from the oracle's fp64 order.  A choice is then
correct when the selection rule applied to SOME order that never puts an
item before another scoring more than tau above it yields it.  These tests
enumerate every such order on tiny inputs (with planted exact and near ties)
and check that the rules accept exactly the results those orders give:
nothing valid is rejected and nothing else is accepted."""
import itertools

import numpy as np
import pytest

from parity import BAND_REL, check_block_choice, check_selection


def _band_orders(items, s, tau):
    """Every order of `items` in which no item precedes one scoring more than tau above it."""
    for perm in itertools.permutations(items):
        if all(s[perm[i]] >= s[perm[j]] - tau for i in range(len(perm)) for j in range(i + 1, len(perm))):
            yield perm


def _greedy(order, sizes, budget, k_max):
    """The semantic-blocks page's rule on one order: take blocks while the
    running token count stays within the budget (the first always), at most k_max."""
    taken, run = [], 0
    for x in order:
        if len(taken) >= k_max or (taken and run + int(sizes[x]) > budget):
            break
        taken.append(x)
        run += int(sizes[x])
    return tuple(sorted(taken))


def _accepts(fn, *args):
    try:
        fn(*args)
        return True
    except AssertionError:
        return False


def _scores(rng, n):
    """Scores on a coarse grid (exact ties) plus sub-band jitter (near ties)."""
    base = rng.integers(1, 4, n).astype(np.float64)
    jitter = rng.choice([0.0, 0.4e-4, -0.4e-4, 0.8e-4, 3e-4], n) * 3.0
    return base + jitter


@pytest.mark.parametrize("seed", range(400))
def test_block_choice_rule_accepts_exactly_the_band_orders(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 7))
    s = _scores(rng, n)
    sizes = rng.integers(0, 6, n)
    if seed % 7 == 0:
        sizes[:] = 0 if seed % 2 else sizes  # nothing to choose in some cases
    budget = int(rng.integers(0, 14))
    k_max = int(rng.integers(1, 5))
    tau = BAND_REL * max(1e-30, float(np.abs(s).max()))
    items = [x for x in range(n) if sizes[x] > 0]
    valid = {_greedy(o, sizes, budget, k_max) for o in _band_orders(items, s, tau)} if items else {()}
    unique = None
    for r in range(0, n + 1):
        for X in itertools.combinations(range(n), r):
            ok = _accepts(check_block_choice, np.array(X, dtype=np.int64), s, sizes, budget, k_max)
            assert ok == (X in valid), dict(X=X, valid=valid, s=s, sizes=sizes, budget=budget, k_max=k_max)
            if ok:
                unique = not check_block_choice(np.array(X, dtype=np.int64), s, sizes, budget, k_max)
    # a row reported free of near ties has exactly one valid choice
    if unique:
        assert len(valid) == 1


@pytest.mark.parametrize("seed", range(200))
def test_page_selection_rule_is_sandwiched_by_the_band_orders(seed):
    """check_selection (page top-k of the paged path, band around the k-th
    score s_k): it accepts the first k pages of every order consistent within
    tau (nothing correct is rejected), and everything it accepts is the first
    k pages of an order consistent within 2 tau (a page more than 2 tau
    above a chosen one is never left out)."""
    rng = np.random.default_rng(1000 + seed)
    npg = int(rng.integers(1, 7))
    s = _scores(rng, npg)
    cand = rng.random(npg) < 0.85
    s_or_nan = np.where(cand, s, np.nan)
    k_max = int(rng.integers(1, 5))
    items = [p for p in range(npg) if cand[p]]
    k = min(k_max, len(items))
    sk = np.sort(s[cand])[::-1][k - 1] if k else 0.0
    tau = BAND_REL * max(abs(sk), 1e-30)
    inner = {tuple(sorted(o[:k])) for o in _band_orders(items, s, tau)} if items else {()}
    outer = {tuple(sorted(o[:k])) for o in _band_orders(items, s, 2 * tau)} if items else {()}
    for X in itertools.combinations(range(npg), k):
        sel = np.full((1, 1, 1, k_max), -1, np.int32)
        sel[0, 0, 0, :k] = X
        cnt = np.full((1, 1, 1), k, np.int32)
        ok = _accepts(check_selection, sel, cnt, s_or_nan[None, None, None], k_max)
        if X in inner:
            assert ok, dict(X=X, inner=inner, s=s_or_nan, k_max=k_max)
        if ok:
            assert X in outer, dict(X=X, outer=outer, s=s_or_nan, k_max=k_max)
