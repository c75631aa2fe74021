"""Comparison rules between the HIP path and the oracle.

Selected pages: scores are fp32 on the GPU and fp64 in the oracle, so pages
whose oracle score lies within a relative 1e-4 of the k-th largest score may
legitimately differ.  With s_k the oracle's k-th largest group score and
tau = 1e-4 * max(|s_k|, 1e-30), the GPU set must have exactly k pages, be
strictly ascending candidate pages, contain every page scoring above
s_k + tau and none scoring below s_k - tau.  The output is then compared with
the oracle re-run on the GPU's own set.

Outputs: max-abs 2e-2 for bf16 K/V (bf16 inputs, fp32 accumulation, bf16
output rounding) and 1e-4 for fp32 K/V.
"""
from __future__ import annotations

import numpy as np

BAND_REL = 1e-4
TOL = {0: 1e-4, 1: 2e-2}  # F32, BF16


def check_selection(sel: np.ndarray, cnt: np.ndarray, scores: np.ndarray, k_max: int):
    """sel [B][Hkv][Q][k_max], cnt [B][Hkv][Q] from the GPU; scores
    [B][Hkv][Q][max_pages] from the oracle (NaN = not a candidate).  Returns
    the number of pages inside the band, summed."""
    in_band = 0
    B, Hkv, Q = cnt.shape
    for b in range(B):
        for h in range(Hkv):
            for i in range(Q):
                s = scores[b, h, i]
                cand = ~np.isnan(s)
                n = int(cand.sum())
                k = min(k_max, n)
                assert cnt[b, h, i] == k, (b, h, i, cnt[b, h, i], k)
                got = sel[b, h, i, :k]
                assert (np.diff(got) > 0).all(), got
                assert cand[got].all(), got
                if k_max > k:
                    assert (sel[b, h, i, k:] == -1).all()
                if k == 0 or k == n:
                    continue
                vals = np.sort(s[cand])[::-1]
                sk = vals[k - 1]
                tau = BAND_REL * max(abs(sk), 1e-30)
                must = np.flatnonzero(cand & (s > sk + tau))
                never = np.flatnonzero(cand & (s < sk - tau))
                gs = set(got.tolist())
                missing = [p for p in must if p not in gs]
                extra = [p for p in never if p in gs]
                assert not missing and not extra, dict(b=b, h=h, i=i, missing=missing, extra=extra)
                in_band += int((cand & (np.abs(s - sk) <= tau)).sum())
    return in_band


def check_output(gpu_out: np.ndarray, ref_out: np.ndarray, dtype: int, what: str = ""):
    err = np.abs(gpu_out.astype(np.float64) - ref_out)
    assert np.isfinite(gpu_out).all(), f"{what}: non-finite output"
    worst = float(err.max()) if err.size else 0.0
    assert worst <= TOL[dtype], f"{what}: max-abs error {worst:.3e} > {TOL[dtype]}"
    return worst


def check_lse(gpu_lse: np.ndarray, ref_lse: np.ndarray, what: str = ""):
    err = np.abs(gpu_lse.astype(np.float64) - ref_lse)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= 1e-4 * max(1.0, float(np.abs(ref_lse).max())), f"{what}: lse error {worst:.3e}"
    return worst


def check_block_choice(got, scores, sizes, budget: int, k_max: int, rel: float = BAND_REL) -> bool:
    """Checks one row's choice of ragged blocks (semantic-blocks page: the
    best blocks by centre score, taken while the running token count stays
    within the budget, the first always, at most k_max; empty blocks never).

    `scores` are the oracle's fp64 group scores, `sizes` the block sizes the
    budget counts.  The GPU ranks fp32 scores, so its order may differ from
    the oracle's between blocks whose scores lie within tau = rel * max|s| of
    each other.  The choice is valid when it is what the greedy rule yields
    for SOME order of the non-empty blocks that never puts a block before
    another scoring more than tau above it.  That holds exactly when
      * the chosen blocks are strictly ascending, non-empty, at most k_max,
        and at least one unless there is nothing to choose;
      * no block left out scores more than tau above a chosen one (so every
        block clearly above the edge is taken and none clearly below it);
      * the chosen sizes fit the budget (one block may exceed it alone);
      * the rule stopped legitimately: k_max reached, nothing left, or some
        block that may come next (within tau of the best left out) does not
        fit.
    Returns True when the row's edge holds a near tie (several choices are
    valid), False when the choice is unique and equal to the oracle's."""
    got = np.asarray(got, dtype=np.int64)
    s = np.asarray(scores, dtype=np.float64)
    sizes = np.asarray(sizes, dtype=np.int64)
    nonempty = np.flatnonzero(sizes > 0)
    tau = rel * max(1e-30, float(np.abs(s).max()) if s.size else 0.0)
    assert np.all(np.diff(got) > 0), got
    assert np.all(sizes[got] > 0), got
    if nonempty.size == 0 or k_max == 0:
        assert got.size == 0, got
        return False
    assert 1 <= got.size <= k_max, got
    chosen = np.zeros(s.size, bool)
    chosen[got] = True
    rest = nonempty[~chosen[nonempty]]
    total = int(sizes[got].sum())
    assert got.size == 1 or total <= budget, (got, total, budget)
    if rest.size:
        top_rest = float(s[rest].max())
        assert float(s[got].min()) >= top_rest - tau, dict(got=got, low=float(s[got].min()), above=top_rest)
        if got.size < k_max:
            may_next = rest[s[rest] >= top_rest - tau]
            assert np.any(total + sizes[may_next] > budget), dict(got=got, total=total, budget=budget,
                                                                   could_take=may_next)
    # near tie at the edge: the oracle's order (score desc, block asc) around its cut
    order = sorted(nonempty.tolist(), key=lambda x: (-s[x], x))
    want, run = [], 0
    for x in order:
        if len(want) >= k_max or (want and run + int(sizes[x]) > budget):
            break
        want.append(x)
        run += int(sizes[x])
    n = len(want)
    edge = s[order[max(0, n - 1):n + 2]]
    tie = len(edge) >= 2 and float(np.min(-np.diff(edge))) <= tau
    if not tie:
        np.testing.assert_array_equal(got, np.sort(want))
    return tie
