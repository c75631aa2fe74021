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
