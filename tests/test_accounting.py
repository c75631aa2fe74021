"""Byte and FLOP accounting against the numbers the pages print."""
import json
import os

import numpy as np
import pytest

from block_sparse_long_page_amd import accounting as acc
from block_sparse_long_page_amd import configs

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))
GiB = float(1 << 30)


def _unit(v, unit):
    return v * (GiB if unit == "GiB" else 1e9)


@pytest.mark.parametrize("e", G["kv_bytes"], ids=lambda e: str(e["layers"]))
def test_kv_bytes(e):
    per = acc.kv_bytes_per_token(e["layers"], e["kv_heads"], e["head_dim"], e["elem_bytes"])
    if "bytes_per_token" in e:
        assert per == e["bytes_per_token"]
    tol = e["tolerance"]
    for tokens, val, unit in e.get("at_tokens", []):
        got = acc.kv_cache_bytes(e["layers"], e["kv_heads"], e["head_dim"], e["elem_bytes"], tokens)
        assert abs(got - _unit(val, unit)) <= tol * _unit(val, unit)
    for tokens, batch, val, unit in e.get("at_batch", []):
        got = acc.kv_cache_bytes(e["layers"], e["kv_heads"], e["head_dim"], e["elem_bytes"], tokens, batch)
        assert abs(got - _unit(val, unit)) <= tol * _unit(val, unit)
    for heads, val, unit in e.get("kv_heads_alt", []):
        got = acc.kv_cache_bytes(e["layers"], heads, e["head_dim"], e["elem_bytes"], e["at_tokens"][0][0])
        assert abs(got - _unit(val, unit)) <= tol * _unit(val, unit)


def test_block_sparse_flop_ratio():
    f = G["flop_ratio"]
    r = acc.block_sparse_flops(f["n"], f["head_dim"], f["block"], f["topk"]) / acc.dense_flops(f["n"], f["head_dim"])
    assert r == pytest.approx(f["ratio"], abs=1e-12)
    assert r == pytest.approx(f["topk"] * f["block"] / f["n"])


def test_read_time_floor():
    r = G["read_time"]
    ms = r["bytes_gib"] * GiB / (r["bandwidth_tb_s"] * 1e12) * 1e3
    assert abs(ms - r["ms"]) <= r["tolerance"] * ms + 0.2


@pytest.mark.parametrize("L,P,S,W", [
    (2048, 16, 16, 64),        # the tiny workload
    (32768, 16, 256, 1024),    # the Qwen3-8B-shaped layer
    (131072, 64, 256, 4096),   # the Llama-3-70B-shaped layer
    (262144 + 5, 32, 256, 2048 + 5),  # a hybrid layer between refreshes (ragged last page)
    (1000, 16, 40, 30),        # sink and window edges inside pages
    (300, 16, 200, 100),       # sink and window meet: no middle region
    (100, 16, 256, 64),        # sink longer than the sequence
])
def test_candidate_counts_match_the_oracle(L, P, S, W):
    """The byte accounting's candidate count equals the number of pages the
    oracle scores (the non-NaN entries of its score row)."""
    import oracle
    from block_sparse_long_page_amd import synth

    pr = synth.random_problem(B=1, Hq=1, Hkv=1, hd=64, P=P, seq_lens=[L], sink=S, window=W, budget=P,
                              dtype="f32", seed=L % 97)
    r = oracle.run(pr.cache, pr.q, mode=oracle.QUEST, Q=1, sink=S, window=W, budget=P, want_scores=True)
    assert int(np.count_nonzero(~np.isnan(r.scores[0, 0, 0]))) == acc.candidate_pages(L, P, S, W)


def test_headline_step_bytes():
    w = configs.LLAMA3_70B
    sb = acc.decode_step_bytes(B=w.batch, Hq=w.num_q_heads, Hkv=w.num_kv_heads, hd=w.head_dim, elem_bytes=2,
                               L=w.context, P=w.page_size, S=w.sink, W=w.window, budget=w.budget, mode=0, splits=32)
    # 256 sink + 4096 window + 128 pages x 64 = 12544 tokens per (b, kv head), 512 B each for K+V
    assert sb.kv == 32 * 12544 * 512
    assert sb.meta == 32 * 1980 * 512
    # the attended share of the dense cache is (S + W + k P) / L
    assert acc.attended_tokens(w.context, w.page_size, w.sink, w.window, w.k_pages) / w.context == pytest.approx(
        12544 / 131072)
