"""Host-side checks of the eviction and prefill workloads and their seeded
inputs (CPU only): the shapes the benchmark and the GPU tests rely on."""
import numpy as np

from block_sparse_long_page_amd import configs, synth


def test_keydiff_workload_holds_one_block_over_the_budget():
    wl = configs.KEYDIFF_8K
    assert wl.context == wl.budget + wl.block
    assert wl.sink < wl.budget and wl.context - wl.sink <= 12288  # one top-k workgroup's candidates
    assert wl.num_q_heads % wl.num_kv_heads == 0


def test_prefill_workload_chunks_tile_the_prompt():
    wl = configs.SEMANTIC_PREFILL_64K
    assert wl.window == wl.q_rows  # the window is the chunk itself
    assert (wl.context - wl.q_rows) % 2048 == 0  # whole clusters of 2048 keys, then the last chunk
    assert wl.context % wl.q_rows == 0  # the chunks tile the prompt
    assert wl.q_rows <= 128  # the grouped decode's row sets


def test_prefill_queries_are_seeded_and_shaped():
    wl = configs.SEMANTIC_512K.scaled(batch=1, num_q_heads=4, num_kv_heads=2, head_dim=32, context=4 * 64 + 8,
                                      page_size=64, window=8, budget=64, q_rows=8)
    pr = synth.semantic_problem(wl, seed=3, blocks=4, block_tokens=64, scatter=True)
    L = int(pr.cache.seq_lens[0])
    a = synth.prefill_queries(pr, seed=7)
    b = synth.prefill_queries(pr, seed=7)
    c = synth.prefill_queries(pr, seed=8)
    assert a.shape == (1, 4, L, 32) and a.dtype == np.uint16
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, c)
    # each row is a unit direction scaled by sqrt(hd), up to bf16 rounding
    n = np.linalg.norm(synth.to_f32(a, pr.cache.dtype).astype(np.float64), axis=-1)
    np.testing.assert_allclose(n, np.sqrt(32), rtol=1e-2)
