"""End-to-end parity at the workloads' full sizes, in the launch configuration
the benchmark times (the library's default split count): the tiny fp32
case, the Qwen3-8B-shaped and Llama-3-70B-shaped layers (the latter also with
compressed-key scores, and one KV head's share of a 1M-token context: 16384
pages, ranked in chunks and merged), the 3-layer hybrid
256k schedule (every refresh step and the last step) and the semantic-block
512K chunk, paged and over a block index built from interleaved keys.  The
oracle computes every output at these sizes (the index: its layout exactly,
every key's assignment within the rounding bound, the last centre update on
samples, and every row's block choice and outputs)."""
import time

import numpy as np
import pytest

import oracle
from block_sparse_long_page_amd import configs, synth
from parity import check_block_choice, check_lse, check_output, check_selection

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from block_sparse_long_page_amd import binding as B  # noqa: E402
from block_sparse_long_page_amd.device import (BlockIndex, DeviceCache, GroupedStep, SparseDecoder,  # noqa: E402
                                               to_device)
from oracle import semantic as sem  # noqa: E402


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("wl", [configs.TINY, configs.QWEN3_8B, configs.LLAMA3_70B,
                                configs.LLAMA3_70B.scaled(name="llama3-70b-layer-128k-compressed", mode="compressed"),
                                # one GPU's share (one KV head, its 8 query heads) of a 1M-token context:
                                # 16384 pages, more than one workgroup ranks, so the selection merges chunks
                                configs.LLAMA3_70B.scaled(name="llama3-70b-layer-1m-one-kv-head", batch=1,
                                                          num_q_heads=8, num_kv_heads=1, context=1 << 20,
                                                          budget=(1 << 20) // 16),
                                configs.SEMANTIC_512K],
                         ids=lambda w: w.name)
def test_single_step_workload(wl):
    t0 = time.time()
    pr = synth.workload_problem(wl)
    _say(f"[{wl.name}] inputs {time.time() - t0:.1f}s")
    dc = DeviceCache.from_host(pr.cache)
    dec = SparseDecoder(dc, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget)
    q = to_device(pr.q)
    dec.build_meta()
    dec.step(q)
    torch.cuda.synchronize()
    sel, cnt = dec.selection()
    _say(f"[{wl.name}] gpu done, splits={dec.splits}")
    r = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget,
                   want_scores=True)
    band = check_selection(sel, cnt, r.scores, pr.k_pages)
    for (b, kvh, p) in pr.needles:
        assert p in set(sel[b, kvh, 0, : cnt[b, kvh, 0]])
    ref = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget,
                     sel=sel, cnt=cnt)
    err = check_output(dec.out_f32(), ref.out, pr.cache.dtype, wl.name)
    check_lse(dec.lse_f32(), ref.lse, wl.name)
    same = int((sel == r.sel).all(axis=-1).sum())
    _say(f"[{wl.name}] max-abs {err:.2e}, pages in band {band}, identical sets {same}/{cnt.size}, "
         f"total {time.time() - t0:.1f}s")
    # the selecting step with the top-k inside the decode kernel (what the benchmark times)
    dec.sel.fill_(-7)
    dec.count.fill_(-7)
    dec.fused_step(q)
    torch.cuda.synchronize()
    sel2, cnt2 = dec.selection()
    np.testing.assert_array_equal(cnt2, cnt)
    np.testing.assert_array_equal(sel2, sel)  # same scores, same ranking
    err2 = check_output(dec.out_f32(), ref.out, pr.cache.dtype, wl.name + " fused")
    check_lse(dec.lse_f32(), ref.lse, wl.name + " fused")
    _say(f"[{wl.name}] fused step max-abs {err2:.2e}")
    if pr.Q > 1 and pr.cache.dtype == B.SA_BF16:
        # several query rows: the decode grouped by page reads each selected page once
        gs = GroupedStep(dec)
        gs.decode(q)
        gs.combine()
        torch.cuda.synchronize()
        err3 = check_output(dec.out_f32(), ref.out, pr.cache.dtype, wl.name + " grouped")
        check_lse(dec.lse_f32(), ref.lse, wl.name + " grouped")
        union = int(gs.ws[: 4 * pr.cache.B * pr.cache.Hkv].view(torch.int32).sum())
        _say(f"[{wl.name}] grouped max-abs {err3:.2e}, pages in the unions {union} "
             f"(per-row lists {int(cnt.sum())})")


def test_hybrid_schedule():
    wl = configs.HYBRID_256K
    t0 = time.time()
    hs = synth.hybrid_schedule(wl)
    _say(f"[{wl.name}] inputs {time.time() - t0:.1f}s")
    L0, T, R = hs.context, hs.steps, hs.refresh
    check_at = set(range(0, T, R)) | {T - 1}
    for li, cache in enumerate(hs.caches):
        W, budget = hs.windows[li], hs.budgets[li]
        cache.seq_lens[:] = L0
        dc = DeviceCache.from_host(cache, max_seq_len=L0 + T)
        dec = SparseDecoder(dc, mode=hs.mode, Q=1, sink=hs.sink, window=W, budget=budget)
        dec.build_meta()
        t_ref = 0
        for t in range(T):
            L = L0 + t
            if t > 0:  # one token appended (the last combine advanced the length): refresh the last page's summary
                last = (L - 1) // dc.P
                dec.build_meta(last, last + 1)
            q = to_device(hs.q[li][t])
            if t % R == 0:  # a selecting step: top-k inside the decode kernel
                t_ref = t
                dec.select_decode(q)
            else:
                dec.decode(q, window=W + (t - t_ref))
            w_eff = W + (t - t_ref)
            dec.combine(advance=1)  # the step's last launch appends the next token
            if t in check_at:
                torch.cuda.synchronize()
                cache.seq_lens[:] = L
                sel, cnt = dec.selection()
                qh = hs.q[li][t]
                if t == t_ref:
                    r = oracle.run(cache, qh, mode=hs.mode, Q=1, sink=hs.sink, window=W, budget=budget,
                                   want_scores=True)
                    check_selection(sel, cnt, r.scores, budget // dc.P)
                ref = oracle.run(cache, qh, mode=hs.mode, Q=1, sink=hs.sink, window=w_eff, budget=budget,
                                 sel=sel, cnt=cnt)
                err = check_output(dec.out_f32(), ref.out, cache.dtype, f"layer {li} step {t}")
                check_lse(dec.lse_f32(), ref.lse, f"layer {li} step {t}")
                _say(f"[{wl.name}] layer {li} step {t} window {w_eff} max-abs {err:.2e}")
        torch.cuda.synchronize()
        assert int(dc.seq_lens[0]) == L0 + T
        del dc, dec
        torch.cuda.empty_cache()
    _say(f"[{wl.name}] total {time.time() - t0:.1f}s")


def test_semantic_index_workload():
    """The 512K semantic chunk with keys interleaved in position order, over
    the index the benchmark builds (one block per 2048 tokens, 8 k-means
    iterations, L/16 token budget, at most 64 blocks per row)."""
    wl = configs.SEMANTIC_512K
    t0 = time.time()
    pr = synth.semantic_problem(wl, scatter=True)
    c = pr.cache
    L = int(c.seq_lens[0])
    N, C = L - pr.window, (L - pr.window) // 2048
    dc = DeviceCache.from_host(c)
    q = to_device(pr.q)
    ix = BlockIndex(dc, N, C, Q=pr.Q, window=pr.window, budget=pr.budget, k_max=64)
    ix.build(7)
    torch.cuda.synchronize()
    prev_c, prev_a = ix.centres.cpu().numpy().astype(np.float64), ix.assignment.cpu().numpy()
    ix.build(8)
    ix.step(q)
    torch.cuda.synchronize()
    cen, asg = ix.centres.cpu().numpy().astype(np.float64), ix.assignment.cpu().numpy()
    off, perm = ix.offsets.cpu().numpy(), ix.positions.cpu().numpy()
    sel, cnt = ix.sel.cpu().numpy(), ix.count.cpu().numpy()
    out, lse = ix.out_f32(), ix.lse_f32()
    _say(f"[{wl.name} index] built and stepped {time.time() - t0:.1f}s")
    rng = np.random.default_rng(0)
    G = c.Hq // c.Hkv
    scale = 1.0 / np.sqrt(c.hd)
    ties = 0
    for b in range(c.B):
        for kvh in range(c.Hkv):
            n_pages = -(-L // c.P)
            phys = c.block_table[b, :n_pages]
            K = synth.to_f32(c.k[phys, kvh], c.dtype).astype(np.float64).reshape(-1, c.hd)[:L]
            V = synth.to_f32(c.v[phys, kvh], c.dtype).astype(np.float64).reshape(-1, c.hd)[:L]
            # the layout of the final assignment, exactly
            p_ref, o_ref = sem.block_layout(asg[b, kvh], C)
            np.testing.assert_array_equal(off[b, kvh], o_ref)
            np.testing.assert_array_equal(perm[b, kvh], p_ref)
            # every key: the best centre within the rounding of bf16 products summed in fp32
            cb = (cen[b, kvh].astype(np.float32).view(np.uint32).astype(np.uint64))
            cb = ((((cb + 0x7FFF + ((cb >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32)
                  .astype(np.float64))
            for k0 in range(0, N, 1 << 16):
                Kc = K[k0:min(N, k0 + (1 << 16))]
                d = Kc @ cb.T
                bound = 1e-5 * (np.abs(Kc) @ np.abs(cb).T).max(axis=1)
                a = asg[b, kvh, k0:k0 + len(Kc)]
                assert np.all(d[np.arange(len(Kc)), a] >= d.max(axis=1) - bound), (b, kvh, k0)
            # the last update of a few blocks from the previous assignment
            u = sem.unit_keys(K[:N])
            for x in rng.choice(C, 6, replace=False):
                members = np.flatnonzero(prev_a[b, kvh] == x)
                if members.size:
                    want = u[members].sum(axis=0)
                    want /= np.linalg.norm(want)
                    np.testing.assert_allclose(cen[b, kvh, x], want, rtol=0, atol=2e-5)
            # every row: its block choice, then the oracle's attention over the GPU's blocks and the window
            sizes = np.diff(off[b, kvh])
            for i in range(pr.Q):
                qg = np.stack([synth.to_f32(pr.q[b, kvh * G + h, i], c.dtype).astype(np.float64) for h in range(G)])
                s_ = sem.block_scores(qg, cen[b, kvh])
                got = sel[b, kvh, i, :cnt[b, kvh, i]]
                assert (sel[b, kvh, i, cnt[b, kvh, i]:] == -1).all()
                ties += check_block_choice(got, s_, sizes, ix.budget, ix.k_max)
                pos = L - pr.Q + i
                toks = np.concatenate([perm[b, kvh, off[b, kvh, x]:off[b, kvh, x + 1]] for x in got] +
                                      [np.arange(L - pr.window, pos + 1)])
                Kt, Vt = K[toks], V[toks]
                for h in range(G):
                    o, l_ = sem.attend(qg[h], Kt, Vt, scale)
                    check_output(out[b, kvh * G + h, i], o, c.dtype, f"b{b} kvh{kvh} row{i} head{h}")
                    check_lse(np.array([lse[b, kvh * G + h, i]]), np.array([l_]), "index lse")
    rows = c.B * c.Hkv * pr.Q
    _say(f"[{wl.name} index] {ties} of {rows} rows with a near tie at the edge")
    assert ties <= max(2, rows // 10)
    _say(f"[{wl.name} index] checked {time.time() - t0:.1f}s; blocks {sizes.min()}..{sizes.max()} tokens")
