"""End-to-end parity at the workloads' full sizes, in the launch configuration
the benchmark times (the library's default split count): the tiny fp32
case, the Qwen3-8B-shaped and Llama-3-70B-shaped layers, the 3-layer hybrid
256k schedule (every refresh step and the last step) and the semantic-block
512K chunk.  The oracle computes every output at these sizes."""
import time

import numpy as np
import pytest

import oracle
from block_sparse_long_page_amd import configs, synth
from parity import check_lse, check_output, check_selection

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from block_sparse_long_page_amd import binding as B  # noqa: E402
from block_sparse_long_page_amd.device import DeviceCache, GroupedStep, SparseDecoder, to_device  # noqa: E402


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("wl", [configs.TINY, configs.QWEN3_8B, configs.LLAMA3_70B, configs.SEMANTIC_512K],
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
            if t > 0:  # one token appended: refresh the summary of the last page only
                dc.seq_lens.fill_(L)
                last = (L - 1) // dc.P
                dec.build_meta(last, last + 1)
            q = to_device(hs.q[li][t])
            if t % R == 0:  # a selecting step: top-k inside the decode kernel
                t_ref = t
                dec.select_decode(q)
            else:
                dec.decode(q, window=W + (t - t_ref))
            w_eff = W + (t - t_ref)
            dec.combine()
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
        del dc, dec
        torch.cuda.empty_cache()
    _say(f"[{wl.name}] total {time.time() - t0:.1f}s")
