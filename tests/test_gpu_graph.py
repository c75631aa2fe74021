"""A decode schedule captured as HIP graphs (one per step, as the benchmark
replays the hybrid schedule): two layers sharing the sequences' lengths,
a selection every 8 steps with the window grown between them, the pages
appended since the last selection summarised before the next one, and the
last combine of every step advancing the lengths.  The graphs are replayed
three times, with the program's own eager work and synchronisations between
the replays, and every step's outputs of every replay must equal the eager
run bit for bit; so must the outputs at the end of every cycle when each
refresh cycle is one graph (as the benchmark replays the schedule).  The
eager run itself is checked against the oracle."""
import numpy as np
import pytest

import oracle
from block_sparse_long_page_amd import synth
from parity import check_lse, check_output, check_selection

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from block_sparse_long_page_amd.device import DeviceCache, SparseDecoder, to_device  # noqa: E402

L0, T, RF, P, SINK = 4096, 20, 8, 32, 64
LAYERS = [(256, 512), (128, 1024)]  # (window, budget)


def _setup():
    caches, qs, layers = [], [], []
    seq_lens = None
    for li, (W, budget) in enumerate(LAYERS):
        pr = synth.random_problem(B=2, Hq=16, Hkv=2, hd=128, P=P, seq_lens=[L0 + T] * 2, sink=SINK, window=W,
                                  budget=budget, mode="quest", dtype="bf16", seed=70 + li, shuffle=True, clusters=8)
        rng = np.random.default_rng(80 + li)
        q = synth.store(rng.standard_normal((T, 2, 16, 1, 128)).astype(np.float32), pr.cache.dtype)
        pr.cache.seq_lens[:] = L0
        dc = DeviceCache.from_host(pr.cache, max_seq_len=L0 + T)
        if seq_lens is None:
            seq_lens = dc.seq_lens
        dc.seq_lens = seq_lens
        dec = SparseDecoder(dc, mode=pr.mode, Q=1, sink=SINK, window=W, budget=budget, splits=4)
        caches.append(pr.cache)
        qs.append(q)
        layers.append((dc, dec, W, [to_device(q[t]) for t in range(T)]))
    return caches, qs, layers, seq_lens


def _reset(layers, seq_lens):
    seq_lens.fill_(L0)
    for dc, dec, W, q in layers:
        dec.build_meta()


def _issue(layers, t):
    t_ref = t - t % RF
    L = L0 + t
    for li, (dc, dec, W, q) in enumerate(layers):
        if t == t_ref:
            if t > 0:
                dec.build_meta((L0 + t_ref - RF - 1) // P, (L - 1) // P + 1)
            dec.select_decode(q[t])
        else:
            dec.decode(q[t], window=W + (t - t_ref))
        dec.combine(advance=1 if li == len(layers) - 1 else 0)


def _outputs(layers):
    return [(dec.out.clone(), dec.lse.clone(), dec.sel.clone(), dec.count.clone()) for dc, dec, W, q in layers]


def test_schedule_replayed_from_graphs_equals_eager():
    caches, qs, layers, seq_lens = _setup()
    _reset(layers, seq_lens)
    eager = []
    for t in range(T):
        _issue(layers, t)
        eager.append(_outputs(layers))
    torch.cuda.synchronize()
    assert int(seq_lens[0]) == L0 + T
    # the eager run against the oracle at every selection and the last step
    for li, (W, budget) in enumerate(LAYERS):
        cache = caches[li]
        for t in sorted(set(range(0, T, RF)) | {T - 1}):
            t_ref = t - t % RF
            cache.seq_lens[:] = L0 + t
            out, lse, sel, cnt = eager[t][li]
            k = budget // P
            s, c = sel.cpu().numpy()[..., :k], cnt.cpu().numpy()
            if t == t_ref:
                r = oracle.run(cache, qs[li][t], mode=0, Q=1, sink=SINK, window=W, budget=budget, want_scores=True)
                check_selection(s, c, r.scores, k)
            ref = oracle.run(cache, qs[li][t], mode=0, Q=1, sink=SINK, window=W + t - t_ref, budget=budget, sel=s,
                             cnt=c)
            o = (out.cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
            check_output(o.reshape(ref.out.shape), ref.out, cache.dtype, f"layer {li} step {t}")
            check_lse(lse.cpu().numpy().reshape(ref.lse.shape), ref.lse, f"layer {li} step {t}")
    # one graph per step
    _reset(layers, seq_lens)
    torch.cuda.synchronize()
    graphs = []
    for t in range(T):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            _issue(layers, t)
        graphs.append(g)
    for rep in range(3):
        _reset(layers, seq_lens)
        scratch = torch.randn(1 << 20, device="cuda").sum()  # the program's own eager work between replays
        torch.cuda.synchronize()
        for t in range(T):
            graphs[t].replay()
            got = _outputs(layers)
            for li in range(len(layers)):
                for a, b in zip(got[li], eager[t][li]):
                    assert torch.equal(a, b), (rep, t, li)
        torch.cuda.synchronize()
        assert int(seq_lens[0]) == L0 + T, rep
        del scratch
    # one graph per refresh cycle (as the benchmark replays): the outputs at the end of every cycle
    _reset(layers, seq_lens)
    torch.cuda.synchronize()
    cycles = []
    for c0 in range(0, T, RF):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for t in range(c0, min(T, c0 + RF)):
                _issue(layers, t)
        cycles.append((g, min(T, c0 + RF) - 1))
    for rep in range(3):
        _reset(layers, seq_lens)
        torch.cuda.synchronize()
        for g, last in cycles:
            g.replay()
            got = _outputs(layers)
            for li in range(len(layers)):
                for a, b in zip(got[li], eager[last][li]):
                    assert torch.equal(a, b), (rep, last, li)
        torch.cuda.synchronize()
        assert int(seq_lens[0]) == L0 + T, rep
