"""Parity of the semantic block index (sparse_attn_build_block_index,
sparse_attn_select_blocks, sparse_attn_decode_blocks) with the fp64 oracle
of oracle/semantic.py.

The k-means assignment is an argmax that the GPU takes with bf16 centres
and fp32 sums on the matrix cores, so each step is checked on the GPU's own
state: every key's block must be within the fp32 rounding bound of the best
centre (computed in fp64 from the same bf16 operands), each centre update
must match the oracle's update of the GPU's previous assignment, and the
block layout, the copied keys and values and the block choice are compared
exactly; the block choice must equal the oracle's where no two block scores
at the budget's edge are within 1e-4 relative of each other, and elsewhere be
what the greedy rule gives for an order consistent within that band
(tests/parity.py::check_block_choice), with the number of such rows bounded.
The decode is compared with the oracle's attention over the GPU's blocks and the window.  Shapes cover both
head dims, several GQA groups, ragged chunk, segment and tile tails, more
than 256 blocks (two rounds of centres in LDS), empty blocks, and keys
interleaved in position order."""
import numpy as np
import pytest

from oracle import semantic as sem
from block_sparse_long_page_amd import configs, synth
from block_sparse_long_page_amd.synth import to_f32
from parity import check_block_choice, check_lse, check_output

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from block_sparse_long_page_amd.device import BlockIndex, DeviceCache, to_device  # noqa: E402

CASES = {
    # (problem kwargs, N, C)
    "hd128-g4-p64-clusters": ("semantic", dict(hd=128), None, 8),
    "hd128-g2-random-ragged": ("random", dict(B=2, Hq=4, Hkv=2, hd=128, P=16, L=3000 + 8, W=8), 3000, 23),
    # the first 1000 keys are one repeated key: the starting centres there coincide, every such key
    # goes to the lowest of them and the others are left empty
    "hd64-g8-random-300-blocks": ("random", dict(B=1, Hq=8, Hkv=1, hd=64, P=32, L=5000 + 16, W=16, dup=1000), 5000,
                                  300),
    "hd128-g1-more-blocks-than-clusters": ("semantic", dict(hd=128, G=1), None, 20),
    # key counts one past a workgroup's 256 keys of the assignment and centre
    # counts one past, one short of and at its rounds of 128 centres
    "hd128-g2-edges-257-129": ("random", dict(B=1, Hq=4, Hkv=2, hd=128, P=16, L=257 + 8, W=8), 257, 129),
    "hd64-g4-p1-edges-1023-128": ("random", dict(B=2, Hq=4, Hkv=1, hd=64, P=1, L=1023 + 16, W=16), 1023, 128),
    "hd128-g1-p64-edges-768-127": ("random", dict(B=1, Hq=2, Hkv=2, hd=128, P=64, L=768 + 8, W=8), 768, 127),
}


def _problem(kind, kw, seed=0):
    if kind == "semantic":
        G = kw.get("G", 4)
        wl = configs.SEMANTIC_512K.scaled(batch=2, num_q_heads=2 * G, num_kv_heads=2, head_dim=kw["hd"],
                                          context=16 * 64 + 8, page_size=64, window=8, budget=4 * 64, q_rows=8)
        return synth.semantic_problem(wl, seed=seed, blocks=16, block_tokens=64, scatter=True)
    pr = synth.random_problem(B=kw["B"], Hq=kw["Hq"], Hkv=kw["Hkv"], hd=kw["hd"], P=kw["P"],
                              seq_lens=[kw["L"]] * kw["B"], sink=0, window=kw["W"], budget=kw["L"] // 16,
                              mode="centroid", dtype="bf16", seed=100 + seed, shuffle=True, clusters=12,
                              Q=kw["W"] // 2)
    c = pr.cache
    for b in range(c.B):
        for t in range(1, kw.get("dup", 0)):
            c.k[c.block_table[b, t // c.P], :, t % c.P] = c.k[c.block_table[b, 0], :, 0]
    return pr


def _setup(name, seed=0):
    kind, kw, N, C = CASES[name]
    pr = _problem(kind, kw, seed)
    c = pr.cache
    L = int(c.seq_lens[0])
    N = N or L - pr.window
    dc = DeviceCache.from_host(c)
    ix = BlockIndex(dc, N, C, Q=pr.Q, window=pr.window, budget=max(64, N // 16), k_max=C)
    return pr, dc, ix, N, C


def _keys(pr, b, kvh, N):
    c = pr.cache
    n_pages = -(-N // c.P)
    phys = c.block_table[b, :n_pages]
    K = to_f32(c.k[phys, kvh], c.dtype).astype(np.float64).reshape(-1, c.hd)[:N]
    V = to_f32(c.v[phys, kvh], c.dtype).astype(np.float64).reshape(-1, c.hd)[:N]
    return K, V


def _bf16(x):
    """fp32 -> bf16 (round to nearest even) -> float64, as the GPU rounds its centres."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _state(ix):
    torch.cuda.synchronize()
    return dict(centres=ix.centres.cpu().numpy().astype(np.float64), assign=ix.assignment.cpu().numpy(),
                offsets=ix.offsets.cpu().numpy(), positions=ix.positions.cpu().numpy(),
                kb=ix.k_blocks.cpu().numpy(), vb=ix.v_blocks.cpu().numpy())


def _check_assignment(K, centres, a):
    """Every key's block is the best centre within the fp32 rounding bound of
    the products (bf16 keys and centres, fp32 sums over hd channels)."""
    cb = _bf16(centres)
    d = K @ cb.T
    best = d.max(axis=1)
    got = d[np.arange(len(a)), a]
    bound = 1e-5 * (np.abs(K) @ np.abs(cb).T).max(axis=1) + 1e-30
    bad = np.flatnonzero(got < best - bound)
    assert bad.size == 0, (bad[:5], got[bad[:5]], best[bad[:5]])
    # ties inside the bound may go either way; everywhere else the choice is unique
    clear = (np.sort(d, axis=1)[:, -2] < best - bound) if d.shape[1] > 1 else np.ones(len(a), bool)
    np.testing.assert_array_equal(a[clear], np.argmax(d, axis=1)[clear])


@pytest.mark.parametrize("name", list(CASES))
def test_build_steps_match_the_oracle(name):
    pr, dc, ix, N, C = _setup(name)
    c = pr.cache
    states = []
    for it in (0, 1, 2, 6):
        ix.build(iterations=it)
        states.append(_state(ix))
    again = BlockIndex(dc, N, C, Q=pr.Q, window=pr.window, budget=ix.budget, k_max=C)
    again.build(iterations=6)
    s2 = _state(again)
    for k in states[-1]:  # bitwise reproducible
        assert np.array_equal(states[-1][k], s2[k]), k
    for b in range(c.B):
        for kvh in range(c.Hkv):
            K, V = _keys(pr, b, kvh, N)
            u = sem.unit_keys(K)
            st = [{k: v[b, kvh] for k, v in s.items()} for s in states]
            np.testing.assert_allclose(st[0]["centres"], sem.init_centres(u, C), rtol=0, atol=2e-6)
            for s in st:
                _check_assignment(K, s["centres"], s["assign"])
            # an update is the oracle's update of the GPU's previous assignment
            for prev, cur in ((st[0], st[1]), (st[1], st[2])):
                want = sem.update(u, prev["assign"], prev["centres"])
                np.testing.assert_allclose(cur["centres"], want, rtol=0, atol=2e-5)
            fin = st[-1]
            perm, off = sem.block_layout(fin["assign"], C)
            np.testing.assert_array_equal(fin["offsets"], off)
            np.testing.assert_array_equal(fin["positions"], perm)
            n_pages = -(-N // c.P)
            rowsK = c.k[c.block_table[b, :n_pages], kvh].reshape(-1, c.hd)[:N]
            rowsV = c.v[c.block_table[b, :n_pages], kvh].reshape(-1, c.hd)[:N]
            np.testing.assert_array_equal(fin["kb"].view(np.uint16), rowsK[perm])
            np.testing.assert_array_equal(fin["vb"].view(np.uint16), rowsV[perm])
            assert (np.diff(off) == 0).any() or name != "hd64-g8-random-300-blocks"  # empty blocks occur


def _query_group(pr, b, kvh, i):
    c = pr.cache
    G = c.Hq // c.Hkv
    return np.stack([to_f32(pr.q[b, kvh * G + h, i], c.dtype).astype(np.float64) for h in range(G)])


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("budget", ["zero", "sixteenth", "all"])
def test_block_choice_matches_the_oracle(name, budget):
    pr, dc, ix, N, C = _setup(name, seed=1)
    c = pr.cache
    ix.budget = {"zero": 0, "sixteenth": max(1, N // 16), "all": 10**9}[budget]
    ix.k_max = C if budget != "all" else max(1, C // 2)
    ix.sel = torch.full((c.B, c.Hkv, pr.Q, ix.k_max), -1, dtype=torch.int32, device="cuda")
    ix.build(iterations=3)
    ix.select(to_device(pr.q))
    st = _state(ix)
    sel, cnt = ix.sel.cpu().numpy(), ix.count.cpu().numpy()
    ties = 0
    for b in range(c.B):
        for kvh in range(c.Hkv):
            mu = st["centres"][b, kvh]
            sizes = np.diff(st["offsets"][b, kvh])
            for i in range(pr.Q):
                s = sem.block_scores(_query_group(pr, b, kvh, i), mu)
                got = sel[b, kvh, i, :cnt[b, kvh, i]]
                assert (sel[b, kvh, i, cnt[b, kvh, i]:] == -1).all()
                # the oracle's choice where the edge is clear; elsewhere the
                # greedy rule's result for an order consistent within the band
                ties += check_block_choice(got, s, sizes, ix.budget, ix.k_max)
    rows = c.B * c.Hkv * pr.Q
    print(f"{name} budget={budget}: {ties} of {rows} rows with a near tie at the edge")
    assert ties <= max(2, rows // 10)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("splits", [(1, 1), (2, 3)])
def test_block_decode_matches_the_oracle(name, splits):
    pr, dc, ix, N, C = _setup(name, seed=2)
    c = pr.cache
    ix.ts, ix.ls = splits
    ix.stride = ix.k_max * ix.ts + ix.ls
    ix.part_o = torch.empty((ix.rows, ix.stride, c.hd), dtype=torch.float32, device="cuda")
    ix.part_ml = torch.empty((ix.rows, ix.stride, 2), dtype=torch.float32, device="cuda")
    q = to_device(pr.q)
    ix.build(iterations=4)
    ix.step(q)
    st = _state(ix)
    out, lse = ix.out_f32(), ix.lse_f32()
    sel, cnt = ix.sel.cpu().numpy(), ix.count.cpu().numpy()
    L = int(c.seq_lens[0])
    G = c.Hq // c.Hkv
    ref_out = np.zeros_like(out, dtype=np.float64)
    ref_lse = np.zeros_like(lse, dtype=np.float64)
    for b in range(c.B):
        for kvh in range(c.Hkv):
            n_pages = -(-L // c.P)
            phys = c.block_table[b, :n_pages]
            K = to_f32(c.k[phys, kvh], c.dtype).astype(np.float64).reshape(-1, c.hd)[:L]
            V = to_f32(c.v[phys, kvh], c.dtype).astype(np.float64).reshape(-1, c.hd)[:L]
            perm, off = st["positions"][b, kvh], st["offsets"][b, kvh]
            for i in range(pr.Q):
                pos = L - pr.Q + i
                blocks = sel[b, kvh, i, :cnt[b, kvh, i]]
                toks = np.concatenate([perm[off[x]:off[x + 1]] for x in blocks] +
                                      [np.arange(L - pr.window, pos + 1)])
                qg = _query_group(pr, b, kvh, i)
                for h in range(G):
                    o, l_ = sem.attend(qg[h], K[toks], V[toks], 1.0 / np.sqrt(c.hd))
                    ref_out[b, kvh * G + h, i] = o
                    ref_lse[b, kvh * G + h, i] = l_
    check_output(out, ref_out, c.dtype, name)
    check_lse(lse, ref_lse, name)
    o1, l1 = ix.out.clone(), ix.lse.clone()
    ix.step(q)
    torch.cuda.synchronize()
    assert torch.equal(ix.out, o1) and torch.equal(ix.lse, l1)
