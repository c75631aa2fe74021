"""Parity of KeyDiff eviction on the GPU with its fp64 oracle
(oracle/keydiff.py): the kept positions of every (sequence, KV head) on
small shapes with ragged pages, shuffled block tables and sequences shorter
than the budget, exact on planted ties; the compaction bit for bit; attention
over the evicted cache against the oracle's attention over the kept tokens;
a blockwise schedule on the GPU's own state; and the full-size eviction of
the Llama-3.1-8B-shaped layer.

The GPU ranks fp32 squared distances, the oracle fp64 distances, so tokens
within a relative 1e-4 of the boundary distance may legitimately differ:
the kept set must hold every candidate farther than d_k (1 + 1e-4), none
nearer than d_k (1 - 1e-4), and exactly budget - sink of them."""
import numpy as np
import pytest

from block_sparse_long_page_amd import configs, synth
from helpers import dense_keys_values, query
from oracle import keydiff as kd
from parity import check_lse, check_output

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from block_sparse_long_page_amd import binding as B  # noqa: E402
from block_sparse_long_page_amd.device import DeviceCache, KeyDiffEviction, SparseDecoder, to_device  # noqa: E402

BAND_REL = 1e-4


def check_kept(kept: np.ndarray, keys: np.ndarray, budget: int, sink: int) -> int:
    """kept: the GPU's positions (ascending) for one (sequence, KV head);
    keys: fp64 [L][hd].  Returns the number of candidates inside the band."""
    L = len(keys)
    if L <= budget:
        np.testing.assert_array_equal(kept, np.arange(L))
        return 0
    s0 = min(sink, L)
    assert len(kept) == budget and np.all(np.diff(kept) > 0) and kept[0] >= 0 and kept[-1] < L
    assert list(kept[:s0]) == list(range(s0))
    d = kd.distances(keys)
    k = budget - s0
    if k == 0:
        return 0
    cand = np.arange(s0, L)
    dk = np.sort(d[cand])[::-1][k - 1]
    tau = BAND_REL * max(dk, 1e-30)
    got = set(kept[s0:].tolist())
    must = [p for p in cand if d[p] > dk + tau]
    never = [p for p in cand if d[p] < dk - tau]
    assert all(p in got for p in must), [p for p in must if p not in got][:10]
    assert not any(p in got for p in never), [p for p in never if p in got][:10]
    return int(np.sum(np.abs(d[cand] - dk) <= tau))


def _evict(pr, budget, sink, dst_P=None):
    c = pr.cache
    src = DeviceCache.from_host(c)
    dst = DeviceCache.empty(c.B, c.Hq, c.Hkv, c.hd, dst_P or c.P, budget, c.dtype)
    ev = KeyDiffEviction(src, dst, budget, sink)
    ev.evict()
    torch.cuda.synchronize()
    return src, dst, ev


CASES = {
    "bf16-hd128-p16": dict(B=2, Hq=8, Hkv=2, hd=128, P=16, seq_lens=[3000, 1777], budget=1024, sink=4,
                           dtype="bf16"),
    "f32-hd64-p7": dict(B=1, Hq=4, Hkv=1, hd=64, P=7, seq_lens=[700], budget=100, sink=0, dtype="f32"),
    "bf16-hd64-short": dict(B=3, Hq=8, Hkv=4, hd=64, P=64, seq_lens=[5000, 64, 20], budget=1000, sink=16,
                            dtype="bf16"),
    "bf16-hd128-sink-only": dict(B=1, Hq=2, Hkv=1, hd=128, P=32, seq_lens=[500], budget=32, sink=32, dtype="bf16"),
    "f32-hd128-one-evicted": dict(B=2, Hq=4, Hkv=2, hd=128, P=16, seq_lens=[257, 256], budget=256, sink=1,
                                  dtype="f32"),
    "bf16-hd128-near-limit": dict(B=1, Hq=8, Hkv=1, hd=128, P=64, seq_lens=[12000], budget=8192, sink=256,
                                  dtype="bf16"),
    # past one workgroup's 12288 candidates: chunks of 8192 pick the tokens to evict, a merge chooses them
    "bf16-hd128-past-limit": dict(B=2, Hq=8, Hkv=1, hd=128, P=64, seq_lens=[20000, 13000], budget=16384, sink=256,
                                  dtype="bf16"),
    "f32-hd64-past-limit-block": dict(B=1, Hq=4, Hkv=2, hd=64, P=16, seq_lens=[30000], budget=28000, sink=4,
                                      dtype="f32"),
    # one-token pages: a wave's 128 rows span 128 pages, two block-table
    # entries per lane; two-token pages: exactly 64
    "bf16-hd128-p1": dict(B=1, Hq=4, Hkv=2, hd=128, P=1, seq_lens=[1500], budget=700, sink=3, dtype="bf16"),
    "f32-hd64-p2": dict(B=2, Hq=2, Hkv=1, hd=64, P=2, seq_lens=[1001, 640], budget=300, sink=2, dtype="f32"),
}


def _problem(name, seed=0):
    kw = dict(CASES[name])
    budget, sink = kw.pop("budget"), kw.pop("sink")
    pr = synth.random_problem(**kw, sink=sink, window=1, budget=budget, seed=500 + seed, shuffle=True,
                              spare_pages=3, clusters=16)
    return pr, budget, sink


@pytest.mark.parametrize("name", list(CASES))
def test_kept_positions(name):
    pr, budget, sink = _problem(name)
    c = pr.cache
    _, _, ev = _evict(pr, budget, sink)
    kept = ev.kept.cpu().numpy()
    cnt = ev.count.cpu().numpy()
    band = 0
    for b in range(c.B):
        L = int(c.seq_lens[b])
        for kvh in range(c.Hkv):
            assert cnt[b, kvh] == min(L, budget)
            assert (kept[b, kvh, cnt[b, kvh]:] == -1).all()
            keys = dense_keys_values(c, b, kvh)[0]
            band += check_kept(kept[b, kvh, : cnt[b, kvh]], keys, budget, sink)
    print(f"{name}: {band} candidates inside the band")


# lengths one short of, at and one past the 512-token chunks of the sum pass
# and the 128 rows a wave streams, with pages of 1 and 2 tokens (a wave's
# rows over 128 and 64 pages) and of 16
@pytest.mark.parametrize("P,lens,budget,sink,hd,dtype", [
    (16, [512, 513, 1023], 300, 4, 128, "bf16"), (1, [127, 128, 129], 100, 1, 128, "bf16"),
    (1, [1024, 1025, 640], 500, 0, 64, "bf16"), (2, [511, 2049, 64], 256, 8, 128, "f32")])
def test_kept_positions_at_chunk_edges(P, lens, budget, sink, hd, dtype):
    pr = synth.random_problem(B=3, Hq=4, Hkv=2, hd=hd, P=P, seq_lens=lens, sink=sink, window=1, budget=budget,
                              dtype=dtype, seed=sum(lens) + P, shuffle=True, spare_pages=3, clusters=16)
    c = pr.cache
    _, _, ev = _evict(pr, budget, sink)
    kept = ev.kept.cpu().numpy()
    cnt = ev.count.cpu().numpy()
    for b in range(c.B):
        L = int(c.seq_lens[b])
        for kvh in range(c.Hkv):
            assert cnt[b, kvh] == min(L, budget)
            assert (kept[b, kvh, cnt[b, kvh]:] == -1).all()
            check_kept(kept[b, kvh, : cnt[b, kvh]], dense_keys_values(c, b, kvh)[0], budget, sink)


@pytest.mark.parametrize("name", ["bf16-hd128-p16", "bf16-hd128-past-limit", "bf16-hd128-p1"])
def test_planted_ties_keep_the_later_position(name):
    """Every key is one of four bf16 vectors, so distances tie exactly on both
    sides and the kept set must equal the oracle's (also when the evicted set
    is chosen per chunk and merged)."""
    pr, budget, sink = _problem(name, seed=1)
    c = pr.cache
    rng = np.random.default_rng(3)
    protos = synth.store(rng.standard_normal((4, c.hd)).astype(np.float32) * [[1.0], [2.0], [3.0], [4.0]], c.dtype)
    lab = rng.integers(0, 4, size=c.k.shape[:3])
    c.k[...] = protos[lab]
    _, _, ev = _evict(pr, budget, sink)
    got = ev.kept_positions()
    for b in range(c.B):
        for kvh in range(c.Hkv):
            keys = dense_keys_values(c, b, kvh)[0]
            np.testing.assert_array_equal(got[b][kvh], kd.keep(keys, budget, sink))


@pytest.mark.parametrize("name,dst_P", [("bf16-hd128-p16", 16), ("bf16-hd128-p16", 64), ("f32-hd64-p7", 10),
                                        ("bf16-hd64-short", 64), ("bf16-hd128-p1", 1), ("f32-hd64-p2", 2)])
def test_compaction_copies_the_kept_rows(name, dst_P):
    pr, budget, sink = _problem(name)
    c = pr.cache
    _, dst, ev = _evict(pr, budget, sink, dst_P=dst_P)
    got = ev.kept_positions()
    dk = dst.k.cpu().numpy()
    dv = dst.v.cpu().numpy()
    dbt = dst.block_table.cpu().numpy()
    assert list(dst.seq_lens.cpu().numpy()) == [min(int(L), budget) for L in c.seq_lens]
    for b in range(c.B):
        n_pages = -(-int(c.seq_lens[b]) // c.P)
        for kvh in range(c.Hkv):
            pos = got[b][kvh]
            sk = c.k[c.block_table[b, :n_pages], kvh].reshape(-1, c.hd)
            sv = c.v[c.block_table[b, :n_pages], kvh].reshape(-1, c.hd)
            rows_k = dk[dbt[b, np.arange(len(pos)) // dst_P], kvh, np.arange(len(pos)) % dst_P]
            rows_v = dv[dbt[b, np.arange(len(pos)) // dst_P], kvh, np.arange(len(pos)) % dst_P]
            np.testing.assert_array_equal(rows_k.view(sk.dtype), sk[pos])
            np.testing.assert_array_equal(rows_v.view(sv.dtype), sv[pos])


@pytest.mark.parametrize("name", ["bf16-hd128-p16", "f32-hd64-p7", "bf16-hd64-short", "bf16-hd128-past-limit"])
def test_attention_over_the_evicted_cache(name):
    """The dense decode of the evicted cache is the oracle's attention over
    the kept tokens of each KV head."""
    pr, budget, sink = _problem(name)
    c = pr.cache
    _, dst, ev = _evict(pr, budget, sink)
    got = ev.kept_positions()
    dec = SparseDecoder(dst, mode=0, Q=1, sink=0, window=1, budget=0)
    q = to_device(pr.q)
    dec.decode(q, dense=True)
    dec.combine()
    torch.cuda.synchronize()
    G = c.Hq // c.Hkv
    ref_o = np.zeros((c.B, c.Hq, 1, c.hd))
    ref_l = np.zeros((c.B, c.Hq, 1))
    for b in range(c.B):
        for kvh in range(c.Hkv):
            K, V = dense_keys_values(c, b, kvh)
            pos = got[b][kvh]
            for h in range(G):
                o, lse = kd.attend(query(pr, b, kvh * G + h, 0), K[pos], V[pos], 1.0 / np.sqrt(c.hd))
                ref_o[b, kvh * G + h, 0], ref_l[b, kvh * G + h, 0] = o, lse
    check_output(dec.out_f32(), ref_o, c.dtype, name)
    check_lse(dec.lse_f32(), ref_l, name)


@pytest.mark.parametrize("carried", [False, True])
def test_blockwise_schedule_on_the_gpu_state(carried):
    """A 4000-token sequence arrives in blocks of 300; after each block the
    cache (kept tokens, then the block) is evicted back to 512 tokens and
    compacted into the other of two buffers.  Each eviction is checked
    against the oracle on the keys the GPU's cache holds at that moment.
    carried: each copy also writes the key sums of every 64 slots it fills
    (checked against the sums of the rows it copied), and the next eviction
    takes the held tokens' mean from them (only the new block's keys are
    summed)."""
    block, budget, sink = 300, 512, 8
    pr = synth.random_problem(B=2, Hq=8, Hkv=2, hd=128, P=16, seq_lens=[4000, 4000], sink=sink, window=1,
                              budget=budget, dtype="bf16", seed=77, clusters=8)
    c = pr.cache
    full_k = np.stack([np.stack([c.k[c.block_table[b, :250], h].reshape(-1, c.hd) for h in range(c.Hkv)])
                       for b in range(c.B)])  # [B][Hkv][4000][hd] storage
    full_v = np.stack([np.stack([c.v[c.block_table[b, :250], h].reshape(-1, c.hd) for h in range(c.Hkv)])
                       for b in range(c.B)])
    cap = budget + block
    bufs = [DeviceCache.empty(c.B, c.Hq, c.Hkv, c.hd, c.P, cap, c.dtype) for _ in range(2)]
    held = [[np.zeros(0, dtype=np.int64) for _ in range(c.Hkv)] for _ in range(c.B)]
    cur = 0
    n_in = 0
    band = 0
    prev = None  # the eviction whose copy filled the current source
    n_carried = 0
    for t0 in range(0, 4000, block):
        src = bufs[cur]
        t1 = min(4000, t0 + block)
        # append the block after the tokens the cache holds (the model would write these rows)
        k_np = src.k.cpu().numpy()
        v_np = src.v.cpu().numpy()
        bt = src.block_table.cpu().numpy()
        for b in range(c.B):
            slots = n_in + np.arange(t1 - t0)
            for h in range(c.Hkv):
                k_np[bt[b, slots // c.P], h, slots % c.P] = full_k[b, h, t0:t1].view(k_np.dtype)
                v_np[bt[b, slots // c.P], h, slots % c.P] = full_v[b, h, t0:t1].view(v_np.dtype)
                held[b][h] = np.concatenate([held[b][h], np.arange(t0, t1)])
        src.k.copy_(torch.from_numpy(k_np))
        src.v.copy_(torch.from_numpy(v_np))
        n_cache = n_in + (t1 - t0)
        src.seq_lens.fill_(n_cache)
        dst = bufs[1 - cur]
        ev = KeyDiffEviction(src, dst, budget, sink, sums=carried)
        if carried and prev is not None:
            ev.select(carried=prev.carried())
            n_carried += int(prev.count.min().item()) // 512
        else:
            ev.select()
        ev.compact()
        torch.cuda.synchronize()
        got = ev.kept_positions()
        for b in range(c.B):
            for h in range(c.Hkv):
                keys = synth.to_f32(full_k[b, h, held[b][h]], c.dtype).astype(np.float64)
                band += check_kept(got[b][h], keys, budget, sink)
                held[b][h] = held[b][h][got[b][h]]
        n_in = min(n_cache, budget)
        assert list(dst.seq_lens.cpu().numpy()) == [n_in] * c.B
        if carried:  # the slot sums: the copied keys of each group of 64 slots
            sums = ev.slot_sums.cpu().numpy()
            for b in range(c.B):
                for h in range(c.Hkv):
                    kk = synth.to_f32(full_k[b, h, held[b][h]], c.dtype).astype(np.float64)
                    for i in range(-(-n_in // 64)):
                        grp = kk[64 * i: 64 * (i + 1)]
                        want = grp.sum(0)
                        tol = 1e-5 * np.abs(grp).sum(0) + 1e-6
                        assert (np.abs(sums[b, h, i] - want) <= tol).all(), (t0, b, h, i)
        prev = ev
        cur = 1 - cur
    for b in range(c.B):
        for h in range(c.Hkv):
            assert list(held[b][h][:sink]) == list(range(sink)) and len(held[b][h]) == budget
    if carried:
        assert n_carried > 0  # some evictions took whole chunks from the carried sums
    print(f"blockwise: {band} candidates inside the band over {-(-4000 // block)} evictions, "
          f"{n_carried} carried chunks")


def test_full_size_eviction():
    """The Llama-3.1-8B-shaped layer at 10240 tokens evicted to 8192: every
    (sequence, KV head)'s kept set within the band, the planted needle
    tokens (distinctive keys) all kept, and sampled compacted rows exact."""
    wl = configs.KEYDIFF_8K
    pr = synth.workload_problem(wl)
    c = pr.cache
    _, dst, ev = _evict(pr, wl.budget, wl.sink)
    got = ev.kept_positions()
    band = 0
    for b in range(c.B):
        for kvh in range(c.Hkv):
            keys = dense_keys_values(c, b, kvh)[0]
            band += check_kept(got[b][kvh], keys, wl.budget, wl.sink)
    for (b, kvh, p) in pr.needles:
        assert set(range(p * c.P, (p + 1) * c.P)) <= set(got[b][kvh].tolist())
    rng = np.random.default_rng(0)
    dk = dst.k.cpu().numpy()
    for _ in range(64):
        b, kvh, j = int(rng.integers(c.B)), int(rng.integers(c.Hkv)), int(rng.integers(wl.budget))
        p = got[b][kvh][j]
        src_row = c.k[c.block_table[b, p // c.P], kvh, p % c.P]
        np.testing.assert_array_equal(dk[j // c.P + b * dst.max_pages, kvh, j % c.P].view(src_row.dtype), src_row)
    print(f"full size: {band} candidates inside the band")


def test_full_size_carried_eviction():
    """The same layer as the steady state of a blockwise eviction: the first
    8192 positions of every (sequence, KV head) as an earlier eviction's copy
    left them (an identity copy writes their slot sums), the last 2048 the
    new block.  The carried selection's kept sets are within the band of the
    oracle on the whole cache (the needle tokens all kept); the count of
    positions that differ from the direct selection is reported."""
    wl = configs.KEYDIFF_8K
    pr = synth.workload_problem(wl)
    c = pr.cache
    src = DeviceCache.from_host(c)
    held = wl.budget
    # the copy that would have filled positions [0, held): identity kept lists into a scratch cache
    scratch = DeviceCache.empty(c.B, c.Hq, c.Hkv, c.hd, c.P, held, c.dtype)
    filler = KeyDiffEviction(src, scratch, held, 0, sums=True)
    filler.kept.copy_(torch.arange(held, dtype=torch.int32, device=filler.kept.device).expand_as(filler.kept))
    filler.count.fill_(held)
    filler.compact()
    dst = DeviceCache.empty(c.B, c.Hq, c.Hkv, c.hd, c.P, wl.budget, c.dtype)
    ev = KeyDiffEviction(src, dst, wl.budget, wl.sink, sums=True)
    ev.select(carried=filler.carried())
    ev.compact()
    direct = KeyDiffEviction(src, dst, wl.budget, wl.sink)
    direct.select()
    torch.cuda.synchronize()
    got, ref = ev.kept_positions(), direct.kept_positions()
    band, differ = 0, 0
    for b in range(c.B):
        for kvh in range(c.Hkv):
            keys = dense_keys_values(c, b, kvh)[0]
            band += check_kept(got[b][kvh], keys, wl.budget, wl.sink)
            differ += len(set(got[b][kvh].tolist()) ^ set(ref[b][kvh].tolist()))
    for (b, kvh, p) in pr.needles:
        assert set(range(p * c.P, (p + 1) * c.P)) <= set(got[b][kvh].tolist())
    print(f"full size, carried: {band} candidates inside the band; {differ} positions differ from the direct "
          f"selection (its mean rounds differently)")


@pytest.mark.parametrize("name", ["f32-hd64-p7", "bf16-hd64-short", "f32-hd128-one-evicted", "bf16-hd128-past-limit",
                                  "bf16-hd128-p1"])
def test_carried_sums_on_every_layout(name):
    """The copy's slot sums (every 64 destination slots: the sum of the keys
    copied there) on fp32 and bf16 caches of head dim 64 and 128, ragged
    counts included; then a second eviction of the evicted cache to 7/8 of
    the budget that carries those sums chooses within the band of the oracle
    on the keys that cache holds."""
    pr, budget, sink = _problem(name, seed=9)
    c = pr.cache
    src = DeviceCache.from_host(c)
    dst = DeviceCache.empty(c.B, c.Hq, c.Hkv, c.hd, c.P, budget, c.dtype)
    ev = KeyDiffEviction(src, dst, budget, sink, sums=True)
    ev.evict()
    torch.cuda.synchronize()
    got = ev.kept_positions()
    sums = ev.slot_sums.cpu().numpy()
    held = [[dense_keys_values(c, b, kvh)[0][got[b][kvh]] for kvh in range(c.Hkv)] for b in range(c.B)]
    for b in range(c.B):
        for kvh in range(c.Hkv):
            kk = held[b][kvh]
            for i in range(-(-len(kk) // 64)):
                grp = kk[64 * i: 64 * (i + 1)]
                tol = 1e-5 * np.abs(grp).sum(0) + 1e-6
                assert (np.abs(sums[b, kvh, i] - grp.sum(0)) <= tol).all(), (name, b, kvh, i)
    budget2 = max(sink, budget - max(1, budget // 8))  # (a small eviction keeps the past-limit case in range)
    dst2 = DeviceCache.empty(c.B, c.Hq, c.Hkv, c.hd, c.P, budget2, c.dtype)
    ev2 = KeyDiffEviction(dst, dst2, budget2, sink)
    ev2.select(carried=ev.carried())
    torch.cuda.synchronize()
    got2 = ev2.kept_positions()
    band = 0
    for b in range(c.B):
        for kvh in range(c.Hkv):
            band += check_kept(got2[b][kvh], held[b][kvh], budget2, sink)
    print(f"{name}: second eviction with carried sums, {band} candidates inside the band")
