"""The entry point that allocates nothing (sparse_attn_decode_step_static,
through the C ABI) against the existing entry points it combines
(sparse_attn_decode_step + sparse_attn_combine with caller buffers): the
same page lists, bitwise the same outputs and log-sum-exps, and the oracle's
attention over them, on two calls in a row, the second with a smaller
input (the static scratch keeps the first call's contents).  A shape whose
workspace and partials exceed the scratch is refused before any launch."""
import numpy as np
import pytest

import oracle
from block_sparse_long_page_amd import synth
from parity import check_lse, check_output, check_selection

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from block_sparse_long_page_amd import binding as B  # noqa: E402
from block_sparse_long_page_amd.device import DeviceCache, SparseDecoder, to_device  # noqa: E402

SHAPES = [
    # first call: the larger input; second: fewer sequences, heads, pages and splits
    dict(B=2, Hq=16, Hkv=2, hd=128, P=64, seq_lens=[6000, 4100], sink=64, window=512, budget=1024, splits=6),
    dict(B=1, Hq=8, Hkv=1, hd=128, P=64, seq_lens=[2500], sink=64, window=256, budget=512, splits=3),
]


def _static_step(dec, q, pr, out, lse, sel, cnt):
    B.sparse_attn_decode_step_static(dec.desc, q, 1, dec.meta, pr.mode, pr.sink, pr.window, pr.budget, 0.0,
                                     dec.splits, sel, cnt, out, dec.out_dtype, lse)


def test_static_step_matches_the_step_with_caller_buffers():
    for i, shape in enumerate(SHAPES):
        kw = dict(shape)
        splits = kw.pop("splits")
        pr = synth.random_problem(**kw, mode="quest", dtype="bf16", seed=40 + i, shuffle=True, clusters=8,
                                  needles_per_head=1)
        print(f"static step, call {i}: {shape}", flush=True)
        dc = DeviceCache.from_host(pr.cache)
        dec = SparseDecoder(dc, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget, splits=splits)
        q = to_device(pr.q)
        dec.build_meta()
        dec.fused_step(q)  # the existing entry points, caller buffers
        out = torch.full_like(dec.out, 7)
        lse = torch.full_like(dec.lse, 7.0)
        sel = torch.full_like(dec.sel, -7)
        cnt = torch.full_like(dec.count, -7)
        _static_step(dec, q, pr, out, lse, sel, cnt)
        torch.cuda.synchronize()
        assert torch.equal(cnt, dec.count)
        k = dec.k_max
        assert torch.equal(sel[..., :k], dec.sel[..., :k])
        assert torch.equal(out, dec.out) and torch.equal(lse, dec.lse)
        # and the oracle on the same lists
        s_np, c_np = sel.cpu().numpy()[..., :k], cnt.cpu().numpy()
        r = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget,
                       want_scores=True)
        check_selection(s_np, c_np, r.scores, k)
        ref = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget,
                         sel=s_np, cnt=c_np)
        o = (out.cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        check_output(o.reshape(ref.out.shape), ref.out, pr.cache.dtype, f"static call {i}")
        check_lse(lse.cpu().numpy().reshape(ref.lse.shape), ref.lse, f"static call {i}")
        del dec, dc
        torch.cuda.empty_cache()


def test_static_step_refuses_shapes_past_its_scratch():
    pr = synth.random_problem(B=1, Hq=8, Hkv=1, hd=128, P=64, seq_lens=[1024], sink=64, window=256, budget=256,
                              mode="quest", dtype="bf16", seed=3)
    dc = DeviceCache.from_host(pr.cache)
    dec = SparseDecoder(dc, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget, splits=64)
    q = to_device(pr.q)
    dec.build_meta()
    # 8 rows x 64 splits of partials fit; 1024 rows x 64 splits (34 MB) do not
    big = synth.random_problem(B=16, Hq=64, Hkv=8, hd=128, P=64, seq_lens=[1024] * 16, sink=64, window=256,
                               budget=256, mode="quest", dtype="bf16", seed=3)
    bdc = DeviceCache.from_host(big.cache)
    bdec = SparseDecoder(bdc, mode=big.mode, Q=1, sink=big.sink, window=big.window, budget=big.budget, splits=64)
    with pytest.raises(B.SparseAttnError) as err:
        _static_step(bdec, to_device(big.q), big, bdec.out, bdec.lse, bdec.sel, bdec.count)
    assert err.value.status == B.SA_ERR_SCRATCH
    _static_step(dec, q, pr, dec.out, dec.lse, dec.sel, dec.count)
    torch.cuda.synchronize()
    assert np.isfinite(dec.out_f32()).all()
