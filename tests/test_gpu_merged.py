"""The decode kernels that merge their split partials in their own last
workgroup (sparse_attn_decode_merged, sparse_attn_decode_step_merged): out
and lse bitwise those of the same kernels followed by the combine kernel,
the fp64 oracle's attention over the GPU's page lists, the counters left
zero, repeated calls, both paths of the selecting step, and lengths
advanced once per sequence after the whole launch."""
import numpy as np
import pytest

import oracle
from parity import check_lse, check_output

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from block_sparse_long_page_amd import binding as B  # noqa: E402
from block_sparse_long_page_amd.device import DeviceCache, SparseDecoder, to_device  # noqa: E402
from test_gpu_kernels import CASES, _problem  # noqa: E402

BF16_CASES = [n for n, c in CASES.items() if c["dtype"] == "bf16"]


def _decoder(name, splits, out_dtype, mode="quest", seed=3):
    pr = _problem(name, mode, seed=seed)
    dc = DeviceCache.from_host(pr.cache)
    dec = SparseDecoder(dc, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget, splits=splits,
                        out_dtype=out_dtype)
    q = to_device(pr.q)
    dec.build_meta()
    return pr, dc, dec, q


def _poison(dec):
    # bf16 outputs are held as their 16-bit patterns: 0x7fc0 is a NaN
    dec.out.fill_(0x7FC0 if dec.out_dtype == B.SA_BF16 else float("nan"))
    dec.lse.fill_(float("nan"))


@pytest.mark.parametrize("name", BF16_CASES)
@pytest.mark.parametrize("splits", [1, 5, 16, 64])
@pytest.mark.parametrize("out_dtype", [B.SA_BF16, B.SA_F32])
def test_decode_merged_equals_decode_and_combine(name, splits, out_dtype):
    pr, dc, dec, q = _decoder(name, splits, out_dtype)
    dec.select(q)
    dec.decode(q)
    dec.combine()
    torch.cuda.synchronize()
    out_ref, lse_ref = dec.out.clone(), dec.lse.clone()
    for _ in range(2):  # the counters return to zero: a second call merges the same way
        _poison(dec)
        dec.decode_merged(q)
        torch.cuda.synchronize()
        assert torch.equal(dec.out, out_ref) and torch.equal(dec.lse, lse_ref), name
        assert int(dec.counters.abs().sum()) == 0
    sel, cnt = dec.selection()
    ref = oracle.run(pr.cache, pr.q, mode=pr.mode, Q=pr.Q, sink=pr.sink, window=pr.window, budget=pr.budget,
                     sel=sel, cnt=cnt)
    # the bf16 cache's arithmetic sets the tolerance, whatever the output dtype
    check_output(dec.out_f32(), ref.out, pr.cache.dtype, name)
    check_lse(dec.lse_f32(), ref.lse, name)


@pytest.mark.parametrize("name", BF16_CASES)
@pytest.mark.parametrize("splits", [None, 3])
def test_step_merged_equals_step_and_combine(name, splits):
    """Both paths of the selecting step (the select-and-decode kernel, or
    the separate selection and the merging decode) give the two-call
    results bit for bit."""
    pr, dc, dec, q = _decoder(name, splits, None, seed=5)
    dec.fused_step(q)
    torch.cuda.synchronize()
    out_ref, lse_ref = dec.out.clone(), dec.lse.clone()
    sel_ref, cnt_ref = dec.selection()
    path = B.sparse_attn_step_path(dec.desc, pr.sink, pr.window, pr.budget, dec.splits, dec.ws)
    for _ in range(2):
        _poison(dec)
        dec.sel.fill_(-7)
        dec.select_decode_merged(q)
        torch.cuda.synchronize()
        sel, cnt = dec.selection()
        np.testing.assert_array_equal(cnt, cnt_ref)
        np.testing.assert_array_equal(sel, sel_ref)
        assert torch.equal(dec.out, out_ref) and torch.equal(dec.lse, lse_ref), f"{name} path {path}"


def test_step_merged_takes_both_paths():
    """The cases above cover the fused and the separate path."""
    paths = set()
    for name in BF16_CASES:
        pr, dc, dec, q = _decoder(name, None, None)
        paths.add(B.sparse_attn_step_path(dec.desc, pr.sink, pr.window, pr.budget, dec.splits, dec.ws))
        paths.add(B.sparse_attn_step_path(dec.desc, pr.sink, pr.window, pr.budget, 3, dec.ws))
    assert paths == {B.SA_STEP_FUSED, B.SA_STEP_SEPARATE}


@pytest.mark.parametrize("name", ["bf16-hd128-g8-p64", "bf16-hd128-g8-q5"])
def test_merged_decode_advances_the_lengths_once(name):
    """advance = 2: every sequence's length grows by exactly 2 after the
    launch, and each launch attends the lengths it started with (the same as
    decode + combine_advance, step after step)."""
    pr, dc, dec, q = _decoder(name, 7, None)
    dec.select(q)
    torch.cuda.synchronize()
    L0 = dc.seq_lens.clone()
    outs = []
    for _ in range(3):
        dec.decode_merged(q, advance=2)
        torch.cuda.synchronize()
        outs.append((dec.out.clone(), dec.lse.clone(), dc.seq_lens.clone()))
    assert torch.equal(outs[-1][2], L0 + 6)
    assert int(dec.counters.abs().sum()) == 0
    dc.seq_lens.copy_(L0)
    for o, l, lens in outs:
        dec.decode(q)
        dec.combine(advance=2)
        torch.cuda.synchronize()
        assert torch.equal(dec.out, o) and torch.equal(dec.lse, l) and torch.equal(dc.seq_lens, lens)
