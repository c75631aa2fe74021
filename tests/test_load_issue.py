"""Streaming kernels keep a round of their loads in flight together.

The KeyDiff sum and distance passes stream each wave's key rows with
16-byte loads, and the index assignment loads its key tiles and a round of
centres.  A load whose result feeds an address (a block-table entry)
between two such loads makes the compiler wait for every earlier load
before the next one, which leaves a wave one load in flight instead of a
round of them.  This compiles the kernels for gfx950 with the library's
flags (device code only, to assembly) and checks that each issues a whole
round of 16-byte loads with no wait on the vector memory counter between
them.  CPU only: hipcc cross-compiles.
"""
import os
import re
import shutil
import subprocess

import pytest

from block_sparse_long_page_amd import _build


def _kernel_bodies(asm: str) -> dict:
    bodies, name, lines = {}, None, []
    for line in asm.split("\n"):
        m = re.match(r"^(_Z[^:\s]+):", line)
        if m:
            name, lines = m.group(1), []
            continue
        if name is None:
            continue
        lines.append(line)
        if re.match(r"^\s+s_endpgm", line):
            bodies[name] = lines
            name = None
    return bodies


def _longest_run(lines, load_pattern: str) -> int:
    """Longest run of matching loads with no s_waitcnt on vmcnt between them."""
    best = run = 0
    for line in lines:
        if re.search(load_pattern, line):
            run += 1
            best = max(best, run)
        elif re.search(r"^\s+s_waitcnt.*vmcnt", line):
            run = 0
    return best


def _device_asm(tmp_path_factory, source: str) -> dict:
    if not os.path.exists(_build.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc is not installed")
    out = tmp_path_factory.mktemp("isa") / (os.path.splitext(source)[0] + ".s")
    cmd = [_build.HIPCC, *_build.FLAGS, "--cuda-device-only", "-S", os.path.join(_build.CSRC, source), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return _kernel_bodies(out.read_text())


@pytest.fixture(scope="module")
def keydiff_asm(tmp_path_factory):
    return _device_asm(tmp_path_factory, "keydiff.hip")


@pytest.fixture(scope="module")
def index_asm(tmp_path_factory):
    return _device_asm(tmp_path_factory, "index.hip")


# (kernel, head dim, bf16): row loads per lane in one round (a wave's 128 rows
# in one round of at most 32 loads for the sum, 16 per round for the distances)
CASES = [("k_kd_sum", 128, True, 32), ("k_kd_sum", 64, True, 16), ("k_kd_sum", 128, False, 32),
         ("k_kd_dist", 128, True, 16), ("k_kd_dist", 64, False, 16)]


@pytest.mark.parametrize("kernel,hd,bf,round_loads", CASES)
def test_row_loads_are_issued_together(keydiff_asm, kernel, hd, bf, round_loads):
    want = f"{kernel}ILi{hd}ELb{1 if bf else 0}E"
    names = [n for n in keydiff_asm if want in n]
    assert len(names) == 1, (want, list(keydiff_asm))
    run = _longest_run(keydiff_asm[names[0]], r"^\s+global_load_dwordx4")
    assert run >= round_loads, f"{kernel}<{hd}, {bf}>: at most {run} row loads in flight, {round_loads} expected"


@pytest.mark.parametrize("hd,loads", [(128, 16 + 8), (64, 8 + 4)])
def test_index_assignment_issues_keys_and_centres_together(index_asm, hd, loads):
    """Four key tiles of hd / 32 loads each, then the first round of centres
    (128 centres of hd bf16 over 256 threads), all in one run."""
    names = [n for n in index_asm if f"k_idx_assignILi{hd}E" in n]
    assert len(names) == 1, list(index_asm)
    run = _longest_run(index_asm[names[0]], r"^\s+global_load_dwordx4")
    assert run >= loads, f"k_idx_assign<{hd}>: at most {run} loads in flight, {loads} expected"
