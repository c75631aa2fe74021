"""Builds libsparse_attn.so in-tree with hipcc for gfx950 (runs on a machine
without a GPU: hipcc cross-compiles)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsparse_attn.so")
# load-only reference kernels the benchmark times beside the path (not part of it)
PROBE_LIB = os.path.join(PKG, "libsa_probe.so")
PROBE_SOURCE = "probe.hip"
SOURCES = ["page_meta.hip", "select.hip", "decode.hip", "group.hip", "index.hip", "prefill.hip", "keydiff.hip",
           "combine.hip", "noalloc.hip", "sparse_attn.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions: scalar fp32 only (the host pass warns about the unknown feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(PKG, os.pardir, "include"),
]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(extra=(), jobs: int = 0) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), SOURCES))
    _link(objs, LIB)
    _link([_compile(PROBE_SOURCE, list(extra))], PROBE_LIB)
    return LIB


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build())
