"""Benchmark: one decode step of block/page-sparse attention on one MI355X.

A step is the whole per-token hot path on one batch: page selection (scores
+ per-KV-head top-k), split-K decode over sink + window + selected pages,
and the log-sum-exp combine.  The workload is the Llama-3-70B-shaped layer
at 128k context with GQA-8 (batch 4, 64 q / 8 KV heads, head dim 128, bf16,
page 64, sink 256, window 4096, budget L/16 = 8192 tokens, Quest min/max
scores, keys from 64 Gaussian clusters), on seeded synthetic inputs already
resident in HBM.

To keep the 256 MB last-level cache from serving repeated reads, the timed
steps rotate over R copies of the cache and of its summaries (distinct
physical pages, the same contents; R = 10 by default, so the copies' summaries
alone exceed the cache), so each step reads data no recent step touched.

Prints one JSON line: selected-KV GB/s (algorithmic bytes / step time),
us/step, the roofline of the decode kernel (HIP-event time of its launches
inside the timed region) and the fp64 CPU oracle timed on the host cores.

    python bench.py [--steps K] [--warmup W] [--replicas R] [--splits S]
                    [--no-cpu-baseline] [--copy-probe]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
CSRC = os.path.join(ROOT, "block_sparse_long_page_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--replicas", type=int, default=0,
                    help="copies of the cache rotated over the steps (0: the workload's default, 10 for the "
                         "headline step, 6 for the eviction, 3 for the semantic chunk)")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--local-splits", type=int, default=0, help="splits of the sink+window decode")
    ap.add_argument("--middle-splits", type=int, default=0, help="splits of the selected-pages decode")
    ap.add_argument("--separate", action="store_true",
                    help="select, decode and combine as three launches instead of the fused select-and-decode step")
    ap.add_argument("--merge", action="store_true",
                    help="llama3-70b-layer-128k / hybrid-3layer-256k: the decode kernel merges its partials in its "
                         "own last workgroups (sparse_attn_decode_step_merged, sparse_attn_decode_merged) instead of "
                         "the separate combine kernel")
    ap.add_argument("--overlap", action="store_true",
                    help="decode sink + window on a second stream beside the selection, then the selected pages")
    ap.add_argument("--dense-steps", type=int, default=10)
    ap.add_argument("--eager", action="store_true",
                    help="hybrid-3layer-256k: launch every step's kernels one by one instead of replaying graphs")
    ap.add_argument("--direct", action="store_true",
                    help="keydiff-llama3.1-8b-8k: sum every held key for the mean instead of carrying the held "
                         "tokens' key sums from the copy that filled the cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe", action="store_true", help="only run a plain device copy of 1 GiB (calibration)")
    ap.add_argument("--traffic-from", default="",
                    help="no GPU: write the HBM traffic record from the rocprofv3 counter runs under this folder "
                         "(prof_fetch, prof_write: the bench under --pmc FETCH_SIZE / WRITE_SIZE, its JSON line in "
                         "fetch.out; prof_cfetch, prof_cwrite: the same counters over --copy-probe)")
    ap.add_argument("--only-timed", action="store_true",
                    help="run only the warmup and the timed region (for profiler runs)")
    ap.add_argument("--token-splits", type=int, default=0,
                    help="semantic-512k: token chunks per page; semantic-prefill-64k: per block (0: default)")
    ap.add_argument("--iterations", type=int, default=8, help="semantic-512k-index: k-means iterations")
    ap.add_argument("--k-max", type=int, default=10, help="semantic-prefill-64k: most blocks a row takes")
    ap.add_argument("--chunks-per-call", type=int, default=16,
                    help="semantic-prefill-64k: consecutive chunks per sparse_attn_prefill_chunks call (1: one "
                         "sparse_attn_prefill_chunk call per chunk)")
    ap.add_argument("--score", default="quest", choices=["quest", "mean", "centroid", "compressed"],
                    help="llama3-70b-layer-128k: page summary and score (compressed: mean keys of two-page "
                         "blocks with a one-page stride)")
    ap.add_argument("--workload", default="llama3-70b-layer-128k",
                    choices=["llama3-70b-layer-128k", "semantic-512k", "semantic-512k-index", "hybrid-3layer-256k",
                             "keydiff-llama3.1-8b-8k", "semantic-prefill-64k"],
                    help="semantic-512k: the 64-row chunk decoded by page (selection, grouped decode, combine); "
                         "semantic-512k-index: the same chunk over a semantic block index built from keys "
                         "interleaved in position order (index build, then block choice, grouped decode of the "
                         "blocks, combine); "
                         "hybrid-3layer-256k: the 128-step schedule of three layers (one token appended every step, "
                         "selection every 32 steps after summarising the pages appended since the last one, "
                         "growing window between); "
                         "keydiff-llama3.1-8b-8k: KeyDiff eviction of a cache of 10240 tokens back to 8192 "
                         "(distances to the mean key, top-k, compaction of the kept K/V rows); "
                         "semantic-prefill-64k: chunked sparse prefill of a 64K prompt over one block index")
    return ap.parse_args()


def oracle_seconds(fn, seconds: float, max_calls: int = 200):
    """Median seconds per call of an oracle call `fn`, repeated until
    `seconds` have passed (at least once); returns (median, calls)."""
    times = []
    t_end = time.time() + seconds
    while not times or time.time() < t_end:
        t1 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t1)
        if len(times) >= max_calls:
            break
    return statistics.median(times), len(times)


def roofline_record(kernel: str, bytes_per_launch: int, launch_ms: float) -> dict:
    """HBM roofline of one launch (or one call of several kernels) from its
    algorithmic bytes and its average duration (HIP events around
    back-to-back launches on their stream)."""
    gbs = bytes_per_launch / (launch_ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBPS, 4), "traffic": None, "bytes_per_launch": int(bytes_per_launch),
            "avg_launch_us": round(launch_ms * 1e3, 2)}


def cpu_model() -> str:
    """The host CPU's model name (for the oracle's record)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


class Probes:
    """The load-only reference kernels of libsa_probe.so (block_sparse_long_page_amd/csrc/probe.hip):
    the attended K/V pages of a step read in the decode's tile pattern, and a contiguous read."""

    def __init__(self):
        import ctypes

        import torch

        path = os.path.join(ROOT, "block_sparse_long_page_amd", "libsa_probe.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with __graft_entry__.build()")
        self.lib = ctypes.CDLL(path)
        P, I = ctypes.c_void_p, ctypes.c_int
        self.lib.sa_probe_pages.restype = I
        self.lib.sa_probe_pages.argtypes = [P, P, P, P, I, I, I, I, I, P, P]
        self.lib.sa_probe_stream.restype = I
        self.lib.sa_probe_stream.argtypes = [P, ctypes.c_size_t, I, P, P]
        self.out = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")

    def pages(self, pool, slabs, offsets, problems, splits):
        import torch

        rc = self.lib.sa_probe_pages(pool.k.data_ptr(), pool.v.data_ptr(), slabs.data_ptr(), offsets.data_ptr(),
                                     problems, splits, pool.P, pool.hd, 2, self.out.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
        assert rc == 0, f"sa_probe_pages: {rc}"

    def stream(self, buf, workgroups):
        import torch

        rc = self.lib.sa_probe_stream(buf.data_ptr(), buf.numel() * buf.element_size(), workgroups,
                                      self.out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert rc == 0, f"sa_probe_stream: {rc}"


def attended_slabs(table, P, Hkv, L, S, W, sel, cnt):
    """Per (sequence, KV head) the physical page slabs a decode step attends
    (sink pages, window pages, selected pages; each once), as a flat int32
    list with offsets: the input of the load-only page probe."""
    import numpy as np

    B_ = table.shape[0]
    slabs, offsets = [], [0]
    n_pages = -(-L // P)
    for b in range(B_):
        for h in range(Hkv):
            pages = set(range(0, -(-min(S, L) // P)))
            pages |= set(range(max(0, L - W) // P, n_pages))
            pages |= set(int(x) for x in sel[b, h, 0, :cnt[b, h, 0]])
            slabs.extend(int(table[b, p]) * Hkv + h for p in sorted(pages))
            offsets.append(len(slabs))
    return np.asarray(slabs, dtype=np.int32), np.asarray(offsets, dtype=np.int32)


def percentiles(ms_list):
    """Median, p10 and p90 in microseconds of durations given in milliseconds."""
    import numpy as np

    a = np.asarray(ms_list, dtype=np.float64) * 1e3
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2)}


def copy_probe():
    import torch

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(10):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / 10
    print(json.dumps({"copy_bytes": n, "ms": ms, "GBps_read_plus_write": 2 * n / ms / 1e6}))


def kernel_sources_sha256() -> str:
    """Digest of every kernel source (the .hip and .hpp files of the library)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp")):
            h.update(name.encode())
            h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()


def traffic_record(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    runs (FETCH_SIZE and WRITE_SIZE scaled by a plain copy's readings), or
    None when a kernel source changed since they were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    if rec.get("kernel_sources_sha256") != kernel_sources_sha256() or rec.get("kernel") != kernel:
        return None
    return rec.get("bytes_per_launch")


def counter_means(folder: str) -> dict:
    """Mean Counter_Value per dispatch of every kernel (by its k_* name) in
    the rocprofv3 counter-collection CSV under `folder`."""
    import csv
    import glob
    import re

    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    tot, n = {}, {}
    for f in files:
        for row in csv.DictReader(open(f)):
            m = re.search(r"\b(k_\w+)", row["Kernel_Name"])
            k = m.group(1) if m else row["Kernel_Name"]
            tot[k] = tot.get(k, 0.0) + float(row["Counter_Value"])
            n[k] = n.get(k, 0) + 1
    return {k: tot[k] / n[k] for k in tot}


def write_traffic_record(folder: str):
    """The committed traffic record: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) of the step's kernels, each scaled by what the same counter
    reads for a 1 GiB device copy (1 GiB read, 1 GiB written), keyed to the
    kernel sources' digest."""
    lines = [ln for ln in open(os.path.join(folder, "fetch.out")) if ln.startswith("{")]
    line = json.loads(lines[-1])
    kernel = line["roofline"]["kernel"]
    copy_kib = (1 << 30) / 1024
    cf = counter_means(os.path.join(folder, "prof_cfetch"))
    cw = counter_means(os.path.join(folder, "prof_cwrite"))
    # the copy is the only kernel of the probe run with a 1 GiB-scale reading
    fetch_copy, write_copy = max(cf.values()), max(cw.values())
    fs, ws = copy_kib / fetch_copy, copy_kib / write_copy
    fetch = counter_means(os.path.join(folder, "prof_fetch"))
    write = counter_means(os.path.join(folder, "prof_write"))
    per = {}
    print(f"| counter | copy reading (KiB / dispatch) | scale |\n|---|---|---|\n"
          f"| FETCH_SIZE | {fetch_copy:.1f} | {fs:.4f} |\n| WRITE_SIZE | {write_copy:.1f} | {ws:.4f} |\n")
    print("| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) | written MB (scaled) |\n|---|---|---|---|---|")
    for k in sorted(fetch, key=lambda k: -fetch[k]):
        if not k.startswith("k_"):
            continue
        rd, wr = int(fetch[k] * 1024 * fs), int(write.get(k, 0.0) * 1024 * ws)
        per[k] = {"read": rd, "written": wr}
        print(f"| `{k}` | {fetch[k]:.1f} | {write.get(k, 0.0):.1f} | {rd / 1e6:.2f} | {wr / 1e6:.2f} |")
    parts = [k.strip() for k in kernel.split("+")]
    total = sum(per[k]["read"] + per[k]["written"] for k in parts)
    rec = {"kernel": kernel, "workload": line["config"]["workload"], "kernel_sources_sha256": kernel_sources_sha256(),
           "bytes_per_launch": total, "fetch_scale": round(fs, 6), "write_scale": round(ws, 6),
           "per_kernel_bytes": per, "algorithmic_bytes_per_launch": line["roofline"]["bytes_per_launch"]}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    alg = rec["algorithmic_bytes_per_launch"]
    print(f"\n{kernel}: {total / 1e6:.2f} MB of HBM traffic against {alg / 1e6:.2f} MB algorithmic: "
          f"ratio {total / alg:.3f}")


def replicate(pool, c, R):
    """R copies of the cache in one physical-page pool and the block table of
    each copy (so repeated steps do not find their pages in the last-level
    cache)."""
    import numpy as np
    import torch

    from block_sparse_long_page_amd.device import to_device

    if R > 1:
        k_all = torch.empty((R * c.num_phys,) + tuple(pool.k.shape[1:]), dtype=pool.k.dtype, device="cuda")
        v_all = torch.empty_like(k_all)
        for r in range(R):
            k_all[r * c.num_phys:(r + 1) * c.num_phys].copy_(pool.k)
            v_all[r * c.num_phys:(r + 1) * c.num_phys].copy_(pool.v)
        pool.k, pool.v, pool.num_phys = k_all, v_all, R * c.num_phys
    tables = []
    for r in range(R):
        bt = c.block_table.astype(np.int64)
        tables.append(to_device(np.where(bt >= 0, bt + r * c.num_phys, -1).astype(np.int32)))
    return tables


def bench_semantic(args):
    """The semantic-block chunk (64 query rows, 2048-token blocks, 16 blocks
    per row at 512K context): selection, the decode grouped by page and the
    combine, against the per-row decode of the same lists."""
    import numpy as np
    import torch

    from block_sparse_long_page_amd import accounting, binding as B, configs, synth
    from block_sparse_long_page_amd.device import DeviceCache, GroupedStep, SparseDecoder, to_device

    wl = configs.SEMANTIC_512K
    t0 = time.time()
    pr = synth.workload_problem(wl)
    c = pr.cache
    log(f"inputs {time.time() - t0:.1f}s")
    R = max(1, min(args.replicas or 3, 3))  # 2 GiB of K+V per copy
    pool = DeviceCache.from_host(c)
    tables = replicate(pool, c, R)
    q = to_device(pr.q)
    Q = pr.Q
    dec = SparseDecoder(pool, mode=pr.mode, Q=Q, sink=pr.sink, window=pr.window, budget=pr.budget,
                        splits=args.splits or None)
    gs = GroupedStep(dec, token_splits=args.token_splits or None)
    descs = [pool.desc(block_table=t) for t in tables]
    metas = [dec.meta] + [pool.new_meta(pr.mode) for _ in range(R - 1)]
    for d, m in zip(descs, metas):
        B.sparse_attn_build_page_meta(d, pr.mode, 0, pool.max_pages, m)
    torch.cuda.synchronize()

    def select(r):
        B.sparse_attn_select(descs[r], q, Q, metas[r], pr.mode, pr.sink, pr.window, pr.budget, dec.sel, dec.count,
                             dec.ws, dec.ws_bytes)

    def step_grouped(r):
        select(r)
        B.sparse_attn_decode_grouped(descs[r], q, Q, dec.sel, dec.count, dec.k_max, pr.sink, pr.window, 0.0, gs.ts,
                                     gs.ls, gs.part_o, gs.part_ml, gs.ws, gs.ws_bytes)
        gs.combine()

    def step_rows(r):
        select(r)
        B.sparse_attn_decode(descs[r], q, Q, dec.sel, dec.count, dec.k_max, pr.sink, pr.window, B.SA_PART_ALL, 0.0,
                             dec.splits, 0, dec.part_o, dec.part_ml)
        dec.combine()

    K = args.steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(step, n):
        for i in range(args.warmup):
            step(i % R)
        torch.cuda.synchronize()
        start.record()
        for i in range(n):
            step(i % R)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / n

    ms = timed(step_grouped, K)
    ms_rows = float("nan") if args.only_timed else timed(step_rows, max(1, K // 5))

    def decode_grouped(r):  # the dominant call alone, on the last step's lists
        B.sparse_attn_decode_grouped(descs[r], q, Q, dec.sel, dec.count, dec.k_max, pr.sink, pr.window, 0.0, gs.ts,
                                     gs.ls, gs.part_o, gs.part_ml, gs.ws, gs.ws_bytes)

    dec_ms = timed(decode_grouped, K)

    # bytes: the union of the rows' pages per (sequence, KV head), read once
    sel, cnt = dec.selection()
    L = int(c.seq_lens[0])
    se, ws = accounting.regions(L, pr.sink, pr.window)
    union_tok = union_pages = list_pages = 0
    flops = 0
    for b in range(c.B):
        for h in range(c.Hkv):
            rows_of = {}
            for i in range(Q):
                for p in sel[b, h, i, : cnt[b, h, i]]:
                    rows_of.setdefault(int(p), []).append(i)
            list_pages += int(cnt[b, h].sum())
            union_pages += len(rows_of)
            for p, rows in rows_of.items():
                n = max(0, min((p + 1) * c.P, ws) - max(p * c.P, se))
                union_tok += n
                flops += 4 * n * c.hd * len(rows) * (c.Hq // c.Hkv)
    local_tok = c.B * c.Hkv * (se + (L - ws))
    flops += 4 * local_tok * c.hd * Q * (c.Hq // c.Hkv)  # an upper bound: rows attend causal parts of the window
    n_cand = accounting.candidate_pages(L, c.P, pr.sink, pr.window)
    sb = accounting.grouped_step_bytes(B=c.B, Hq=c.Hq, Hkv=c.Hkv, hd=c.hd, elem_bytes=2, Q=Q, n_cand=n_cand,
                                       k_max=dec.k_max, mode=pr.mode, union_tokens=union_tok,
                                       local_tokens=local_tok, stride=gs.stride)
    gbs = sb.total / (ms * 1e-3) / 1e9
    # the grouped call reads the page lists, q and the K/V of the unions and
    # of the windows once, and writes the partials
    dec_bytes = sb.kv + sb.q + sb.partials // 2 + c.B * c.Hkv * Q * (dec.k_max + 1) * 4
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        oracle.build(force=False)
        med, calls = oracle_seconds(lambda: oracle.run(c, pr.q, mode=pr.mode, Q=Q, sink=pr.sink, window=pr.window,
                                                       budget=pr.budget), args.cpu_seconds)
        cpu = {"value": round(sb.total / med / 1e9, 3), "unit": "GB/s", "cores": oracle.max_threads(),
               "kind": "oracle", "sample": f"the full 64-row step (centroids of every page, scores, top-k, "
                                           f"attention) in fp64, {calls} run(s); median {med * 1e3:.0f} ms/step",
               "ms_per_step": round(med * 1e3, 1)}
    print(json.dumps({
        "metric": "selected-KV GB/s (% of HBM peak) + us/decode step, 512K ctx semantic blocks, 64-row chunk",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "us_per_step": round(ms * 1e3, 2), "pct_hbm_peak": round(100 * gbs / 8000, 1),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded): 256 vMF clusters of 2048 keys per (b, kvh), V N(0,1), rows around 4 topics",
        "config": {"workload": wl.name, "batch": c.B, "q_heads": c.Hq, "kv_heads": c.Hkv, "head_dim": c.hd,
                   "context": L, "page": c.P, "rows": Q, "budget": pr.budget, "window": pr.window,
                   "score": "centroid", "replicas": R, "token_splits": gs.ts, "local_splits": gs.ls,
                   "step": "select + grouped decode + combine"},
        "union_pages": union_pages, "listed_pages": list_pages,
        "mfma_tflops": round(flops / (ms * 1e-3) / 1e12, 1), "flops_per_step": flops,
        "per_row_us_per_step": None if ms_rows != ms_rows else round(ms_rows * 1e3, 2),
        "speedup_vs_per_row": None if ms_rows != ms_rows else round(ms_rows / ms, 2),
        "bytes_per_step": sb.as_dict(),
        "roofline": roofline_record("sparse_attn_decode_grouped (k_group_plan + k_group_decode_mfma + k_decode_mfma)",
                                    dec_bytes, dec_ms),
        "cpu_baseline": cpu,
    }))


def bench_semantic_index(args):
    """The semantic-block chunk at 512K with keys interleaved in position
    order: the block index is built (spherical k-means, block layout of K and
    V), then each step chooses the rows' blocks under the L/16 token budget,
    decodes the union of the chosen blocks once per (sequence, KV head) plus
    the 64-token window, and combines."""
    import numpy as np
    import torch

    from block_sparse_long_page_amd import configs, synth
    from block_sparse_long_page_amd.device import BlockIndex, DeviceCache, to_device

    wl = configs.SEMANTIC_512K
    t0 = time.time()
    pr = synth.semantic_problem(wl, scatter=True)
    c = pr.cache
    log(f"inputs {time.time() - t0:.1f}s")
    L = int(c.seq_lens[0])
    N = L - pr.window
    C = N // 2048
    dc = DeviceCache.from_host(c)
    q = to_device(pr.q)
    ix = BlockIndex(dc, N, C, Q=pr.Q, window=pr.window, budget=pr.budget, k_max=64)
    nbk, hd, it = c.B * c.Hkv, c.hd, args.iterations
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    ix.build(it)
    torch.cuda.synchronize()
    nb = 3
    start.record()
    for _ in range(nb):
        ix.build(it)
    stop.record()
    torch.cuda.synchronize()
    build_ms = start.elapsed_time(stop) / nb
    # bytes the build must move: keys once for the lengths, twice per
    # iteration (assignment, centre update), once for the final assignment,
    # keys and values read and written by the layout copy
    row = hd * 2
    build_bytes = nbk * N * row * (1 + 2 * it + 1 + 4)
    build_flops = 2 * nbk * N * C * hd * (it + 1)

    for _ in range(args.warmup):
        ix.step(q)
    torch.cuda.synchronize()
    K = args.steps
    start.record()
    for _ in range(K):
        ix.step(q)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / K
    # the block decode alone (plan + grouped decode of the blocks + window), on the last step's lists
    start.record()
    for _ in range(K):
        ix.decode(q)
    stop.record()
    torch.cuda.synchronize()
    dec_ms = start.elapsed_time(stop) / K

    sel, cnt = ix.sel.cpu().numpy(), ix.count.cpu().numpy()
    off = ix.offsets.cpu().numpy()
    sizes = np.diff(off, axis=-1)
    union_tok = union_blocks = listed = 0
    for b in range(c.B):
        for h in range(c.Hkv):
            u = set()
            for i in range(pr.Q):
                u.update(int(x) for x in sel[b, h, i, :cnt[b, h, i]])
            listed += int(cnt[b, h].sum())
            union_blocks += len(u)
            union_tok += int(sum(sizes[b, h, x] for x in u))
    Q = pr.Q
    local_tok = nbk * pr.window
    # partials: a used slot (a listed block's chunk or the window's split)
    # holds o and (m, l) for every head, an unused one only (m, l)
    used = (c.Hq // c.Hkv) * (listed * ix.ts + nbk * Q * ix.ls)
    partial_bytes = (used * (hd + 2) + (c.B * c.Hq * Q * ix.stride - used) * 2) * 4
    step_bytes = (union_tok * row * 2 + local_tok * row * 2 + nbk * C * (hd * 4 + 4) + c.B * c.Hq * Q * hd * 2 * 2
                  + 2 * partial_bytes)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    dec_bytes = union_tok * row * 2 + local_tok * row * 2 + c.B * c.Hq * Q * hd * 2 + partial_bytes \
        + nbk * Q * (ix.k_max + 1) * 4
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's block choice and attention for the 64 rows of one
        # (sequence, KV head), over the index the GPU built (fp64 numpy, one thread)
        from threadpoolctl import threadpool_limits

        from oracle import semantic as sem

        cent = ix.centres.cpu().numpy().astype(np.float64)[0, 0]
        perm0, off0 = ix.positions.cpu().numpy()[0, 0], ix.offsets.cpu().numpy()[0, 0]
        n_pages = -(-L // c.P)
        Kf = synth.to_f32(c.k[c.block_table[0, :n_pages], 0], c.dtype).reshape(-1, hd)[:L].astype(np.float64)
        Vf = synth.to_f32(c.v[c.block_table[0, :n_pages], 0], c.dtype).reshape(-1, hd)[:L].astype(np.float64)
        G = c.Hq // c.Hkv
        qf = synth.to_f32(pr.q[0, :G], c.dtype).astype(np.float64)  # [G][Q][hd]

        def rows():
            for i in range(Q):
                blocks = sem.select_blocks(sem.block_scores(qf[:, i], cent), sizes[0, 0], pr.budget, ix.k_max)
                toks = np.concatenate([perm0[off0[x]:off0[x + 1]] for x in blocks] + [np.arange(N, L - Q + i + 1)])
                for h in range(G):
                    sem.attend(qf[h, i], Kf[toks], Vf[toks], 1.0 / np.sqrt(hd))

        with threadpool_limits(1):
            med, calls = oracle_seconds(rows, args.cpu_seconds)
        cpu = {"value": round(step_bytes / nbk / med / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"(sequence 0, KV head 0): block choice and attention of its {Q} rows over the GPU-built "
                         f"index in fp64 numpy, {calls} run(s), median {med * 1e3:.0f} ms, scaled by the "
                         f"{nbk} (sequence, KV head) pairs of the step's bytes"}
    print(json.dumps({
        "metric": "selected-KV GB/s (% of HBM peak) + us/decode step, 512K ctx semantic block index, 64-row chunk",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "us_per_step": round(ms * 1e3, 2), "pct_hbm_peak": round(100 * gbs / 8000, 1),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded): 256 vMF clusters of 2048 keys per (b, kvh) interleaved in position order, "
                "V N(0,1), rows around 4 topics",
        "config": {"workload": "semantic-512k-index", "batch": c.B, "q_heads": c.Hq, "kv_heads": c.Hkv,
                   "head_dim": hd, "context": L, "indexed_tokens": N, "blocks": C, "iterations": it, "rows": Q,
                   "budget": pr.budget, "window": pr.window, "k_max": ix.k_max,
                   "step": "block choice + grouped decode of the blocks + combine"},
        "build_ms": round(build_ms, 3), "build_GBps": round(build_bytes / (build_ms * 1e-3) / 1e9, 1),
        "build_tflops": round(build_flops / (build_ms * 1e-3) / 1e12, 1),
        "block_tokens": {"min": int(sizes.min()), "mean": float(sizes.mean()), "max": int(sizes.max()),
                         "empty": int((sizes == 0).sum())},
        "union_blocks": union_blocks, "listed_blocks": listed, "bytes_per_step": step_bytes,
        "roofline": roofline_record("sparse_attn_decode_blocks (k_group_plan + k_group_decode_mfma + k_decode_mfma)",
                                    dec_bytes, dec_ms),
        "cpu_baseline": cpu,
    }))


def bench_keydiff(args):
    """KeyDiff eviction of a Llama-3.1-8B-shaped layer (batch 8, 32 q / 8 KV
    heads, bf16) whose cache holds an 8192-token budget plus one 2048-token
    block: each step ranks every token of every (sequence, KV head) by the
    distance of its key to the mean key, keeps the sink and the farthest
    tokens up to the budget, and copies the kept K and V rows into the
    evicted cache.  By default the step is the steady state of a blockwise
    eviction: the first 8192 positions are what the previous eviction's copy
    left, with the key sums of their slots (written untimed, by an identity
    copy, before timing), so the mean sums only the new block's keys; the
    step's copy writes the sums the next eviction would carry.  --direct sums
    every held key instead."""
    import torch

    from block_sparse_long_page_amd import binding as B, configs, synth
    from block_sparse_long_page_amd.device import DeviceCache, KeyDiffEviction

    wl = configs.KEYDIFF_8K
    t0 = time.time()
    pr = synth.workload_problem(wl)
    c = pr.cache
    log(f"inputs {time.time() - t0:.1f}s")
    R = max(1, args.replicas or 6)
    pool = DeviceCache.from_host(c)
    tables = replicate(pool, c, R)
    dst = DeviceCache.empty(c.B, c.Hq, c.Hkv, c.hd, c.P, wl.budget, c.dtype)
    carried = not args.direct
    evs, carry = [], []
    for r in range(R):
        ev = KeyDiffEviction(pool, dst, wl.budget, wl.sink, sums=carried)
        ev.src_desc = pool.desc(tables[r])
        evs.append(ev)
        if carried:  # the copy that left positions [0, budget) of this replica (untimed)
            filler = KeyDiffEviction(pool, dst, wl.budget, 0, sums=True)
            filler.src_desc = pool.desc(tables[r])
            filler.kept.copy_(torch.arange(wl.budget, dtype=torch.int32, device=filler.kept.device)
                              .expand_as(filler.kept))
            filler.count.fill_(wl.budget)
            B.sparse_attn_keydiff_compact_sums(filler.src_desc, filler.kept, filler.count, wl.budget,
                                               filler.dst_desc, filler.slot_sums)
            carry.append(filler.carried())
    torch.cuda.synchronize()

    def select(r):
        evs[r].select(carried=carry[r] if carried else None)

    def compact(r):
        if carried:
            B.sparse_attn_keydiff_compact_sums(evs[r].src_desc, evs[r].kept, evs[r].count, wl.budget,
                                               evs[r].dst_desc, evs[r].slot_sums)
        else:
            B.sparse_attn_keydiff_compact(evs[r].src_desc, evs[r].kept, evs[r].count, wl.budget, evs[r].dst_desc)

    def step(r):
        select(r)
        compact(r)

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, K):
        torch.cuda.synchronize()
        start.record()
        for i in range(K):
            fn(i % R)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / K

    for i in range(args.warmup):
        step(i % R)
    K = args.steps
    ms = timed(step, K)
    sel_ms = timed(select, K)
    comp_ms = timed(compact, K)

    nbk, L, row = c.B * c.Hkv, int(c.seq_lens[0]), c.hd * 2
    kept_n = min(L, wl.budget)
    nch = -(-pool.max_seq_len // 512)  # chunks of 512 tokens
    # keys once, the chunk sums written and read once, the distances' order
    # keys written and read, kept positions written; the copy reads the kept
    # positions and the kept K and V rows and writes the rows
    sel_bytes = nbk * (L * row + nch * c.hd * 4 * 2 + L * 4 * 2 + wl.budget * 4)
    comp_bytes = nbk * (kept_n * 4 + kept_n * row * 2 * 2)
    if carried:  # the carried slot sums read, the next ones written
        groups = B.sparse_attn_keydiff_slot_groups(wl.budget)
        sel_bytes += nbk * groups * c.hd * 4
        comp_bytes += nbk * groups * c.hd * 4
    step_bytes = sel_bytes + comp_bytes
    gbs = step_bytes / (ms * 1e-3) / 1e9
    comp_gbs = comp_bytes / (comp_ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's eviction (distances, kept set) and the copy of the kept
        # rows for (sequence, KV head) pairs in turn (fp64 numpy, one thread)
        import numpy as np
        from threadpoolctl import threadpool_limits

        from oracle import keydiff as kd

        n_pages = -(-L // c.P)
        pairs = [(b, h) for b in range(c.B) for h in range(c.Hkv)][:8]
        kv = [(synth.to_f32(c.k[c.block_table[b, :n_pages], h], c.dtype).reshape(-1, c.hd)[:L].astype(np.float64),
               synth.to_f32(c.v[c.block_table[b, :n_pages], h], c.dtype).reshape(-1, c.hd)[:L].astype(np.float64))
              for b, h in pairs]

        def evict_pairs():
            for Kf, Vf in kv:
                kept = kd.keep(Kf, wl.budget, wl.sink)
                _ = (Kf[kept], Vf[kept])  # the copy into the evicted cache

        with threadpool_limits(1):
            med, calls = oracle_seconds(evict_pairs, args.cpu_seconds)
        cpu = {"value": round(step_bytes * len(pairs) / nbk / med / 1e9, 3), "unit": "GB/s", "cores": 1,
               "kind": "oracle", "sample": f"{len(pairs)} of the {nbk} (sequence, KV head) pairs evicted in fp64 "
                                           f"numpy, {calls} run(s), median {med * 1e3:.0f} ms, against their share "
                                           f"of the step's bytes"}
    print(json.dumps({
        "metric": "evicted-cache GB/s + us per eviction, 10240 -> 8192 tokens, Llama-3.1-8B-shaped layer",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "us_per_step": round(ms * 1e3, 2), "pct_hbm_peak": round(100 * gbs / 8000, 1),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded): K from 64 Gaussian clusters with 4 needle pages per (b, kvh), V N(0,1)",
        "config": {"workload": wl.name, "batch": c.B, "q_heads": c.Hq, "kv_heads": c.Hkv, "head_dim": c.hd,
                   "cache_tokens": L, "budget": wl.budget, "block": wl.block, "sink": wl.sink, "page": c.P,
                   "replicas": R, "carried_sums": carried,
                   "step": ("keydiff select with the held tokens' key sums carried (the new block summed, distances, "
                            "top-k) + compaction writing the next sums") if carried else
                           "keydiff select (sums, distances, top-k) + compaction"},
        "roofline": {"bound": "hbm", "kernel": "k_kd_compact", "achieved": round(comp_gbs, 1), "peak": 8000.0,
                     "unit": "GB/s", "frac": round(comp_gbs / 8000.0, 4), "traffic": None,
                     "bytes_per_launch": comp_bytes, "avg_launch_us": round(comp_ms * 1e3, 2)},
        "select_us": round(sel_ms * 1e3, 2), "select_GBps": round(sel_bytes / (sel_ms * 1e-3) / 1e9, 1),
        "bytes_per_step": step_bytes,
        "cpu_baseline": cpu,
    }))


def bench_prefill(args):
    """Chunked sparse prefill of a 64K-token prompt (batch 2, 16 q / 4 KV
    heads, keys of 32 semantic clusters interleaved in position order): one
    block index of the whole prompt is built, then the prompt's rows are
    processed 128 at a time, one sparse_attn_prefill_chunk call (three
    launches) per chunk; each chunk sees the index only before its own
    tokens, chooses blocks per row under a budget of 1/16 of its length,
    reads each chosen block once for all its rows and attends its own tokens
    causally.  The same chunks with every visible block chosen (dense over
    the prefix, same kernels, no index build) are timed beside it, unless
    --only-timed."""
    import numpy as np
    import torch

    from block_sparse_long_page_amd import configs, synth
    from block_sparse_long_page_amd.device import BlockIndex, ChunkedPrefill, DeviceCache, to_device

    wl = configs.SEMANTIC_PREFILL_64K
    t0 = time.time()
    pr = synth.semantic_problem(wl, scatter=True, blocks=(wl.context - wl.q_rows) // 2048)
    q_all = synth.prefill_queries(pr, seed=wl.seed)
    c = pr.cache
    L = int(c.seq_lens[0])
    T, W = wl.q_rows, wl.window
    nch = L // T
    C = L // 2048
    log(f"inputs {time.time() - t0:.1f}s")
    dc = DeviceCache.from_host(c)
    # chunk-major queries: chunk j is the contiguous [B][Hq][T][hd] block j
    q_dev = to_device(q_all).view(c.B, c.Hq, nch, T, c.hd).permute(2, 0, 1, 3, 4).contiguous()
    q0 = np.ascontiguousarray(q_all[0, :c.Hq // c.Hkv])  # sequence 0's first group, for the CPU baseline
    del q_all
    ix = BlockIndex(dc, L, C, Q=T, window=W, budget=0, k_max=C)
    # at most 10 blocks per row (the budget, 1/16 of at most 65664 tokens,
    # holds about 2 blocks of the average 2048 tokens; rows that reach the cap
    # are counted below).  With one chunk per call each block is read in 3
    # token chunks so that the few blocks a chunk reads spread over the GPU;
    # with several chunks per call they fill it already, and one token chunk
    # per block keeps the partials (written, then read by the combine) few.
    # The dense run takes every block.
    per = max(1, args.chunks_per_call)
    ts = args.token_splits or (3 if per == 1 else 1)
    pf = ChunkedPrefill(ix, T, W, k_max=min(C, args.k_max), token_splits=ts, per_call=per)
    pf_dense = ChunkedPrefill(ix, T, W, k_max=C, token_splits=1, per_call=per)
    # one call per chunk, for the byte count's pass (its lists are the same bit for bit)
    pf1 = pf if per == 1 else ChunkedPrefill(ix, T, W, k_max=pf.k_max, token_splits=pf.ts)
    # the calls: consecutive chunks, their rows contiguous ([B][Hq][n * T][hd])
    calls = []
    for j0 in range(0, nch, per):
        n = min(per, nch - j0)
        qg = q_dev[j0:j0 + n].permute(1, 2, 0, 3, 4).contiguous().view(c.B, c.Hq, n * T, c.hd)
        calls.append((j0, qg, [max(1, (j + 1) * T // 16) for j in range(j0, j0 + n)]))
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        torch.cuda.synchronize()
        start.record()
        fn()
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop)

    def window_slots(Lc):
        """Partial slots of the window the chunk's rows use (length Lc): the
        window pages' token chunks a row sees (each page of [Lc - W, Lc) is
        split into token_splits chunks), or one per row (per-row decode)."""
        if not pf.fused:
            return T * pf.ls
        n = 0
        a = max(0, Lc - W)
        for p in range(a // c.P, (Lc - 1) // c.P + 1):
            a0, a1 = max(p * c.P, a), min((p + 1) * c.P, Lc)
            csz = -(-(a1 - a0) // pf.ts)
            for s in range(pf.ts):
                t0 = a0 + min(a1 - a0, s * csz)
                if min(a1, t0 + csz) > t0:  # rows at or after t0 see the chunk
                    n += max(0, min(T, Lc - t0))
        return n

    def build():
        ix.build(args.iterations)

    def chunks(dense):
        for j0, qg, budgets in calls:
            if per == 1:
                (pf_dense if dense else pf).chunk(q_dev[j0], j0 * T, 10**9 if dense else budgets[0])
            elif dense:
                pf_dense.chunks(qg, j0 * T, [10**9] * len(budgets))
            else:
                pf.chunks(qg, j0 * T, budgets)

    build()
    chunks(False)
    if not args.only_timed:
        chunks(True)
    build_ms = timed(build)
    sparse_ms = timed(lambda: chunks(False))
    dense_ms = float("nan") if args.only_timed else timed(lambda: chunks(True))
    total_ms = build_ms + sparse_ms
    toks = c.B * L

    # algorithmic bytes of the sparse chunks (an untimed pass that reads each
    # chunk's lists back): the visible K/V of the union of the rows' blocks
    # and of the window, once per (sequence, KV head), q, the page lists, the
    # partials written and read, the output
    nbk, row, G = c.B * c.Hkv, c.hd * 2, c.Hq // c.Hkv
    chunk_bytes = 0
    at_cap = 0
    for j in range(nch):
        pf1.chunk(q_dev[j], j * T, max(1, (j + 1) * T // 16))
        sel, cnt = pf1.sel.cpu().numpy(), pf1.count.cpu().numpy()
        at_cap += int((cnt == pf.k_max).sum())
        ends, off = pf1.ends.cpu().numpy(), ix.offsets.cpu().numpy()
        vis_tok = 0
        for b in range(c.B):
            for h in range(c.Hkv):
                u = set()
                for i in range(T):
                    u.update(int(x) for x in sel[b, h, i, :cnt[b, h, i]])
                vis_tok += sum(int(ends[b, h, x] - off[b, h, x]) for x in u)
        win = min(W, (j + 1) * T)
        # a used slot (a listed block's token chunk, or a window chunk the row
        # sees) holds o and (m, l) for every head, an unused one only (m, l);
        # written, then read by the combine
        used = G * (int(cnt.sum()) * pf.ts + nbk * window_slots(j * T + T))
        partials = 2 * (used * (c.hd + 2) + (c.B * c.Hq * T * pf.stride - used) * 2) * 4
        chunk_bytes += ((vis_tok + nbk * win) * row * 2 + c.B * c.Hq * T * c.hd * 2 * 2
                        + nbk * T * (pf.k_max + 1) * 4 + partials + nbk * C * 4)
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's prefill of one (sequence, KV head): its index (spherical
        # k-means of the whole prompt, layout) once, and chunks spread over the
        # prompt; the whole prompt's time is projected from their average
        from threadpoolctl import threadpool_limits

        from oracle import semantic as sem

        n_pages = -(-L // c.P)
        Kf = synth.to_f32(c.k[c.block_table[0, :n_pages], 0], c.dtype).reshape(-1, c.hd)[:L].astype(np.float64)
        Vf = synth.to_f32(c.v[c.block_table[0, :n_pages], 0], c.dtype).reshape(-1, c.hd)[:L].astype(np.float64)
        qf = synth.to_f32(q0, c.dtype).astype(np.float64).transpose(1, 0, 2)  # [L][G][hd]
        with threadpool_limits(1):
            t1 = time.perf_counter()
            mu, a, _ = sem.spherical_kmeans(Kf, C, args.iterations)
            perm, offs = sem.block_layout(a, C)
            t_index = time.perf_counter() - t1
            picks = np.linspace(0, nch - 1, 9).astype(int)
            times = []
            t_end = time.time() + args.cpu_seconds
            for j in picks:
                t1 = time.perf_counter()
                sem.prefill_chunk(Kf, Vf, qf[j * T:(j + 1) * T], mu, perm, offs, j * T, W, max(1, (j + 1) * T // 16),
                                  pf.k_max, 1.0 / np.sqrt(c.hd))
                times.append(time.perf_counter() - t1)
                if time.time() > t_end:
                    break
        per_pair = t_index + nch * float(np.mean(times))
        cpu = {"value": round(toks / (nbk * per_pair), 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"(sequence 0, KV head 0): the index ({t_index:.2f} s) and {len(times)} chunks spread over "
                         f"the prompt (mean {1e3 * float(np.mean(times)):.0f} ms) in fp64 numpy; the prompt's "
                         f"{nch} chunks and {nbk} (sequence, KV head) pairs projected from them"}
    print(json.dumps({
        "metric": "prefill tokens/s, 64K prompt, semantic block index, 128-row chunks",
        "value": round(toks / (total_ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": 1,
        "warmup": 1, "ms_per_step": round(total_ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded): 32 vMF clusters of 2048 keys per (b, kvh) interleaved in position order, "
                "V N(0,1), query rows around 4 topics per (b, kvh)",
        "config": {"workload": wl.name, "batch": c.B, "q_heads": c.Hq, "kv_heads": c.Hkv, "head_dim": c.hd,
                   "prompt": L, "chunk": T, "window": W, "blocks": C, "iterations": args.iterations,
                   "k_max": pf.k_max, "token_splits": pf.ts, "chunks_per_call": per,
                   "budget": "1/16 of the chunk's length"},
        "index_build_ms": round(build_ms, 3), "sparse_chunks_ms": round(sparse_ms, 3),
        "dense_chunks_ms": None if args.only_timed else round(dense_ms, 3),
        "speedup_vs_dense": None if args.only_timed else round(dense_ms / total_ms, 2),
        "us_per_chunk": round(sparse_ms * 1e3 / nch, 2),
        "bytes_sparse_chunks": chunk_bytes, "rows_at_k_max": at_cap,
        "roofline": roofline_record("every launch of the sparse chunks (the front: visible ends, block choice and "
                                    "slot table; the grouped decode of the blocks and the window's pages; the "
                                    "combine)", chunk_bytes, sparse_ms),
        "cpu_baseline": cpu,
    }))


def bench_hybrid(args):
    """The hybrid model's three full-attention layers at 256k over 128 decode
    steps: every step appends a token to every sequence; steps 0, 32, 64, 96
    summarise the pages appended since the previous selection and select and
    decode with the top-k inside the decode kernel, the others decode the
    kept pages with the window grown by the steps since the selection; then
    the combine, whose last launch of a step also advances the sequences'
    lengths (the next step's token appended), so a step is only library
    launches.  By default every refresh cycle (a selecting step and the 31
    decode steps after it) is captured as a HIP graph before the timed
    region, which then replays the four graphs; --eager launches the kernels
    one by one.  Reports the average per layer-step over the schedule."""
    import torch

    from block_sparse_long_page_amd import accounting, configs, synth
    from block_sparse_long_page_amd.device import DeviceCache, SparseDecoder, to_device

    wl = configs.HYBRID_256K
    t0 = time.time()
    hs = synth.hybrid_schedule(wl)
    L0, T, RF = hs.context, hs.steps, hs.refresh
    log(f"inputs {time.time() - t0:.1f}s")
    layers = []
    seq_lens = None  # the layers of one model share the sequences' lengths
    for li in range(len(hs.caches)):
        cache = hs.caches[li]
        cache.seq_lens[:] = L0
        dc = DeviceCache.from_host(cache, max_seq_len=L0 + T)
        if seq_lens is None:
            seq_lens = dc.seq_lens
        dc.seq_lens = seq_lens
        dec = SparseDecoder(dc, mode=hs.mode, Q=1, sink=hs.sink, window=hs.windows[li], budget=hs.budgets[li],
                            splits=args.splits or None)
        dec.build_meta()
        layers.append((dc, dec, hs.windows[li], [to_device(hs.q[li][t]) for t in range(T)]))
    torch.cuda.synchronize()
    P = layers[0][0].P

    merge = args.merge  # the decode kernels merge their partials (no combine launch)

    def reset():
        seq_lens.fill_(L0)
        for dc, dec, W, qs in layers:
            dec.build_meta((L0 - 1) // P, dc.max_pages)

    def issue(t):
        """The launches of step t (the lengths read L0 + t when it starts).
        The summaries are read only when selecting, so the pages appended
        since the last selection are summarised right before the next one
        (the same summaries as folding each token in as it arrives)."""
        t_ref = t - t % RF
        L = L0 + t
        for li, (dc, dec, W, qs) in enumerate(layers):
            adv = 1 if li == len(layers) - 1 else 0
            if t == t_ref:
                if t > 0:
                    first = (L0 + t_ref - RF - 1) // P  # the page that held the last token at the previous selection
                    dec.build_meta(first, (L - 1) // P + 1)
                if merge:
                    dec.select_decode_merged(qs[t], advance=adv)
                else:
                    dec.select_decode(qs[t])
            elif merge:
                dec.decode_merged(qs[t], window=W + (t - t_ref), advance=adv)
            else:
                dec.decode(qs[t], window=W + (t - t_ref))
            if not merge:
                dec.combine(advance=adv)

    # one graph per refresh cycle: its selecting step and the decode steps until the next
    graphs = None
    if not args.eager:
        graphs = []
        reset()
        torch.cuda.synchronize()
        for t0 in range(0, T, RF):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for t in range(t0, min(T, t0 + RF)):
                    issue(t)
            graphs.append(g)
        torch.cuda.synchronize()

    def schedule(steps):
        if graphs is None:
            for t in range(steps):
                issue(t)
        else:
            for c in range(-(-steps // RF)):
                graphs[c].replay()

    reset()
    schedule(min(args.warmup, T))
    torch.cuda.synchronize()
    reset()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    schedule(T)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop)
    assert int(seq_lens[0]) == L0 + T  # every step appended its token

    # the dominant call alone: layer 0's decode of its kept pages one step
    # after a selection (window grown by one), back to back
    dc0, dec0, W0, qs0 = layers[0]
    reset()
    dec0.select_decode(qs0[0])
    seq_lens.fill_(L0 + 1)
    torch.cuda.synchronize()
    K = 50
    start.record()
    for _ in range(K):
        if merge:
            dec0.decode_merged(qs0[1], window=W0 + 1)
        else:
            dec0.decode(qs0[1], window=W0 + 1)
    stop.record()
    torch.cuda.synchronize()
    dec_ms = start.elapsed_time(stop) / K
    sel0, cnt0 = dec0.selection()
    ntok = sum(accounting.attended_tokens_exact(L0 + 1, P, hs.sink, W0 + 1, sel0[b, h, 0, :cnt0[b, h, 0]])
               for b in range(dc0.B) for h in range(dc0.Hkv))
    dec_bytes = accounting.decode_kernel_bytes(B=dc0.B, Hq=dc0.Hq, Hkv=dc0.Hkv, hd=dc0.hd, elem_bytes=2,
                                               ntok_total=ntok, splits=dec0.splits, sel_entries=int(cnt0.sum()))
    if merge:  # the merge in the last workgroups: the partials read back, out and lse written
        dec_bytes += dec0.rows * (dec0.splits * (dc0.hd + 2) * 4 + dc0.hd * 2 + 4)

    # algorithmic bytes of the schedule
    total = 0
    c0 = layers[0][0]
    for dc, dec, W, qs in layers:
        t_ref = 0
        for t in range(T):
            L = L0 + t
            if t % RF == 0:
                t_ref = t
            w_eff = W + (t - t_ref)
            sb = accounting.decode_step_bytes(B=dc.B, Hq=dc.Hq, Hkv=dc.Hkv, hd=dc.hd, elem_bytes=2, L=L, P=P,
                                              S=hs.sink, W=w_eff, budget=dec.budget, mode=0, splits=dec.splits)
            step = sb.total if t == t_ref else sb.total - sb.meta  # summaries are read when selecting
            if t == t_ref and t > 0:  # the pages appended since the last selection summarised
                pages = (L - 1) // P - (L0 + t - RF - 1) // P + 1
                step += dc.B * dc.Hkv * pages * (P * dc.hd * 2 + 2 * dc.hd * 2)
            total += step

    cpu = None
    if not args.no_cpu_baseline:
        # the oracle runs the same schedule: all 128 steps of the three layers
        # (a selection at every refresh, the window grown between refreshes)
        import oracle

        oracle.build(force=False)
        del layers, graphs
        torch.cuda.empty_cache()
        t_start = time.perf_counter()
        n_sel = 0
        for li, host in enumerate(hs.caches):
            W, budget = hs.windows[li], hs.budgets[li]
            sel_ref = cnt_ref = None
            t_ref = 0
            for t in range(T):
                host.seq_lens[:] = L0 + t
                if t % RF == 0:
                    t_ref = t
                    r = oracle.run(host, hs.q[li][t], mode=hs.mode, Q=1, sink=hs.sink, window=W, budget=budget)
                    sel_ref, cnt_ref = r.sel, r.cnt
                    n_sel += 1
                else:
                    oracle.run(host, hs.q[li][t], mode=hs.mode, Q=1, sink=hs.sink, window=W + (t - t_ref),
                               budget=budget, sel=sel_ref, cnt=cnt_ref)
        sec = time.perf_counter() - t_start
        cpu = {"value": round(total / sec / 1e9, 3), "unit": "GB/s", "cores": oracle.max_threads(),
               "cpu_model": cpu_model(), "kind": "oracle",
               "sample": f"the whole schedule in fp64: 128 steps of the three layers ({n_sel} selecting "
                         f"layer-steps with summaries of every page), against the schedule's algorithmic bytes; "
                         f"{sec:.2f} s in all, {1e3 * sec / T:.1f} ms per step",
               "ms_per_step": round(1e3 * sec / T, 2)}

    n = T * len(hs.caches)
    gbs = total / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "selected-KV GB/s (% of HBM peak) + us/decode step, hybrid 3-layer 256k, average over 128 steps",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": T, "warmup": min(args.warmup, T),
        "ms_per_step": round(ms / T, 5), "us_per_step": round(1e3 * ms / T, 2),
        "us_per_layer_step": round(1e3 * ms / n, 2), "pct_hbm_peak": round(100 * gbs / 8000, 1),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded): K, V, q N(0,1); one token appended per step and layer",
        "config": {"workload": wl.name, "batch": c0.B, "q_heads": c0.Hq, "kv_heads": c0.Hkv, "head_dim": c0.hd,
                   "context": L0, "page": P, "sink": hs.sink, "layers": [
                       {"window": W, "budget": b_, "splits": s_} for W, b_, s_ in
                       zip(hs.windows, hs.budgets, [dec0.splits] * len(hs.windows))],
                   "refresh": RF, "launch": "eager" if args.eager else "a HIP graph per refresh cycle, captured beforehand",
                   "step": ("summary refresh + (select-and-decode | decode) per layer, each decode kernel merging "
                            "its partials in its last workgroups; the last layer's advances the lengths") if merge else
                           ("summary refresh + (select-and-decode | decode) + combine per layer; the last combine "
                            "advances the lengths")},
        "bytes_per_schedule": total,
        "roofline": roofline_record("k_decode_mfma (kept pages, first layer, one step after a selection"
                                    + (", merging its partials)" if merge else ")"), dec_bytes, dec_ms),
        "cpu_baseline": cpu,
    }))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path has no collectives; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.traffic_from:
        write_traffic_record(args.traffic_from)
        return

    import numpy as np
    import torch

    if args.copy_probe:
        copy_probe()
        return

    if args.workload == "semantic-512k":
        bench_semantic(args)
        return
    if args.workload == "hybrid-3layer-256k":
        bench_hybrid(args)
        return
    if args.workload == "semantic-512k-index":
        bench_semantic_index(args)
        return
    if args.workload == "keydiff-llama3.1-8b-8k":
        bench_keydiff(args)
        return
    if args.workload == "semantic-prefill-64k":
        bench_prefill(args)
        return

    from block_sparse_long_page_amd import accounting, binding as B, configs, synth
    from block_sparse_long_page_amd.device import DeviceCache, OverlappedStep, SparseDecoder, to_device

    wl = configs.LLAMA3_70B.scaled(mode=args.score)
    t0 = time.time()
    pr = synth.workload_problem(wl)
    c = pr.cache
    log(f"inputs {time.time() - t0:.1f}s")

    # R copies of the cache in one physical-page pool; replica r's table points at its own pages.
    # Ten copies: the K/V a step reads (205 MB) and the summaries (33 MB per
    # copy, 330 MB in all) both exceed the 256 MB last-level cache, so no step
    # finds the data of a recent one there.
    R = max(1, args.replicas or 10)
    pool = DeviceCache.from_host(c)
    tables = replicate(pool, c, R)
    q = to_device(pr.q)

    dec = SparseDecoder(pool, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget,
                        splits=args.splits or None)
    descs = [pool.desc(block_table=t) for t in tables]
    metas = [dec.meta] + [pool.new_meta(pr.mode) for _ in range(R - 1)]  # summaries per replica
    for d, m in zip(descs, metas):
        B.sparse_attn_build_page_meta(d, pr.mode, 0, pool.max_pages, m)
    torch.cuda.synchronize()

    ov = OverlappedStep(dec, local_splits=args.local_splits or None, middle_splits=args.middle_splits or None)

    def step_sequential(r, ev=None):
        d = descs[r]
        B.sparse_attn_select(d, q, 1, metas[r], pr.mode, pr.sink, pr.window, pr.budget, dec.sel, dec.count,
                             dec.ws, dec.ws_bytes)
        if ev is not None:
            ev[0].record()
        B.sparse_attn_decode(d, q, 1, dec.sel, dec.count, dec.k_max, pr.sink, pr.window, B.SA_PART_ALL, 0.0,
                             dec.splits, 0, dec.part_o, dec.part_ml)
        if ev is not None:
            ev[1].record()
        B.sparse_attn_combine(dec.rows, c.hd, dec.splits, dec.part_o, dec.part_ml, dec.out, dec.out_dtype,
                              dec.lse)

    def step_overlapped(r, ev=None):
        ov.step(q, desc=descs[r], meta=metas[r], middle_events=ev)

    def select_decode(r):
        B.sparse_attn_decode_step(descs[r], q, 1, metas[r], pr.mode, pr.sink, pr.window, pr.budget, 0.0, dec.splits,
                                  dec.sel, dec.count, dec.ws, dec.ws_bytes, dec.part_o, dec.part_ml)

    def step_fused(r, ev=None):
        select_decode(r)
        B.sparse_attn_combine(dec.rows, c.hd, dec.splits, dec.part_o, dec.part_ml, dec.out, dec.out_dtype,
                              dec.lse)

    def select_decode_merged(r):
        B.sparse_attn_decode_step_merged(descs[r], q, 1, metas[r], pr.mode, pr.sink, pr.window, pr.budget, 0.0,
                                         dec.splits, dec.sel, dec.count, dec.ws, dec.ws_bytes, dec.part_o,
                                         dec.part_ml, dec.out, dec.out_dtype, dec.lse, 0)

    def step_merged(r, ev=None):
        select_decode_merged(r)

    mode = ("overlap" if args.overlap else "separate" if args.separate else "fused+merge" if args.merge
            else "fused")
    step = {"overlap": step_overlapped, "separate": step_sequential, "fused": step_fused,
            "fused+merge": step_merged}[mode]

    for i in range(args.warmup):
        step(i % R)
    torch.cuda.synchronize()
    sel, cnt = dec.selection()

    # algorithmic bytes of one step and of one decode launch
    L = int(c.seq_lens[0])
    attended = [accounting.attended_tokens_exact(L, c.P, pr.sink, pr.window, sel[b, h, 0, : cnt[b, h, 0]])
                for b in range(c.B) for h in range(c.Hkv)]
    sb = accounting.decode_step_bytes(B=c.B, Hq=c.Hq, Hkv=c.Hkv, hd=c.hd, elem_bytes=2, L=L, P=c.P, S=pr.sink,
                                      W=pr.window, budget=pr.budget, mode=pr.mode, splits=dec.splits,
                                      attended=attended)
    n_cand = accounting.candidate_pages(L, c.P, pr.sink, pr.window)
    if mode in ("fused", "fused+merge"):
        # the launch pair of sparse_attn_decode_step: page scores, then top-k + decode (+ the merge of the
        # partials in the decode kernel's last workgroups: the partials read back, out and lse written)
        dec_kernel = ("k_score_quest_mfma" if pr.mode == B.SA_QUEST else "k_score") + " + k_select_decode_mfma"
        dec_bytes = accounting.select_decode_bytes(B=c.B, Hq=c.Hq, Hkv=c.Hkv, hd=c.hd, elem_bytes=2,
                                                   ntok_total=sum(attended), splits=dec.splits, meta=sb.meta,
                                                   n_cand=n_cand, k_max=dec.k_max)
        if mode == "fused+merge":
            dec_bytes += dec.rows * (dec.splits * (c.hd + 2) * 4 + c.hd * 2 + 4)
    elif mode == "separate":
        # one decode launch over sink + window + selected pages
        dec_kernel = "k_decode_mfma"
        dec_bytes = accounting.decode_kernel_bytes(B=c.B, Hq=c.Hq, Hkv=c.Hkv, hd=c.hd, elem_bytes=2,
                                                   ntok_total=sum(attended), splits=dec.splits,
                                                   sel_entries=int(cnt.sum()))
    else:
        # the timed launch is the selected pages' decode; sink + window run beside the selection
        local = accounting.attended_tokens_exact(L, c.P, pr.sink, pr.window, [])
        dec_kernel = "k_decode_mfma (selected pages)"
        dec_bytes = accounting.decode_kernel_bytes(B=c.B, Hq=c.Hq, Hkv=c.Hkv, hd=c.hd, elem_bytes=2,
                                                   ntok_total=sum(attended) - local * c.B * c.Hkv, splits=ov.sm,
                                                   sel_entries=int(cnt.sum()))

    # timed region: K steps back to back
    K = args.steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        step(i % R)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / K

    # the dominant launch(es) alone: K calls back to back on the stream they run
    # on, between two HIP events (an event record between kernels would add a
    # few microseconds to each), rotating over the replicas like the steps
    if mode == "fused":
        def launch(r):
            select_decode(r)
    elif mode == "fused+merge":
        def launch(r):
            select_decode_merged(r)
    elif mode == "separate":
        def launch(r):
            B.sparse_attn_decode(descs[r], q, 1, dec.sel, dec.count, dec.k_max, pr.sink, pr.window, B.SA_PART_ALL,
                                 0.0, dec.splits, 0, dec.part_o, dec.part_ml)
    else:
        def launch(r):
            ov.decode_middle(q, descs[r], pr.window)
    for i in range(3):
        launch(i % R)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        launch(i % R)
    stop.record()
    torch.cuda.synchronize()
    dec_avg_ms = start.elapsed_time(stop) / K

    # per-step distribution: one event between consecutive steps (each
    # difference is a step plus one event record)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(K):
        step(i % R)
        evs[i + 1].record()
    torch.cuda.synchronize()
    step_dist = percentiles([evs[i].elapsed_time(evs[i + 1]) for i in range(K)])
    step_dist["method"] = f"{K} steps, an event between consecutive steps, replicas rotated"

    # load-only references on the same box: the step's attended K/V pages in
    # the decode's tile pattern and launch shape, and a contiguous read
    probes = Probes()
    slab_lists = []
    for r in range(R):
        s_np, o_np = attended_slabs(tables[r].cpu().numpy(), c.P, c.Hkv, L, pr.sink, pr.window, sel, cnt)
        slab_lists.append((torch.from_numpy(s_np).cuda(), torch.from_numpy(o_np).cuda()))
    probe_bytes = int(len(s_np)) * 2 * c.P * c.hd * 2
    for i in range(3):
        probes.pages(pool, *slab_lists[i % R], c.B * c.Hkv, dec.splits)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        probes.pages(pool, *slab_lists[i % R], c.B * c.Hkv, dec.splits)
    stop.record()
    torch.cuda.synchronize()
    probe_ms = start.elapsed_time(stop) / K
    sbuf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    sbuf.fill_(1)
    for i in range(2):
        probes.stream(sbuf, 256 * 16)
    torch.cuda.synchronize()
    start.record()
    for i in range(5):
        probes.stream(sbuf, 256 * 16)
    stop.record()
    torch.cuda.synchronize()
    stream_ms = start.elapsed_time(stop) / 5
    del sbuf
    probe_gbps = probe_bytes / (probe_ms * 1e-3) / 1e9
    stream_ref = {"kernel": "k_probe_pages", "what": "load-only read of the step's attended K/V pages in 16-token "
                                                     "tiles, the decode's launch shape, replicas rotated",
                  "bytes": probe_bytes, "us": round(probe_ms * 1e3, 2), "GBps": round(probe_gbps, 1),
                  "contiguous_read_GBps": round((1 << 30) / (stream_ms * 1e-3) / 1e9, 1)}

    ms_hot = dense_ms = float('nan')
    if not args.only_timed:
        # one replica (repeated reads may hit the last-level cache)
        torch.cuda.synchronize()
        start.record()
        for i in range(K):
            step(0)
        stop.record()
        torch.cuda.synchronize()
        ms_hot = start.elapsed_time(stop) / K

        # dense decode of the same cache: every page, same kernels, no selection
        ddec = SparseDecoder(pool, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pool.max_pages * c.P)
        for i in range(2):
            ddec.desc = descs[i % R]
            ddec.decode(q, dense=True)
            ddec.combine()
        torch.cuda.synchronize()
        start.record()
        for i in range(args.dense_steps):
            ddec.desc = descs[i % R]
            ddec.decode(q, dense=True)
            ddec.combine()
        stop.record()
        torch.cuda.synchronize()
        dense_ms = start.elapsed_time(stop) / args.dense_steps

    gbps = sb.total / (ms * 1e-3) / 1e9
    dec_gbps = dec_bytes / (dec_avg_ms * 1e-3) / 1e9

    cpu = None
    accuracy = None
    if not args.no_cpu_baseline:
        import numpy as np

        import oracle

        oracle.build(force=False)
        times = []
        own = None
        t_end = time.time() + args.cpu_seconds
        while len(times) < 3 or time.time() < t_end:
            t1 = time.perf_counter()
            own = oracle.run(c, pr.q, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget)
            times.append(time.perf_counter() - t1)
            if len(times) >= 200:
                break
        med = statistics.median(times)
        cpu = {"value": round(sb.total / med / 1e9, 3), "unit": "GB/s", "cores": oracle.max_threads(),
               "kind": "oracle", "sample": f"the full step (summaries of all pages, scores, top-k, attention) "
                                           f"in fp64, repeated {len(times)} times; median {med * 1e3:.1f} ms/step",
               "ms_per_step": round(med * 1e3, 2), "cpu_model": cpu_model()}
        if mode != "overlap":
            # The step's accuracy, outside the timed region: one step on the
            # first copy (the host cache's own block table), its output
            # against the oracle attending the same page lists in fp64, and
            # its page lists against the oracle's own selection.
            step(0)
            torch.cuda.synchronize()
            gsel, gcnt = dec.selection()
            ref = oracle.run(c, pr.q, mode=pr.mode, Q=1, sink=pr.sink, window=pr.window, budget=pr.budget,
                             sel=gsel, cnt=gcnt)
            err = float(np.abs(dec.out_f32().astype(np.float64) - ref.out).max())
            accuracy = {"max_abs_err": float(f"{err:.3e}"), "tolerance": 2e-2 if c.dtype == B.SA_BF16 else 1e-4,
                        "reference": "the fp64 oracle attending the step's own page lists (first copy)",
                        "identical_page_lists": f"{int((gsel == own.sel).all(axis=-1).sum())}/{gcnt.size}"}

    rec = {
        "metric": "selected-KV GB/s (% of HBM peak) + us/decode step, 128k ctx GQA-8",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2),
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded): K from 64 Gaussian clusters, V and q N(0,1)",
        "config": {"workload": wl.name, "batch": c.B, "q_heads": c.Hq, "kv_heads": c.Hkv, "head_dim": c.hd,
                   "context": L, "page": c.P, "sink": pr.sink, "window": pr.window, "budget": pr.budget,
                   "score": wl.mode, "replicas": R,
                   "splits": dec.splits if mode != "overlap" else {"sink_window": ov.sl, "selected": ov.sm},
                   "step": mode},
        "roofline": {"bound": "hbm", "kernel": dec_kernel, "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_record(dec_kernel), "bytes_per_launch": dec_bytes,
                     "avg_launch_us": round(dec_avg_ms * 1e3, 2)},
        "cpu_baseline": cpu,
        "accuracy": accuracy,
        "step_us": step_dist,
        "stream_ref": stream_ref,
        "stream_ref_us": stream_ref["us"],
        "frac_of_stream": round(gbps / probe_gbps, 4),
        "pair_frac_of_stream": round(dec_gbps / probe_gbps, 4),
        "bytes_per_step": sb.as_dict(),
        "us_per_step_one_replica": None if args.only_timed else round(ms_hot * 1e3, 2),
        "dense_us_per_step": None if args.only_timed else round(dense_ms * 1e3, 2),
        "speedup_vs_dense": None if args.only_timed else round(dense_ms / ms, 2),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
