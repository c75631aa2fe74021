// C ABI: host-side validation and dispatch to the gfx950 kernels.
// Every check runs before any HIP call, so a rejected call queues nothing
// and touches no device state.  With SPARSE_ATTN_SYNC=1 in the environment
// every entry point synchronises its stream and reports asynchronous
// failures as SA_ERR_HIP (a debugging aid; off by default).
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cstdint>

#include "../../include/sparse_attn.h"
#include "kernels.hpp"

namespace {

constexpr int kMaxSplits = 1024;
constexpr int kMaxSelectPages = 12288;  // one top-k workgroup holds one key per page in LDS
constexpr int kMaxChunks = 64;          // chunks of the two-stage selection (524288 pages)
constexpr long kMaxGridY = 65535;
constexpr int kMaxTokenSplits = 64;  // token chunks per page of the grouped decode

// debugging aids, read at every call
bool sync_mode()
{
    const char* e = getenv("SPARSE_ATTN_SYNC");
    return e && e[0] == '1';
}

// bound on the selecting kernel's wait for its page list (rounds of three
// tiles); SPARSE_ATTN_SPIN_LIMIT lowers it to exercise the give-up path
int spin_limit()
{
    constexpr int kDefault = 1 << 24;
    const char* e = getenv("SPARSE_ATTN_SPIN_LIMIT");
    if (!e || !e[0]) return kDefault;
    const long v = strtol(e, nullptr, 10);
    return v >= 1 && v < kDefault ? (int)v : kDefault;
}

int finish(hipError_t launch, hipStream_t s)
{
    if (launch != hipSuccess) return SA_ERR_HIP;
    if (sync_mode()) {
        if (hipStreamSynchronize(s) != hipSuccess) return SA_ERR_HIP;
        if (hipGetLastError() != hipSuccess) return SA_ERR_HIP;
    }
    return SA_OK;
}

bool pow2_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

// A launch of `wgs` workgroups of `threads` work-items each fits the
// dispatch packet, whose grid size is a 32-bit count of work-items.
bool grid_fits(long wgs, long threads) { return wgs >= 0 && wgs * threads <= 0xffffffffl; }
constexpr long kDecodeThreads = 512;  // the largest decode workgroup (8 waves)

// Validates the cache descriptor; fills `g` on success.
int check_kv(const sa_kv_desc* kv, sa::Geometry* g)
{
    if (!kv) return SA_ERR_INVALID_ARG;
    if (kv->batch < 1 || kv->num_kv_heads < 1 || kv->num_q_heads < 1 || kv->page_size < 1 ||
        kv->max_pages_per_seq < 1 || kv->num_phys_pages < 1 || kv->max_seq_len < 1)
        return SA_ERR_INVALID_ARG;
    if (kv->num_q_heads % kv->num_kv_heads != 0) return SA_ERR_INVALID_ARG;
    if (kv->page_size > 16384) return SA_ERR_UNSUPPORTED;
    if ((long)kv->max_seq_len > (long)kv->max_pages_per_seq * kv->page_size) return SA_ERR_INVALID_ARG;
    if ((long)kv->max_pages_per_seq * kv->page_size >= (1l << 30)) return SA_ERR_UNSUPPORTED;
    // K/V rows are indexed with 32-bit integers
    if ((long)kv->num_phys_pages * kv->num_kv_heads * kv->page_size >= (1l << 31)) return SA_ERR_UNSUPPORTED;
    if (!kv->k_cache || !kv->v_cache || !kv->block_table || !kv->seq_lens) return SA_ERR_INVALID_ARG;
    if (kv->dtype != SA_F32 && kv->dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
    if (kv->head_dim != 64 && kv->head_dim != 128) return SA_ERR_UNSUPPORTED;
    const int G = kv->num_q_heads / kv->num_kv_heads;
    if (!pow2_group(G)) return SA_ERR_UNSUPPORTED;
    const sa::FastDivHost pd = sa::make_fastdiv((uint32_t)kv->page_size);
    *g = sa::Geometry{kv->batch, kv->num_q_heads, kv->num_kv_heads, G, kv->head_dim, kv->page_size,
                      kv->max_pages_per_seq, kv->num_phys_pages, kv->dtype, kv->k_cache, kv->v_cache,
                      kv->block_table, kv->seq_lens, pd};
    return SA_OK;
}

// resident decode workgroups per CU, queried once per kernel shape
int occupancy(int hd, int G, int dtype)
{
    static std::atomic<int> cache[2][2][5];
    if ((hd != 64 && hd != 128) || (dtype != SA_F32 && dtype != SA_BF16) || !pow2_group(G)) return 1;
    int gi = 0;
    while ((1 << gi) < G) ++gi;
    std::atomic<int>& c = cache[hd == 128][dtype == SA_BF16][gi];
    int v = c.load(std::memory_order_relaxed);
    if (v == 0) {
        v = sa::decode_wgs_per_cu(hd, G, dtype);
        c.store(v, std::memory_order_relaxed);
    }
    return v;
}

// workgroups of the persistent grouped decode on the current device (CUs
// times resident workgroups per CU), queried once per device and shape
int group_grid(int hd, int G)
{
    constexpr int kDevices = 64;
    static std::atomic<int> cache[kDevices][2][5];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if ((hd != 64 && hd != 128) || !pow2_group(G)) return 8;
    int gi = 0;
    while ((1 << gi) < G) ++gi;
    if (dev < 0 || dev >= kDevices) return sa::group_workgroups(hd, G);
    std::atomic<int>& c = cache[dev][hd == 128][gi];
    int v = c.load(std::memory_order_relaxed);
    if (v == 0) {
        v = sa::group_workgroups(hd, G);
        c.store(v, std::memory_order_relaxed);
    }
    return v;
}

// fewest splits that leave every workgroup of the select-and-decode kernel
// at most kRowsWG row-table entries: a share of the sink + window rounded up
// to a multiple of 16 (up to 16 more than toks / s) plus a share of the
// selected pages (up to 1 more)
long fused_min_splits(int32_t sink_len, int32_t window_len, int32_t k_max, int32_t page_size)
{
    const long toks = (long)(sink_len > 0 ? sink_len : 0) + (window_len > 0 ? window_len : 0) +
                      (long)(k_max > 0 ? k_max : 0) * page_size;
    return (toks + sa::kRowsWG - 18) / (sa::kRowsWG - 17);
}

// Whether sparse_attn_decode_step runs the select-and-decode kernel (else
// the separate top-k and decode).  The kernel reads the block-table and score
// rows as 16-byte vectors.
bool fused_step_ok(const sa_kv_desc* kv, int32_t sink_len, int32_t window_len, int32_t k_max, int32_t num_splits,
                   const void* workspace)
{
    const bool aligned = kv->max_pages_per_seq % 4 == 0 && ((uintptr_t)kv->block_table & 15) == 0 &&
                         ((uintptr_t)workspace & 15) == 0;
    return kv->dtype == SA_BF16 && k_max >= 1 && k_max <= sa::kSelCap && kv->max_pages_per_seq <= sa::kFusedMaxCand &&
           aligned && num_splits >= fused_min_splits(sink_len, window_len, k_max, kv->page_size);
}

// workspace of the KeyDiff selection: the chunk key sums, then the order
// keys of the distances (rows padded to a multiple of 4), each 256-byte
// aligned
// (past kKdMaxCand candidates, also each chunk's picks of tokens to evict:
// inverted keys, then candidate indices)
struct KeydiffWs {
    int nchunks, Tk, ecnk;
    size_t partial, okeys, part_keys, part_idx, total;
};
KeydiffWs keydiff_ws(const sa_kv_desc* kv, int32_t sink_len, int32_t budget)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t bh = (size_t)kv->batch * kv->num_kv_heads;
    KeydiffWs w;
    w.nchunks = (kv->max_seq_len + sa::kKdChunk - 1) / sa::kKdChunk;
    w.Tk = (kv->max_seq_len + 3) & ~3;
    w.partial = 0;
    w.okeys = up(bh * (size_t)w.nchunks * kv->head_dim * sizeof(float));
    w.total = up(w.okeys + bh * (size_t)w.Tk * sizeof(uint32_t));
    w.ecnk = 0;
    w.part_keys = w.part_idx = 0;
    const long cand = (long)kv->max_seq_len - (sink_len > 0 ? sink_len : 0);
    if (kv->max_seq_len > budget && cand > sa::kKdMaxCand) {
        w.ecnk = (int)((cand + sa::kTopkChunk - 1) / sa::kTopkChunk);
        const size_t part = up(bh * (size_t)w.ecnk * sa::kTopkChunk * sizeof(uint32_t));
        w.part_keys = w.total;
        w.part_idx = w.part_keys + part;
        w.total = w.part_idx + part;
    }
    return w;
}

// Whether the eviction can rank the longest sequence's candidates: one
// workgroup holds kKdMaxCand; past that, at most kKdMaxChunks chunks whose
// picks (min(evicted, kTopkChunk) each) fit the merge workgroup.
bool keydiff_fits(const sa_kv_desc* kv, int32_t sink_len, int32_t budget)
{
    const long cand = (long)kv->max_seq_len - sink_len;
    if (kv->max_seq_len <= budget || cand <= sa::kKdMaxCand) return true;
    const long chunks = (cand + sa::kTopkChunk - 1) / sa::kTopkChunk;
    const long evicted = (long)kv->max_seq_len - budget;
    return chunks <= sa::kKdMaxChunks && chunks * std::min<long>(evicted, sa::kTopkChunk) <= sa::kTopkMerge;
}

// workspace of the grouped decode: byte offsets of its three arrays, each
// 256-byte aligned
struct GroupedWs {
    size_t nunion, upages, slots, total;
};
// npg: candidate units per (sequence, KV head) (pages, or an index's blocks)
GroupedWs grouped_ws(const sa_kv_desc* kv, long npg)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t bh = (size_t)kv->batch * kv->num_kv_heads, mp = (size_t)npg;
    GroupedWs w;
    w.nunion = 0;
    w.upages = up(w.nunion + bh * sizeof(int32_t));
    w.slots = up(w.upages + bh * mp * sizeof(sa::GroupPage));
    w.total = up(w.slots + bh * mp * sa::kGroupMaxRows * sizeof(int16_t));
    return w;
}

// The prefill front's workspace: the slot table [B][Hkv][C][kGroupMaxRows]
// (int16), the rows of each row group of 8 that chose each block
// [B][Hkv][C][16] (uint8), the decode's item counters [B][Hkv], each
// 256-byte aligned.
struct PrefillWs {
    size_t slots, rows, ctr, total;
};
// nck: prompt chunks per call (each has its own slot table, row counts and counters)
PrefillWs prefill_ws(const sa_kv_desc* kv, long C, long nck = 1)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t bh = (size_t)kv->batch * kv->num_kv_heads * nck;
    PrefillWs w;
    w.slots = 0;
    w.rows = up(bh * (size_t)C * sa::kGroupMaxRows * sizeof(int16_t));
    w.ctr = up(w.rows + bh * (size_t)C * 16);
    w.total = up(w.ctr + bh * sizeof(int32_t));
    return w;
}

// Window units of a prefill chunk: the pages that [L - W, L) can touch.
long prefill_window_units(long window_len, long page_size) { return (window_len - 1) / page_size + 2; }

// The selection's workspace: the fp32 scores [B][Hkv][Q][max_pages]; past
// kMaxSelectPages pages per sequence also every chunk's winners (order keys,
// then candidate indices, [B][Hkv][Q][nchunks][kTopkChunk] each), 256-byte
// aligned.
struct SelectWs {
    int nchunks;  // 0: one workgroup ranks all of a problem's candidates
    size_t part_keys, part_idx, total;
};
SelectWs select_ws(const sa_kv_desc* kv, int32_t rows)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t problems = (size_t)kv->batch * kv->num_kv_heads * rows;
    SelectWs w;
    w.total = sizeof(float) * problems * kv->max_pages_per_seq;
    w.nchunks = 0;
    w.part_keys = w.part_idx = 0;
    if (kv->max_pages_per_seq > kMaxSelectPages) {
        w.nchunks = (kv->max_pages_per_seq + sa::kTopkChunk - 1) / sa::kTopkChunk;
        const size_t part = sizeof(uint32_t) * problems * w.nchunks * sa::kTopkChunk;
        w.part_keys = up(w.total);
        w.part_idx = w.part_keys + up(part);
        w.total = w.part_idx + up(part);
    }
    return w;
}
size_t select_ws_bytes(const sa_kv_desc* kv, int32_t rows) { return select_ws(kv, rows).total; }

// Whether the selection can rank k_max of max_pages candidates: one
// workgroup holds up to kMaxSelectPages; past that, at most kMaxChunks chunks
// whose winners (min(k_max, kTopkChunk) each) fit the merge workgroup.
bool select_fits(const sa_kv_desc* kv, int32_t k_max)
{
    if (k_max <= 0 || kv->max_pages_per_seq <= kMaxSelectPages) return true;
    const long nchunks = (kv->max_pages_per_seq + sa::kTopkChunk - 1) / sa::kTopkChunk;
    return nchunks <= kMaxChunks && nchunks * std::min<long>(k_max, sa::kTopkChunk) <= sa::kTopkMerge;
}

// the selecting step's workspace: the scores, then (256-byte aligned) its
// status word
size_t status_offset(const sa_kv_desc* kv, int32_t rows) { return (select_ws_bytes(kv, rows) + 255) & ~(size_t)255; }
// the merge's counters: one per (sequence, KV head, row), then one per sequence
long merge_counters(const sa_kv_desc* kv, int32_t rows) { return (long)kv->batch * kv->num_kv_heads * rows + kv->batch; }
size_t counters_offset(const sa_kv_desc* kv, int32_t rows) { return status_offset(kv, rows) + 256; }
size_t step_ws_bytes(const sa_kv_desc* kv, int32_t rows)
{
    return counters_offset(kv, rows) + (((size_t)merge_counters(kv, rows) * sizeof(uint32_t) + 255) & ~(size_t)255);
}
sa::MergeArgs merge_args(const sa_kv_desc* kv, int32_t rows, void* out, int32_t out_dtype, float* lse,
                         uint32_t* counters, int32_t advance)
{
    sa::MergeArgs m{};
    m.out = out;
    m.out_dtype = out_dtype == SA_BF16 ? 1 : 0;
    m.lse = lse;
    m.arrive = counters;
    m.batch_done = counters + (long)kv->batch * kv->num_kv_heads * rows;
    m.seq_lens = advance > 0 ? (int32_t*)kv->seq_lens : nullptr;
    m.advance = advance;
    return m;
}

// The checks of sparse_attn_decode_step's arguments other than its
// workspace and partials (shared with the variant that keeps them in the
// static scratch).
int check_step(const sa_kv_desc* kv, const void* q, int32_t num_q_rows, const void* meta, int32_t score_mode,
               int32_t sink_len, int32_t window_len, int32_t token_budget, float softmax_scale, int32_t num_splits,
               const int32_t* sel_pages, const int32_t* sel_count)
{
    sa::Geometry g;
    const int rc = check_kv(kv, &g);
    if (rc != SA_OK) return rc;
    if (score_mode < SA_QUEST || score_mode > SA_COMPRESSED) return SA_ERR_UNSUPPORTED;
    if (!q || !meta || !sel_count || num_q_rows < 1 || sink_len < 0 || window_len < 1 || token_budget < 0)
        return SA_ERR_INVALID_ARG;
    if (num_q_rows > kv->max_seq_len) return SA_ERR_INVALID_ARG;
    const int k_max = token_budget / kv->page_size;
    if (k_max > 0 && !sel_pages) return SA_ERR_INVALID_ARG;
    if (num_splits < 1 || num_splits > kMaxSplits) return SA_ERR_INVALID_ARG;
    if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return SA_ERR_INVALID_ARG;
    if ((long)kv->batch * kv->num_kv_heads * num_q_rows > kMaxGridY) return SA_ERR_UNSUPPORTED;
    if (!grid_fits((long)kv->batch * kv->num_kv_heads * num_q_rows * num_splits, kDecodeThreads))
        return SA_ERR_UNSUPPORTED;
    if (!select_fits(kv, k_max)) return SA_ERR_UNSUPPORTED;
    return SA_OK;
}

}  // namespace

extern "C" {

const char* sparse_attn_status_string(int status)
{
    switch (status) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID_ARG: return "invalid argument";
    case SA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SA_ERR_HIP: return "HIP launch error";
    case SA_ERR_SCRATCH: return "needs more than the library's static scratch (16 MiB)";
    default: return "unknown status";
    }
}

size_t sparse_attn_workspace_bytes(const sa_kv_desc* kv, int32_t num_q_rows)
{
    if (!kv || num_q_rows < 1 || kv->batch < 1 || kv->num_kv_heads < 1 || kv->max_pages_per_seq < 1) return 0;
    return step_ws_bytes(kv, num_q_rows);
}

int sparse_attn_build_page_meta(const sa_kv_desc* kv, int32_t score_mode, int32_t page_begin, int32_t page_end,
                                void* meta, hipStream_t stream)
{
    sa::Geometry g;
    const int rc = check_kv(kv, &g);
    if (rc != SA_OK) return rc;
    if (!meta || page_begin < 0 || page_end < page_begin) return SA_ERR_INVALID_ARG;
    if (score_mode < SA_QUEST || score_mode > SA_COMPRESSED) return SA_ERR_UNSUPPORTED;
    const int end = page_end < g.max_pages ? page_end : g.max_pages;
    if (end <= page_begin) return SA_OK;
    // one wave per (sequence, page, KV head)
    if (!grid_fits((long)kv->batch * (end - page_begin) * kv->num_kv_heads, 64)) return SA_ERR_UNSUPPORTED;
    sa::MetaArgs a{g, score_mode, page_begin, end, meta};
    return finish(sa::launch_page_meta(a, stream), stream);
}

int sparse_attn_select(const sa_kv_desc* kv, const void* q, int32_t num_q_rows, const void* meta,
                       int32_t score_mode, int32_t sink_len, int32_t window_len, int32_t token_budget,
                       int32_t* sel_pages, int32_t* sel_count, void* workspace, size_t workspace_bytes,
                       hipStream_t stream)
{
    sa::Geometry g;
    const int rc = check_kv(kv, &g);
    if (rc != SA_OK) return rc;
    if (score_mode < SA_QUEST || score_mode > SA_COMPRESSED) return SA_ERR_UNSUPPORTED;
    if (!q || !meta || !sel_count || num_q_rows < 1 || sink_len < 0 || window_len < 1 || token_budget < 0)
        return SA_ERR_INVALID_ARG;
    if (num_q_rows > kv->max_seq_len) return SA_ERR_INVALID_ARG;
    const int k_max = token_budget / kv->page_size;
    if (k_max > 0 && !sel_pages) return SA_ERR_INVALID_ARG;
    if ((long)kv->batch * kv->num_kv_heads * num_q_rows > kMaxGridY) return SA_ERR_UNSUPPORTED;
    if (k_max > 0) {
        if (!select_fits(kv, k_max)) return SA_ERR_UNSUPPORTED;
        if (!workspace || workspace_bytes < select_ws_bytes(kv, num_q_rows)) return SA_ERR_INVALID_ARG;
    }
    const SelectWs w = select_ws(kv, num_q_rows);
    char* base = (char*)workspace;
    sa::SelectArgs a{g,         q,          num_q_rows, meta,      score_mode,        sink_len, window_len,
                     k_max,     sel_pages,  sel_count,  (float*)workspace, 0,          nullptr,  w.nchunks,
                     sa::kTopkChunk, w.nchunks ? (uint32_t*)(base + w.part_keys) : nullptr,
                     w.nchunks ? (int32_t*)(base + w.part_idx) : nullptr};
    return finish(sa::launch_select(a, stream), stream);
}

int32_t sparse_attn_default_splits(const sa_kv_desc* kv, int32_t num_q_rows, int32_t sink_len, int32_t window_len,
                                   int32_t k_max)
{
    if (!kv || kv->batch < 1 || kv->num_kv_heads < 1 || num_q_rows < 1 || kv->page_size < 1) return 1;
    // attended tokens per (sequence, KV head, row), at most
    const long L = kv->max_seq_len;
    long ntok = (long)(sink_len < 0 ? 0 : sink_len) + (window_len < 1 ? 1 : window_len) +
                (long)(k_max < 0 ? 0 : k_max) * kv->page_size;
    if (ntok > L) ntok = L;
    const long problems = (long)kv->batch * kv->num_kv_heads * num_q_rows;
    // one round of workgroups over the device: CUs x resident workgroups per CU,
    // with at least 256 tokens per workgroup
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    const int G = kv->num_kv_heads > 0 ? kv->num_q_heads / kv->num_kv_heads : 1;
    const long slots = (long)cus * occupancy(kv->head_dim, G, kv->dtype);
    long s = (slots + problems - 1) / problems;
    const long by_tokens = ntok / 256 > 0 ? ntok / 256 : 1;
    if (s > by_tokens) s = by_tokens;
    if (s < 1) s = 1;
    const long fused = fused_min_splits(sink_len, window_len, k_max, kv->page_size);
    if (s < fused) s = fused;
    if (s > kMaxSplits) s = kMaxSplits;
    return (int32_t)s;
}

int sparse_attn_decode(const sa_kv_desc* kv, const void* q, int32_t num_q_rows, const int32_t* sel_pages,
                       const int32_t* sel_count, int32_t k_max, int32_t sink_len, int32_t window_len, int32_t parts,
                       float softmax_scale, int32_t num_splits, int32_t split_stride, float* part_o, float* part_ml,
                       hipStream_t stream)
{
    sa::Geometry g;
    const int rc = check_kv(kv, &g);
    if (rc != SA_OK) return rc;
    if (!q || !part_o || !part_ml || num_q_rows < 1 || sink_len < 0 || window_len < 1 || k_max < 0)
        return SA_ERR_INVALID_ARG;
    if (num_q_rows > kv->max_seq_len) return SA_ERR_INVALID_ARG;
    if (sel_pages && !sel_count) return SA_ERR_INVALID_ARG;
    if (num_splits < 1 || num_splits > kMaxSplits) return SA_ERR_INVALID_ARG;
    if (split_stride == 0) split_stride = num_splits;
    if (split_stride < num_splits || split_stride > kMaxSplits) return SA_ERR_INVALID_ARG;
    if (parts < SA_PART_LOCAL || parts > SA_PART_ALL) return SA_ERR_INVALID_ARG;
    if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return SA_ERR_INVALID_ARG;
    if (!grid_fits((long)kv->batch * kv->num_kv_heads * num_q_rows * num_splits, kDecodeThreads))
        return SA_ERR_UNSUPPORTED;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)kv->head_dim);
    sa::DecodeArgs a{g,        q,          num_q_rows, sel_pages, sel_count, sel_pages ? k_max : 0,
                     sink_len, window_len, parts,      scale * 1.4426950408889634f,   num_splits,
                     split_stride, part_o, part_ml};
    return finish(sa::launch_decode(a, stream), stream);
}

int sparse_attn_decode_step(const sa_kv_desc* kv, const void* q, int32_t num_q_rows, const void* meta,
                            int32_t score_mode, int32_t sink_len, int32_t window_len, int32_t token_budget,
                            float softmax_scale, int32_t num_splits, int32_t* sel_pages, int32_t* sel_count,
                            void* workspace, size_t workspace_bytes, float* part_o, float* part_ml,
                            hipStream_t stream)
{
    const int rc = check_step(kv, q, num_q_rows, meta, score_mode, sink_len, window_len, token_budget, softmax_scale,
                              num_splits, sel_pages, sel_count);
    if (rc != SA_OK) return rc;
    if (!part_o || !part_ml) return SA_ERR_INVALID_ARG;
    const int k_max = token_budget / kv->page_size;
    if (k_max > 0 && (!workspace || workspace_bytes < step_ws_bytes(kv, num_q_rows))) return SA_ERR_INVALID_ARG;
    sa::Geometry g;
    (void)check_kv(kv, &g);  // validated above: fills g
    const bool fused = fused_step_ok(kv, sink_len, window_len, k_max, num_splits, workspace);
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)kv->head_dim);
    if (!fused) {
        const int r1 = sparse_attn_select(kv, q, num_q_rows, meta, score_mode, sink_len, window_len, token_budget,
                                          sel_pages, sel_count, workspace, workspace_bytes, stream);
        if (r1 != SA_OK) return r1;
        return sparse_attn_decode(kv, q, num_q_rows, sel_pages, sel_count, k_max, sink_len, window_len, SA_PART_ALL,
                                  softmax_scale, num_splits, num_splits, part_o, part_ml, stream);
    }
    uint32_t* status = (uint32_t*)((char*)workspace + status_offset(kv, num_q_rows));
    sa::SelectArgs sarg{g,     q,         num_q_rows, meta, score_mode, sink_len, window_len, k_max, sel_pages,
                        sel_count, (float*)workspace, 1, status, 0, 0, nullptr, nullptr};
    const int r1 = finish(sa::launch_select(sarg, stream), stream);
    if (r1 != SA_OK) return r1;
    sa::SelectDecodeArgs d{g,          q,          num_q_rows, (const float*)workspace,
                           k_max,      sink_len,   window_len, scale * 1.4426950408889634f,
                           num_splits, num_splits, part_o,     part_ml,
                           sel_pages,  sel_count,  status,     spin_limit()};
    const int r2 = finish(sa::launch_select_decode(d, stream), stream);
    if (r2 != SA_OK || !sync_mode()) return r2;
    // synchronised: a workgroup whose bounded wait ran out left NaN partials
    uint32_t st = 0;
    if (hipMemcpy(&st, status, sizeof(st), hipMemcpyDeviceToHost) != hipSuccess) return SA_ERR_HIP;
    return st == 0 ? SA_OK : SA_ERR_HIP;
}

int32_t sparse_attn_merge_counters(const sa_kv_desc* kv, int32_t num_q_rows)
{
    if (!kv || kv->batch < 1 || kv->num_kv_heads < 1 || num_q_rows < 1) return -SA_ERR_INVALID_ARG;
    const long n = merge_counters(kv, num_q_rows);
    return n > 0x7fffffffl ? -SA_ERR_UNSUPPORTED : (int32_t)n;
}

int sparse_attn_decode_merged(const sa_kv_desc* kv, const void* q, int32_t num_q_rows, const int32_t* sel_pages,
                              const int32_t* sel_count, int32_t k_max, int32_t sink_len, int32_t window_len,
                              float softmax_scale, int32_t num_splits, float* part_o, float* part_ml, void* out,
                              int32_t out_dtype, float* lse, int32_t advance, uint32_t* counters, hipStream_t stream)
{
    sa::Geometry g;
    const int rc = check_kv(kv, &g);
    if (rc != SA_OK) return rc;
    if (!q || !part_o || !part_ml || !out || !counters || num_q_rows < 1 || sink_len < 0 || window_len < 1 ||
        k_max < 0 || advance < 0)
        return SA_ERR_INVALID_ARG;
    if (num_q_rows > kv->max_seq_len) return SA_ERR_INVALID_ARG;
    if (sel_pages && !sel_count) return SA_ERR_INVALID_ARG;
    if (num_splits < 1 || num_splits > sa::kMergeMaxSplits) return SA_ERR_INVALID_ARG;
    if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return SA_ERR_INVALID_ARG;
    if (kv->dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
    if (out_dtype != SA_F32 && out_dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
    if (!grid_fits((long)kv->batch * kv->num_kv_heads * num_q_rows * num_splits, kDecodeThreads))
        return SA_ERR_UNSUPPORTED;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)kv->head_dim);
    sa::DecodeArgs a{g,        q,          num_q_rows,  sel_pages, sel_count, sel_pages ? k_max : 0,
                     sink_len, window_len, SA_PART_ALL, scale * 1.4426950408889634f,   num_splits,
                     num_splits, part_o,   part_ml};
    a.m = merge_args(kv, num_q_rows, out, out_dtype, lse, counters, advance);
    return finish(sa::launch_decode(a, stream), stream);
}

int sparse_attn_decode_step_merged(const sa_kv_desc* kv, const void* q, int32_t num_q_rows, const void* meta,
                                   int32_t score_mode, int32_t sink_len, int32_t window_len, int32_t token_budget,
                                   float softmax_scale, int32_t num_splits, int32_t* sel_pages, int32_t* sel_count,
                                   void* workspace, size_t workspace_bytes, float* part_o, float* part_ml, void* out,
                                   int32_t out_dtype, float* lse, int32_t advance, hipStream_t stream)
{
    const int rc = check_step(kv, q, num_q_rows, meta, score_mode, sink_len, window_len, token_budget, softmax_scale,
                              num_splits, sel_pages, sel_count);
    if (rc != SA_OK) return rc;
    if (!part_o || !part_ml || !out || advance < 0) return SA_ERR_INVALID_ARG;
    if (num_splits > sa::kMergeMaxSplits) return SA_ERR_INVALID_ARG;
    if (kv->dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
    if (out_dtype != SA_F32 && out_dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < step_ws_bytes(kv, num_q_rows)) return SA_ERR_INVALID_ARG;
    const int k_max = token_budget / kv->page_size;
    sa::Geometry g;
    (void)check_kv(kv, &g);  // validated above: fills g
    uint32_t* counters = (uint32_t*)((char*)workspace + counters_offset(kv, num_q_rows));
    const bool fused = k_max > 0 && fused_step_ok(kv, sink_len, window_len, k_max, num_splits, workspace);
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)kv->head_dim);
    if (!fused) {
        const int r0 = finish(sa::launch_zero_u32(counters, merge_counters(kv, num_q_rows), stream), stream);
        if (r0 != SA_OK) return r0;
        const int r1 = sparse_attn_select(kv, q, num_q_rows, meta, score_mode, sink_len, window_len, token_budget,
                                          sel_pages, sel_count, workspace, workspace_bytes, stream);
        if (r1 != SA_OK) return r1;
        return sparse_attn_decode_merged(kv, q, num_q_rows, sel_pages, sel_count, k_max, sink_len, window_len,
                                         softmax_scale, num_splits, part_o, part_ml, out, out_dtype, lse, advance,
                                         counters, stream);
    }
    uint32_t* status = (uint32_t*)((char*)workspace + status_offset(kv, num_q_rows));
    sa::SelectArgs sarg{g,     q,         num_q_rows, meta, score_mode, sink_len, window_len, k_max, sel_pages,
                        sel_count, (float*)workspace, 1, status, 0, 0, nullptr, nullptr,
                        counters, (int)merge_counters(kv, num_q_rows)};
    const int r1 = finish(sa::launch_select(sarg, stream), stream);
    if (r1 != SA_OK) return r1;
    sa::SelectDecodeArgs d{g,          q,          num_q_rows, (const float*)workspace,
                           k_max,      sink_len,   window_len, scale * 1.4426950408889634f,
                           num_splits, num_splits, part_o,     part_ml,
                           sel_pages,  sel_count,  status,     spin_limit()};
    d.m = merge_args(kv, num_q_rows, out, out_dtype, lse, counters, advance);
    const int r2 = finish(sa::launch_select_decode(d, stream), stream);
    if (r2 != SA_OK || !sync_mode()) return r2;
    uint32_t st = 0;
    if (hipMemcpy(&st, status, sizeof(st), hipMemcpyDeviceToHost) != hipSuccess) return SA_ERR_HIP;
    return st == 0 ? SA_OK : SA_ERR_HIP;
}

int32_t sparse_attn_step_path(const sa_kv_desc* kv, int32_t sink_len, int32_t window_len, int32_t token_budget,
                              int32_t num_splits, const void* workspace)
{
    sa::Geometry g;
    if (check_kv(kv, &g) != SA_OK || sink_len < 0 || window_len < 1 || token_budget < 0 || num_splits < 1)
        return -SA_ERR_INVALID_ARG;
    return fused_step_ok(kv, sink_len, window_len, token_budget / kv->page_size, num_splits, workspace)
               ? SA_STEP_FUSED
               : SA_STEP_SEPARATE;
}

size_t sparse_attn_grouped_workspace_bytes(const sa_kv_desc* kv)
{
    if (!kv || kv->batch < 1 || kv->num_kv_heads < 1 || kv->max_pages_per_seq < 1) return 0;
    return grouped_ws(kv, kv->max_pages_per_seq).total;
}

}  // extern "C"

namespace {

// The union plan and grouped decode of the rows' lists of units (pages of
// the paged cache, or blocks of an index with blk_off != nullptr), then the
// per-row decode of the sink and window into the slots after the units'.
int grouped_impl(const sa_kv_desc* kv, const sa::Geometry& g, const void* q, int32_t num_q_rows,
                 const int32_t* sel, const int32_t* cnt, int32_t k_max, int32_t sink_len, int32_t window_len,
                 float softmax_scale, int32_t token_splits, int32_t local_splits, float* part_o, float* part_ml,
                 void* workspace, size_t workspace_bytes, int npg, const int32_t* blk_off, const void* blk_k,
                 const void* blk_v, int blk_n, const int32_t* blk_end, hipStream_t stream)
{
    if (!q || !part_o || !part_ml || num_q_rows < 1 || sink_len < 0 || window_len < 1 || k_max < 0)
        return SA_ERR_INVALID_ARG;
    if (k_max > 0 && (!sel || !cnt)) return SA_ERR_INVALID_ARG;
    if (num_q_rows > kv->max_seq_len) return SA_ERR_INVALID_ARG;
    if (token_splits < 1 || token_splits > kMaxTokenSplits || local_splits < 1) return SA_ERR_INVALID_ARG;
    if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return SA_ERR_INVALID_ARG;
    const long stride = (long)k_max * token_splits + local_splits;
    if (stride > kMaxSplits) return SA_ERR_INVALID_ARG;
    if (kv->dtype != SA_BF16 || num_q_rows > sa::kGroupMaxRows || npg > sa::kGroupMaxPages)
        return SA_ERR_UNSUPPORTED;
    if ((long)kv->batch * kv->num_kv_heads > kMaxGridY) return SA_ERR_UNSUPPORTED;
    if (!grid_fits((long)kv->batch * kv->num_kv_heads * num_q_rows * local_splits, kDecodeThreads))
        return SA_ERR_UNSUPPORTED;
    const long max_union = std::min<long>(npg, (long)num_q_rows * k_max);
    if (!grid_fits(max_union * token_splits * kv->batch * kv->num_kv_heads, kDecodeThreads))
        return SA_ERR_UNSUPPORTED;
    const GroupedWs w = grouped_ws(kv, npg);
    if (k_max > 0 && (!workspace || workspace_bytes < w.total || ((uintptr_t)workspace & 255) != 0))
        return SA_ERR_INVALID_ARG;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)kv->head_dim);
    const float sl2 = scale * 1.4426950408889634f;
    if (k_max > 0) {
        char* base = (char*)workspace;
        sa::GroupArgs a{g,          q,          num_q_rows, sel,     cnt,
                        k_max,      sink_len,   window_len, sl2,     token_splits,
                        (int)stride, part_o,    part_ml,    (int32_t*)(base + w.nunion),
                        (sa::GroupPage*)(base + w.upages), (int16_t*)(base + w.slots),
                        npg,        blk_off,    blk_k,      blk_v,   blk_n,
                        blk_end,    0,          nullptr,    nullptr, 1};
        const int r1 = finish(sa::launch_group(a, (int)max_union, stream), stream);
        if (r1 != SA_OK) return r1;
    }
    const long off = (long)k_max * token_splits;
    sa::DecodeArgs d{g,        q,          num_q_rows, nullptr,       nullptr, 0,
                     sink_len, window_len, SA_PART_LOCAL, sl2,        local_splits,
                     (int)stride, part_o + off * kv->head_dim, part_ml + off * 2};
    return finish(sa::launch_decode(d, stream), stream);
}

// the index's arrays, and its sizes against the cache
int check_index(const sa_kv_desc* kv, const sa_block_index* idx)
{
    if (!idx || !idx->offsets || !idx->positions || !idx->centres || !idx->k_blocks || !idx->v_blocks)
        return SA_ERR_INVALID_ARG;
    if (idx->num_tokens < 1 || idx->num_tokens > kv->max_seq_len) return SA_ERR_INVALID_ARG;
    if (idx->num_blocks < 1 || idx->num_blocks > idx->num_tokens) return SA_ERR_INVALID_ARG;
    if (idx->num_blocks > sa::kIndexMaxBlocks) return SA_ERR_UNSUPPORTED;
    if ((long)kv->batch * kv->num_kv_heads * idx->num_tokens >= (1l << 31)) return SA_ERR_UNSUPPORTED;
    // 16-byte rows are read and written whole
    if (((uintptr_t)idx->k_blocks & 15) || ((uintptr_t)idx->v_blocks & 15) || ((uintptr_t)idx->centres & 15))
        return SA_ERR_INVALID_ARG;
    return SA_OK;
}

struct IndexWs {
    size_t inv_norm, cent_bf, assign, cnt, seg_base, seg_block, seg_sum, total;
    int nchunks, nseg;
};
IndexWs index_ws(const sa_kv_desc* kv, long N, long C)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t bh = (size_t)kv->batch * kv->num_kv_heads;
    IndexWs w;
    w.nchunks = (int)((N + sa::kIndexChunk - 1) / sa::kIndexChunk);
    w.nseg = (int)((N + sa::kIndexSegment - 1) / sa::kIndexSegment + C);
    w.inv_norm = 0;
    w.cent_bf = up(w.inv_norm + bh * N * sizeof(float));
    w.assign = up(w.cent_bf + bh * C * kv->head_dim * sizeof(uint16_t));
    w.cnt = up(w.assign + bh * N * sizeof(int32_t));
    w.seg_base = up(w.cnt + bh * w.nchunks * C * sizeof(int32_t));
    w.seg_block = up(w.seg_base + bh * (C + 1) * sizeof(int32_t));
    w.seg_sum = up(w.seg_block + bh * w.nseg * sizeof(int32_t));
    w.total = up(w.seg_sum + bh * w.nseg * kv->head_dim * sizeof(float));
    return w;
}

}  // namespace

extern "C" {

size_t sparse_attn_index_workspace_bytes(const sa_kv_desc* kv, int32_t num_tokens, int32_t num_blocks)
{
    if (!kv || kv->batch < 1 || kv->num_kv_heads < 1 || (kv->head_dim != 64 && kv->head_dim != 128) ||
        num_tokens < 1 || num_blocks < 1)
        return 0;
    return index_ws(kv, num_tokens, num_blocks).total;
}

int sparse_attn_build_block_index(const sa_kv_desc* kv, int32_t iterations, const sa_block_index* index,
                                  int32_t* assignment, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    sa::Geometry g;
    const int rc = check_kv(kv, &g);
    if (rc != SA_OK) return rc;
    const int ri = check_index(kv, index);
    if (ri != SA_OK) return ri;
    if (kv->dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
    if (iterations < 0 || iterations > 64) return SA_ERR_INVALID_ARG;
    if ((long)kv->batch * kv->num_kv_heads > kMaxGridY) return SA_ERR_UNSUPPORTED;
    // the widest launch: one work-item per 16-byte piece of a key row (plus a workgroup of rounding)
    if (!grid_fits((long)index->num_tokens * kv->head_dim / 8 + 256, 1)) return SA_ERR_UNSUPPORTED;
    const IndexWs w = index_ws(kv, index->num_tokens, index->num_blocks);
    if (!workspace || workspace_bytes < w.total || ((uintptr_t)workspace & 255) != 0) return SA_ERR_INVALID_ARG;
    char* base = (char*)workspace;
    sa::IndexArgs a{g,
                    index->num_tokens,
                    index->num_blocks,
                    iterations,
                    index->offsets,
                    index->positions,
                    index->centres,
                    index->k_blocks,
                    index->v_blocks,
                    assignment,
                    (float*)(base + w.inv_norm),
                    (uint16_t*)(base + w.cent_bf),
                    (int32_t*)(base + w.assign),
                    (int32_t*)(base + w.cnt),
                    (int32_t*)(base + w.seg_base),
                    (int32_t*)(base + w.seg_block),
                    (float*)(base + w.seg_sum),
                    w.nchunks,
                    w.nseg};
    return finish(sa::launch_index_build(a, stream), stream);
}

int sparse_attn_select_blocks(const sa_kv_desc* kv, const sa_block_index* index, const void* q, int32_t num_q_rows,
                              int32_t token_budget, int32_t k_max, int32_t* sel_blocks, int32_t* sel_count,
                              hipStream_t stream)
{
    sa::Geometry g;
    const int rc = check_kv(kv, &g);
    if (rc != SA_OK) return rc;
    const int ri = check_index(kv, index);
    if (ri != SA_OK) return ri;
    if (kv->dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
    if (!q || !sel_blocks || !sel_count || num_q_rows < 1 || token_budget < 0) return SA_ERR_INVALID_ARG;
    if (k_max < 1 || k_max > index->num_blocks) return SA_ERR_INVALID_ARG;
    if (!grid_fits((long)kv->batch * kv->num_kv_heads * num_q_rows, 256)) return SA_ERR_UNSUPPORTED;
    sa::SelectBlocksArgs a{g,          q,     num_q_rows, index->num_blocks, index->offsets, index->centres,
                           token_budget, k_max, sel_blocks, sel_count, index->visible_end};
    return finish(sa::launch_select_blocks(a, stream), stream);
}

int sparse_attn_blocks_visible(const sa_kv_desc* kv, const sa_block_index* index, int32_t window_len,
                               int32_t* visible_end, hipStream_t stream)
{
    sa::Geometry g;
    const int rc = check_kv(kv, &g);
    if (rc != SA_OK) return rc;
    const int ri = check_index(kv, index);
    if (ri != SA_OK) return ri;
    if (!visible_end || window_len < 0) return SA_ERR_INVALID_ARG;
    sa::VisibleArgs a{g, index->num_tokens, index->num_blocks, window_len, index->offsets, index->positions,
                      visible_end};
    return finish(sa::launch_blocks_visible(a, stream), stream);
}

size_t sparse_attn_blocks_workspace_bytes(const sa_kv_desc* kv, const sa_block_index* index)
{
    if (!kv || !index || kv->batch < 1 || kv->num_kv_heads < 1 || index->num_blocks < 1) return 0;
    return grouped_ws(kv, index->num_blocks).total;
}

int sparse_attn_decode_blocks(const sa_kv_desc* kv, const sa_block_index* index, const void* q, int32_t num_q_rows,
                              const int32_t* sel_blocks, const int32_t* sel_count, int32_t k_max, int32_t window_len,
                              float softmax_scale, int32_t token_splits, int32_t local_splits, float* part_o,
                              float* part_ml, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    sa::Geometry g;
    const int rc = check_kv(kv, &g);
    if (rc != SA_OK) return rc;
    const int ri = check_index(kv, index);
    if (ri != SA_OK) return ri;
    // the rows' window holds the current fragment, and the blocks' tokens precede it
    if (window_len < num_q_rows || k_max > index->num_blocks) return SA_ERR_INVALID_ARG;
    return grouped_impl(kv, g, q, num_q_rows, sel_blocks, sel_count, k_max, 0, window_len, softmax_scale,
                        token_splits, local_splits, part_o, part_ml, workspace, workspace_bytes, index->num_blocks,
                        index->offsets, index->k_blocks, index->v_blocks, index->num_tokens, index->visible_end,
                        stream);
}

int32_t sparse_attn_prefill_num_splits(const sa_kv_desc* kv, int32_t window_len, int32_t k_max, int32_t token_splits)
{
    if (!kv || kv->page_size < 1 || window_len < 1 || k_max < 1 || token_splits < 1 ||
        token_splits > kMaxTokenSplits)
        return -SA_ERR_INVALID_ARG;
    const long s = (k_max + prefill_window_units(window_len, kv->page_size)) * (long)token_splits;
    return s > kMaxSplits ? -SA_ERR_UNSUPPORTED : (int32_t)s;
}

size_t sparse_attn_prefill_workspace_bytes(const sa_kv_desc* kv, const sa_block_index* index)
{
    return sparse_attn_prefill_chunks_workspace_bytes(kv, index, 1);
}

size_t sparse_attn_prefill_chunks_workspace_bytes(const sa_kv_desc* kv, const sa_block_index* index,
                                                  int32_t num_chunks)
{
    if (!kv || !index || kv->batch < 1 || kv->num_kv_heads < 1 || index->num_blocks < 1 || num_chunks < 1 ||
        num_chunks > sa::kPfMaxChunks)
        return 0;
    return prefill_ws(kv, index->num_blocks, num_chunks).total;
}

namespace {

// num_chunks consecutive chunks of num_q_rows rows (rows j * num_q_rows ..
// of q, the lists and the partials for chunk j, whose length is
// seq_lens[b] + j * num_q_rows), token_budgets[j] each
int prefill_impl(const sa_kv_desc* kv, const sa_block_index* index, const void* q, int32_t num_q_rows,
                 int32_t num_chunks, int32_t window_len, const int32_t* token_budgets, int32_t k_max,
                 float softmax_scale, int32_t token_splits, int32_t* visible_end, int32_t* sel_blocks,
                 int32_t* sel_count, float* part_o, float* part_ml, void* out, int32_t out_dtype, float* lse,
                 int32_t advance, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    sa::Geometry g;
    const int rc = check_kv(kv, &g);
    if (rc != SA_OK) return rc;
    const int ri = check_index(kv, index);
    if (ri != SA_OK) return ri;
    if (!q || !visible_end || !sel_blocks || !sel_count || !part_o || !part_ml || !out || !token_budgets)
        return SA_ERR_INVALID_ARG;
    if (num_chunks < 1 || num_chunks > sa::kPfMaxChunks) return SA_ERR_INVALID_ARG;
    if (num_q_rows < 1 || (long)num_q_rows * num_chunks > kv->max_seq_len || window_len < num_q_rows ||
        advance < 0)
        return SA_ERR_INVALID_ARG;
    for (int jc = 0; jc < num_chunks; ++jc)
        if (token_budgets[jc] < 0) return SA_ERR_INVALID_ARG;
    if (k_max < 1 || k_max > index->num_blocks) return SA_ERR_INVALID_ARG;
    if (token_splits < 1 || token_splits > kMaxTokenSplits) return SA_ERR_INVALID_ARG;
    if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return SA_ERR_INVALID_ARG;
    if (kv->dtype != SA_BF16 || num_q_rows > sa::kGroupMaxRows || index->num_blocks > sa::kPfMaxBlocks)
        return SA_ERR_UNSUPPORTED;
    if (out_dtype != SA_F32 && out_dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
    const int32_t stride = sparse_attn_prefill_num_splits(kv, window_len, k_max, token_splits);
    if (stride < 0) return -stride;
    const long nwin = prefill_window_units(window_len, kv->page_size);
    const long nbk = (long)kv->batch * kv->num_kv_heads, C = index->num_blocks;
    const long rows = (long)kv->batch * kv->num_q_heads * num_q_rows * num_chunks;
    if (nwin + C > sa::kGroupMaxPages) return SA_ERR_UNSUPPORTED;
    if (!grid_fits(nbk * num_chunks * ((num_q_rows + 7) / 8), kDecodeThreads) || !grid_fits(rows, 64))
        return SA_ERR_UNSUPPORTED;
    const PrefillWs w = prefill_ws(kv, C, num_chunks);
    if (!workspace || workspace_bytes < w.total || ((uintptr_t)workspace & 255) != 0) return SA_ERR_INVALID_ARG;
    char* base = (char*)workspace;
    int16_t* slots = (int16_t*)(base + w.slots);
    unsigned char* chosen_rows = (unsigned char*)(base + w.rows);
    int32_t* ctr = (int32_t*)(base + w.ctr);
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)kv->head_dim);

    sa::PrefillArgs f{};
    f.g = g;
    f.q = q;
    f.Q = num_q_rows;
    f.N = index->num_tokens;
    f.C = (int)C;
    f.nck = num_chunks;
    f.offsets = index->offsets;
    f.positions = index->positions;
    f.centres = index->centres;
    for (int jc = 0; jc < num_chunks; ++jc) f.budget[jc] = token_budgets[jc];
    f.k_max = k_max;
    f.W = window_len;
    f.tsplit = token_splits;
    f.split_stride = stride;
    f.ends = visible_end;
    f.sel = sel_blocks;
    f.count = sel_count;
    f.slots = slots;
    f.part_ml = part_ml;
    f.rows = chosen_rows;
    f.ctr = ctr;
    const int r1 = finish(sa::launch_prefill_choose(f, stream), stream);
    if (r1 != SA_OK) return r1;
    sa::GroupArgs d{};
    d.g = g;
    d.q = q;
    d.Q = num_q_rows;
    d.k_max = k_max;
    d.S = 0;
    d.W = window_len;
    d.scale_log2 = scale * 1.4426950408889634f;
    d.tsplit = token_splits;
    d.split_stride = stride;
    d.part_o = part_o;
    d.part_ml = part_ml;
    d.slots = slots;
    d.npg = (int)C;
    d.blk_off = index->offsets;
    d.blk_k = index->k_blocks;
    d.blk_v = index->v_blocks;
    d.blk_n = index->num_tokens;
    d.blk_end = visible_end;
    d.nwin = (int)nwin;
    d.pf_rows = chosen_rows;
    d.ctr = ctr;
    d.nck = num_chunks;
    const int r2 = finish(sa::launch_group_prefill(d, group_grid(kv->head_dim, g.G), stream), stream);
    if (r2 != SA_OK) return r2;
    sa::CombineArgs m{(int)rows, kv->head_dim, stride, out_dtype, part_o, part_ml, out, lse,
                      advance > 0 ? (int32_t*)kv->seq_lens : nullptr, kv->batch, advance};
    return finish(sa::launch_combine(m, stream), stream);
}

}  // namespace

int sparse_attn_prefill_chunk(const sa_kv_desc* kv, const sa_block_index* index, const void* q, int32_t num_q_rows,
                              int32_t window_len, int32_t token_budget, int32_t k_max, float softmax_scale,
                              int32_t token_splits, int32_t* visible_end, int32_t* sel_blocks, int32_t* sel_count,
                              float* part_o, float* part_ml, void* out, int32_t out_dtype, float* lse,
                              int32_t advance, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    return prefill_impl(kv, index, q, num_q_rows, 1, window_len, &token_budget, k_max, softmax_scale, token_splits,
                        visible_end, sel_blocks, sel_count, part_o, part_ml, out, out_dtype, lse, advance, workspace,
                        workspace_bytes, stream);
}

int sparse_attn_prefill_chunks(const sa_kv_desc* kv, const sa_block_index* index, const void* q, int32_t num_q_rows,
                               int32_t num_chunks, int32_t window_len, const int32_t* token_budgets, int32_t k_max,
                               float softmax_scale, int32_t token_splits, int32_t* visible_end, int32_t* sel_blocks,
                               int32_t* sel_count, float* part_o, float* part_ml, void* out, int32_t out_dtype,
                               float* lse, int32_t advance, void* workspace, size_t workspace_bytes,
                               hipStream_t stream)
{
    return prefill_impl(kv, index, q, num_q_rows, num_chunks, window_len, token_budgets, k_max, softmax_scale,
                        token_splits, visible_end, sel_blocks, sel_count, part_o, part_ml, out, out_dtype, lse,
                        advance, workspace, workspace_bytes, stream);
}

int sparse_attn_decode_grouped(const sa_kv_desc* kv, const void* q, int32_t num_q_rows, const int32_t* sel_pages,
                               const int32_t* sel_count, int32_t k_max, int32_t sink_len, int32_t window_len,
                               float softmax_scale, int32_t token_splits, int32_t local_splits, float* part_o,
                               float* part_ml, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    sa::Geometry g;
    const int rc = check_kv(kv, &g);
    if (rc != SA_OK) return rc;
    return grouped_impl(kv, g, q, num_q_rows, sel_pages, sel_count, k_max, sink_len, window_len, softmax_scale,
                        token_splits, local_splits, part_o, part_ml, workspace, workspace_bytes,
                        kv->max_pages_per_seq, nullptr, nullptr, nullptr, 0, nullptr, stream);
}

size_t sparse_attn_keydiff_workspace_bytes(const sa_kv_desc* kv, int32_t sink_len, int32_t budget)
{
    sa::Geometry g;
    if (check_kv(kv, &g) != SA_OK || sink_len < 0 || budget < 1) return 0;
    return keydiff_ws(kv, sink_len, budget).total;
}

namespace {

int keydiff_select_impl(const sa_kv_desc* kv, int32_t sink_len, int32_t budget, const float* slot_sums,
                        int32_t slot_groups, const int32_t* carried_count, int32_t* kept, int32_t* kept_count,
                        void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    sa::Geometry g;
    const int rc = check_kv(kv, &g);
    if (rc != SA_OK) return rc;
    if (!kept || !kept_count || sink_len < 0 || budget < 1 || budget < sink_len) return SA_ERR_INVALID_ARG;
    if ((long)kv->batch * kv->num_kv_heads > kMaxGridY) return SA_ERR_UNSUPPORTED;
    if (!keydiff_fits(kv, sink_len, budget)) return SA_ERR_UNSUPPORTED;
    const KeydiffWs w = keydiff_ws(kv, sink_len, budget);
    // the top-k reads the order keys as 16-byte vectors
    if (!workspace || workspace_bytes < w.total || ((uintptr_t)workspace & 15) != 0) return SA_ERR_INVALID_ARG;
    char* base = (char*)workspace;
    sa::KeydiffArgs a{g,
                      kv->max_seq_len,
                      w.Tk,
                      sink_len,
                      budget,
                      w.nchunks,
                      (float*)(base + w.partial),
                      (uint32_t*)(base + w.okeys),
                      kept,
                      kept_count,
                      w.ecnk,
                      w.ecnk ? (uint32_t*)(base + w.part_keys) : nullptr,
                      w.ecnk ? (int32_t*)(base + w.part_idx) : nullptr,
                      slot_sums,
                      carried_count,
                      slot_groups};
    return finish(sa::launch_keydiff_select(a, stream), stream);
}

int keydiff_compact_impl(const sa_kv_desc* src, const int32_t* kept, const int32_t* kept_count, int32_t budget,
                         const sa_kv_desc* dst, float* slot_sums, hipStream_t stream)
{
    sa::Geometry gs, gd;
    const int rs = check_kv(src, &gs);
    if (rs != SA_OK) return rs;
    const int rd = check_kv(dst, &gd);
    if (rd != SA_OK) return rd;
    if (!kept || !kept_count || budget < 1) return SA_ERR_INVALID_ARG;
    if (dst->batch != src->batch || dst->num_kv_heads != src->num_kv_heads || dst->head_dim != src->head_dim ||
        dst->dtype != src->dtype)
        return SA_ERR_INVALID_ARG;
    if ((long)dst->max_pages_per_seq * dst->page_size < budget) return SA_ERR_INVALID_ARG;
    if ((long)src->batch * src->num_kv_heads > kMaxGridY) return SA_ERR_UNSUPPORTED;
    if (!grid_fits(((long)budget + sa::kKdSlots - 1) / sa::kKdSlots, 256)) return SA_ERR_UNSUPPORTED;
    sa::CompactArgs a{gs, gd, budget, kept, kept_count, slot_sums};
    return finish(sa::launch_keydiff_compact(a, stream), stream);
}

}  // namespace

int sparse_attn_keydiff_select(const sa_kv_desc* kv, int32_t sink_len, int32_t budget, int32_t* kept,
                               int32_t* kept_count, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    return keydiff_select_impl(kv, sink_len, budget, nullptr, 0, nullptr, kept, kept_count, workspace,
                               workspace_bytes, stream);
}

int sparse_attn_keydiff_select_carried(const sa_kv_desc* kv, int32_t sink_len, int32_t budget,
                                       const float* slot_sums, int32_t slot_groups, const int32_t* carried_count,
                                       int32_t* kept, int32_t* kept_count, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream)
{
    if (!slot_sums || !carried_count || slot_groups < 1) return SA_ERR_INVALID_ARG;
    return keydiff_select_impl(kv, sink_len, budget, slot_sums, slot_groups, carried_count, kept, kept_count,
                               workspace, workspace_bytes, stream);
}

int32_t sparse_attn_keydiff_slot_groups(int32_t budget)
{
    if (budget < 1) return -SA_ERR_INVALID_ARG;
    return (budget + sa::kKdSlots - 1) / sa::kKdSlots;
}

int sparse_attn_keydiff_compact(const sa_kv_desc* src, const int32_t* kept, const int32_t* kept_count,
                                int32_t budget, const sa_kv_desc* dst, hipStream_t stream)
{
    return keydiff_compact_impl(src, kept, kept_count, budget, dst, nullptr, stream);
}

int sparse_attn_keydiff_compact_sums(const sa_kv_desc* src, const int32_t* kept, const int32_t* kept_count,
                                     int32_t budget, const sa_kv_desc* dst, float* slot_sums, hipStream_t stream)
{
    if (!slot_sums) return SA_ERR_INVALID_ARG;
    return keydiff_compact_impl(src, kept, kept_count, budget, dst, slot_sums, stream);
}

int sparse_attn_decode_step_static(const sa_kv_desc* kv, const void* q, int32_t num_q_rows, const void* meta,
                                   int32_t score_mode, int32_t sink_len, int32_t window_len, int32_t token_budget,
                                   float softmax_scale, int32_t num_splits, int32_t* sel_pages, int32_t* sel_count,
                                   void* out, int32_t out_dtype, float* lse, hipStream_t stream)
{
    // every check of both calls before any HIP call
    sa::Geometry g;
    const int rc = check_kv(kv, &g);
    if (rc != SA_OK) return rc;
    if (!out || num_q_rows < 1) return SA_ERR_INVALID_ARG;
    if (out_dtype != SA_F32 && out_dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
    if (num_splits < 1 || num_splits > kMaxSplits) return SA_ERR_INVALID_ARG;
    const long rows = (long)kv->batch * kv->num_q_heads * num_q_rows;
    if (!grid_fits(rows, 64)) return SA_ERR_UNSUPPORTED;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t ws = up(step_ws_bytes(kv, num_q_rows));
    const size_t po_bytes = up((size_t)rows * num_splits * kv->head_dim * sizeof(float));
    const size_t pml_bytes = up((size_t)rows * num_splits * 2 * sizeof(float));
    if (ws + po_bytes + pml_bytes > sa::kStaticScratchBytes) return SA_ERR_SCRATCH;
    const int r0 = check_step(kv, q, num_q_rows, meta, score_mode, sink_len, window_len, token_budget,
                              softmax_scale, num_splits, sel_pages, sel_count);
    if (r0 != SA_OK) return r0;
    void* base = nullptr;
    if (sa::static_scratch(&base) != hipSuccess) return SA_ERR_HIP;
    float* part_o = (float*)((char*)base + ws);
    float* part_ml = (float*)((char*)base + ws + po_bytes);
    const int r1 = sparse_attn_decode_step(kv, q, num_q_rows, meta, score_mode, sink_len, window_len, token_budget,
                                           softmax_scale, num_splits, sel_pages, sel_count, base, ws, part_o, part_ml,
                                           stream);
    if (r1 != SA_OK) return r1;
    return sparse_attn_combine((int32_t)rows, kv->head_dim, num_splits, part_o, part_ml, out, out_dtype, lse, stream);
}

int sparse_attn_combine_advance(int32_t num_rows, int32_t head_dim, int32_t num_splits, const float* part_o,
                                const float* part_ml, void* out, int32_t out_dtype, float* lse, int32_t* seq_lens,
                                int32_t batch, int32_t advance, hipStream_t stream)
{
    if (!seq_lens || batch < 1 || advance < 0) return SA_ERR_INVALID_ARG;
    if (!part_o || !part_ml || !out || num_rows < 1) return SA_ERR_INVALID_ARG;
    if (num_splits < 1 || num_splits > kMaxSplits) return SA_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return SA_ERR_UNSUPPORTED;
    if (out_dtype != SA_F32 && out_dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
    if (!grid_fits(num_rows, 64)) return SA_ERR_UNSUPPORTED;
    sa::CombineArgs a{num_rows, head_dim, num_splits, out_dtype, part_o, part_ml, out, lse, seq_lens, batch, advance};
    return finish(sa::launch_combine(a, stream), stream);
}

int sparse_attn_combine(int32_t num_rows, int32_t head_dim, int32_t num_splits, const float* part_o,
                        const float* part_ml, void* out, int32_t out_dtype, float* lse, hipStream_t stream)
{
    if (!part_o || !part_ml || !out || num_rows < 1) return SA_ERR_INVALID_ARG;
    if (num_splits < 1 || num_splits > kMaxSplits) return SA_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return SA_ERR_UNSUPPORTED;
    if (out_dtype != SA_F32 && out_dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
    if (!grid_fits(num_rows, 64)) return SA_ERR_UNSUPPORTED;
    sa::CombineArgs a{num_rows, head_dim, num_splits, out_dtype, part_o, part_ml, out, lse, nullptr, 0, 0};
    return finish(sa::launch_combine(a, stream), stream);
}

}  // extern "C"
