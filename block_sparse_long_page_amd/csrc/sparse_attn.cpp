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
constexpr int kMaxSelectPages = 12288;  // the top-k workgroup holds one key per page in LDS
constexpr long kMaxGridY = 65535;
constexpr int kMaxTokenSplits = 64;  // token chunks per page of the grouped decode

bool sync_mode()
{
    static const int on = [] {
        const char* e = getenv("SPARSE_ATTN_SYNC");
        return e && e[0] == '1' ? 1 : 0;
    }();
    return on != 0;
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

// workspace of the KeyDiff selection: the chunk key sums, then the order
// keys of the distances (rows padded to a multiple of 4), each 256-byte
// aligned
struct KeydiffWs {
    int nchunks, Tk;
    size_t partial, okeys, total;
};
KeydiffWs keydiff_ws(const sa_kv_desc* kv)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t bh = (size_t)kv->batch * kv->num_kv_heads;
    KeydiffWs w;
    w.nchunks = (kv->max_seq_len + sa::kKdChunk - 1) / sa::kKdChunk;
    w.Tk = (kv->max_seq_len + 3) & ~3;
    w.partial = 0;
    w.okeys = up(bh * (size_t)w.nchunks * kv->head_dim * sizeof(float));
    w.total = up(w.okeys + bh * (size_t)w.Tk * sizeof(uint32_t));
    return w;
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

size_t select_ws_bytes(const sa_kv_desc* kv, int32_t rows)
{
    return sizeof(float) * (size_t)kv->batch * kv->num_kv_heads * rows * kv->max_pages_per_seq;
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
    default: return "unknown status";
    }
}

size_t sparse_attn_workspace_bytes(const sa_kv_desc* kv, int32_t num_q_rows)
{
    if (!kv || num_q_rows < 1 || kv->batch < 1 || kv->num_kv_heads < 1 || kv->max_pages_per_seq < 1) return 0;
    return select_ws_bytes(kv, num_q_rows);
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
        if (kv->max_pages_per_seq > kMaxSelectPages) return SA_ERR_UNSUPPORTED;
        if (!workspace || workspace_bytes < select_ws_bytes(kv, num_q_rows)) return SA_ERR_INVALID_ARG;
    }
    sa::SelectArgs a{g, q, num_q_rows, meta, score_mode, sink_len, window_len, k_max, sel_pages, sel_count,
                     (float*)workspace, 0};
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
    const long wgs = (long)kv->batch * kv->num_kv_heads * num_q_rows * num_splits;
    if (wgs > 0x7fffffffl) return SA_ERR_UNSUPPORTED;
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
    sa::Geometry g;
    const int rc = check_kv(kv, &g);
    if (rc != SA_OK) return rc;
    if (score_mode < SA_QUEST || score_mode > SA_COMPRESSED) return SA_ERR_UNSUPPORTED;
    if (!q || !meta || !sel_count || !part_o || !part_ml || num_q_rows < 1 || sink_len < 0 || window_len < 1 ||
        token_budget < 0)
        return SA_ERR_INVALID_ARG;
    if (num_q_rows > kv->max_seq_len) return SA_ERR_INVALID_ARG;
    const int k_max = token_budget / kv->page_size;
    if (k_max > 0 && !sel_pages) return SA_ERR_INVALID_ARG;
    if (num_splits < 1 || num_splits > kMaxSplits) return SA_ERR_INVALID_ARG;
    if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return SA_ERR_INVALID_ARG;
    if ((long)kv->batch * kv->num_kv_heads * num_q_rows > kMaxGridY) return SA_ERR_UNSUPPORTED;
    if ((long)kv->batch * kv->num_kv_heads * num_q_rows * num_splits > 0x7fffffffl) return SA_ERR_UNSUPPORTED;
    if (k_max > 0) {
        if (kv->max_pages_per_seq > kMaxSelectPages) return SA_ERR_UNSUPPORTED;
        if (!workspace || workspace_bytes < select_ws_bytes(kv, num_q_rows)) return SA_ERR_INVALID_ARG;
    }
    // the fused kernel reads the block-table and score rows as 16-byte vectors
    const bool aligned = kv->max_pages_per_seq % 4 == 0 && ((uintptr_t)kv->block_table & 15) == 0 &&
                         ((uintptr_t)workspace & 15) == 0;
    const bool fused = kv->dtype == SA_BF16 && k_max >= 1 && k_max <= sa::kSelCap &&
                       kv->max_pages_per_seq <= sa::kFusedMaxCand && aligned &&
                       num_splits >= fused_min_splits(sink_len, window_len, k_max, kv->page_size);
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)kv->head_dim);
    if (!fused) {
        const int r1 = sparse_attn_select(kv, q, num_q_rows, meta, score_mode, sink_len, window_len, token_budget,
                                          sel_pages, sel_count, workspace, workspace_bytes, stream);
        if (r1 != SA_OK) return r1;
        return sparse_attn_decode(kv, q, num_q_rows, sel_pages, sel_count, k_max, sink_len, window_len, SA_PART_ALL,
                                  softmax_scale, num_splits, num_splits, part_o, part_ml, stream);
    }
    sa::SelectArgs sarg{g,        q,          num_q_rows, meta,      score_mode, sink_len, window_len,
                        k_max,    sel_pages,  sel_count,  (float*)workspace, 1};
    const int r1 = finish(sa::launch_select(sarg, stream), stream);
    if (r1 != SA_OK) return r1;
    sa::SelectDecodeArgs d{g,          q,          num_q_rows, (const float*)workspace,
                           k_max,      sink_len,   window_len, scale * 1.4426950408889634f,
                           num_splits, num_splits, part_o,     part_ml,
                           sel_pages,  sel_count};
    return finish(sa::launch_select_decode(d, stream), stream);
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
    if ((long)kv->batch * kv->num_kv_heads * num_q_rows * local_splits > 0x7fffffffl) return SA_ERR_UNSUPPORTED;
    const GroupedWs w = grouped_ws(kv, npg);
    if (k_max > 0 && (!workspace || workspace_bytes < w.total || ((uintptr_t)workspace & 255) != 0))
        return SA_ERR_INVALID_ARG;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)kv->head_dim);
    const float sl2 = scale * 1.4426950408889634f;
    if (k_max > 0) {
        char* base = (char*)workspace;
        const long max_union = std::min<long>(npg, (long)num_q_rows * k_max);
        sa::GroupArgs a{g,          q,          num_q_rows, sel,     cnt,
                        k_max,      sink_len,   window_len, sl2,     token_splits,
                        (int)stride, part_o,    part_ml,    (int32_t*)(base + w.nunion),
                        (sa::GroupPage*)(base + w.upages), (int16_t*)(base + w.slots),
                        npg,        blk_off,    blk_k,      blk_v,   blk_n,
                        blk_end};
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
    if ((long)kv->batch * kv->num_kv_heads * num_q_rows > 0x7fffffffl) return SA_ERR_UNSUPPORTED;
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

size_t sparse_attn_keydiff_workspace_bytes(const sa_kv_desc* kv)
{
    sa::Geometry g;
    if (check_kv(kv, &g) != SA_OK) return 0;
    return keydiff_ws(kv).total;
}

int sparse_attn_keydiff_select(const sa_kv_desc* kv, int32_t sink_len, int32_t budget, int32_t* kept,
                               int32_t* kept_count, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    sa::Geometry g;
    const int rc = check_kv(kv, &g);
    if (rc != SA_OK) return rc;
    if (!kept || !kept_count || sink_len < 0 || budget < 1 || budget < sink_len) return SA_ERR_INVALID_ARG;
    if ((long)kv->batch * kv->num_kv_heads > kMaxGridY) return SA_ERR_UNSUPPORTED;
    // the top-k workgroup holds every candidate's key in LDS
    if (kv->max_seq_len > budget && (long)kv->max_seq_len - sink_len > sa::kKdMaxCand) return SA_ERR_UNSUPPORTED;
    const KeydiffWs w = keydiff_ws(kv);
    // the top-k reads the order keys as 16-byte vectors
    if (!workspace || workspace_bytes < w.total || ((uintptr_t)workspace & 15) != 0) return SA_ERR_INVALID_ARG;
    char* base = (char*)workspace;
    sa::KeydiffArgs a{g,         kv->max_seq_len, w.Tk, sink_len, budget, w.nchunks, (float*)(base + w.partial),
                      (uint32_t*)(base + w.okeys), kept, kept_count};
    return finish(sa::launch_keydiff_select(a, stream), stream);
}

int sparse_attn_keydiff_compact(const sa_kv_desc* src, const int32_t* kept, const int32_t* kept_count,
                                int32_t budget, const sa_kv_desc* dst, hipStream_t stream)
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
    sa::CompactArgs a{gs, gd, budget, kept, kept_count};
    return finish(sa::launch_keydiff_compact(a, stream), stream);
}

int sparse_attn_combine(int32_t num_rows, int32_t head_dim, int32_t num_splits, const float* part_o,
                        const float* part_ml, void* out, int32_t out_dtype, float* lse, hipStream_t stream)
{
    if (!part_o || !part_ml || !out || num_rows < 1) return SA_ERR_INVALID_ARG;
    if (num_splits < 1 || num_splits > kMaxSplits) return SA_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return SA_ERR_UNSUPPORTED;
    if (out_dtype != SA_F32 && out_dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
    sa::CombineArgs a{num_rows, head_dim, num_splits, out_dtype, part_o, part_ml, out, lse};
    return finish(sa::launch_combine(a, stream), stream);
}

}  // extern "C"
