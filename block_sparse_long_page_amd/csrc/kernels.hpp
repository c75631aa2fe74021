// Internal launcher interface between the C ABI (host validation and
// dispatch) and the gfx950 kernels.  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

constexpr int kSelCap = 1024;        // page-list entries the bf16 decode stages in LDS
constexpr int kRowsWG = 2048;        // rows a decode workgroup resolves per prologue round
constexpr int kFusedMaxCand = 8448;  // pages per sequence the select-and-decode kernel stages in LDS (256k + 8k tokens at P 32)
constexpr int kGroupMaxPages = 4096; // pages per sequence the grouped decode's plan holds in LDS (20 B each)
constexpr int kGroupMaxRows = 128;   // query rows of the grouped decode (two 64-bit mask words per page)

struct FastDivHost {
    uint32_t d, magic, shift;
};

// magic pair for n / d with 0 <= n < 2^31, d >= 1
inline FastDivHost make_fastdiv(uint32_t d)
{
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    uint64_t magic = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
    return FastDivHost{d, (uint32_t)magic, s};
}

struct Geometry {
    int B, Hq, Hkv, G, hd, P, max_pages, num_phys, dtype;
    const void* k;
    const void* v;
    const int32_t* block_table;
    const int32_t* seq_lens;
    FastDivHost pdiv;
};

struct MetaArgs {
    Geometry g;
    int mode;
    int page_begin, page_end;  // logical range (clipped per sequence in the kernel)
    void* meta;
};

struct SelectArgs {
    Geometry g;
    const void* q;
    int Q;
    const void* meta;
    int mode;
    int S, W, k_max;
    int32_t* sel;
    int32_t* count;
    float* scores;   // workspace [B][Hkv][Q][max_pages]
    int score_only;  // 1: scores only (the select-and-decode kernel ranks them)
};

struct DecodeArgs {
    Geometry g;
    const void* q;
    int Q;
    const int32_t* sel;
    const int32_t* count;
    int k_max, S, W;
    int parts;         // bit 0: sink + window, bit 1: selected middle tokens
    float scale_log2;  // softmax scale * log2(e)
    int splits;
    int split_stride;  // partial slots per row
    float* part_o;
    float* part_ml;
};

struct SelectDecodeArgs {
    Geometry g;
    const void* q;
    int Q;
    const float* scores;  // [B][Hkv][Q][max_pages], written by the score kernel
    int k_max, S, W;
    float scale_log2;
    int splits, split_stride;
    float* part_o;
    float* part_ml;
    int32_t* sel;
    int32_t* count;
};

// A page of the union of the rows' page lists of one (sequence, KV head).
struct __attribute__((aligned(16))) GroupPage {
    int32_t page;   // logical page
    int32_t phys;   // its physical page, -1 when unmapped
    int32_t nrows;  // rows that chose it (the slot table names them)
    int32_t pad;
};

// Multi-query decode grouped by page: the union of the rows' page lists is
// streamed once per (sequence, KV head).
struct GroupArgs {
    Geometry g;
    const void* q;
    int Q;
    const int32_t* sel;    // [B][Hkv][Q][k_max], each row ascending
    const int32_t* count;  // [B][Hkv][Q]
    int k_max, S, W;
    float scale_log2;
    int tsplit;        // token chunks per page; slot of (list index j, chunk s) = j * tsplit + s
    int split_stride;  // partial slots per row
    float* part_o;
    float* part_ml;
    // workspace: the plan
    int32_t* nunion;    // [B][Hkv] pages in the union
    GroupPage* upages;  // [B][Hkv][npg] the union in launch order (costliest first)
    int16_t* slots;     // [B][Hkv][npg][kGroupMaxRows] each row's list index of each union page (same
                        // order), -1 for a row that did not choose it
    int npg;            // candidate units per (sequence, KV head): max_pages, or the index's blocks
    // block mode (semantic index; blk_off == nullptr: pages of the paged
    // cache): the units are the blocks of a contiguous per-(b, KV head)
    // layout, whose tokens all precede every row's window
    const int32_t* blk_off;  // [B][Hkv][npg + 1] first row of each block
    const void* blk_k;       // [B][Hkv][blk_n][hd]
    const void* blk_v;
    int blk_n;               // rows per (sequence, KV head)
    const int32_t* blk_end;  // [B][Hkv][npg] end row of each block's visible part, or null (whole blocks)
};

// Semantic block index: spherical k-means of the unit keys of positions
// [0, N) of every (sequence, KV head) into C blocks, and the block layout.
struct IndexArgs {
    Geometry g;
    int N, C, iters;
    // the index (caller's buffers)
    int32_t* offsets;    // [B][Hkv][C + 1]
    int32_t* positions;  // [B][Hkv][N] position of each row of the block layout
    float* centres;      // [B][Hkv][C][hd]
    void* k_blocks;      // [B][Hkv][N][hd]
    void* v_blocks;
    int32_t* assign_out;  // optional copy of the final assignment [B][Hkv][N]
    // workspace
    float* inv_norm;     // [B][Hkv][N] 1 / |k_t| (0 for a zero key)
    uint16_t* cent_bf;   // [B][Hkv][C][hd] the centres rounded to bf16 (the assignment's operand)
    int32_t* assign;     // [B][Hkv][N]
    int32_t* cnt;        // [B][Hkv][C][nchunks] per-chunk block counts, then each chunk's first row
    int32_t* seg_base;   // [B][Hkv][C + 1] first update segment of each block
    int32_t* seg_block;  // [B][Hkv][nseg] block of each segment
    float* seg_sum;      // [B][Hkv][nseg][hd] sum of a segment's unit keys
    int nchunks, nseg;
};

constexpr int kIndexChunk = 1024;    // tokens per counting-sort chunk
constexpr int kIndexSegment = 128;   // rows per centre-update segment
constexpr int kIndexMaxBlocks = 4096;

// Block choice of one (sequence, KV head, row) against an index.
struct SelectBlocksArgs {
    Geometry g;
    const void* q;
    int Q;
    int C;
    const int32_t* offsets;  // [B][Hkv][C + 1]
    const float* centres;    // [B][Hkv][C][hd]
    int budget, k_max;
    int32_t* sel;            // [B][Hkv][Q][k_max] ascending, -1 after the count
    int32_t* count;          // [B][Hkv][Q]
    const int32_t* ends;     // [B][Hkv][C] end row of each block's visible part, or null (whole blocks)
};

// end row of the visible part of every block: the rows of positions before
// L - W (positions ascend inside a block, so the part is a prefix)
struct VisibleArgs {
    Geometry g;
    int N, C, W;
    const int32_t* offsets;    // [B][Hkv][C + 1]
    const int32_t* positions;  // [B][Hkv][N]
    int32_t* ends;             // [B][Hkv][C]
};

// KeyDiff eviction of a cache back to a token budget (distance of each key to
// the mean key; the sink is kept)
constexpr int kKdChunk = 512;      // tokens per workgroup of the sum and distance passes
constexpr int kKdMaxCand = 12288;  // candidates the top-k workgroup holds in LDS

struct KeydiffArgs {
    Geometry g;
    int T;             // longest sequence (the descriptor's max_seq_len)
    int Tk;            // row stride of okeys: T rounded up to a multiple of 4
    int sink, budget;
    int nchunks;       // ceil(T / kKdChunk)
    float* partial;    // [B][Hkv][nchunks][hd] fp32 key sums of each chunk
    uint32_t* okeys;   // [B][Hkv][Tk] order keys of the squared distances to the mean
                       // key, position t at index L-1-t (the candidates come first)
    int32_t* kept;     // [B][Hkv][budget] kept positions ascending, -1 after the count
    int32_t* count;    // [B][Hkv]
};

struct CompactArgs {
    Geometry src, dst;
    int budget;
    const int32_t* kept;
    const int32_t* count;
};

struct CombineArgs {
    int rows, hd, splits, out_dtype;
    const float* part_o;
    const float* part_ml;
    void* out;
    float* lse;
};

// Each returns hipSuccess or the launch error; 1 for an unsupported
// template combination (the host layer checks these first).
hipError_t launch_page_meta(const MetaArgs& a, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_select_decode(const SelectDecodeArgs& a, hipStream_t s);
// resident decode workgroups per CU for this shape (occupancy query)
int decode_wgs_per_cu(int hd, int G, int dtype);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
// plan kernel, then the grouped decode over max_union pages per (sequence, KV head)
hipError_t launch_group(const GroupArgs& a, int max_union, hipStream_t s);
// the whole index build (every kernel of every iteration)
hipError_t launch_index_build(const IndexArgs& a, hipStream_t s);
hipError_t launch_select_blocks(const SelectBlocksArgs& a, hipStream_t s);
hipError_t launch_blocks_visible(const VisibleArgs& a, hipStream_t s);
// key sums, distances and the kept positions
hipError_t launch_keydiff_select(const KeydiffArgs& a, hipStream_t s);
hipError_t launch_keydiff_compact(const CompactArgs& a, hipStream_t s);

}  // namespace sa
