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
    uint32_t* status;  // the step's status word, cleared by the score kernel (or null)
    // Selection over more candidates than one workgroup holds: a local top-k
    // per chunk of kTopkChunk candidates, then a merge of the chunks' winners
    // (nchunks == 0: one workgroup per problem ranks all its candidates).
    int nchunks;           // chunks per problem
    int kc;                // winners per chunk: min(k_max, kTopkChunk)
    uint32_t* part_keys;   // [B][Hkv][Q][nchunks][kc] order keys of each chunk's winners
    int32_t* part_idx;     // [B][Hkv][Q][nchunks][kc] their candidate indices, ascending
    uint32_t* counters;    // the merging decode's counters, cleared by the score kernel (or null)
    int ncounters;
};

constexpr int kTopkChunk = 8192;   // candidates a chunk of the two-stage selection ranks
constexpr int kTopkMerge = 12288;  // winners the merge workgroup ranks (nchunks * kc)

// The merge of a decode kernel's split partials in its own last workgroup
// per (sequence, KV head, row) (out == null: partials only).  The partials
// go out with agent-scope stores, then each workgroup counts itself in; the
// last one reads them back with agent-scope loads and merges as the combine
// kernel does.  The counters return to zero by the end of every launch.
constexpr int kMergeMaxSplits = 64;  // splits a merging decode supports
struct MergeArgs {
    void* out;              // [B * Hq * Q][hd], out_dtype
    int out_dtype;          // 1: bf16, else fp32
    float* lse;             // [B * Hq * Q] or null
    uint32_t* arrive;       // [B][Hkv][Q] workgroups arrived
    uint32_t* batch_done;   // [B] (sequence, KV head, row)s merged
    int32_t* seq_lens;      // or null: seq_lens[b] += advance once every problem of b has merged
    int advance;
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
    MergeArgs m;
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
    uint32_t* status;  // set to kStatusGaveUp by a workgroup whose bounded wait ran out
    int spin_max;      // bound on the wait for the page list (rounds)
    MergeArgs m;
};

constexpr uint32_t kStatusGaveUp = 1;  // a share of the attended set was not computed

// A unit of the union of the rows' lists of one (sequence, KV head): a page
// of the paged cache, or a block of an index.
struct __attribute__((aligned(16))) GroupPage {
    int32_t page;   // logical page, or block
    int32_t phys;   // page: its physical page, -1 when unmapped; block: its first row in the block layout
    int32_t nrows;  // rows that chose it (the slot table names them)
    int32_t pad;    // block: the end of its (visible) rows; page: 0
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
    // prefill mode (pf_rows != null; block mode, no plan): units 0 .. nwin-1
    // are the pages of the rows' window [L - W, L), attended causally by the
    // rows at or after each token chunk's start (list index k_max + unit);
    // then the blocks, each attended by the rows whose slot in
    // slots[b][kvh][block][row] is >= 0 (the slot table is indexed by block)
    int nwin;                      // window units per (sequence, KV head)
    const unsigned char* pf_rows;  // [nck][B][Hkv][npg][16] rows of each row group of 8 that chose each block
    int32_t* ctr;                  // [nck][B][Hkv] prefill: item counters, zero when the decode starts
    // prefill: chunks of Q rows in the call (1 otherwise); chunk j's rows are
    // rows j*Q .. of q and the partials (row stride nck*Q), its length
    // seq_lens[b] + j*Q, and slots, pf_rows, blk_end and ctr hold one copy
    // per chunk (index vb = j * B * Hkv + bk)
    int nck;
};

// Query columns (row, head) of one pass of a grouped-decode workgroup (16 per
// wave, 8 waves); a unit with more columns is split into items of one pass.
constexpr int kGroupPassCols = 128;
// Fewest tokens of a token chunk: a unit of n tokens has min(tsplit,
// ceil(n / kGroupChunkMin)) chunks (one item streams a chunk).
constexpr int kGroupChunkMin = 512;

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
constexpr int kIndexRowsPerThread = 4;  // keys a lane group of the norms handles
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
    // More candidates than one workgroup holds: each chunk of kTopkChunk
    // candidates (position order) picks its tokens to evict, and a merge
    // picks the evicted set among them (ecnk == 0: one workgroup ranks all)
    int ecnk;             // chunks per (sequence, KV head)
    uint32_t* part_keys;  // [B][Hkv][ecnk][kTopkChunk] inverted order keys of each chunk's picks
    int32_t* part_idx;    // [B][Hkv][ecnk][kTopkChunk] their candidate indices, ascending
    // Key sums carried from the compaction that filled the cache (null: none):
    // group i of (b, kvh) is the sum of the keys of positions [64i, 64i + 64);
    // a chunk of positions below carried_count[b][kvh] takes its sum from its
    // groups instead of the keys.
    const float* carried;          // [B][Hkv][carried_groups][hd]
    const int32_t* carried_count;  // [B][Hkv]
    int carried_groups;
};
constexpr int kKdMaxChunks = 16;  // chunks of the two-stage eviction (131072 candidates)

// The front of a sparse prefill chunk over a block index: visible ends,
// block choice of every row and the grouped decode's slot table.
constexpr int kPfMaxBlocks = 512;  // index blocks the front holds (8 block keys per lane)
// One call serves nck consecutive chunks of Q rows: chunk j's rows are rows
// j*Q .. j*Q + Q-1 of the row dimension (nck*Q rows of q, lists and
// partials), its length is seq_lens[b] + j*Q, and its per-chunk arrays are
// indexed by vb = j * B * Hkv + b * Hkv + kvh.
constexpr int kPfMaxChunks = 16;
struct PrefillArgs {
    Geometry g;
    const void* q;             // [B][Hq][nck * Q][hd]
    int Q, N, C, nck;
    const int32_t* offsets;    // [B][Hkv][C + 1]
    const int32_t* positions;  // [B][Hkv][N]
    const float* centres;      // [B][Hkv][C][hd]
    int budget[kPfMaxChunks];  // token budget of each chunk
    int k_max, W;
    int tsplit, split_stride;  // token chunks per block; partial slots per row
    int32_t* ends;             // [nck][B][Hkv][C] out: end row of each block's visible part
    int32_t* sel;              // [B][Hkv][nck * Q][k_max] out
    int32_t* count;            // [B][Hkv][nck * Q] out
    int16_t* slots;            // [nck][B][Hkv][C][kGroupMaxRows] out: each row's list index of each block, -1 if not chosen
    float* part_ml;            // the (m, l) of the list slots a row leaves unused are set empty
    unsigned char* rows;       // [nck][B][Hkv][C][16] out: rows of each row group of 8 that chose each block (0 past the groups)
    int32_t* ctr;              // [nck][B][Hkv] the grouped decode's item counters, cleared here
};

struct CompactArgs {
    Geometry src, dst;
    int budget;
    const int32_t* kept;
    const int32_t* count;
    float* slot_sums;  // null, or [B][Hkv][ceil(budget / kKdSlots)][hd]: the key sum of each group of slots
};
constexpr int kKdSlots = 64;  // destination slots per compaction workgroup, and per carried key sum

struct CombineArgs {
    int rows, hd, splits, out_dtype;
    const float* part_o;
    const float* part_ml;
    void* out;
    float* lse;
    int32_t* seq_lens;  // or null: after the merge, seq_lens[b] += advance for b < batch
    int batch, advance;
};

// The static device scratch of the entry point that allocates nothing:
// its size, and its device address on the current device (taken once per
// device with hipGetSymbolAddress, then kept).
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
hipError_t static_scratch(void** ptr);

// Each returns hipSuccess or the launch error; 1 for an unsupported
// template combination (the host layer checks these first).
hipError_t launch_page_meta(const MetaArgs& a, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_select_decode(const SelectDecodeArgs& a, hipStream_t s);
// resident decode workgroups per CU for this shape (occupancy query)
int decode_wgs_per_cu(int hd, int G, int dtype);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
// n zeros at p (a kernel, so that a captured graph holds no memset node)
hipError_t launch_zero_u32(uint32_t* p, long n, hipStream_t s);
// plan kernel, then the grouped decode over max_union units per (sequence, KV head)
hipError_t launch_group(const GroupArgs& a, int max_union, hipStream_t s);
// the grouped decode in prefill mode (no plan kernel; persistent: `workgroups`, a multiple of 8)
hipError_t launch_group_prefill(const GroupArgs& a, int workgroups, hipStream_t s);
// resident grouped-decode workgroups on the device (CUs times occupancy), a multiple of 8
int group_workgroups(int hd, int G);
hipError_t launch_prefill_choose(const PrefillArgs& a, hipStream_t s);
// the whole index build (every kernel of every iteration)
hipError_t launch_index_build(const IndexArgs& a, hipStream_t s);
hipError_t launch_select_blocks(const SelectBlocksArgs& a, hipStream_t s);
hipError_t launch_blocks_visible(const VisibleArgs& a, hipStream_t s);
// key sums, distances and the kept positions
hipError_t launch_keydiff_select(const KeydiffArgs& a, hipStream_t s);
hipError_t launch_keydiff_compact(const CompactArgs& a, hipStream_t s);

}  // namespace sa
