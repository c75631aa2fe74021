/*
 * sparse_attn.h -- C ABI of block/page-sparse long-context decode attention
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (hybrid sparse attention page: full-attention layers attend a
 * 256-token prefix, a recent window and the pages that Quest scores highest;
 * semantic-blocks page: queries are compared with block centres and attend
 * the chosen blocks; course module 14, sections 14.2-14.3: attention sink +
 * window, block gating) runs as four calls on a caller-owned HIP stream:
 *
 *   sparse_attn_build_page_meta  page summaries (min/max, mean or centroid)
 *   sparse_attn_select           score pages, per-KV-head top-k
 *   sparse_attn_decode           exact softmax attention over sink, window and
 *                                the selected pages, split over the token set
 *   sparse_attn_combine          log-sum-exp merge of the split partials
 *   sparse_attn_decode_grouped   multi-query decode that reads each selected
 *                                page once for all the rows that chose it
 *
 * and, for the semantic block index (semantic-blocks page: spherical k-means
 * of the normalised keys into blocks, keys and values laid out block by
 * block, blocks chosen by centre score up to a token budget):
 *
 *   sparse_attn_build_block_index  k-means and the block layout
 *   sparse_attn_select_blocks      per-row block choice under a token budget
 *   sparse_attn_decode_blocks      grouped decode over the chosen blocks plus
 *                                  the window of recent tokens
 *   sparse_attn_blocks_visible     the part of each block before a prompt
 *                                  chunk's window (chunked prefill over an
 *                                  index of the whole prompt)
 *   sparse_attn_prefill_chunk(s)   one chunk (or up to 16 consecutive
 *                                  chunks) of that prefill in three launches
 *
 * and, for KeyDiff eviction (course module 14, section 14.4: tokens whose
 * keys lie closest to the mean key are evicted, the sink never, blockwise so
 * the cache never exceeds its budget by more than a block):
 *
 *   sparse_attn_keydiff_select     the tokens each (sequence, KV head) keeps
 *   sparse_attn_keydiff_compact    their K and V rows, in order, into a cache
 *                                  of the budget's size
 *   sparse_attn_keydiff_compact_sums, sparse_attn_keydiff_select_carried
 *                                  the same with the held keys' sums carried
 *                                  from one eviction to the next
 *
 * sparse_attn_decode_step runs select and decode of a selecting step with the
 * top-k inside the decode kernel (two launches instead of three).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership.  The caller allocates and owns every device buffer and the
 *   stream.  The library allocates nothing, frees nothing and never
 *   synchronises; its process-wide state is a table of occupancy figures,
 *   each queried from the runtime once per kernel shape and read-only
 *   afterwards, and the static scratch of sparse_attn_decode_step_static
 *   (a device array of the code object, with its address per device).  Calls on different streams are independent.  Work
 *   is queued on `stream` and is complete when the stream is.  All pointers
 *   are device pointers unless stated otherwise.
 * Errors.  Every argument is checked on the host before any HIP call; a bad
 *   argument returns SA_ERR_INVALID_ARG or SA_ERR_UNSUPPORTED and queues
 *   nothing.  A call whose launches would exceed the dispatch limit of 2^32
 *   work-items returns SA_ERR_UNSUPPORTED.  SA_ERR_HIP reports a failed
 *   kernel launch.  No C++ exception
 *   crosses the boundary.  Device-side contents (seq_lens, block_table,
 *   selected pages) cannot be checked on the host: the kernels clamp
 *   seq_lens[b] to [0, max_pages_per_seq*page_size], ignore block-table
 *   entries outside [0, num_phys_pages) and selected pages outside the
 *   candidate range, so bad contents give wrong numbers, never stray memory
 *   accesses.
 * Positions.  seq_lens[b] = L counts every token in the cache, the current
 *   one(s) included.  With Q query rows, row i sits at position L - Q + i and
 *   attends causally (positions <= its own).
 * Regions (StreamingLLM sink + window, course module 14, section 14.2; window
 *   of the w most recent positions, self-indexing attention page, "Sliding
 *   window").  sink = [0, min(S, L)); window = [max(sink end, L - W), L)
 *   (the current token is in the window, so W >= 1); middle = between them.
 *   A page is a candidate when it holds at least one middle token.  The
 *   attended set is sink + window + the middle tokens of the selected pages,
 *   each token once.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define SA_OK 0
#define SA_ERR_INVALID_ARG 1  /* null pointer, bad size or range, workspace too small */
#define SA_ERR_UNSUPPORTED 2  /* valid but not built: head_dim, GQA ratio, dtype, mode */
#define SA_ERR_HIP 3          /* a kernel launch failed (hipGetLastError) */
#define SA_ERR_SCRATCH 4      /* sparse_attn_decode_step_static: more than the static scratch holds */

/* element types of K, V, q, Quest summaries and outputs */
#define SA_F32 0
#define SA_BF16 1

/* parts of the attended set a decode call covers */
#define SA_PART_LOCAL 1  /* the sink and the window */
#define SA_PART_MIDDLE 2 /* the middle-region tokens of the selected pages */
#define SA_PART_ALL 3

/* page-summary / scoring modes */
#define SA_QUEST 0    /* per-channel min and max; score = sum_c max(q_c*min_c, q_c*max_c) */
#define SA_MEAN 1     /* mean key of the page (MoBA-style block key); score = q.mean */
#define SA_CENTROID 2 /* unit-norm mean of unit-norm keys (semantic block centre); score = q.c */
#define SA_COMPRESSED 3 /* mean key of the block of two pages starting at the page (compressed keys
                           with block length 2P and stride P); score = max(q.c_p, q.c_{p-1}) */

/*
 * The paged KV cache (PagedAttention-style page management, attention-
 * mechanisms article, "Basic math and real cost").
 *
 *   k_cache, v_cache  [num_phys_pages][num_kv_heads][page_size][head_dim]
 *                     in `dtype`; one (page, KV head) slab is contiguous.
 *   block_table       int32 [batch][max_pages_per_seq]: logical page ->
 *                     physical page.  Entries past a sequence's last page
 *                     are never read.
 *   seq_lens          int32 [batch]: tokens in each sequence (see above).
 *
 * Limits: batch >= 1; num_kv_heads >= 1; num_q_heads = G * num_kv_heads with
 * G (the GQA ratio) in {1, 2, 4, 8, 16}; head_dim in {64, 128};
 * 1 <= page_size <= 16384; max_pages_per_seq >= 1; num_phys_pages >= 1;
 * 1 <= max_seq_len <= max_pages_per_seq * page_size and max_seq_len < 2^30
 * (host-side bound on every seq_lens[b], used for grid sizing).
 */
typedef struct sa_kv_desc {
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t max_pages_per_seq;
    int32_t num_phys_pages;
    int32_t max_seq_len;
    int32_t dtype; /* SA_F32 or SA_BF16 */
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_table;
    const int32_t* seq_lens;
} sa_kv_desc;

/*
 * Page summaries (hybrid sparse attention page: Quest pages; course module
 * 14, section 14.3: one key per block; semantic-blocks page: block centres
 * from normalised keys).
 *
 * For every sequence b, KV head and logical page p in
 * [page_begin, min(page_end, ceil(L_b / page_size))) whose block-table entry
 * is a valid physical page, summarises the page's valid tokens
 * [p*P, min((p+1)*P, L_b)) into meta at (b, KV head, p):
 *   SA_QUEST     meta [batch][num_kv_heads][max_pages_per_seq][2][head_dim]
 *                in `dtype`: [0] = per-channel min, [1] = per-channel max
 *                (exact).
 *   SA_MEAN      meta [batch][num_kv_heads][max_pages_per_seq][head_dim]
 *                fp32: mean key.
 *   SA_CENTROID  same layout: u = sum_t k_t/|k_t| (zero keys skipped),
 *                meta = u/|u| (zeros when u = 0).
 *   SA_COMPRESSED same layout: mean of the valid keys of pages p and p+1
 *                (self-indexing attention page, "Compressed keys": blocks of
 *                2P keys with stride P, mean-pooled); page p+1 counts only
 *                when page p is full and p+1 is mapped.  A change to page p
 *                also changes summary p-1, so after an append rebuild
 *                [last-1, last+1).
 * Summaries are indexed by logical page, so selection streams one
 * contiguous run per (sequence, KV head) without going through the block
 * table.  Sums run in fp32.  Pages outside the range are left untouched, so
 * after a one-token append only the last page needs rebuilding.
 * Errors: kv or meta null, page_begin < 0, page_end < page_begin, bad mode.
 */
int sparse_attn_build_page_meta(const sa_kv_desc* kv, int32_t score_mode, int32_t page_begin, int32_t page_end,
                                void* meta, hipStream_t stream);

/*
 * Page selection: scores, then a per-KV-head top-k (hybrid sparse attention
 * page: Quest pages per head; attention-mechanisms article, "Learned top-k
 * sparse attention": top-16 blocks per GQA group; semantic-blocks page:
 * budget L/16).
 *
 *   q           [batch][num_q_heads][num_q_rows][head_dim] in `dtype`.
 *   meta        summaries from sparse_attn_build_page_meta, same score_mode.
 *   sink_len S >= 0, window_len W >= 1 (the window of the selecting step),
 *   token_budget >= 0: k_max = token_budget / page_size pages per KV head.
 *   sel_pages   int32 [batch][num_kv_heads][num_q_rows][k_max] (written only
 *               when k_max > 0): the chosen logical pages in ascending order,
 *               -1 after the last.
 *   sel_count   int32 [batch][num_kv_heads][num_q_rows]: min(k_max, #candidates).
 *   workspace   device scratch of at least sparse_attn_workspace_bytes() bytes;
 *               on return its first B*Hkv*Q*max_pages_per_seq floats hold the
 *               group scores, [batch][num_kv_heads][num_q_rows][max_pages],
 *               of the candidate pages (other entries undefined).
 *
 * For every (b, KV head, row) and candidate page p, each of the G query heads
 * of the group scores the page (SA_QUEST: the exact maximum of q.x over the
 * page's per-channel bounding box, an upper bound on max_t q.k_t; SA_MEAN /
 * SA_CENTROID: q.summary; SA_COMPRESSED: the larger of q.summary_p and, when
 * page p-1 is mapped, q.summary_{p-1}, since both blocks cover page p); the
 * group score is the maximum over the G heads.
 * Scores are fp32 products with fp32 sums (with a bf16 cache the fp32
 * summaries of the dot-product modes enter the matrix cores as three exact
 * bf16 parts).  Pages are ranked by (group score desc, page index asc) in
 * fp32 and the first k kept.  When k_max >= #candidates every candidate is kept (the
 * dense fallback at short context).  Up to 12288 pages per sequence one
 * workgroup ranks a problem's candidates; past that, each chunk of 8192
 * candidates is ranked by its own workgroup and one workgroup per problem
 * ranks the chunks' winners (the same pages: every page among the k best is
 * among its chunk's best).  This needs at most 64 chunks (524288 pages per
 * sequence) and chunks * min(k_max, 8192) <= 12288, e.g. 16384 pages (1M
 * tokens of 64-token pages) with k_max <= 6144.
 * Errors: null pointers (sel_pages may be null only when k_max == 0),
 * num_q_rows < 1, S < 0, W < 1, token_budget < 0, workspace too small;
 * SA_ERR_UNSUPPORTED past the two-stage limits above.
 */
int sparse_attn_select(const sa_kv_desc* kv, const void* q, int32_t num_q_rows, const void* meta,
                       int32_t score_mode, int32_t sink_len, int32_t window_len, int32_t token_budget,
                       int32_t* sel_pages, int32_t* sel_count, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Bytes of device workspace sparse_attn_select and sparse_attn_decode_step
 * need for this cache and row count (the scores and the step's status word). */
size_t sparse_attn_workspace_bytes(const sa_kv_desc* kv, int32_t num_q_rows);

/*
 * Exact softmax attention over the attended set, split over its tokens
 * (FlashAttention's block-by-block softmax with a running maximum and sum,
 * attention-mechanisms article, "FlashAttention does not change what the
 * model looks at"; course module 14, exercise 14.1: logits q.k/sqrt(d)).
 *
 *   q            [batch][num_q_heads][num_q_rows][head_dim] in `dtype`.
 *   sel_pages    [batch][num_kv_heads][num_q_rows][k_max] as written by
 *                sparse_attn_select (ascending candidate pages), with
 *                sel_count [batch][num_kv_heads][num_q_rows]; or NULL for
 *                dense attention (every middle page).
 *   window_len   the effective window: after a refresh the caller passes
 *                W + (steps since the selection), so tokens appended since
 *                stay visible (hybrid sparse attention page: selection
 *                refreshed every 32 steps while the window grows).
 *   parts        SA_PART_ALL, or one of SA_PART_LOCAL (sink and window:
 *                independent of the selection, so it can run on another
 *                stream while sparse_attn_select runs) and SA_PART_MIDDLE
 *                (the selected pages' middle tokens); the two partial
 *                results merge in sparse_attn_combine like any other splits.
 *   softmax_scale  <= 0 selects 1/sqrt(head_dim).
 *   num_splits   1..1024 parts of each row's token set (see
 *                sparse_attn_default_splits); each part is one workgroup.
 *   split_stride slots per row in part_o / part_ml (0 means num_splits,
 *                else >= num_splits); this call writes slots [0, num_splits)
 *                of every row, so a second call can fill the slots after
 *                them through offset pointers.
 *   part_o       fp32 [batch][num_q_heads][num_q_rows][split_stride][head_dim]:
 *                the split's normalised output sum_t e^{z_t-m} v_t / l.
 *   part_ml      fp32 [batch][num_q_heads][num_q_rows][split_stride][2]:
 *                (m, l): m is a reference logit (natural units) within
 *                8 ln 2 below the split's largest logit and l = sum_t e^{z_t-m}.
 *                An empty split writes (-inf, 0) and o = 0.
 * No float atomics; results are bitwise reproducible.
 * Errors: null pointers (sel_count may be null only with sel_pages null),
 * num_q_rows < 1, S < 0, W < 1, k_max < 0, parts not in 1..3, num_splits or
 * split_stride out of range.
 */
int sparse_attn_decode(const sa_kv_desc* kv, const void* q, int32_t num_q_rows, const int32_t* sel_pages,
                       const int32_t* sel_count, int32_t k_max, int32_t sink_len, int32_t window_len, int32_t parts,
                       float softmax_scale, int32_t num_splits, int32_t split_stride, float* part_o, float* part_ml,
                       hipStream_t stream);

/*
 * One selecting step in two launches: the page scores of sparse_attn_select,
 * then one kernel that ranks the pages and decodes.  Each of its workgroups
 * stages its row's block-table row and scores, then one of its waves ranks
 * the pages (the selection depends only on the scores, so every workgroup of
 * a row computes the same page list) while the others stream the
 * workgroup's share of the sink and window tokens; then all its waves take
 * their share of the selected pages' middle tokens.
 * Same arithmetic as sparse_attn_select followed by sparse_attn_decode with
 * parts = SA_PART_ALL; the tokens of a row are split over the workgroups
 * differently, so the partials differ from sparse_attn_decode's by rounding
 * only, and their merge by sparse_attn_combine is the same attention.
 *   Arguments as in sparse_attn_select and sparse_attn_decode (split_stride
 *   = num_splits).  Writes sel_pages / sel_count as sparse_attn_select does,
 *   and part_o / part_ml for sparse_attn_combine.
 *   workspace   at least sparse_attn_workspace_bytes(kv, num_q_rows) bytes:
 *               the scores, then a status word (cleared by the step's first
 *               kernel), then the counters of sparse_attn_decode_step_merged.
 * The fused kernel runs for bf16 caches with 1 <= k_max <= 1024, at most 8448
 * pages per sequence, max_pages_per_seq a multiple of 4, block_table and
 * workspace 16-byte aligned, and num_splits >= (S + W + k_max * page_size) /
 * 2031 (at most 2048 row-table entries per workgroup, 15 of them padding);
 * any other valid call runs sparse_attn_select and then sparse_attn_decode,
 * with the same results.  sparse_attn_step_path tells the caller which.
 * A workgroup of the fused kernel waits for its page list (published by one
 * of its own waves) for a bounded number of rounds; should the bound ever
 * run out, the workgroup writes NaN partials (l = NaN, so the combined row
 * is NaN, never a silently wrong value) and sets the status word.
 * Errors: those of sparse_attn_select and sparse_attn_decode; with
 * SPARSE_ATTN_SYNC=1, SA_ERR_HIP also when the status word is set.
 */
int sparse_attn_decode_step(const sa_kv_desc* kv, const void* q, int32_t num_q_rows, const void* meta,
                            int32_t score_mode, int32_t sink_len, int32_t window_len, int32_t token_budget,
                            float softmax_scale, int32_t num_splits, int32_t* sel_pages, int32_t* sel_count,
                            void* workspace, size_t workspace_bytes, float* part_o, float* part_ml,
                            hipStream_t stream);

/*
 * Multi-query decode grouped by page (semantic-blocks page: the query rows
 * that chose the same block are collected and the block's keys and values
 * are loaded once for all of them).  The same attention as sparse_attn_decode
 * with parts = SA_PART_ALL for num_q_rows rows with per-row page lists: per
 * (sequence, KV head) the union of the rows' selected pages is streamed once,
 * and every page's middle-region tokens are attended by each row (and each
 * of the G heads of the group) that listed it, on the matrix cores.  The sink
 * and window tokens run through the per-row decode.
 *   sel_pages, sel_count, k_max  per-row page lists as sparse_attn_select
 *                writes them: ascending, distinct candidate pages.  An entry
 *                outside the candidate pages, or not above the entry before
 *                it (a repeated page among them), is not attended: its slot
 *                holds an empty partial.  k_max = 0 attends the sink and
 *                window only.
 *   token_splits 1..64 chunks of each page's middle tokens, one workgroup
 *                each (more workgroups for few, long pages).
 *   local_splits >= 1 splits of each row's sink and window tokens.
 *   part_o, part_ml  as in sparse_attn_decode with split_stride =
 *                k_max * token_splits + local_splits (<= 1024): slot
 *                j * token_splits + c holds chunk c of the row's j-th page,
 *                slots k_max * token_splits + s the sink/window split s; an
 *                unused slot holds (m, l) = (-inf, 0) and its o is left
 *                as it was (the combine skips it).  Merge them with
 *                sparse_attn_combine(num_splits = split_stride).
 *   workspace    >= sparse_attn_grouped_workspace_bytes(kv) bytes, 256-byte
 *                aligned (the per-(sequence, KV head) plan: the page union
 *                with its row masks in launch order, the rows' slots);
 *                needed when k_max > 0.
 * bf16 caches, num_q_rows <= 128, max_pages_per_seq <= 4096.  Results are
 * bitwise reproducible (fixed slots, fixed merge order).
 * Errors: those of sparse_attn_decode; SA_ERR_UNSUPPORTED outside the limits
 * above; SA_ERR_INVALID_ARG for a bad split count, a small or misaligned
 * workspace or missing page lists.
 */
int sparse_attn_decode_grouped(const sa_kv_desc* kv, const void* q, int32_t num_q_rows, const int32_t* sel_pages,
                               const int32_t* sel_count, int32_t k_max, int32_t sink_len, int32_t window_len,
                               float softmax_scale, int32_t token_splits, int32_t local_splits, float* part_o,
                               float* part_ml, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of sparse_attn_decode_grouped for this cache (host only; 0 for a bad descriptor). */
size_t sparse_attn_grouped_workspace_bytes(const sa_kv_desc* kv);

/*
 * Semantic block index of a cache (semantic-blocks page: per request, layer
 * and KV head the normalised keys are grouped into semantic blocks by
 * spherical k-means, and the keys and values are laid out again block by
 * block).  It covers positions [0, num_tokens) of every sequence; every
 * sequence must hold at least num_tokens tokens.  All buffers are the
 * caller's device memory; k_blocks, v_blocks and centres 16-byte aligned.
 */
typedef struct sa_block_index {
    int32_t num_tokens;  /* N: indexed positions per sequence, 1 <= N <= max_seq_len */
    int32_t num_blocks;  /* C: 1 <= C <= min(N, 4096) */
    int32_t* offsets;    /* [batch][num_kv_heads][C + 1] first row of each block (CSR) */
    int32_t* positions;  /* [batch][num_kv_heads][N] position of each row of the block layout */
    float* centres;      /* [batch][num_kv_heads][C][head_dim] unit-length block centres */
    void* k_blocks;      /* [batch][num_kv_heads][N][head_dim] keys in block order, KV dtype */
    void* v_blocks;      /* [batch][num_kv_heads][N][head_dim] values in block order */
    /* optional [batch][num_kv_heads][C]: the end row of each block's visible
       part (sparse_attn_blocks_visible); NULL: whole blocks.  Read by
       sparse_attn_select_blocks (block sizes) and sparse_attn_decode_blocks
       (rows attended); the build ignores it. */
    const int32_t* visible_end;
} sa_block_index;

/* Workspace bytes of sparse_attn_build_block_index (host only; 0 for bad sizes). */
size_t sparse_attn_index_workspace_bytes(const sa_kv_desc* kv, int32_t num_tokens, int32_t num_blocks);

/*
 * Builds `index` from the keys and values of kv, per (sequence, KV head):
 * unit keys u_t = k_t / |k_t| (a zero key stays zero); centre c starts as
 * the unit key at position floor(c N / C); `iterations` times each key goes
 * to the centre with the largest dot product (ties: the lower centre; the
 * products use the centres rounded to bf16 and the bf16 keys, summed in
 * fp32 on the matrix cores) and each centre becomes the normalised sum of
 * its unit keys in fp32 (a centre without keys keeps its value).  A last
 * assignment to the final centres defines the blocks: block c holds the
 * keys assigned to c, rows in position order, blocks in order.  offsets,
 * positions, centres and the K/V copies are written; `assignment` (nullable,
 * [batch][num_kv_heads][N] int32) receives that last assignment.  Every sum
 * runs in a fixed order, so the result is bitwise reproducible.
 *   iterations  0..64 (0: the starting centres)
 *   workspace   >= sparse_attn_index_workspace_bytes(kv, N, C) bytes,
 *               256-byte aligned
 * bf16 caches only.  Errors: SA_ERR_INVALID_ARG for missing or misaligned
 * buffers, sizes out of range or a small workspace; SA_ERR_UNSUPPORTED for
 * other dtypes or C > 4096.
 */
int sparse_attn_build_block_index(const sa_kv_desc* kv, int32_t iterations, const sa_block_index* index,
                                  int32_t* assignment, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Block choice of every (sequence, KV head, row) (semantic-blocks page: the
 * query is compared with the block centres and the best blocks are taken up
 * to a budget of tokens): block c scores max over the group's heads of
 * q_h . centre_c (fp32); blocks are taken in order of (score desc, block
 * asc) while the running token count stays <= token_budget, at least one
 * and at most k_max; blocks without tokens are never taken.  With
 * index->visible_end set, a block's size is its visible part (blocks with
 * none are never taken).
 *   q           [batch][num_q_heads][num_q_rows][head_dim], bf16
 *   sel_blocks  [batch][num_kv_heads][num_q_rows][k_max]: the chosen blocks
 *               ascending, -1 after the last; sel_count [..][num_q_rows]
 *   k_max       1..C
 * Errors: as sparse_attn_build_block_index; SA_ERR_INVALID_ARG for k_max out
 * of range or a negative budget.
 */
int sparse_attn_select_blocks(const sa_kv_desc* kv, const sa_block_index* index, const void* q, int32_t num_q_rows,
                              int32_t token_budget, int32_t k_max, int32_t* sel_blocks, int32_t* sel_count,
                              hipStream_t stream);

/*
 * The visible part of every block for a chunk of rows (semantic-blocks page:
 * one index serves the prompt's processing as well as generation, and a
 * prompt chunk attends its own tokens and the recent history without
 * selection): visible_end[b][kvh][c] = the first row of block c whose
 * position is >= L_b - window_len (positions ascend inside a block, so the
 * rows before it, of positions < L_b - window_len, are its visible part).
 * With visible_end stored in index->visible_end, sparse_attn_select_blocks
 * sizes the blocks by their visible parts and sparse_attn_decode_blocks
 * attends only those rows, so an index of the whole prompt serves every
 * chunk: the chunk's rows see the index only before their window.
 *   visible_end  int32 [batch][num_kv_heads][C]
 * Errors: those of the index checks; SA_ERR_INVALID_ARG for a null
 * visible_end or window_len < 0.
 */
int sparse_attn_blocks_visible(const sa_kv_desc* kv, const sa_block_index* index, int32_t window_len,
                               int32_t* visible_end, hipStream_t stream);

/* Workspace bytes of sparse_attn_decode_blocks for this index (host only; 0 for bad sizes). */
size_t sparse_attn_blocks_workspace_bytes(const sa_kv_desc* kv, const sa_block_index* index);

/*
 * The attention of num_q_rows rows over their chosen blocks and the window:
 * each block of the union of the rows' lists (per sequence and KV head) is
 * read once from the block layout and attended by every row that listed it
 * (the grouped decode of sparse_attn_decode_grouped, with blocks for pages),
 * and the window [L - window_len, L) of the paged cache by the per-row
 * decode (no sink).  The blocks' tokens are attended without a causal test:
 * the caller keeps the index to positions before every row's window, i.e.
 * num_tokens <= L - window_len for every sequence, or sets
 * index->visible_end from sparse_attn_blocks_visible with the same
 * window_len (then only the rows before the window are attended), and
 * window_len >= num_q_rows so that the window holds the rows themselves.
 *   sel_blocks, sel_count, k_max  as sparse_attn_select_blocks writes them
 *   token_splits, local_splits, part_o, part_ml  as in
 *               sparse_attn_decode_grouped (slot j * token_splits + c holds
 *               chunk c of the row's j-th block); merge with
 *               sparse_attn_combine(num_splits = k_max * token_splits +
 *               local_splits)
 *   workspace   >= sparse_attn_blocks_workspace_bytes(kv, index) bytes,
 *               256-byte aligned; needed when k_max > 0
 * bf16 caches, num_q_rows <= 128.  Results are bitwise reproducible.
 * Errors: those of sparse_attn_decode_grouped and of the index checks;
 * SA_ERR_INVALID_ARG when window_len < num_q_rows or k_max > C.
 */
int sparse_attn_decode_blocks(const sa_kv_desc* kv, const sa_block_index* index, const void* q, int32_t num_q_rows,
                              const int32_t* sel_blocks, const int32_t* sel_count, int32_t k_max, int32_t window_len,
                              float softmax_scale, int32_t token_splits, int32_t local_splits, float* part_o,
                              float* part_ml, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One chunk of a sparse prefill over a block index of the prompt, in three
 * launches (semantic-blocks page: one index serves the prompt's processing;
 * the queries that chose the same block are grouped so that the block is
 * read once for all of them; the current fragment is attended without
 * selection).  The rows at positions [L - num_q_rows, L) of every sequence
 * (L = its length) see the index only before their window [L - window_len,
 * L):
 *   1. the front, one workgroup per 8 rows: the visible part of every block
 *      (as sparse_attn_blocks_visible), each row's block choice (as
 *      sparse_attn_select_blocks with those visible parts), and the grouped
 *      decode's slot table;
 *   2. the grouped decode: every block chosen by some row is read once
 *      (its visible rows, in token_splits chunks) for all the rows that
 *      chose it, and every page of the window once for all the rows,
 *      causally (row i at position L - num_q_rows + i sees window tokens
 *      up to its own position);
 *   3. the merge of each row's partials (sparse_attn_combine_advance).
 * Same arithmetic as sparse_attn_blocks_visible, sparse_attn_select_blocks,
 * sparse_attn_decode_blocks (local_splits = 1) and sparse_attn_combine: the
 * lists are the same, and the window's tokens are split over the partials
 * differently (per page and token chunk), so outputs differ by rounding only.
 *   q            [batch][num_q_heads][num_q_rows][head_dim], bf16
 *   window_len   >= num_q_rows (the window holds the rows themselves)
 *   token_budget, k_max  as sparse_attn_select_blocks (1 <= k_max <= C)
 *   token_splits 1..64: token chunks per chosen block and per window page
 *   visible_end  out, int32 [batch][num_kv_heads][C] (as
 *                sparse_attn_blocks_visible writes it); index->visible_end
 *                is not read
 *   sel_blocks, sel_count  out, as sparse_attn_select_blocks
 *   part_o, part_ml  [batch * num_q_heads * num_q_rows][num_splits][head_dim]
 *                and [..][num_splits][2] fp32, num_splits =
 *                sparse_attn_prefill_num_splits(kv, window_len, k_max,
 *                token_splits); every slot is written
 *   out, out_dtype, lse  as sparse_attn_combine (lse nullable)
 *   advance      >= 0: kv->seq_lens[b] += advance for every sequence after
 *                the merge (0: the lengths are not written; > 0: seq_lens
 *                must be writable device memory), so a caller can chain the
 *                chunks of a prompt without touching the lengths itself
 *   workspace    >= sparse_attn_prefill_workspace_bytes(kv, index) bytes,
 *                256-byte aligned
 * The caller keeps every sequence's prompt positions before L - window_len
 * inside the index (num_tokens >= L - window_len); rows of positions
 * outside [0, num_tokens) are never visible.  Results are bitwise
 * reproducible.  bf16 caches, num_q_rows <= 128, C <= 512.
 * Errors: those of the index checks; SA_ERR_INVALID_ARG for null outputs,
 * num_q_rows < 1, window_len < num_q_rows, a negative budget or advance,
 * k_max or token_splits out of range, a non-finite scale or a small or
 * misaligned workspace; SA_ERR_UNSUPPORTED for other dtypes, more than 128
 * rows or 512 blocks, num_splits above 1024 or a grid too large.
 */
int sparse_attn_prefill_chunk(const sa_kv_desc* kv, const sa_block_index* index, const void* q, int32_t num_q_rows,
                              int32_t window_len, int32_t token_budget, int32_t k_max, float softmax_scale,
                              int32_t token_splits, int32_t* visible_end, int32_t* sel_blocks, int32_t* sel_count,
                              float* part_o, float* part_ml, void* out, int32_t out_dtype, float* lse,
                              int32_t advance, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Several consecutive chunks of a prompt in one call: the same as
 * num_chunks calls of sparse_attn_prefill_chunk, chunk j on rows
 * j*num_q_rows .. (j+1)*num_q_rows - 1 at length L_b + j*num_q_rows (L_b =
 * kv->seq_lens[b] when the call starts, chunk 0's rows included) with token
 * budget token_budgets[j], and with the same results bit for bit; the three
 * launches serve every chunk, so their fixed costs are paid once.  Chunks are
 * independent once the index is built (each sees the index's tokens before
 * its own window and attends its window causally).
 *   q            [batch][num_q_heads][num_chunks * num_q_rows][head_dim], bf16
 *   num_chunks   1..16
 *   token_budgets  host array of num_chunks budgets (>= 0)
 *   visible_end  out, int32 [num_chunks][batch][num_kv_heads][C]
 *   sel_blocks, sel_count  out, [batch][num_kv_heads][num_chunks *
 *                num_q_rows][k_max] and [..][num_chunks * num_q_rows]
 *   part_o, part_ml  [batch * num_q_heads * num_chunks * num_q_rows]
 *                [num_splits][head_dim] / [..][num_splits][2]
 *   out, lse     [batch][num_q_heads][num_chunks * num_q_rows][head_dim] / [..]
 *   advance      as in sparse_attn_prefill_chunk (num_chunks * num_q_rows to
 *                chain calls)
 *   workspace    >= sparse_attn_prefill_chunks_workspace_bytes(kv, index,
 *                num_chunks) bytes, 256-byte aligned
 * The rest as in sparse_attn_prefill_chunk.  The caller keeps L_b +
 * num_chunks*num_q_rows within the cache (lengths past it are clamped).
 * Errors: those of sparse_attn_prefill_chunk; SA_ERR_INVALID_ARG for
 * num_chunks outside 1..16, a null token_budgets or a negative budget.
 */
int sparse_attn_prefill_chunks(const sa_kv_desc* kv, const sa_block_index* index, const void* q, int32_t num_q_rows,
                               int32_t num_chunks, int32_t window_len, const int32_t* token_budgets, int32_t k_max,
                               float softmax_scale, int32_t token_splits, int32_t* visible_end, int32_t* sel_blocks,
                               int32_t* sel_count, float* part_o, float* part_ml, void* out, int32_t out_dtype,
                               float* lse, int32_t advance, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Workspace bytes of sparse_attn_prefill_chunks for this index and chunk
 * count (host only; 0 for bad sizes or num_chunks outside 1..16). */
size_t sparse_attn_prefill_chunks_workspace_bytes(const sa_kv_desc* kv, const sa_block_index* index,
                                                  int32_t num_chunks);

/* Partial slots per row of sparse_attn_prefill_chunk: (k_max + the window's
 * pages, (window_len - 1) / page_size + 2) * token_splits; negative error
 * code for bad arguments or more than 1024 (host only). */
int32_t sparse_attn_prefill_num_splits(const sa_kv_desc* kv, int32_t window_len, int32_t k_max,
                                       int32_t token_splits);

/* Workspace bytes of sparse_attn_prefill_chunk for this index (host only; 0 for bad sizes). */
size_t sparse_attn_prefill_workspace_bytes(const sa_kv_desc* kv, const sa_block_index* index);

/* Workspace bytes of sparse_attn_keydiff_select for this cache, sink and
 * budget (host only; 0 for a bad descriptor, sink_len < 0 or budget < 1). */
size_t sparse_attn_keydiff_workspace_bytes(const sa_kv_desc* kv, int32_t sink_len, int32_t budget);

/*
 * KeyDiff eviction, the choice (course module 14, section 14.4 and exercise
 * 14.2: importance of a token = how far its key lies from the mean key of the
 * tokens the cache holds; the least distinctive are evicted; the first
 * positions are never evicted).
 *
 * For every sequence b and KV head, over the tokens [0, L_b) the cache holds:
 * m = the mean key (fp32 sums), d_t = |k_t - m|^2 (fp32).  When L_b <= budget
 * every token is kept.  Otherwise the positions [0, min(sink_len, L_b)) and
 * the budget - sink_len others with the largest d_t are kept; among equal
 * distances the later position is kept (the earlier is evicted first).  One
 * call evicts down to the budget at once (the mean is the whole cache's).
 *   kept        int32 [batch][num_kv_heads][budget]: kept positions ascending,
 *               -1 after the count.
 *   kept_count  int32 [batch][num_kv_heads]: min(L_b, budget).
 *   workspace   device scratch of sparse_attn_keydiff_workspace_bytes(kv,
 *               sink_len, budget), 16-byte aligned.
 * Called after each block of new tokens, this keeps a cache within budget +
 * block tokens.  A token whose page is unmapped counts as a zero key.
 * Up to 12288 candidates (max_seq_len - sink_len) one workgroup per
 * (sequence, KV head) ranks them; past that the tokens to evict are chosen
 * instead (the same set): each chunk of 8192 candidates picks its
 * min(evicted, 8192) nearest to the mean (earlier position first among
 * equal distances) and one workgroup per (sequence, KV head) picks the
 * evicted among those and writes the others.  This needs at most 16 chunks
 * (131072 candidates) and chunks * min(max_seq_len - budget, 8192) <= 12288,
 * e.g. a 2048-token block evicted from up to 49152 held tokens.
 * Errors: null pointers, sink_len < 0, budget < 1 or < sink_len, workspace
 * too small or misaligned; SA_ERR_UNSUPPORTED past the limits above or when
 * batch * num_kv_heads > 65535.
 */
int sparse_attn_keydiff_select(const sa_kv_desc* kv, int32_t sink_len, int32_t budget, int32_t* kept,
                               int32_t* kept_count, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * KeyDiff eviction, the copy: the K and V rows of the kept positions of
 * every (sequence, KV head), in order, into slots 0 .. kept_count-1 of the
 * same sequence and KV head in `dst` (the evicted cache is physically
 * shorter).  src and dst share batch, num_kv_heads, head_dim and dtype; dst
 * holds at least `budget` tokens per sequence (max_pages_per_seq *
 * page_size); its page size may differ.  dst's pages must not overlap the
 * pages src reads (rows are copied by many workgroups at once).  The caller
 * sets dst's seq_lens to kept_count.  Kept positions outside src's pages or
 * on unmapped pages, and unmapped dst pages, are skipped.
 * Errors: null pointers, mismatched descriptors, budget < 1 or above dst's
 * capacity.
 */
int sparse_attn_keydiff_compact(const sa_kv_desc* src, const int32_t* kept, const int32_t* kept_count,
                                int32_t budget, const sa_kv_desc* dst, hipStream_t stream);

/*
 * KeyDiff eviction with the held keys' sums carried from the last eviction
 * (course module 14, section 14.4: blockwise eviction; the mean key of the
 * held set is what each eviction measures distances to).  After an eviction
 * the cache holds the kept tokens, whose key sums that eviction's copy can
 * leave behind (sparse_attn_keydiff_compact_sums); until the next eviction
 * only new tokens are appended, so its mean needs the keys of the new block
 * and those sums, not the keys of the whole cache.
 *
 * sparse_attn_keydiff_compact_sums: sparse_attn_keydiff_compact, and for
 * every (sequence, KV head) the fp32 sum of the keys copied into each group
 * of 64 destination slots [64i, 64i + 64) (a key not copied counts as zero),
 * added in a fixed order (bitwise reproducible); groups at or past
 * kept_count are not written.
 *   slot_sums  fp32 [batch][num_kv_heads][sparse_attn_keydiff_slot_groups(
 *              budget)][head_dim]
 *
 * sparse_attn_keydiff_select_carried: sparse_attn_keydiff_select on a cache
 * whose positions [0, carried_count[b][kvh]) hold the keys that a
 * sparse_attn_keydiff_compact_sums call copied there (its slot_sums and its
 * kept_count, for this cache as its dst); new tokens may follow them.  Each
 * 512-position chunk of a (sequence, KV head) that lies wholly below
 * min(carried_count, L_b) takes its key sum from its 8 groups' sums instead
 * of its keys; the others are summed from the keys.  The choice rule is
 * sparse_attn_keydiff_select's; the mean differs from it by fp32 rounding
 * only (the order of the additions).  The caller keeps the carried positions
 * unchanged between the two calls.
 *   slot_sums, slot_groups  as written by the compaction, slot_groups =
 *              sparse_attn_keydiff_slot_groups(its budget)
 *   carried_count  int32 [batch][num_kv_heads], the compaction's kept_count
 *              (values past 64 * slot_groups count as 64 * slot_groups)
 *   the rest as in sparse_attn_keydiff_select (same workspace size).
 * Errors: those of sparse_attn_keydiff_select and sparse_attn_keydiff_compact;
 * SA_ERR_INVALID_ARG for a null slot_sums or carried_count, or slot_groups < 1.
 */
int sparse_attn_keydiff_compact_sums(const sa_kv_desc* src, const int32_t* kept, const int32_t* kept_count,
                                     int32_t budget, const sa_kv_desc* dst, float* slot_sums, hipStream_t stream);
int sparse_attn_keydiff_select_carried(const sa_kv_desc* kv, int32_t sink_len, int32_t budget,
                                       const float* slot_sums, int32_t slot_groups, const int32_t* carried_count,
                                       int32_t* kept, int32_t* kept_count, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/* Groups of 64 slots whose key sums sparse_attn_keydiff_compact_sums writes
 * per (sequence, KV head) for this budget: ceil(budget / 64) (host only;
 * -SA_ERR_INVALID_ARG for budget < 1). */
int32_t sparse_attn_keydiff_slot_groups(int32_t budget);

/* Which kernels sparse_attn_decode_step queues for these arguments (host
 * only): SA_STEP_FUSED (score kernel, then the select-and-decode kernel) or
 * SA_STEP_SEPARATE (sparse_attn_select, then sparse_attn_decode);
 * -SA_ERR_INVALID_ARG for a bad descriptor or range. */
#define SA_STEP_SEPARATE 0
#define SA_STEP_FUSED 1
int32_t sparse_attn_step_path(const sa_kv_desc* kv, int32_t sink_len, int32_t window_len, int32_t token_budget,
                              int32_t num_splits, const void* workspace);

/* A split count that fills the GPU for this shape and suits sparse_attn_decode_step (host only). */
int32_t sparse_attn_default_splits(const sa_kv_desc* kv, int32_t num_q_rows, int32_t sink_len, int32_t window_len,
                                   int32_t k_max);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): one whole
 * selecting step, sparse_attn_decode_step followed by sparse_attn_combine,
 * whose workspace and split partials live in a static device array of the
 * library (16 MiB per GPU, held from the library's load until the process
 * ends) instead of caller buffers.  The caller passes the inputs and the
 * outputs only.
 *   Arguments as in sparse_attn_decode_step (sel_pages, sel_count written
 *   the same way) and sparse_attn_combine (out [batch][num_q_heads]
 *   [num_q_rows][head_dim] in out_dtype, lse fp32 or NULL).
 * The scratch needs the step's workspace (sparse_attn_workspace_bytes) plus
 * batch * num_q_heads * num_q_rows * num_splits * (head_dim + 2) * 4 bytes of
 * partials, each rounded up to 256 bytes; a call needing more than 16 MiB
 * returns SA_ERR_SCRATCH and queues nothing.  Nothing is allocated: the
 * array's device address is looked up once per device, on the first call
 * with that device current.  Every call on a GPU uses that GPU's one array,
 * so calls that overlap on one GPU (on different streams, or from several
 * threads) race and must be serialised by the caller; calls in a row on one
 * stream are fine.  The kernels write every scratch byte they read in the
 * same call (the status word is cleared by the step's first kernel), so the
 * contents a previous call left do not matter.  Results are identical to
 * sparse_attn_decode_step + sparse_attn_combine with the same arguments.
 * Errors: those of the two calls, checked before any HIP call;
 * SA_ERR_SCRATCH as above.
 */
int sparse_attn_decode_step_static(const sa_kv_desc* kv, const void* q, int32_t num_q_rows, const void* meta,
                                   int32_t score_mode, int32_t sink_len, int32_t window_len, int32_t token_budget,
                                   float softmax_scale, int32_t num_splits, int32_t* sel_pages, int32_t* sel_count,
                                   void* out, int32_t out_dtype, float* lse, hipStream_t stream);

/*
 * Log-sum-exp merge of split partials (attention-mechanisms article,
 * DeepSeek-V4 section: combining partial results; the same running-max
 * rescaling as FlashAttention's online softmax).
 *
 * For each of num_rows rows: m* = max_s m_s over non-empty parts,
 * l = sum_s e^{m_s-m*} l_s, out = sum_s e^{m_s-m*} l_s o_s / l,
 * lse = m* + ln l, in a fixed order over s (deterministic).
 *   part_o [num_rows][num_splits][head_dim], part_ml [num_rows][num_splits][2]
 *   out    [num_rows][head_dim] in out_dtype (SA_BF16: round to nearest even)
 *   lse    fp32 [num_rows] or NULL.
 * A part with l = 0 is empty: its o is not read into the sum (it may hold
 * anything).  A row whose parts are all empty gets out = 0 and lse = -inf.
 * A part with l = NaN marks a share that was not computed (see
 * sparse_attn_decode_step): the row's out and lse are NaN.
 * Errors: null pointers, num_rows < 1, head_dim not 64/128, num_splits
 * outside 1..1024, bad out_dtype.
 */
int sparse_attn_combine(int32_t num_rows, int32_t head_dim, int32_t num_splits, const float* part_o,
                        const float* part_ml, void* out, int32_t out_dtype, float* lse, hipStream_t stream);

/*
 * sparse_attn_combine, then every sequence's length advanced:
 * seq_lens[b] += advance for b < batch, inside the same launch.  For the
 * last kernel of a decode step, so that the next step attends the token it
 * appends (hybrid sparse attention page: one token appended per step while
 * the window grows until the next selection) with no separate update of the
 * lengths, which also lets a step be captured in a HIP graph and replayed.
 *   seq_lens   int32 [batch], the descriptor's lengths; no other kernel may
 *              read or write them while the call runs.
 * Errors: those of sparse_attn_combine; SA_ERR_INVALID_ARG for a null
 * seq_lens, batch < 1 or advance < 0.
 */
int sparse_attn_combine_advance(int32_t num_rows, int32_t head_dim, int32_t num_splits, const float* part_o,
                                const float* part_ml, void* out, int32_t out_dtype, float* lse, int32_t* seq_lens,
                                int32_t batch, int32_t advance, hipStream_t stream);

/*
 * The split-K decode with the log-sum-exp merge in its own last workgroups
 * (one launch where sparse_attn_decode + sparse_attn_combine take two; the
 * merge's arithmetic is the combine's, so out and lse are bitwise those of
 * the two calls).  Every workgroup of a (sequence, KV head, row) writes its
 * partials with agent-scope stores (coherent across the XCDs' caches),
 * waits for them to complete and counts itself in; the last of the
 * num_splits to arrive reads the problem's partials back with agent-scope
 * loads, merges its group's rows and clears its counter.  With advance > 0
 * the last problem of each sequence to merge then adds `advance` to the
 * sequence's length (kv->seq_lens is written: device memory), when no
 * workgroup of the launch reads it any more.
 *   Arguments as in sparse_attn_decode with parts = SA_PART_ALL and
 *   split_stride = num_splits, and as in sparse_attn_combine for out,
 *   out_dtype and lse.
 *   num_splits  1..64
 *   counters    uint32 [sparse_attn_merge_counters(kv, num_q_rows)]: zero
 *               before the first call; every call that completes leaves them
 *               zero.  Calls that overlap on one counter array race.
 * bf16 caches.  Errors: those of sparse_attn_decode; SA_ERR_INVALID_ARG for a
 * null out or counters, advance < 0 or num_splits past 64;
 * SA_ERR_UNSUPPORTED for fp32 caches or another out_dtype.
 */
int sparse_attn_decode_merged(const sa_kv_desc* kv, const void* q, int32_t num_q_rows, const int32_t* sel_pages,
                              const int32_t* sel_count, int32_t k_max, int32_t sink_len, int32_t window_len,
                              float softmax_scale, int32_t num_splits, float* part_o, float* part_ml, void* out,
                              int32_t out_dtype, float* lse, int32_t advance, uint32_t* counters, hipStream_t stream);

/* Counters of the merging decode for this shape: one per (sequence, KV head,
 * row) and one per sequence (host only; a negative error code for bad
 * arguments). */
int32_t sparse_attn_merge_counters(const sa_kv_desc* kv, int32_t num_q_rows);

/*
 * A selecting step with the merge in its decode kernel:
 * sparse_attn_decode_step whose select-and-decode kernel (or, on the
 * separate path, whose decode) merges as sparse_attn_decode_merged does; the
 * counters live in the workspace after the status word and are cleared by
 * the step's first kernel (on the separate path by a small fill kernel), so
 * the workspace needs no preparation.  out and lse are bitwise those of
 * sparse_attn_decode_step + sparse_attn_combine.
 *   Arguments as in sparse_attn_decode_step, plus out, out_dtype, lse (as in
 *   sparse_attn_combine) and advance (as in sparse_attn_decode_merged).
 *   workspace  at least sparse_attn_workspace_bytes(kv, num_q_rows) bytes.
 * Errors: those of sparse_attn_decode_step and sparse_attn_decode_merged.
 */
int sparse_attn_decode_step_merged(const sa_kv_desc* kv, const void* q, int32_t num_q_rows, const void* meta,
                                   int32_t score_mode, int32_t sink_len, int32_t window_len, int32_t token_budget,
                                   float softmax_scale, int32_t num_splits, int32_t* sel_pages, int32_t* sel_count,
                                   void* workspace, size_t workspace_bytes, float* part_o, float* part_ml, void* out,
                                   int32_t out_dtype, float* lse, int32_t advance, hipStream_t stream);

/* A static string naming a status code. */
const char* sparse_attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
