// Multi-query decode grouped by page (semantic-blocks page: the queries that
// chose the same block are collected and the block's K/V is loaded once for
// all of them).  Each query row has its own page list (the per-row selection
// of sparse_attn_select with Q rows); this path inverts the lists into, per
// (sequence, KV head), the union of selected pages with a bit mask of the
// rows that chose each page, and then streams every page of the union once.
//
// k_group_plan: one workgroup per (sequence, KV head).  Builds the row masks
// (two 64-bit words per page, up to 128 rows) in LDS with atomic ORs, writes
// the pages that carry a mask as records (page, physical page, rows) in
// launch order (costliest first), records for every row its index in its
// own list of each page of the union (the row's slot for that page; -1 for
// the rows that did not choose it), and marks every slot a row does not use
// (entries past its count, outside the candidates, or not above the entry
// before it) as an empty partial (m = -inf, l = 0; the combine leaves its o
// out).
//
// k_group_decode_mfma: an item is (unit of the union, token chunk of the
// unit, pass) of one (sequence, KV head); a pass holds up to 128 query
// columns.  Two schedules share the item code:
//  * plan mode (after k_group_plan): one workgroup per (launch rank,
//    (sequence, KV head), token chunk), all passes of its unit in turn; the
//    plan's records are in launch order, the costliest units (tokens times
//    rows) first;
//  * prefill mode: persistent, one workgroup per CU slot; each builds the
//    units of its (sequence, KV head)s in LDS and takes items from a
//    per-(sequence, KV head) counter in that order, so the rows of a unit
//    chosen by many rows are split over several workgroups.  (A grid of one
//    workgroup per possible unit spent tens of microseconds launching
//    workgroups that had nothing to do.)
// The chunk's middle-region tokens are contiguous rows of one physical page; 64-token stages of K and V go
// through LDS (three stages in flight in registers, two in LDS) and are read
// by every wave.  Query columns are (row, head) pairs of the rows in the
// mask, 16 per MFMA column block; each wave owns one column block per pass
// (more columns take more passes over the chunk) and, with fewer blocks
// than waves, the waves of a block share its subtiles and merge their
// states through LDS.  q.k is
// v_mfma_f32_16x16x32_bf16 with the keys as A, p.v v_mfma_f32_16x16x16_bf16
// with the weights as A and the values read column-wise from a padded LDS
// layout; the softmax is the lazily rescaled base-2 online softmax of the
// per-row decode.  Every column's normalised partial and (m, l) go to its
// row's slot for this (page, chunk): slot j * token_splits + chunk, j the
// page's index in the row's list, so the merge order is fixed and the
// results do not depend on timing.
//
// Prefill mode (one or several consecutive chunks of a prompt over a block
// index, after the front of prefill.hip, with no plan kernel; each chunk
// has its own length, slot table and counters): the units of a (chunk,
// sequence, KV head) are
// first the pages of the rows' window [L - W, L), each token chunk attended
// causally by the rows at or after its first token (the others get an empty
// partial for that slot), then the index's blocks, largest visible part
// first, each attended by the rows whose entry in the front's slot table
// (indexed by block) is >= 0; a block no row chose ends its workgroups at
// once.
#include "device_common.hpp"
#include "kernels.hpp"

namespace sa {

namespace {

typedef __bf16 gbf16x8_t __attribute__((ext_vector_type(8)));
typedef short gi16x4_t __attribute__((ext_vector_type(4)));
typedef float gf32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPlanThreads = 256;
constexpr int kPlanBatch = 8;  // list entries per thread whose loads go out together
constexpr int kGW = 8;           // waves of a grouped-decode workgroup
constexpr int kStage = 64;       // tokens per LDS stage
constexpr float kGSlack = 8.0f;  // log2 units, as the per-row decode

// LDS byte offset of (token t, byte b) in a 16-token value tile: rows of
// VROW bytes, 32 bytes of padding after every 4 tokens, so the column reads
// of the p.v operand (tokens 4j .. 4j+3, one channel) hit distinct banks
template <int VROW>
__device__ __forceinline__ int gvt_off(int t, int b)
{
    return t * VROW + (t >> 2) * 32 + b;
}

// the (sequence, KV head)'s candidate range from its length
struct Regions {
    int L, se, ws, plo, phi;
    // extra: tokens past the sequence's length (a later prefill chunk of the same call)
    __device__ __forceinline__ Regions(const Geometry& g, int b, int S, int W, int extra = 0)
    {
        L = imax(0, imin(g.seq_lens[b] + extra, g.max_pages * g.P));
        se = imin(S, L);
        ws = imax(se, L - W);
        plo = se / g.P;
        phi = ws > se ? (ws - 1) / g.P : plo - 1;
    }
};

__global__ __launch_bounds__(kPlanThreads) void k_group_plan(GroupArgs a)
{
    extern __shared__ unsigned long long mask[];  // [npg][2] (rows 0-63, 64-127), then each unit's launch rank
    __shared__ int by_cost[256];
    __shared__ int s_nunion;
    const Geometry& g = a.g;
    const int npg = a.npg;
    int* rank = (int*)(mask + 2 * npg);
    const int bk = blockIdx.x, b = bk / g.Hkv, kvh = bk - b * g.Hkv;
    const int tid = threadIdx.x;
    const Regions rg(g, b, a.S, a.W);
    // candidates: the pages with middle-region tokens, or every block
    const int lo = a.blk_off ? 0 : rg.plo, hi = a.blk_off ? npg - 1 : rg.phi;
    for (int p = tid; p < 2 * npg; p += kPlanThreads) mask[p] = 0ull;
    __syncthreads();

    const int32_t* sel = a.sel + (long)bk * a.Q * a.k_max;
    const int32_t* cnt = a.count + (long)bk * a.Q;
    // The unit of entry idx = (row r, list index j) when the row uses it, it
    // names a candidate unit and it lies above the entry before it (lists
    // are ascending), else -1.  Entries past the count, outside the
    // candidates, or not above their predecessor (a repeated unit among
    // them) are not attended: their slots hold empty partials, so a page is
    // attended at most once per row and the results stay deterministic.
    // The entries a thread handles are read kPlanBatch at a time, every
    // load of a batch in flight together: the entry, the one before it and
    // the row's count.
    const int nent = a.Q * a.k_max;
    struct Listed {
        int p[kPlanBatch];
    };
    auto listed_batch = [&](int base) {
        int pv[kPlanBatch], pb[kPlanBatch], cr[kPlanBatch];
#pragma unroll
        for (int u = 0; u < kPlanBatch; ++u) {
            const int idx = base + u * kPlanThreads + tid;
            const int r = idx / a.k_max, j = idx - r * a.k_max;
            pv[u] = idx < nent ? sel[idx] : -1;
            pb[u] = idx < nent && j > 0 ? sel[idx - 1] : -1;
            cr[u] = idx < nent ? cnt[r] : 0;
        }
        Listed l;
#pragma unroll
        for (int u = 0; u < kPlanBatch; ++u) {
            const int idx = base + u * kPlanThreads + tid;
            const int r = idx / a.k_max, j = idx - r * a.k_max;
            const int p = pv[u];
            const bool used = idx < nent && j < imax(0, imin(cr[u], a.k_max)) && p >= lo && p <= hi;
            l.p[u] = used && (j == 0 || p > pb[u]) ? p : -1;
        }
        return l;
    };
    for (int base = 0; base < nent; base += kPlanBatch * kPlanThreads) {
        const Listed l = listed_batch(base);
#pragma unroll
        for (int u = 0; u < kPlanBatch; ++u) {
            const int idx = base + u * kPlanThreads + tid;
            if (idx >= nent) break;
            const int r = idx / a.k_max, j = idx - r * a.k_max;
            const int p = l.p[u];
            if (p >= 0) {
                atomicOr(&mask[2 * p + (r >> 6)], 1ull << (r & 63));
            } else {
                // a slot this row does not use: an empty partial (m = -inf, l = 0)
                // for every head and chunk; the combine does not read its o
                for (int h = 0; h < g.G; ++h) {
                    const long prow = ((long)b * g.Hq + kvh * g.G + h) * a.Q + r;
                    for (int s = 0; s < a.tsplit; ++s) {
                        const long slot = prow * a.split_stride + (long)j * a.tsplit + s;
                        a.part_ml[slot * 2 + 0] = -INFINITY;
                        a.part_ml[slot * 2 + 1] = 0.f;
                    }
                }
            }
        }
    }
    __syncthreads();

    // The union in launch order: the costliest units first, so the longest
    // workgroups start first and the last to start are short.  A unit's cost
    // is its tokens times (8 + the rows that chose it) (more rows, more
    // matrix-core work per token); a counting sort over quarter-octave
    // buckets of the cost.  The order within a bucket follows the atomics;
    // it affects timing only.  Each unit's record carries what its
    // workgroup needs first (page or block, physical page, row mask).
    auto cost_bucket = [&](int p) {
        int ntok;
        if (a.blk_off) {
            const int32_t* bo = a.blk_off + (long)bk * (npg + 1);
            const int end = a.blk_end ? imax(bo[p], imin(a.blk_end[(long)bk * npg + p], bo[p + 1])) : bo[p + 1];
            ntok = end - bo[p];
        } else {
            ntok = imin((p + 1) * g.P, rg.ws) - imax(p * g.P, rg.se);
        }
        const int nrows = __builtin_popcountll(mask[2 * p]) + __builtin_popcountll(mask[2 * p + 1]);
        const uint64_t cost = (uint64_t)imax(1, ntok) * (uint64_t)(8 + nrows);
        const int lb = 63 - __builtin_clzll(cost);
        const int frac = lb >= 2 ? (int)((cost >> (lb - 2)) & 3u) : 0;
        return 255 - (4 * lb + frac);  // 0: the costliest
    };
    for (int c = tid; c < 256; c += kPlanThreads) by_cost[c] = 0;
    __syncthreads();
    for (int p = tid; p < npg; p += kPlanThreads)
        if ((mask[2 * p] | mask[2 * p + 1]) != 0ull) atomicAdd(&by_cost[cost_bucket(p)], 1);
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int c = 0; c < 256; ++c) {
            const int nc = by_cost[c];
            by_cost[c] = acc;
            acc += nc;
        }
        a.nunion[bk] = acc;
        s_nunion = acc;
    }
    __syncthreads();
    GroupPage* up = a.upages + (long)bk * npg;
    const int32_t* btr = g.block_table + (long)b * g.max_pages;
    for (int p = tid; p < npg; p += kPlanThreads) {
        const unsigned long long m0 = mask[2 * p], m1 = mask[2 * p + 1];
        if ((m0 | m1) != 0ull) {
            const int at = atomicAdd(&by_cost[cost_bucket(p)], 1);
            GroupPage e;
            e.page = p;
            e.nrows = __builtin_popcountll(m0) + __builtin_popcountll(m1);
            if (a.blk_off) {  // blocks: the (visible) rows of the block layout
                const int32_t* bo = a.blk_off + (long)bk * (npg + 1);
                e.phys = bo[p];
                e.pad = a.blk_end ? imax(bo[p], imin(a.blk_end[(long)bk * npg + p], bo[p + 1])) : bo[p + 1];
            } else {
                const int ph = btr[p];
                e.phys = ph >= 0 && ph < g.num_phys ? ph : -1;
                e.pad = 0;
            }
            up[at] = e;
            rank[p] = at;
        }
    }
    // every row's slot of every union page starts as "not chosen"
    int16_t* sl = a.slots + (long)bk * npg * kGroupMaxRows;
    for (int idx = tid; idx < s_nunion * kGroupMaxRows; idx += kPlanThreads) sl[idx] = -1;
    __syncthreads();

    // each row's index j of every page it lists: its slot for that page
    for (int base = 0; base < nent; base += kPlanBatch * kPlanThreads) {
        const Listed l = listed_batch(base);
#pragma unroll
        for (int u = 0; u < kPlanBatch; ++u) {
            const int idx = base + u * kPlanThreads + tid;
            if (idx >= nent) break;
            const int r = idx / a.k_max, j = idx - r * a.k_max;
            if (l.p[u] >= 0) sl[rank[l.p[u]] * kGroupMaxRows + r] = (int16_t)j;
        }
    }
}

template <int HD, int G, bool PF>
__global__ __launch_bounds__(64 * kGW) void k_group_decode_mfma(GroupArgs a)
{
    constexpr int KK = HD / 32;          // q.k products per 16-token subtile (32 channels each)
    constexpr int NB = HD / 16;          // p.v products per subtile (16 channels each)
    constexpr int CPT = HD * 2 / 16;     // 16-byte chunks per token row
    constexpr int KROW = HD * 2 + 16;    // LDS bytes per key row (padded)
    constexpr int VROW = HD * 2;
    constexpr int VTILE = 16 * VROW + 4 * 32;
    constexpr int SUB = kStage / 16;     // subtiles per stage
    constexpr int LPS = kStage * CPT / (64 * kGW);  // 16-byte loads per thread per stage, K and V each
    static_assert(LPS >= 1 && kStage * CPT == LPS * 64 * kGW, "stage loads tile the workgroup");
    static_assert(16 % G == 0, "column blocks hold whole rows");

    // stage buffers (two of K, two of V), reused for the merge of the waves' states
    constexpr int KBUF = kStage * KROW, VBUF = SUB * VTILE;
    constexpr int STAGE_BYTES = 2 * (KBUF + VBUF), MERGE_BYTES = kGW * 16 * (HD + 2) * 4;
    __shared__ __attribute__((aligned(16))) unsigned char smem[STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES];
    auto kl = [&](int buf) { return smem + buf * KBUF; };
    auto vl = [&](int buf) { return smem + 2 * KBUF + buf * VBUF; };
    __shared__ int rows_l[kGroupMaxRows], slot_l[kGroupMaxRows];
    static_assert(kGroupMaxRows == 128, "two slot entries per lane");
    static_assert(kStage % 16 == 0, "stages hold whole subtiles");

    const Geometry& g = a.g;
    const int nbk = g.B * g.Hkv;
    const int QS = a.Q * a.nck;  // row stride of q and the partials (a.Q rows per chunk)
    const int lane = threadIdx.x & 63, wave = wave_index();
    const int r = lane & 15, j = lane >> 4;
    constexpr bool prefill = PF;  // prefill mode (persistent), else plan mode

    // One item: passes pidx, pidx + np, ... of token chunk s (of nch) of unit
    // u of (prompt chunk, sequence, KV head) vb (vb = bk in plan mode).
    // Units: the plan's records in order, or in prefill mode the window's
    // pages (u < nwin) and then the index's blocks (block u - nwin).
    int next_item = -1;  // thread 0: the next item's index, when the item fetched it
    // each lane's two rows' list index of unit u (-1: the row does not attend it)
    auto load_slots = [&](const int vb, const int u, int16_t& slot0, int16_t& slot1) {
        slot0 = -1;
        slot1 = -1;
        if (!prefill) {
            const long ui = (long)vb * a.npg + u;
            slot0 = a.slots[ui * kGroupMaxRows + lane];
            slot1 = a.slots[ui * kGroupMaxRows + 64 + lane];
        } else if (u >= a.nwin) {
            const long ui = (long)vb * a.npg + (u - a.nwin);
            if (lane < a.Q) slot0 = a.slots[ui * kGroupMaxRows + lane];
            if (64 + lane < a.Q) slot1 = a.slots[ui * kGroupMaxRows + 64 + lane];
        }
    };
    auto process = [&](const int vb, const int u, const int s, const int pidx, const int np, const int nch,
                       const int a0, const int a1, const int x, int16_t slot0, int16_t slot1) {
        const int ck = vb / nbk, bk = vb - ck * nbk, b = bk / g.Hkv, kvh = bk - b * g.Hkv;
        const int rb = ck * a.Q;  // the chunk's first row
        const Regions rg(g, b, a.S, a.W, rb);
        const bool win = prefill && u < a.nwin;  // a page of the rows' window (prefill)
        const bool blocks = a.blk_off != nullptr && !win;
        const int phys = blocks ? 0 : x;
        const int p = blocks ? 0 : a0 / g.P;  // the page of a page unit

        // this chunk of the unit's tokens: contiguous rows of one physical
        // page (an unmapped page attends nothing), or of the block layout
        const int n = imax(0, a1 - a0);
        const int csz = (n + nch - 1) / nch;
        const int t0 = a0 + imin(n, s * csz);
        const bool mapped = blocks || phys >= 0;
        const int t1 = mapped ? imin(a1, t0 + csz) : t0;

        const int nst = (imax(0, t1 - t0) + kStage - 1) / kStage;
        // K/V row of token t0 (inside the page or the sequence's rows even when the chunk is empty)
        const long row0 = blocks   ? (long)bk * a.blk_n + imin(t0, a.blk_n - 1)
                          : mapped ? ((long)phys * g.Hkv + kvh) * g.P + imin(t0 - p * g.P, g.P - 1)
                                   : 0;
        const uint16_t* kp = (const uint16_t*)(blocks ? a.blk_k : g.k) + row0 * HD;
        const uint16_t* vp = (const uint16_t*)(blocks ? a.blk_v : g.v) + row0 * HD;
        const int ntok = t1 - t0;

        // stage st: this thread's 16-byte chunks of the K and V rows of
        // tokens t0 + 64 st .. ; chunks past the chunk's end re-read its
        // first row and are masked (values written as zeros)
        struct Staged {
            uint4 k[LPS], v[LPS];
        };
        auto fetch = [&](int st, Staged& x) {
            static_for<0, LPS>([&](auto U) {
                constexpr int u = decltype(U)::value;
                const int e = u * 64 * kGW + threadIdx.x;  // chunk of the stage
                const int tt = st * kStage + e / CPT;
                const long off = (tt < ntok ? (long)tt * HD : 0) + (e % CPT) * 8;
                // plan mode (a decode step's pages, read once) non-temporal;
                // prefill chunks read blocks their neighbours read again
                x.k[u] = PF ? *(const uint4*)(kp + off) : ld_stream(kp + off);
                x.v[u] = PF ? *(const uint4*)(vp + off) : ld_stream(vp + off);
            });
        };
        auto stash = [&](int st, int buf, const Staged& x) {
            static_for<0, LPS>([&](auto U) {
                constexpr int u = decltype(U)::value;
                const int e = u * 64 * kGW + threadIdx.x;
                const int tl = e / CPT, part = e % CPT;
                const bool ok = st * kStage + tl < ntok;
                const uint4 kw = x.k[u];
                *(uint4*)(kl(buf) + tl * KROW + part * 16) = make_uint4(kw.x, kw.y, kw.z, kw.w);
                const uint4 w = x.v[u];
                *(uint4*)(vl(buf) + (tl >> 4) * VTILE + gvt_off<VROW>(tl & 15, part * 16)) =
                    make_uint4(ok ? w.x : 0u, ok ? w.y : 0u, ok ? w.z : 0u, ok ? w.w : 0u);
            });
        };
        // The first pass's three stages are issued now, with the rows' slots
        // in flight: their addresses need only the unit's token range.
        Staged X0, X1, X2;
        fetch(0, X0);
        __builtin_amdgcn_sched_barrier(0);  // keep the stages' loads in stage order
        fetch(1, X1);
        __builtin_amdgcn_sched_barrier(0);
        fetch(2, X2);
        __builtin_amdgcn_sched_barrier(0);

        if (win) {
            // The rows at or after the chunk's first token attend it (list index
            // k_max + unit); every other row gets an empty partial for this
            // slot, and the first chunk's item empties every row's slots of the
            // chunks the unit does not have.
            const int first = t1 > t0 ? t0 - (rg.L - a.Q) : a.Q;  // first row that sees the chunk
            const int16_t ws = (int16_t)(a.k_max + u);
            slot0 = lane >= first && lane < a.Q ? ws : (int16_t)-1;
            slot1 = 64 + lane >= first && 64 + lane < a.Q ? ws : (int16_t)-1;
            const int nout = imin(imax(first, 0), a.Q);
            if (pidx == 0) {
                for (int e2 = threadIdx.x; e2 < nout * G; e2 += 64 * kGW) {
                    const int row = e2 / G, h = e2 - row * G;
                    const long prow = ((long)b * g.Hq + kvh * G + h) * QS + rb + row;
                    const long slot = prow * a.split_stride + (long)ws * a.tsplit + s;
                    *(float2*)(a.part_ml + slot * 2) = make_float2(-INFINITY, 0.f);
                }
                const int nx = s == 0 ? a.tsplit - nch : 0;
                for (int e2 = threadIdx.x; e2 < a.Q * G * nx; e2 += 64 * kGW) {
                    const int row = e2 / (G * nx), rest = e2 - row * (G * nx), h = rest / nx, s2 = nch + rest % nx;
                    const long prow = ((long)b * g.Hq + kvh * G + h) * QS + rb + row;
                    const long slot = prow * a.split_stride + (long)ws * a.tsplit + s2;
                    *(float2*)(a.part_ml + slot * 2) = make_float2(-INFINITY, 0.f);
                }
            }
            if (nout >= a.Q) return;
        }

        // the rows that attend the unit, ascending, and the unit's index in each
        // row's list (every wave takes the same ballots)
        const uint64_t M0 = __builtin_amdgcn_ballot_w64(slot0 >= 0), M1 = __builtin_amdgcn_ballot_w64(slot1 >= 0);
        const int n0 = __builtin_popcountll(M0);
        const int nr = n0 + __builtin_popcountll(M1);
        if (wave == 0) {
            if (slot0 >= 0) {
                rows_l[lanes_below(M0)] = lane;
                slot_l[lanes_below(M0)] = slot0;
            }
            if (slot1 >= 0) {
                rows_l[n0 + lanes_below(M1)] = 64 + lane;
                slot_l[n0 + lanes_below(M1)] = slot1;
            }
        }
        __syncthreads();
        // a unit with fewer token chunks than tsplit: its rows' slots of the
        // missing chunks are empty (written by the first chunk's first pass)
        if (!win && s == 0 && pidx == 0 && nch < a.tsplit) {
            const int nx = a.tsplit - nch;
            for (int e2 = threadIdx.x; e2 < nr * G * nx; e2 += 64 * kGW) {
                const int ri = e2 / (G * nx), rest = e2 - ri * (G * nx), h = rest / nx, s2 = nch + rest % nx;
                const long prow = ((long)b * g.Hq + kvh * G + h) * QS + rb + rows_l[ri];
                const long slot = prow * a.split_stride + (long)slot_l[ri] * a.tsplit + s2;
                *(float2*)(a.part_ml + slot * 2) = make_float2(-INFINITY, 0.f);
            }
        }


        const float sl2 = a.scale_log2, slack = kGSlack / sl2;
        const int ncol = nr * G, ncb = (ncol + 15) / 16;
        if (pidx * kGW >= ncb) return;  // no column block in this workgroup's passes

        // Pass = up to kGW column blocks, one per wave; this workgroup takes
        // passes pidx, pidx + npass, ... (the rows' slots are disjoint between
        // passes, so each is written once).  With fewer blocks than waves, the
        // waves of a block take turns over the 16-token subtiles of each stage
        // and their states merge through LDS at the end of the pass, so the
        // work follows the live columns.  (The assignment is fixed, so the
        // results do not depend on timing.)
        for (int pass = pidx; pass * kGW < ncb; pass += np) {
            const int npb = imin(kGW, ncb - pass * kGW);         // blocks this pass
            const int cbi = wave % npb, gi = wave / npb;          // this wave's block, its index in the block's group
            const int gsz = imin((kGW - cbi + npb - 1) / npb, SUB);  // waves that compute on the block
            const bool computes = gi < gsz;
            const int cb = pass * kGW + cbi;
            // lane r is column 16 cb + r
            gbf16x8_t qb[KK];
            gf32x4_t o[NB];
            float m_run = -INFINITY, l_run = 0.f;
            int cpos;  // position of the column's row (causal limit)
            {
                const int col = 16 * cb + r, ri = col / G, h = col - ri * G;
                const bool live = ri < nr;
                const int row = live ? rows_l[ri] : 0;
                // a block's tokens precede every row's window: no causal test
                cpos = !live ? -1 : blocks ? 0x7fffffff : rg.L - a.Q + row;
    #pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    uint4 w = make_uint4(0, 0, 0, 0);
                    if (live)
                        w = *(const uint4*)((const uint16_t*)a.q +
                                            (((long)b * g.Hq + kvh * G + h) * QS + rb + row) * HD + 32 * kk + 8 * j);
                    qb[kk] = __builtin_bit_cast(gbf16x8_t, w);
                }
    #pragma unroll
                for (int m = 0; m < NB; ++m) o[m] = gf32x4_t{0.f, 0.f, 0.f, 0.f};
            }

            // this wave's subtiles of stage st: gi, gi + gsz, ...
            auto compute = [&](int st, int buf) {
                if (!computes || st >= nst) return;  // a stage past the chunk's end attends nothing
                for (int sub = gi; sub < SUB; sub += gsz) {
                    const int tb = st * kStage + sub * 16;  // chunk-relative index of the subtile's token 0
                    const unsigned char* kt = kl(buf) + sub * 16 * KROW;
                    gbf16x8_t ka[KK];
    #pragma unroll
                    for (int kk = 0; kk < KK; ++kk)
                        ka[kk] = __builtin_bit_cast(gbf16x8_t, *(const uint4*)(kt + r * KROW + kk * 64 + j * 16));
                    gf32x4_t s = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                    for (int kk = 0; kk < KK; ++kk) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kk], qb[kk], s, 0, 0, 0);
                    // lane (r, j): column r, tokens 4j .. 4j+3 of the subtile
                    float z[4];
    #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int tt = tb + 4 * j + i;
                        z[i] = tt < ntok && t0 + tt <= cpos ? s[i] : -INFINITY;
                    }
                    float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
                    mx = fmaxf(mx, xor_lanes<16>(mx));
                    mx = fmaxf(mx, xor_lanes<32>(mx));
                    const bool need = mx > m_run + slack;
                    if (__builtin_amdgcn_ballot_w64(need) != 0) {
                        const float mn = need ? mx : m_run;
                        const float alpha = need ? __builtin_amdgcn_exp2f((m_run - mn) * sl2) : 1.f;
                        l_run *= alpha;
                        m_run = mn;
                        // accumulator rows are columns 4j + i: fetch their factors
    #pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float ai = __shfl(alpha, 4 * j + i);
    #pragma unroll
                            for (int m = 0; m < NB; ++m) o[m][i] *= ai;
                        }
                    }
                    const float mref = m_run == -INFINITY ? 0.f : -m_run * sl2;
                    float pz[4];
    #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        pz[i] = __builtin_amdgcn_exp2f(fmaf(z[i], sl2, mref));  // -inf -> 0
                        l_run += pz[i];
                    }
                    const gi16x4_t pa =
                        __builtin_bit_cast(gi16x4_t, make_uint2(pack_bf16(pz[0], pz[1]), pack_bf16(pz[2], pz[3])));
                    // p.v: B = values of tokens 4j .. 4j+3 at channel 16m + r
                    const unsigned char* vcol = vl(buf) + sub * VTILE + 2 * r;
    #pragma unroll
                    for (int m = 0; m < NB; ++m) {
                        gi16x4_t vb;
    #pragma unroll
                        for (int i = 0; i < 4; ++i) vb[i] = *(const short*)(vcol + gvt_off<VROW>(4 * j + i, 32 * m));
                        o[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, o[m], 0, 0, 0);
                    }
                }
            };

            // Stages: three in flight in registers, two in LDS.  Every step
            // issues its loads and the loop's only exit is at the end of a round
            // of three, so the waits count one stage each; stages past the end
            // re-read the chunk's first row and are not computed.  (Leaving the
            // loop at a chunk's last stage instead made the compiler wait for
            // every load in flight at the top of the loop: slower.)
            if (pass != pidx) {  // the first pass's stages were issued with the unit
                fetch(0, X0);
                __builtin_amdgcn_sched_barrier(0);
                fetch(1, X1);
                __builtin_amdgcn_sched_barrier(0);
                fetch(2, X2);
                __builtin_amdgcn_sched_barrier(0);
            }
            for (int st = 0; st < nst; st += 3) {
                stash(st, 0, X0);
                __syncthreads();
                fetch(st + 3, X0);
                compute(st, 0);
                stash(st + 1, 1, X1);
                __syncthreads();
                fetch(st + 4, X1);
                compute(st + 1, 1);
                __syncthreads();  // stage st is no longer read from buffer 0
                stash(st + 2, 0, X2);
                __syncthreads();
                fetch(st + 5, X2);
                compute(st + 2, 0);
                __syncthreads();  // buffers 0 and 1 are free for the next round
            }
            // the next item's index, taken while this one merges
            if (prefill && threadIdx.x == 0 && (pass + np) * kGW >= ncb) next_item = atomicAdd(a.ctr + vb, 1);

            // Merge the states of a block's waves (group order) through LDS,
            // then the first wave of each block writes its partials.  Lane (r, j)
            // holds columns 4j + i at channel 16m + r.
            l_run += xor_lanes<16>(l_run);
            l_run += xor_lanes<32>(l_run);
            float* wo = (float*)smem;                   // [kGW][16][HD]
            float* wm = wo + kGW * 16 * HD;             // [kGW][16]
            float* wl = wm + kGW * 16;                  // [kGW][16]
            __syncthreads();  // the stage buffers are no longer read
            if (computes) {
    #pragma unroll
                for (int m = 0; m < NB; ++m)
    #pragma unroll
                    for (int i = 0; i < 4; ++i) wo[(wave * 16 + 4 * j + i) * HD + 16 * m + r] = o[m][i];
                if (j == 0) {
                    wm[wave * 16 + r] = m_run;
                    wl[wave * 16 + r] = l_run;
                }
            }
            __syncthreads();
            if (gi == 0) {
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int qc = 4 * j + i;
                    float mm = -INFINITY;
                    for (int k = 0; k < gsz; ++k) mm = fmaxf(mm, wm[(cbi + k * npb) * 16 + qc]);
                    float ls = 0.f, os[NB];
    #pragma unroll
                    for (int m = 0; m < NB; ++m) os[m] = 0.f;
                    for (int k = 0; k < gsz; ++k) {
                        const int w = cbi + k * npb;
                        const float mw = wm[w * 16 + qc];
                        const float wt = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mw - mm) * sl2);
                        ls = fmaf(wl[w * 16 + qc], wt, ls);
    #pragma unroll
                        for (int m = 0; m < NB; ++m) os[m] = fmaf(wo[(w * 16 + qc) * HD + 16 * m + r], wt, os[m]);
                    }
                    const int col = 16 * cb + qc, ri = col / G, h = col - ri * G;
                    if (ri >= nr) continue;
                    const long prow = ((long)b * g.Hq + kvh * G + h) * QS + rb + rows_l[ri];
                    const long slot = prow * a.split_stride + (long)slot_l[ri] * a.tsplit + s;
                    const float inv = ls > 0.f ? 1.0f / ls : 0.f;
    #pragma unroll
                    for (int m = 0; m < NB; ++m) a.part_o[slot * HD + 16 * m + r] = os[m] * inv;
                    if (r == 0) {
                        a.part_ml[slot * 2 + 0] = ls > 0.f ? mm * sl2 * kLn2 : -INFINITY;
                        a.part_ml[slot * 2 + 1] = ls;
                    }
                }
            }
            __syncthreads();  // the next pass restages the buffers
        }
    };

    // A unit's token range, physical page and passes from the plan's record.
    auto plan_unit = [&](const GroupPage& e, const Regions& rg, int& x0, int& x1, int& x) {
        if (a.blk_off) {  // blocks: the plan records the row range
            x0 = e.phys;
            x1 = e.pad;
            x = 0;
        } else {
            x0 = imax(e.page * g.P, rg.se);
            x1 = imin((e.page + 1) * g.P, rg.ws);
            x = e.phys;
        }
    };
    auto unit_chunks = [&](int ntk) { return imin(a.tsplit, imax(1, (ntk + kGroupChunkMin - 1) / kGroupChunkMin)); };

    if constexpr (!PF) {
        // Plan mode: one workgroup per (unit of the union, token chunk); id =
        // (rank * B * Hkv + bk) * tsplit + chunk, the costliest units of every
        // (sequence, KV head) first.  Nearly every unit of the bound is in the
        // union here, so a grid sized to it launches few idle workgroups.
        const int chunk = blockIdx.x % a.tsplit, rest = blockIdx.x / a.tsplit;
        const int bk = rest % nbk, rank = rest / nbk;
        const GroupPage e = a.upages[(long)bk * a.npg + rank];  // rank < npg: the record exists
        int16_t slot0, slot1;
        load_slots(bk, rank, slot0, slot1);  // with the record, not after it
        if (rank >= a.nunion[bk]) return;
        const Regions rg(g, bk / g.Hkv, a.S, a.W);
        int x0, x1, x;
        plan_unit(e, rg, x0, x1, x);
        const int nch = unit_chunks(imax(0, x1 - x0));
        if (chunk >= nch) return;  // the first chunk's workgroup empties this chunk's slots
        process(bk, rank, chunk, 0, 1, nch, x0, x1, x, slot0, slot1);
    } else {
    // The units of the (sequence, KV head) being served: token range [a0, a1)
    // (rows of the block layout for blocks, positions for pages), physical
    // page, passes and token chunks, their launch order and the prefix of
    // their items in that order (filled per (sequence, KV head) below).
    __shared__ int u_a0[kGroupMaxPages], u_a1[kGroupMaxPages], u_x[kGroupMaxPages];
    __shared__ int item_pre[kGroupMaxPages + 1];
    __shared__ unsigned short u_ord[kGroupMaxPages];
    __shared__ unsigned char u_np[kGroupMaxPages], u_nch[kGroupMaxPages], u_bkt[kGroupMaxPages];
    __shared__ int hist[256];
    __shared__ int wsum[kGW];
    __shared__ int s_item;

    // Persistent schedule: one workgroup per CU, in columns of 8 (one per
    // XCD); column col serves (prompt chunk, sequence, KV head)s col, col +
    // ncol, ... (or col mod their number when there are fewer of them than
    // columns).  The workgroups of a (chunk, sequence, KV head) take its
    // items (unit, token chunk, pass) in the units' launch order (costliest
    // first) from a counter the kernel before this one cleared, so none waits
    // for work another could do and none is launched without work.  A unit has one pass per
    // kGroupPassCols query columns of its rows and up to tsplit token chunks
    // of at least kGroupChunkMin tokens.
    const int tid = threadIdx.x;
    const int ncol = gridDim.x >> 3, col = blockIdx.x >> 3;
    const int nvb = nbk * a.nck;  // (prompt chunk, sequence, KV head)s
    const int vb0 = nvb >= ncol ? col : col % nvb, vstep = nvb >= ncol ? ncol : nvb;
    for (int vb = vb0; vb < nvb; vb += vstep) {
        // the first item's index is fetched with the units' loads: its round
        // trip overlaps theirs
        const int first_item = tid == 0 ? atomicAdd(a.ctr + vb, 1) : -1;
        const int ck = vb / nbk, bk = vb - ck * nbk, b = bk / g.Hkv;
        const Regions rg(g, b, a.S, a.W, ck * a.Q);
        // the units, loads in one round
        const int nu = a.nwin + a.npg;
        const int wstart = imax(0, rg.L - a.W);
        for (int u = tid; u < nu; u += 64 * kGW) {
            int x0, x1, x = 0, nrows;
            if (u < a.nwin) {
                const int pg = wstart / g.P + u;
                x0 = imax(pg * g.P, wstart);
                x1 = imin((pg + 1) * g.P, rg.L);
                const int ph = pg < g.max_pages ? g.block_table[(long)b * g.max_pages + pg] : -1;
                x = ph >= 0 && ph < g.num_phys ? ph : -1;
                nrows = imax(1, imin(a.Q, rg.L - x0));  // one item at least: it writes the rows' empty partials
            } else {
                const int c = u - a.nwin;
                const int32_t* bo = a.blk_off + (long)bk * (a.npg + 1);
                x0 = bo[c];
                x1 = imax(x0, imin(a.blk_end[(long)vb * a.npg + c], bo[c + 1]));
                const uint4 cr = *(const uint4*)(a.pf_rows + ((long)vb * a.npg + c) * 16);
                const uint32_t w4[4] = {cr.x, cr.y, cr.z, cr.w};
                nrows = 0;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    nrows += (int)((w4[q4] & 0xff) + ((w4[q4] >> 8) & 0xff) + ((w4[q4] >> 16) & 0xff) + (w4[q4] >> 24));
            }
            const int ntk = imax(0, x1 - x0);
            const int npass = nrows > 0 ? (nrows * G + kGroupPassCols - 1) / kGroupPassCols : 0;
            const int nch = unit_chunks(ntk);
            u_a0[u] = x0;
            u_a1[u] = x1;
            u_x[u] = x;
            u_np[u] = (unsigned char)npass;
            u_nch[u] = (unsigned char)nch;
            // cost bucket (0: the costliest): tokens times (8 + rows), quarter octaves
            const uint64_t cost = (uint64_t)imax(1, ntk) * (uint64_t)(8 + nrows);
            const int lb = 63 - __builtin_clzll(cost);
            const int fr = lb >= 2 ? (int)((cost >> (lb - 2)) & 3u) : 0;
            u_bkt[u] = (unsigned char)(255 - imin(255, 4 * lb + fr));
        }
        __syncthreads();

        // launch order: a stable counting sort of the units by cost bucket,
        // the same in every workgroup of the (sequence, KV head)
        {
            for (int i = tid; i < 256; i += 64 * kGW) hist[i] = 0;
            __syncthreads();
            for (int u = tid; u < nu; u += 64 * kGW) atomicAdd(&hist[u_bkt[u]], 1);
            __syncthreads();
            if (wave == 0) {
                int v[4], sum = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[i] = hist[4 * lane + i];
                    sum += v[i];
                }
                int run = wave_inclusive_scan(sum) - sum;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    hist[4 * lane + i] = run;
                    run += v[i];
                }
                // units in order, 64 at a time: a unit's place is its bucket's
                // base plus the units of that bucket before it
                const uint64_t below = (1ull << lane) - 1ull;
                for (int k0 = 0; k0 < nu; k0 += 64) {
                    const int u = k0 + lane;
                    const bool valid = u < nu;
                    const int bkt = valid ? u_bkt[u] : 0;
                    uint64_t same = __builtin_amdgcn_ballot_w64(valid);
#pragma unroll
                    for (int bit = 0; bit < 8; ++bit) {
                        const bool on = ((bkt >> bit) & 1) != 0;
                        const uint64_t m = __builtin_amdgcn_ballot_w64(on);
                        same &= on ? m : ~m;
                    }
                    if (valid) {
                        u_ord[hist[bkt] + __builtin_popcountll(same & below)] = (unsigned short)u;
                        if ((same >> lane) == 1ull) hist[bkt] += __builtin_popcountll(same);  // the group's last lane
                    }
                }
            }
            __syncthreads();
        }

        // the prefix of the items in launch order, 8 units a thread
        constexpr int UPT = (kGroupMaxPages + 64 * kGW - 1) / (64 * kGW);
        int cnt[UPT], mine = 0;
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int k = tid * UPT + i;
            cnt[i] = 0;
            if (k < nu) {
                const int u = u_ord[k];
                cnt[i] = (int)u_np[u] * (int)u_nch[u];
            }
            mine += cnt[i];
        }
        int total;
        int run = block_exclusive_scan<64 * kGW>(mine, wsum, total);
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int k = tid * UPT + i;
            if (k < nu) item_pre[k] = run;
            run += cnt[i];
        }
        __syncthreads();

        next_item = first_item;
        for (;;) {
            if (tid == 0) s_item = next_item >= 0 ? next_item : atomicAdd(a.ctr + vb, 1);
            __syncthreads();
            const int it = s_item;
            next_item = -1;
            __syncthreads();  // s_item is read before the next item's fetch
            if (it >= total) break;
            // the unit: the last in launch order with item_pre <= it (units
            // without items share the next one's prefix and are skipped)
            int lo = 0, hi = nu - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (item_pre[mid] <= it)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            const int u = u_ord[lo];
            const int np = u_np[u], nch = u_nch[u], kk = it - item_pre[lo];
            int16_t slot0, slot1;
            load_slots(vb, u, slot0, slot1);
            process(vb, u, kk / np, kk % np, np, nch, u_a0[u], u_a1[u], u_x[u], slot0, slot1);
            __syncthreads();  // LDS of this item is no longer read
        }
    }
    }
}

template <int HD, bool PF>
hipError_t launch_group_g(const GroupArgs& a, dim3 grid, hipStream_t s)
{
    const dim3 block(64 * kGW);
    switch (a.g.G) {
    case 1: hipLaunchKernelGGL((k_group_decode_mfma<HD, 1, PF>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_group_decode_mfma<HD, 2, PF>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_group_decode_mfma<HD, 4, PF>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_group_decode_mfma<HD, 8, PF>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_group_decode_mfma<HD, 16, PF>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_group(const GroupArgs& a, int max_union, hipStream_t s)
{
    const Geometry& g = a.g;
    if (g.dtype != 1 || a.Q > kGroupMaxRows || a.npg > kGroupMaxPages || a.pf_rows || a.nck != 1)
        return hipErrorInvalidValue;
    const size_t lds = (2 * sizeof(unsigned long long) + sizeof(int)) * (size_t)a.npg;
    hipLaunchKernelGGL(k_group_plan, dim3((unsigned)(g.B * g.Hkv)), dim3(kPlanThreads), lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || max_union < 1) return e;
    const dim3 grid((unsigned)((long)max_union * a.tsplit * g.B * g.Hkv));
    if (g.hd == 128) return launch_group_g<128, false>(a, grid, s);
    if (g.hd == 64) return launch_group_g<64, false>(a, grid, s);
    return hipErrorInvalidValue;
}

hipError_t launch_group_prefill(const GroupArgs& a, int workgroups, hipStream_t s)
{
    const Geometry& g = a.g;
    if (g.dtype != 1 || a.Q > kGroupMaxRows || a.nwin + a.npg > kGroupMaxPages || !a.pf_rows || !a.blk_off ||
        !a.blk_end || a.nwin < 1 || !a.ctr || workgroups < 8 || workgroups % 8 || a.nck < 1 || a.nck > kPfMaxChunks)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)workgroups);
    if (g.hd == 128) return launch_group_g<128, true>(a, grid, s);
    if (g.hd == 64) return launch_group_g<64, true>(a, grid, s);
    return hipErrorInvalidValue;
}

namespace {
template <int HD>
int resident_g(int G)
{
    const int bs = 64 * kGW;
    int n = 0;
    hipError_t e = hipErrorInvalidValue;
    switch (G) {
    case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_group_decode_mfma<HD, 1, true>, bs, 0); break;
    case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_group_decode_mfma<HD, 2, true>, bs, 0); break;
    case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_group_decode_mfma<HD, 4, true>, bs, 0); break;
    case 8: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_group_decode_mfma<HD, 8, true>, bs, 0); break;
    case 16: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_group_decode_mfma<HD, 16, true>, bs, 0); break;
    default: break;
    }
    return e == hipSuccess && n > 0 ? n : 1;
}
}  // namespace

int group_workgroups(int hd, int G)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    const int per = hd == 64 ? resident_g<64>(G) : resident_g<128>(G);
    return (cus * per + 7) / 8 * 8;
}

}  // namespace sa
