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
// (entries past its count) as an empty partial (m = -inf, l = 0; the
// combine leaves its o out).
//
// k_group_decode_mfma: one workgroup per (sequence, KV head, page of the
// union, token chunk of the page), launched with the costliest pages (tokens
// times rows) first.  The chunk's middle-region tokens are
// contiguous rows of one physical page; 64-token stages of K and V go
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
#include "device_common.hpp"
#include "kernels.hpp"

namespace sa {

namespace {

typedef __bf16 gbf16x8_t __attribute__((ext_vector_type(8)));
typedef short gi16x4_t __attribute__((ext_vector_type(4)));
typedef float gf32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPlanThreads = 256;
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
    __device__ __forceinline__ Regions(const Geometry& g, int b, int S, int W)
    {
        L = imax(0, imin(g.seq_lens[b], g.max_pages * g.P));
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
    for (int idx = tid; idx < a.Q * a.k_max; idx += kPlanThreads) {
        const int r = idx / a.k_max, j = idx - r * a.k_max;
        const int c = imax(0, imin(cnt[r], a.k_max));
        if (j < c) {
            const int p = sel[idx];
            if (p >= lo && p <= hi) atomicOr(&mask[2 * p + (r >> 6)], 1ull << (r & 63));
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
            const int ph = a.blk_off ? 0 : btr[p];  // blocks: rows of the block layout
            GroupPage e;
            e.page = p;
            e.phys = ph >= 0 && ph < g.num_phys ? ph : -1;
            e.nrows = __builtin_popcountll(m0) + __builtin_popcountll(m1);
            e.pad = 0;
            up[at] = e;
            rank[p] = at;
        }
    }
    // every row's slot of every union page starts as "not chosen"
    int16_t* sl = a.slots + (long)bk * npg * kGroupMaxRows;
    for (int idx = tid; idx < s_nunion * kGroupMaxRows; idx += kPlanThreads) sl[idx] = -1;
    __syncthreads();

    // each row's index j of every page it lists: its slot for that page
    for (int idx = tid; idx < a.Q * a.k_max; idx += kPlanThreads) {
        const int r = idx / a.k_max, j = idx - r * a.k_max;
        if (j < imax(0, imin(cnt[r], a.k_max))) {
            const int p = sel[idx];
            if (p >= lo && p <= hi) sl[rank[p] * kGroupMaxRows + r] = (int16_t)j;
        }
    }
}

template <int HD, int G>
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
    // workgroup id = (rank * B * Hkv + bk) * tsplit + chunk: the pages of
    // every (sequence, KV head) in their launch order, interleaved
    const int nbk = g.B * g.Hkv;
    const int chunk = blockIdx.x % a.tsplit, rest = blockIdx.x / a.tsplit;
    const int bk = rest % nbk, rank = rest / nbk, b = bk / g.Hkv, kvh = bk - b * g.Hkv;
    const long ui = (long)bk * a.npg + rank;  // rank < npg: the record exists
    const GroupPage e = a.upages[ui];
    // this lane's two rows' slots, loaded with the record, not after it
    const int16_t slot0 = a.slots[ui * kGroupMaxRows + (threadIdx.x & 63)];
    const int16_t slot1 = a.slots[ui * kGroupMaxRows + 64 + (threadIdx.x & 63)];
    if (rank >= a.nunion[bk]) return;
    const int p = e.page;
    const int lane = threadIdx.x & 63, wave = wave_index();
    const int r = lane & 15, j = lane >> 4;
    const Regions rg(g, b, a.S, a.W);

    // the rows that chose the page, ascending, and the page's index in each
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

    // this chunk of the page's middle-region tokens: contiguous rows of one
    // physical page (an unmapped page attends nothing); or of the block's
    // rows in the block layout
    const bool blocks = a.blk_off != nullptr;
    int a0, a1;
    if (blocks) {
        const int32_t* bo = a.blk_off + (long)bk * (a.npg + 1);
        a0 = bo[p];
        a1 = a.blk_end ? imax(a0, imin(a.blk_end[(long)bk * a.npg + p], bo[p + 1])) : bo[p + 1];
    } else {
        a0 = imax(p * g.P, rg.se);
        a1 = imin((p + 1) * g.P, rg.ws);
    }
    const int n = imax(0, a1 - a0);
    const int csz = (n + a.tsplit - 1) / a.tsplit;
    const int t0 = a0 + imin(n, chunk * csz);
    const int phys = e.phys;
    const bool mapped = phys >= 0;
    const int t1 = mapped ? imin(a1, t0 + csz) : t0;
    const int nst = (imax(0, t1 - t0) + kStage - 1) / kStage;
    // K/V row of token t0 (inside the page or the sequence's rows even when the chunk is empty)
    const long row0 = blocks   ? (long)bk * a.blk_n + imin(t0, a.blk_n - 1)
                      : mapped ? ((long)phys * g.Hkv + kvh) * g.P + imin(t0 - p * g.P, g.P - 1)
                               : 0;
    const uint16_t* kp = (const uint16_t*)(blocks ? a.blk_k : g.k) + row0 * HD;
    const uint16_t* vp = (const uint16_t*)(blocks ? a.blk_v : g.v) + row0 * HD;
    const int ntok = t1 - t0;

    const float sl2 = a.scale_log2, slack = kGSlack / sl2;
    const int ncol = nr * G, ncb = (ncol + 15) / 16;

    // Pass = up to kGW column blocks, one per wave.  With fewer blocks than
    // waves, the waves of a block take turns over the 16-token subtiles of
    // each stage and their states merge through LDS at the end of the pass,
    // so the work follows the live columns.  (The assignment is fixed, so
    // the results do not depend on timing.)
    for (int pass = 0; pass * kGW < ncb; ++pass) {
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
                    w = *(const uint4*)((const uint16_t*)a.q + (((long)b * g.Hq + kvh * G + h) * a.Q + row) * HD +
                                        32 * kk + 8 * j);
                qb[kk] = __builtin_bit_cast(gbf16x8_t, w);
            }
#pragma unroll
            for (int m = 0; m < NB; ++m) o[m] = gf32x4_t{0.f, 0.f, 0.f, 0.f};
        }

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
                x.k[u] = *(const uint4*)(kp + off);
                x.v[u] = *(const uint4*)(vp + off);
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
        // this wave's subtiles of stage st: gi, gi + gsz, ...
        auto compute = [&](int st, int buf) {
            if (!computes) return;
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
        // re-read the chunk's first row and compute nothing.
        Staged X0, X1, X2;
        fetch(0, X0);
        __builtin_amdgcn_sched_barrier(0);  // keep the stages' loads in stage order
        fetch(1, X1);
        __builtin_amdgcn_sched_barrier(0);
        fetch(2, X2);
        __builtin_amdgcn_sched_barrier(0);
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
                const long prow = ((long)b * g.Hq + kvh * G + h) * a.Q + rows_l[ri];
                const long slot = prow * a.split_stride + (long)slot_l[ri] * a.tsplit + chunk;
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
}

template <int HD>
hipError_t launch_group_g(const GroupArgs& a, dim3 grid, hipStream_t s)
{
    const dim3 block(64 * kGW);
    switch (a.g.G) {
    case 1: hipLaunchKernelGGL((k_group_decode_mfma<HD, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_group_decode_mfma<HD, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_group_decode_mfma<HD, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_group_decode_mfma<HD, 8>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_group_decode_mfma<HD, 16>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_group(const GroupArgs& a, int max_union, hipStream_t s)
{
    const Geometry& g = a.g;
    if (g.dtype != 1 || a.Q > kGroupMaxRows || a.npg > kGroupMaxPages) return hipErrorInvalidValue;
    const size_t lds = (2 * sizeof(unsigned long long) + sizeof(int)) * (size_t)a.npg;
    hipLaunchKernelGGL(k_group_plan, dim3((unsigned)(g.B * g.Hkv)), dim3(kPlanThreads), lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || max_union < 1) return e;
    const dim3 grid((unsigned)((long)max_union * a.tsplit * g.B * g.Hkv));
    if (g.hd == 128) return launch_group_g<128>(a, grid, s);
    if (g.hd == 64) return launch_group_g<64>(a, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace sa
