// Page selection (hybrid sparse attention page: the Quest pages most relevant
// to the current query, chosen per head; attention-mechanisms article,
// "Learned top-k sparse attention": top-k blocks per GQA group).
//
// Two kernels:
//  * k_score_quest_mfma (Quest, bf16 cache) / k_score_f32_mfma (fp32
//    summaries): many workgroups per (sequence, KV head, row) stream the page
//    summaries of the candidate pages once, score each page against the G
//    query heads of the group on the matrix cores and keep the group
//    maximum, fp32, in the workspace.  Selection reads megabytes of summaries
//    per step, so it is spread over the whole GPU rather than run by one
//    workgroup per problem.
//  * k_topk: one workgroup per (sequence, KV head, row) keeps the order keys
//    of the candidates in registers, radix-selects the k-th largest starting
//    at the highest bit where the keys differ, and writes the chosen pages in
//    ascending order.  Ties go to the lower page index.
#include "device_common.hpp"
#include "kernels.hpp"
#include "topk_block.hpp"

namespace sa {

namespace {

constexpr int kScoreWaves = 4;

typedef __bf16 sbf16x8_t __attribute__((ext_vector_type(8)));
typedef float sf32x4_t __attribute__((ext_vector_type(4)));

#ifndef SA_SCORE_TW
#define SA_SCORE_TW 2
#endif

// Scores of fp32 summary rows on the matrix cores (fp32 product, fp32 sums):
// the scores of 16 pages for the G heads are one product of the pages'
// summary rows (A: row = page) with the heads' query rows (B: column = head;
// heads past G are zero) over K = the row length, four channels per step.
// Lane (r, j) = (lane % 16, lane / 16) loads channels 4j .. 4j+3 of every
// 16-channel group of its row as one 16-byte vector, and step (s, i) takes
// channel 16 s + 4j + i of both operands; lane (r, j) of the result holds
// head r's scores of pages 4j .. 4j+3, and the group maximum is a DPP max
// over the 16 lanes of its row.
//   KIND 0 (Quest, fp32 cache): rows [mn | mx] against [q- | q+] (K = 2 hd),
//     since max(q_c mn_c, q_c mx_c) = q-_c mn_c + q+_c mx_c term by term.
//   KIND 1 (mean, centroid): rows = the summary, score = q . summary.
//   KIND 2 (compressed keys): as KIND 1, and page p also takes the score of
//     the block starting at p-1 (it covers p too) when p-1 is mapped.  A wave
//     then scores the page before its first output page as well, and each
//     output page takes the larger of its own score and its predecessor's
//     (same lane, the lane group before, or the tile before).
// With a bf16 cache (KIND 1 and 2) the queries are exact in bf16 and each
// fp32 summary element splits exactly into three bf16 parts, hi + mid + lo
// (each the rounded remainder of the one before; 24 bits in all), so the
// product runs as three bf16 products with fp32 sums (16x16x32 steps, lane
// (r, j) holding channels 8j .. 8j+7 of every 32-channel group): an fp32
// product at a third of the matrix-core time, since the fp32 steps would
// spend half their columns on absent heads when G = 8.
template <int HD, int G, bool BF, int KIND>
__global__ __launch_bounds__(64 * kScoreWaves) void k_score_f32_mfma(SelectArgs a)
{
    constexpr bool QUEST = KIND == 0, PREV = KIND == 2;
    constexpr bool SPLIT = BF && !QUEST;               // three bf16 parts per summary element
    constexpr int RL = QUEST ? 2 * HD : HD;           // fp32 elements per summary row
    constexpr int KV = RL / 16;                        // 16-byte pieces per lane per row
    constexpr int QP = HD / 16;                        // query pieces per lane (fp32 steps)
    constexpr int KC = HD / 32;                        // 32-channel groups (bf16 steps)
    constexpr int TW = QUEST ? 1 : SA_SCORE_TW;        // tiles of 16 pages per wave
    constexpr int OUT_PER_WAVE = 16 * TW - (PREV ? 1 : 0);
    constexpr int OUT_PER_WG = OUT_PER_WAVE * kScoreWaves;
    static_assert(G <= 16, "one MFMA column per head");
    const Geometry& g = a.g;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, j = lane >> 4;

    if (a.status && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a.status = 0u;
    if (a.counters && blockIdx.x == 0 && blockIdx.y == 0)
        for (int i = threadIdx.x; i < a.ncounters; i += blockDim.x) a.counters[i] = 0u;
    int pid = blockIdx.y;
    const int row = pid % a.Q;
    pid /= a.Q;
    const int kvh = pid % g.Hkv;
    const int b = pid / g.Hkv;

    const int L = imax(0, imin(g.seq_lens[b], g.max_pages * g.P));
    const int se = imin(a.S, L), ws = imax(se, L - a.W);
    if (ws <= se) return;
    const int plo = se / g.P, phi = (ws - 1) / g.P;
    const int first_out = plo + blockIdx.x * OUT_PER_WG + wave * OUT_PER_WAVE;
    if (first_out > phi) return;
    const int first = first_out - (PREV ? 1 : 0);  // page of tile row 0 (-1 when there is none)

    // A: summary rows of this wave's pages, all in flight at once
    const long meta_row = ((long)b * g.Hkv + kvh) * g.max_pages;
    const float* meta = (const float*)a.meta;
    float4 am[TW][KV];
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        const int p = first + 16 * t + r;
#pragma unroll
        for (int s = 0; s < KV; ++s) {
            // fp32 steps: channels 16 s + 4j .. +3; bf16 steps: piece s covers
            // channels 32 (s/2) + 8j + 4 (s%2) .. +3
            const int ch = SPLIT ? 32 * (s >> 1) + 8 * j + 4 * (s & 1) : 16 * s + 4 * j;
            am[t][s] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (p >= 0 && p <= phi) am[t][s] = *(const float4*)(meta + (meta_row + p) * RL + ch);
        }
    }
    // block-table entries of pages 4j .. 4j+3 of each tile (unmapped pages score -inf)
    const int32_t* bt = g.block_table + (long)b * g.max_pages;
    bool ok[TW][4];
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = first + 16 * t + 4 * j + i;
            const int ph = p >= 0 && p <= phi ? bt[p] : -1;
            ok[t][i] = ph >= 0 && ph < g.num_phys;
        }
    // B: head r's channels, in fp32 (16 s + 4j .. +3) or bf16 (32 s + 8j .. +7)
    const long qoff = (((long)b * g.Hq + kvh * G + r) * a.Q + row) * HD;
    float4 qv[SPLIT ? 1 : QP];
    uint4 qb[SPLIT ? KC : 1];
    if constexpr (SPLIT) {
#pragma unroll
        for (int s = 0; s < KC; ++s)
            qb[s] = r < G ? *(const uint4*)((const uint16_t*)a.q + qoff + 32 * s + 8 * j) : make_uint4(0, 0, 0, 0);
    } else {
#pragma unroll
        for (int s = 0; s < QP; ++s) {
            qv[s] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < G) {
                if constexpr (BF) {
                    const uint2 w = *(const uint2*)((const uint16_t*)a.q + qoff + 16 * s + 4 * j);
                    qv[s] = make_float4(bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y));
                } else {
                    qv[s] = *(const float4*)((const float*)a.q + qoff + 16 * s + 4 * j);
                }
            }
        }
    }

    float* out = a.scores + (((long)b * g.Hkv + kvh) * a.Q + row) * g.max_pages;
    float prev3 = -INFINITY;  // the tile before's score of its last page (PREV)
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        sf32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (SPLIT) {
#pragma unroll
            for (int s = 0; s < KC; ++s) {
                const float* x = (const float*)&am[t][2 * s];  // 8 channels (two adjacent pieces)
                const float* y = (const float*)&am[t][2 * s + 1];
                float v[8] = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
#pragma unroll
                for (int part = 0; part < 3; ++part) {
                    uint4 w;
                    uint32_t* ww = (uint32_t*)&w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ww[e] = pack_bf16(v[2 * e], v[2 * e + 1]);
                        v[2 * e] -= bf_lo(ww[e]);  // exact: the remainder of a rounding
                        v[2 * e + 1] -= bf_hi(ww[e]);
                    }
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sbf16x8_t, w),
                                                                  __builtin_bit_cast(sbf16x8_t, qb[s]), acc, 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < KV; ++s) {
                const float* av = (const float*)&am[t][s];
                float bq[4];
                if constexpr (QUEST) {
                    // pieces 0 .. QP-1 are the min row (q-), QP .. 2QP-1 the max row (q+)
                    const float* qq = (const float*)&qv[s % QP];
#pragma unroll
                    for (int i = 0; i < 4; ++i) bq[i] = s < QP ? fminf(qq[i], 0.f) : fmaxf(qq[i], 0.f);
                } else {
                    const float* qq = (const float*)&qv[s];
#pragma unroll
                    for (int i = 0; i < 4; ++i) bq[i] = qq[i];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bq[i], acc, 0, 0, 0);
            }
        }
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float best = group_max<16>(r < G ? acc[i] : -INFINITY);
            sc[i] = ok[t][i] ? best : -INFINITY;
        }
        if constexpr (PREV) {
            // predecessor of page 4j: the lane group before (j > 0) or the tile before (j == 0)
            const int src = (lane + 48) & 63;
            const float from_group = __shfl(sc[3], src);
            const float pred0 = j > 0 ? from_group : prev3;
            prev3 = __shfl(sc[3], (lane & 15) + 48);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ri = 16 * t + 4 * j + i;
                const int p = first + ri;
                const float pred = i > 0 ? sc[i - 1] : pred0;
                if (r == 0 && ri > 0 && p <= phi) out[p] = ok[t][i] ? fmaxf(sc[i], pred) : -INFINITY;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p = first + 16 * t + 4 * j + i;
                if (r == 0 && p <= phi) out[p] = sc[i];
            }
        }
    }
}

// Quest scores of bf16 summaries on the matrix cores.  With q+ = max(q, 0) and
// q- = min(q, 0), max(q_c mx_c, q_c mn_c) = q+_c mx_c + q-_c mn_c term by term,
// so the bounds of 16 pages for the G heads are one product of the pages'
// summary rows [mn | mx] (A: row = page, 8 elements per lane straight from
// global memory) with the heads' [q- | q+] (B: column = head; heads past G are
// zero), over K = 2 * head_dim.  Lane (r, j) = (lane % 16, lane / 16) then
// holds head r's bounds of pages 4j .. 4j+3; the group maximum is a DPP max
// over the 16 lanes of its row.  Each wave scores TW tiles of 16 pages with
// every summary load issued up front.
template <int HD, int G>
__global__ __launch_bounds__(64 * kScoreWaves) void k_score_quest_mfma(SelectArgs a)
{
    constexpr int KQ = HD / 32;        // 32-channel groups per summary row half
    constexpr int KS = 2 * KQ;         // products per tile (mn half, then mx half)
    constexpr int TW = SA_SCORE_TW;    // tiles per wave
    constexpr int PAGES_PER_WG = 16 * TW * kScoreWaves;
    static_assert(G <= 16, "one MFMA column per head");
    const Geometry& g = a.g;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, j = lane >> 4;

    if (a.status && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a.status = 0u;
    if (a.counters && blockIdx.x == 0 && blockIdx.y == 0)
        for (int i = threadIdx.x; i < a.ncounters; i += blockDim.x) a.counters[i] = 0u;
    int pid = blockIdx.y;
    const int row = pid % a.Q;
    pid /= a.Q;
    const int kvh = pid % g.Hkv;
    const int b = pid / g.Hkv;

    const int L = imax(0, imin(g.seq_lens[b], g.max_pages * g.P));
    const int se = imin(a.S, L), ws = imax(se, L - a.W);
    if (ws <= se) return;
    const int plo = se / g.P, phi = (ws - 1) / g.P;
    const int first = plo + blockIdx.x * PAGES_PER_WG + wave * 16 * TW;
    if (first > phi) return;

    // A: summary rows of this wave's pages, all in flight at once
    const long meta_row = ((long)b * g.Hkv + kvh) * g.max_pages;
    const uint16_t* meta = (const uint16_t*)a.meta;
    uint4 am[TW][KS];
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        const int p = first + 16 * t + r;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            am[t][s] = make_uint4(0, 0, 0, 0);
            if (p <= phi) am[t][s] = *(const uint4*)(meta + (meta_row + p) * 2 * HD + 32 * s + 8 * j);
        }
    }
    // block-table entries of pages 4j .. 4j+3 of each tile (unmapped pages score -inf)
    const int32_t* bt = g.block_table + (long)b * g.max_pages;
    int ph[TW][4];
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = first + 16 * t + 4 * j + i;
            ph[t][i] = p <= phi ? bt[p] : -1;
        }
    // B: head r's q- (for the mn half) and q+ (for the mx half), 8 channels per lane
    uint4 qn[KQ], qp[KQ];
#pragma unroll
    for (int s = 0; s < KQ; ++s) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (r < G) w = *(const uint4*)((const uint16_t*)a.q + (((long)b * g.Hq + kvh * G + r) * a.Q + row) * HD +
                                       32 * s + 8 * j);
        uint32_t* wn = (uint32_t*)&qn[s];
        uint32_t* wp = (uint32_t*)&qp[s];
        const uint32_t* ww = (const uint32_t*)&w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t neg = ((ww[e] >> 15) & 1u) * 0xffffu | ((ww[e] >> 31) & 1u) * 0xffff0000u;
            wn[e] = ww[e] & neg;
            wp[e] = ww[e] & ~neg;
        }
    }

    float* out = a.scores + (((long)b * g.Hkv + kvh) * a.Q + row) * g.max_pages;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        sf32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sbf16x8_t, am[t][s]),
                                                          __builtin_bit_cast(sbf16x8_t, s < KQ ? qn[s] : qp[s - KQ]),
                                                          acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float best = group_max<16>(r < G ? acc[i] : -INFINITY);
            const int p = first + 16 * t + 4 * j + i;
            if (r == 0 && p <= phi) out[p] = ph[t][i] >= 0 && ph[t][i] < g.num_phys ? best : -INFINITY;
        }
    }
}

// One workgroup per (sequence, KV head, row): the block top-k of its
// candidates' scores, written in ascending page order.
__global__ __launch_bounds__(kTopkThreads) void k_topk(SelectArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint32_t keys[];  // [n]
    __shared__ TopkScratch sh;
    const Geometry& g = a.g;
    int pid = blockIdx.x;
    const int row = pid % a.Q;
    pid /= a.Q;
    const int kvh = pid % g.Hkv;
    const int b = pid / g.Hkv;
    const long prob = ((long)b * g.Hkv + kvh) * a.Q + row;
    int32_t* sel = a.sel ? a.sel + prob * a.k_max : nullptr;

    const int L = imax(0, imin(g.seq_lens[b], g.max_pages * g.P));
    const int se = imin(a.S, L), ws = imax(se, L - a.W);
    const int plo = se / g.P;
    const int n = ws > se ? (ws - 1) / g.P - plo + 1 : 0;
    const int k = imin(a.k_max, n);
    const int tid = threadIdx.x;
    if (tid == 0) a.count[prob] = k;
    if (sel)
        for (int i = k + tid; i < a.k_max; i += kTopkThreads) sel[i] = -1;
    if (k == 0) return;
    if (k == n) {
        for (int i = tid; i < n; i += kTopkThreads) sel[i] = plo + i;
        return;
    }
    uint32_t lo, hi;
    topk_load_keys(a.scores + prob * g.max_pages + plo, n, keys, lo, hi);
    block_topk_fast(n, k, keys, lo, hi, sh, [&](int pos, int i) { sel[pos] = plo + i; });
}

// Two-stage selection, stage 1: workgroup (chunk c, problem) ranks the
// candidates [c * kTopkChunk, (c + 1) * kTopkChunk) of its problem and
// writes its min(k, chunk size) best (ties to the lower index) as order keys
// and candidate indices, ascending.  Every candidate among the problem's k
// best is among its chunk's best, so the merge of the winners is exact.
__global__ __launch_bounds__(kTopkThreads) void k_topk_chunk(SelectArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint32_t keys[];  // [kTopkChunk]
    __shared__ TopkScratch sh;
    const Geometry& g = a.g;
    const int c = blockIdx.x;
    int pid = blockIdx.y;
    const int row = pid % a.Q;
    pid /= a.Q;
    const int kvh = pid % g.Hkv;
    const int b = pid / g.Hkv;
    const long prob = ((long)b * g.Hkv + kvh) * a.Q + row;

    const int L = imax(0, imin(g.seq_lens[b], g.max_pages * g.P));
    const int se = imin(a.S, L), ws = imax(se, L - a.W);
    const int plo = se / g.P;
    const int n = ws > se ? (ws - 1) / g.P - plo + 1 : 0;
    const int k = imin(a.k_max, n);
    const int c0 = c * kTopkChunk;
    const int nc = imin(n - c0, kTopkChunk);
    if (k == 0 || k == n || nc <= 0) return;  // the merge needs no winners from this chunk
    const int kc = imin(k, nc);
    uint32_t* pk = a.part_keys + (prob * a.nchunks + c) * a.kc;
    int32_t* pi = a.part_idx + (prob * a.nchunks + c) * a.kc;
    uint32_t lo, hi;
    topk_load_keys(a.scores + prob * g.max_pages + plo + c0, nc, keys, lo, hi);
    if (kc == nc) {  // the whole chunk
        __syncthreads();
        for (int i = threadIdx.x; i < nc; i += kTopkThreads) {
            pk[i] = keys[i];
            pi[i] = c0 + i;
        }
        return;
    }
    block_topk_fast(nc, kc, keys, lo, hi, sh, [&](int pos, int i) {
        pk[pos] = keys[i];
        pi[pos] = c0 + i;
    });
}

// Stage 2: one workgroup per problem ranks the chunks' winners, laid out
// chunk after chunk (so ascending candidate order and ties to the lower
// page carry over), and writes the k best pages ascending.
__global__ __launch_bounds__(kTopkThreads) void k_topk_merge(SelectArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint32_t keys[];  // [kTopkMerge]
    __shared__ TopkScratch sh;
    __shared__ int off[kTopkMerge / 64 + 2];  // first merged position of each chunk's winners
    const Geometry& g = a.g;
    int pid = blockIdx.x;
    const int row = pid % a.Q;
    pid /= a.Q;
    const int kvh = pid % g.Hkv;
    const int b = pid / g.Hkv;
    const long prob = ((long)b * g.Hkv + kvh) * a.Q + row;
    int32_t* sel = a.sel + prob * a.k_max;

    const int L = imax(0, imin(g.seq_lens[b], g.max_pages * g.P));
    const int se = imin(a.S, L), ws = imax(se, L - a.W);
    const int plo = se / g.P;
    const int n = ws > se ? (ws - 1) / g.P - plo + 1 : 0;
    const int k = imin(a.k_max, n);
    const int tid = threadIdx.x;
    if (tid == 0) a.count[prob] = k;
    for (int i = k + tid; i < a.k_max; i += kTopkThreads) sel[i] = -1;
    if (k == 0) return;
    if (k == n) {
        for (int i = tid; i < n; i += kTopkThreads) sel[i] = plo + i;
        return;
    }
    const int nch = (n + kTopkChunk - 1) / kTopkChunk;  // <= a.nchunks
    if (tid == 0) {
        int m = 0;
        for (int c = 0; c < nch; ++c) {
            off[c] = m;
            m += imin(k, imin(n - c * kTopkChunk, kTopkChunk));
        }
        off[nch] = m;
    }
    __syncthreads();
    const int m = off[nch];  // <= kTopkMerge (host-checked)
    const uint32_t* pk = a.part_keys + prob * a.nchunks * a.kc;
    const int32_t* pi = a.part_idx + prob * a.nchunks * a.kc;
    uint32_t lo = 0xffffffffu, hi = 0;
    for (int c = 0; c < nch; ++c) {
        const int cnt = off[c + 1] - off[c];
        for (int i = tid; i < cnt; i += kTopkThreads) {
            const uint32_t key = pk[c * a.kc + i];
            keys[off[c] + i] = key;
            lo = min(lo, key);
            hi = max(hi, key);
        }
    }
    block_topk_fast(m, k, keys, lo, hi, sh, [&](int pos, int i) {
        int c = 0;
        while (c + 1 < nch && off[c + 1] <= i) ++c;
        sel[pos] = plo + pi[c * a.kc + (i - off[c])];
    });
}

template <int HD, int G, bool BF>
hipError_t launch_score_f32(const SelectArgs& a, hipStream_t s)
{
    const int kind = a.mode == 0 ? 0 : a.mode == 3 ? 2 : 1;
    const int tw = kind == 0 ? 1 : SA_SCORE_TW;
    const int per_wg = (16 * tw - (kind == 2 ? 1 : 0)) * kScoreWaves;
    const dim3 grid((unsigned)((a.g.max_pages + per_wg - 1) / per_wg), (unsigned)(a.g.B * a.g.Hkv * a.Q));
    const dim3 block(64 * kScoreWaves);
    if (kind == 0) {
        if constexpr (BF) return hipErrorInvalidValue;  // bf16 Quest bounds: k_score_quest_mfma
        else hipLaunchKernelGGL((k_score_f32_mfma<HD, G, BF, 0>), grid, block, 0, s, a);
    } else if (kind == 1)
        hipLaunchKernelGGL((k_score_f32_mfma<HD, G, BF, 1>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_score_f32_mfma<HD, G, BF, 2>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int HD, int G>
hipError_t launch_score_quest_bf16(const SelectArgs& a, hipStream_t s)
{
    constexpr int per_wg = 16 * SA_SCORE_TW * kScoreWaves;
    const dim3 grid((unsigned)((a.g.max_pages + per_wg - 1) / per_wg), (unsigned)(a.g.B * a.g.Hkv * a.Q));
    hipLaunchKernelGGL((k_score_quest_mfma<HD, G>), grid, dim3(64 * kScoreWaves), 0, s, a);
    return hipGetLastError();
}

template <int HD>
hipError_t launch_score_quest_bf16_g(const SelectArgs& a, hipStream_t s)
{
    switch (a.g.G) {
    case 1: return launch_score_quest_bf16<HD, 1>(a, s);
    case 2: return launch_score_quest_bf16<HD, 2>(a, s);
    case 4: return launch_score_quest_bf16<HD, 4>(a, s);
    case 8: return launch_score_quest_bf16<HD, 8>(a, s);
    case 16: return launch_score_quest_bf16<HD, 16>(a, s);
    default: return hipErrorInvalidValue;
    }
}

template <int HD, bool BF>
hipError_t launch_score_f32_g(const SelectArgs& a, hipStream_t s)
{
    switch (a.g.G) {
    case 1: return launch_score_f32<HD, 1, BF>(a, s);
    case 2: return launch_score_f32<HD, 2, BF>(a, s);
    case 4: return launch_score_f32<HD, 4, BF>(a, s);
    case 8: return launch_score_f32<HD, 8, BF>(a, s);
    case 16: return launch_score_f32<HD, 16, BF>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t s)
{
    const Geometry& g = a.g;
    const int problems = g.B * g.Hkv * a.Q;
    if (a.k_max > 0 && a.mode == 0 && g.dtype == 1) {
        const hipError_t e = g.hd == 128 ? launch_score_quest_bf16_g<128>(a, s) : launch_score_quest_bf16_g<64>(a, s);
        if (e != hipSuccess) return e;
    } else if (a.k_max > 0) {
        // fp32 summaries (and Quest bounds of an fp32 cache)
        const bool bf = g.dtype == 1;
        hipError_t e;
        if (g.hd == 128)
            e = bf ? launch_score_f32_g<128, true>(a, s) : launch_score_f32_g<128, false>(a, s);
        else if (g.hd == 64)
            e = bf ? launch_score_f32_g<64, true>(a, s) : launch_score_f32_g<64, false>(a, s);
        else
            return hipErrorInvalidValue;
        if (e != hipSuccess) return e;
    }
    if (a.score_only) return hipSuccess;
    if (a.nchunks > 0 && a.k_max > 0) {  // more candidates than one workgroup ranks
        hipLaunchKernelGGL(k_topk_chunk, dim3((unsigned)a.nchunks, (unsigned)problems), dim3(kTopkThreads),
                           sizeof(uint32_t) * kTopkChunk, s, a);
        hipLaunchKernelGGL(k_topk_merge, dim3((unsigned)problems), dim3(kTopkThreads), sizeof(uint32_t) * kTopkMerge,
                           s, a);
        return hipGetLastError();
    }
    const size_t lds = sizeof(uint32_t) * (size_t)(a.k_max > 0 ? g.max_pages : 1);  // <= 48 KiB (host-checked)
    hipLaunchKernelGGL(k_topk, dim3((unsigned)problems), dim3(kTopkThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace sa
