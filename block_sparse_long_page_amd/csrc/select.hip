// Page selection (hybrid sparse attention page: the Quest pages most relevant
// to the current query, chosen per head; attention-mechanisms article,
// "Learned top-k sparse attention": top-k blocks per GQA group).
//
// Two kernels:
//  * k_score: many workgroups per (sequence, KV head, row) stream the page
//    summaries of the candidate pages once, score each page against the G
//    query heads of the group and keep the group maximum, fp32, in the
//    workspace.  Selection reads megabytes of summaries per step, so it is
//    spread over the whole GPU rather than run by one workgroup per problem.
//  * k_topk: one workgroup per (sequence, KV head, row) keeps the order keys
//    of the candidates in registers, radix-selects the k-th largest starting
//    at the highest bit where the keys differ, and writes the chosen pages in
//    ascending order.  Ties go to the lower page index.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "topk_block.hpp"

namespace sa {

namespace {

#ifndef SA_SCORE_U
#define SA_SCORE_U 8
#endif
constexpr int kScoreWaves = 4;
constexpr int kScoreU = SA_SCORE_U;  // page rows per lane, all loaded at once

// Each wave scores RPW * U consecutive candidate pages with every summary load
// issued up front (selection is latency-bound: one round trip per wave); the
// workgroup stages the group's queries in LDS once.
// PREV (compressed keys): a page also scores against the summary of the
// page before when that page is mapped (the block starting there covers this
// page too); its score is the larger of the two.
template <int HD, int G, bool BF, bool QUEST, bool PREV>
__global__ __launch_bounds__(64 * kScoreWaves) void k_score(SelectArgs a)
{
    // lanes per page row: Quest reads min and max rows in the cache dtype,
    // mean/centroid read one fp32 row
    constexpr int EB = QUEST ? (BF ? 2 : 4) : 4;
    constexpr int CH = 16 / EB;
    constexpr int LPT = HD / CH;
    constexpr int RPW = 64 / LPT;
    constexpr int U = kScoreU;
    constexpr int PER_WAVE = RPW * U;
    constexpr int PAGES_PER_WG = PER_WAVE * kScoreWaves;
    // packed-bf16 Quest scores reduce-scatter the G head sums (LPT <= 16)
    constexpr bool RS = QUEST && BF && LPT <= 16;
    constexpr int HPL = RS && G > LPT ? G / LPT : 1;
    constexpr int QB = BF ? 2 : 4;             // bytes per query element
    constexpr int QV = HD * QB / 16;           // 16-byte vectors per query row
    typedef typename std::conditional<BF, uint16_t, float>::type E;
    __shared__ uint4 q_lds[G * QV];
    const Geometry& g = a.g;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPT, rg = lane / LPT;

    int pid = blockIdx.y;
    const int row = pid % a.Q;
    pid /= a.Q;
    const int kvh = pid % g.Hkv;
    const int b = pid / g.Hkv;

    const int L = imax(0, imin(g.seq_lens[b], g.max_pages * g.P));
    const int se = imin(a.S, L), ws = imax(se, L - a.W);
    if (ws <= se) return;
    const int plo = se / g.P, phi = (ws - 1) / g.P;
    const int wg_first = plo + blockIdx.x * PAGES_PER_WG;
    if (wg_first > phi) return;

    // every summary row of this wave's pages and their block-table entries
    // are requested before the query staging, so the two round trips overlap
    const int first = wg_first + wave * PER_WAVE;
    const long meta_row = ((long)b * g.Hkv + kvh) * g.max_pages;
    const int32_t* bt = g.block_table + (long)b * g.max_pages;
    uint4 w0[U], w1[U];
    bool ok[U], okp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int p = first + u * RPW + rg;
        const bool in = p <= phi;
        const int phys = in ? bt[p] : -1;
        ok[u] = phys >= 0 && phys < g.num_phys;
        if constexpr (PREV) {
            const int pp = in && p > 0 ? bt[p - 1] : -1;
            okp[u] = pp >= 0 && pp < g.num_phys;
        }
        if constexpr (QUEST) {
            const E* m = (const E*)a.meta + (meta_row + p) * 2 * HD + sub * CH;
            w0[u] = in ? *(const uint4*)m : make_uint4(0, 0, 0, 0);
            w1[u] = in ? *(const uint4*)(m + HD) : make_uint4(0, 0, 0, 0);
        } else {
            const float* m = (const float*)a.meta + (meta_row + p) * HD + sub * CH;
            w0[u] = in ? *(const uint4*)m : make_uint4(0, 0, 0, 0);
            if constexpr (PREV) w1[u] = okp[u] ? *(const uint4*)(m - HD) : make_uint4(0, 0, 0, 0);
        }
    }

    const long qrow0 = (((long)b * g.Hq + kvh * G) * a.Q + row) * HD;
    for (int i = threadIdx.x; i < G * QV; i += 64 * kScoreWaves) {
        const int h = i / QV, v = i % QV;
        q_lds[i] = ((const uint4*)((const E*)a.q + qrow0 + (long)h * a.Q * HD))[v];
    }
    __syncthreads();
    if (first > phi) return;

    // this lane's channels of the G queries
    uint32_t qw[G][4];   // Quest + bf16: packed pairs
    uint32_t neg[G][4];  // Quest + bf16: 0xffff in each half whose q is negative
    float qf[G][CH];     // otherwise: fp32 channels
    for (int h = 0; h < G; ++h) {
        if constexpr (QUEST && BF) {
            const uint4 w = q_lds[h * QV + sub];
            qw[h][0] = w.x;
            qw[h][1] = w.y;
            qw[h][2] = w.z;
            qw[h][3] = w.w;
            for (int j = 0; j < 4; ++j)
                neg[h][j] = ((qw[h][j] >> 15) & 1u) * 0xffffu | ((qw[h][j] >> 31) & 1u) * 0xffff0000u;
        } else {
            const E* qh = (const E*)&q_lds[h * QV];
            for (int c = 0; c < CH; ++c) {
                if constexpr (BF)
                    qf[h][c] = __uint_as_float((uint32_t)((const uint16_t*)qh)[sub * CH + c] << 16);
                else
                    qf[h][c] = ((const float*)qh)[sub * CH + c];
            }
        }
    }

    float* out = a.scores + (((long)b * g.Hkv + kvh) * a.Q + row) * g.max_pages;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int p = first + u * RPW + rg;
        const uint32_t* a0 = (const uint32_t*)&w0[u];
        const uint32_t* a1 = (const uint32_t*)&w1[u];
        float best;
        if constexpr (RS) {
            // max(q*mn, q*mx) = q * (q >= 0 ? mx : mn), picked per bf16 half by q's sign
            float d[G];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) s = dot2_bf16(qw[h][j], (a0[j] & neg[h][j]) | (a1[j] & ~neg[h][j]), s);
                d[h] = s;
            }
            reduce_scatter<G, log2c<LPT>() - 1>(d, lane);
            best = d[0];
#pragma unroll
            for (int j = 1; j < HPL; ++j) best = fmaxf(best, d[j]);
            best = group_max<LPT>(best);
        } else {
            best = -INFINITY;
            for (int h = 0; h < G; ++h) {
                float s = 0.f;
                if constexpr (QUEST) {
                    for (int c = 0; c < CH; ++c) {
                        const float q = qf[h][c];
                        s = fmaf(q, q >= 0.f ? __uint_as_float(a1[c]) : __uint_as_float(a0[c]), s);
                    }
                } else {
                    for (int c = 0; c < CH; ++c) s = fmaf(qf[h][c], __uint_as_float(a0[c]), s);
                }
                best = fmaxf(best, group_sum<LPT>(s));
                if constexpr (PREV) {
                    float s1 = 0.f;
                    for (int c = 0; c < CH; ++c) s1 = fmaf(qf[h][c], __uint_as_float(a1[c]), s1);
                    s1 = group_sum<LPT>(s1);
                    if (okp[u]) best = fmaxf(best, s1);
                }
            }
        }
        if (sub == 0 && p <= phi) out[p] = ok[u] ? best : -INFINITY;
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
typedef __bf16 sbf16x8_t __attribute__((ext_vector_type(8)));
typedef float sf32x4_t __attribute__((ext_vector_type(4)));

#ifndef SA_SCORE_TW
#define SA_SCORE_TW 2
#endif

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

template <int HD, int G, bool BF>
hipError_t launch_score_mode(const SelectArgs& a, dim3 grid, hipStream_t s)
{
    if (a.mode == 0)
        hipLaunchKernelGGL((k_score<HD, G, BF, true, false>), grid, dim3(64 * kScoreWaves), 0, s, a);
    else if (a.mode == 3)
        hipLaunchKernelGGL((k_score<HD, G, BF, false, true>), grid, dim3(64 * kScoreWaves), 0, s, a);
    else
        hipLaunchKernelGGL((k_score<HD, G, BF, false, false>), grid, dim3(64 * kScoreWaves), 0, s, a);
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
hipError_t launch_score_g(const SelectArgs& a, dim3 grid, hipStream_t s)
{
    switch (a.g.G) {
    case 1: return launch_score_mode<HD, 1, BF>(a, grid, s);
    case 2: return launch_score_mode<HD, 2, BF>(a, grid, s);
    case 4: return launch_score_mode<HD, 4, BF>(a, grid, s);
    case 8: return launch_score_mode<HD, 8, BF>(a, grid, s);
    case 16: return launch_score_mode<HD, 16, BF>(a, grid, s);
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
        // rows per wave load of the score kernel, as in k_score
        const int eb = a.mode == 0 ? (g.dtype == 1 ? 2 : 4) : 4;
        const int lpt = g.hd / (16 / eb);
        const int pages_per_wg = (64 / lpt) * kScoreU * kScoreWaves;
        const dim3 grid((unsigned)((g.max_pages + pages_per_wg - 1) / pages_per_wg), (unsigned)problems);
        const bool bf = g.dtype == 1;
        hipError_t e;
        if (g.hd == 128)
            e = bf ? launch_score_g<128, true>(a, grid, s) : launch_score_g<128, false>(a, grid, s);
        else if (g.hd == 64)
            e = bf ? launch_score_g<64, true>(a, grid, s) : launch_score_g<64, false>(a, grid, s);
        else
            return hipErrorInvalidValue;
        if (e != hipSuccess) return e;
    }
    if (a.score_only) return hipSuccess;
    const size_t lds = sizeof(uint32_t) * (size_t)(a.k_max > 0 ? g.max_pages : 1);  // <= 48 KiB (host-checked)
    hipLaunchKernelGGL(k_topk, dim3((unsigned)problems), dim3(kTopkThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace sa
