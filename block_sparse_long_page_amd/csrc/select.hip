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
//  * k_topk: one workgroup per (sequence, KV head, row) radix-selects the k-th
//    largest order key in LDS and writes the chosen pages in ascending order.
//    Ties go to the lower page index.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace sa {

namespace {

constexpr int kScoreWaves = 4;
constexpr int kScoreU = 4;  // page rows in flight per lane

// Quest bound for one channel pair: max(q*mn, q*mx) = q * (q >= 0 ? mx : mn),
// taken per bf16 half with a bit-select on q's sign bits.
__device__ __forceinline__ uint32_t quest_pick(uint32_t qw, uint32_t mn, uint32_t mx)
{
    // 0xffff in each half whose q is negative
    const uint32_t neg = ((qw >> 15) & 1u) * 0xffffu | ((qw >> 31) & 1u) * 0xffff0000u;
    return (mn & neg) | (mx & ~neg);
}

template <int HD, int G, bool BF, bool QUEST>
__global__ __launch_bounds__(64 * kScoreWaves) void k_score(SelectArgs a)
{
    // lanes per page row: Quest reads min and max rows in the cache dtype,
    // mean/centroid read one fp32 row
    constexpr int EB = QUEST ? (BF ? 2 : 4) : 4;
    constexpr int CH = 16 / EB;
    constexpr int LPT = HD / CH;
    constexpr int RPW = 64 / LPT;
    constexpr int U = kScoreU;
    constexpr int PAGES_PER_WG = RPW * U * kScoreWaves;
    const Geometry& g = a.g;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPT, rg = lane / LPT;

    int pid = blockIdx.y;
    const int row = pid % a.Q;
    pid /= a.Q;
    const int kvh = pid % g.Hkv;
    const int b = pid / g.Hkv;

    int L = imax(0, imin(g.seq_lens[b], g.max_pages * g.P));
    const int se = imin(a.S, L), ws = imax(se, L - a.W);
    if (ws <= se) return;
    const int plo = se / g.P, phi = (ws - 1) / g.P;
    const int first = plo + blockIdx.x * PAGES_PER_WG + wave * RPW * U;
    if (first > phi) return;

    // this lane's channels of the G queries of the group
    typedef typename std::conditional<BF, uint16_t, float>::type E;
    const long qrow0 = (((long)b * g.Hq + kvh * G) * a.Q + row) * HD;
    const long qstride = (long)a.Q * HD;
    uint32_t qw[G][4];   // QUEST && BF: packed bf16 pairs
    float qf[G][CH];     // otherwise: fp32 channels
    for (int h = 0; h < G; ++h) {
        const E* qp = (const E*)a.q + qrow0 + h * qstride;
        if constexpr (QUEST && BF) {
            const uint4 w = *(const uint4*)(qp + sub * CH);
            qw[h][0] = w.x;
            qw[h][1] = w.y;
            qw[h][2] = w.z;
            qw[h][3] = w.w;
        } else {
            for (int c = 0; c < CH; ++c) {
                if constexpr (BF)
                    qf[h][c] = __uint_as_float((uint32_t)((const uint16_t*)qp)[sub * CH + c] << 16);
                else
                    qf[h][c] = ((const float*)qp)[sub * CH + c];
            }
        }
    }

    float* out = a.scores + (((long)b * g.Hkv + kvh) * a.Q + row) * g.max_pages;
    uint4 w0[U], w1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int p = first + u * RPW + rg;
        int phys = p <= phi ? g.block_table[(long)b * g.max_pages + p] : -1;
        const bool ok = phys >= 0 && phys < g.num_phys;
        if constexpr (QUEST) {
            const E* m = (const E*)a.meta + ((long)phys * g.Hkv + kvh) * 2 * HD + sub * CH;
            w0[u] = ok ? *(const uint4*)m : make_uint4(0, 0, 0, 0);
            w1[u] = ok ? *(const uint4*)(m + HD) : make_uint4(0, 0, 0, 0);
        } else {
            const float* m = (const float*)a.meta + ((long)phys * g.Hkv + kvh) * HD + sub * CH;
            w0[u] = ok ? *(const uint4*)m : make_uint4(0, 0, 0, 0);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int p = first + u * RPW + rg;
        const int phys = p <= phi ? g.block_table[(long)b * g.max_pages + p] : -1;
        const bool ok = phys >= 0 && phys < g.num_phys;
        const uint32_t* a0 = (const uint32_t*)&w0[u];
        const uint32_t* a1 = (const uint32_t*)&w1[u];
        float best = -INFINITY;
        for (int h = 0; h < G; ++h) {
            float s = 0.f;
            if constexpr (QUEST && BF) {
                for (int j = 0; j < 4; ++j) s = dot2_bf16(qw[h][j], quest_pick(qw[h][j], a0[j], a1[j]), s);
            } else if constexpr (QUEST) {
                for (int c = 0; c < CH; ++c) {
                    const float q = qf[h][c];
                    s = fmaf(q, q >= 0.f ? __uint_as_float(a1[c]) : __uint_as_float(a0[c]), s);
                }
            } else {
                for (int c = 0; c < CH; ++c) s = fmaf(qf[h][c], __uint_as_float(a0[c]), s);
            }
            s = group_sum<LPT>(s);
            best = fmaxf(best, s);
        }
        if (sub == 0 && p <= phi) out[p] = ok ? best : -INFINITY;
    }
}

// order-preserving float -> uint32 (larger float, larger key); -0 maps to +0
__device__ __forceinline__ uint32_t order_key(float f)
{
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopkThreads = 256;

// Inclusive sum over the workgroup; returns the total in *total.
__device__ int block_inclusive_scan(int x, int* lds, int* total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) lds[wave] = x;
    __syncthreads();
    int before = 0, all = 0;
    for (int w = 0; w < kTopkThreads / 64; ++w) {
        const int v = lds[w];
        before += w < wave ? v : 0;
        all += v;
    }
    __syncthreads();
    *total = all;
    return x + before;
}

__global__ __launch_bounds__(kTopkThreads) void k_topk(SelectArgs a)
{
    extern __shared__ uint32_t keys[];  // [phi - plo + 1]
    __shared__ int hist[256];
    __shared__ int scan_tmp[kTopkThreads / 64];
    __shared__ int pick[2];
    const Geometry& g = a.g;
    int pid = blockIdx.x;
    const int row = pid % a.Q;
    pid /= a.Q;
    const int kvh = pid % g.Hkv;
    const int b = pid / g.Hkv;
    const long prob = ((long)b * g.Hkv + kvh) * a.Q + row;
    int32_t* sel = a.sel ? a.sel + prob * a.k_max : nullptr;

    int L = imax(0, imin(g.seq_lens[b], g.max_pages * g.P));
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
    const float* sc = a.scores + prob * g.max_pages + plo;
    for (int i = tid; i < n; i += kTopkThreads) keys[i] = order_key(sc[i]);

    // radix select of the k-th largest key, 8 bits at a time from the top
    uint32_t prefix = 0, mask = 0;
    int need = k;  // keys still to take among those matching `prefix`
    for (int shift = 24; shift >= 0; shift -= 8) {
        hist[tid] = 0;  // kTopkThreads == 256 bins
        __syncthreads();
        for (int i = tid; i < n; i += kTopkThreads) {
            const uint32_t key = keys[i];
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
        __syncthreads();
        if (tid < 64) {
            // lane j owns digits 255-4j .. 252-4j; suffix counts from the top
            int c[4], s = 0;
            for (int d = 0; d < 4; ++d) {
                c[d] = hist[255 - 4 * tid - d];
                s += c[d];
            }
            int incl = s;
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(incl, off);
                if (tid >= off) incl += y;
            }
            int above = incl - s;  // keys with a larger digit than this lane's first
            for (int d = 0; d < 4; ++d) {
                if (above < need && above + c[d] >= need) {
                    pick[0] = 255 - 4 * tid - d;
                    pick[1] = above;
                }
                above += c[d];
            }
        }
        __syncthreads();
        prefix |= (uint32_t)pick[0] << shift;
        mask |= 255u << shift;
        need -= pick[1];
        __syncthreads();
    }
    const uint32_t kth = prefix;  // keys > kth are in; `need` of the keys == kth, lowest pages first

    // ranks among equal keys and output slots, both in ascending page order
    constexpr int PER = 32;  // pages per thread per pass
    int eq_base = 0, out_base = 0;
    for (int base = 0; base < n; base += kTopkThreads * PER) {
        const int i0 = base + tid * PER;
        int eq = 0, gt = 0;
        for (int j = 0; j < PER; ++j) {
            const int i = i0 + j;
            if (i < n) {
                eq += keys[i] == kth;
                gt += keys[i] > kth;
            }
        }
        int eq_total;
        const int eq_before = block_inclusive_scan(eq, scan_tmp, &eq_total) - eq + eq_base;
        // a thread takes min(eq, max(0, need - eq_before)) of its equal keys
        const int take_eq = imin(eq, imax(0, need - eq_before));
        int out_total;
        const int out_before = block_inclusive_scan(gt + take_eq, scan_tmp, &out_total) - (gt + take_eq) + out_base;
        int slot = out_before, taken = 0;
        for (int j = 0; j < PER; ++j) {
            const int i = i0 + j;
            if (i < n) {
                const uint32_t key = keys[i];
                bool in = key > kth;
                if (key == kth && taken < take_eq) {
                    in = true;
                    ++taken;
                }
                if (in) sel[slot++] = plo + i;
            }
        }
        eq_base += eq_total;
        out_base += out_total;
    }
}

template <int HD, int G, bool BF>
hipError_t launch_score_mode(const SelectArgs& a, dim3 grid, hipStream_t s)
{
    if (a.mode == 0)
        hipLaunchKernelGGL((k_score<HD, G, BF, true>), grid, dim3(64 * kScoreWaves), 0, s, a);
    else
        hipLaunchKernelGGL((k_score<HD, G, BF, false>), grid, dim3(64 * kScoreWaves), 0, s, a);
    return hipGetLastError();
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
    if (a.k_max > 0) {
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
    const size_t lds = sizeof(uint32_t) * (size_t)(a.k_max > 0 ? g.max_pages : 1);
    hipLaunchKernelGGL(k_topk, dim3((unsigned)problems), dim3(kTopkThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace sa
