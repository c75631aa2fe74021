// Page summaries: per (physical page, KV head) slab of P x hd keys, the
// per-channel min and max (Quest pages, hybrid sparse attention page), the
// mean key (a block key for MoBA-style gating, course module 14, section
// 14.3), the unit-norm mean of unit-norm keys (semantic block centres,
// semantic-blocks page), or the mean key of the two pages starting at the
// page (compressed key of a block of 2P keys with stride P, self-indexing
// attention page, "Compressed keys", mean-pooled).
//
// One wave per (sequence, logical page, KV head).  The wave reads the slab
// with 16-byte loads: LPT lanes cover one key row (8 bf16 or 4 fp32 channels
// each), 64/LPT rows per load, U loads in flight.  Partial results of the
// row groups are folded with cross-lane shuffles at the end.
#include "device_common.hpp"
#include "kernels.hpp"

namespace sa {

namespace {

constexpr int kWaves = 4;  // independent slabs per workgroup

template <int HD, bool BF, int MODE>
__global__ __launch_bounds__(64 * kWaves) void k_page_meta(MetaArgs a)
{
    constexpr int CH = BF ? 8 : 4;
    constexpr int LPT = HD / CH;
    constexpr int RPW = 64 / LPT;  // key rows per wave load
    constexpr int U = 4;
    const Geometry& g = a.g;
    const int lane = threadIdx.x & 63;
    const int sub = lane % LPT, rg = lane / LPT;

    const int range = a.page_end - a.page_begin;
    long item = (long)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const long items = (long)g.B * range * g.Hkv;
    if (item >= items) return;
    const int kvh = (int)(item % g.Hkv);
    item /= g.Hkv;
    const int page = a.page_begin + (int)(item % range);
    const int b = (int)(item / range);

    int L = g.seq_lens[b];
    L = imax(0, imin(L, g.max_pages * g.P));
    const int t0 = page * g.P;
    const int n = imin(g.P, L - t0);  // valid tokens of this page
    if (n <= 0) return;
    const int phys = g.block_table[(long)b * g.max_pages + page];
    if (phys < 0 || phys >= g.num_phys) return;

    typedef typename std::conditional<BF, uint16_t, float>::type E;
    const E* slab = (const E*)g.k + ((long)phys * g.Hkv + kvh) * (long)g.P * HD + sub * CH;
    // compressed keys: rows P .. 2P-1 are the next page's (when this page is
    // full and the next one is mapped)
    const E* slab1 = slab;
    int nt = n;  // rows summarised
    if constexpr (MODE == 3) {
        const int ph1 = page + 1 < g.max_pages ? g.block_table[(long)b * g.max_pages + page + 1] : -1;
        const int n1 = n == g.P && ph1 >= 0 && ph1 < g.num_phys ? imin(g.P, L - t0 - g.P) : 0;
        if (n1 > 0) {
            slab1 = (const E*)g.k + ((long)ph1 * g.Hkv + kvh) * (long)g.P * HD + sub * CH;
            nt = n + n1;
        }
    }

    float acc0[CH], acc1[CH];  // Quest: min / max; mean, centroid: running sum in acc0
    for (int c = 0; c < CH; ++c) {
        acc0[c] = MODE == 0 ? INFINITY : 0.f;
        acc1[c] = -INFINITY;
    }

    for (int base = 0; base < nt; base += RPW * U) {
        uint4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = base + u * RPW + rg;
            const E* row = r < g.P ? slab + (long)r * HD : slab1 + (long)(r - g.P) * HD;
            w[u] = r < nt ? ld_stream(row) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = base + u * RPW + rg;
            const bool valid = r < nt;
            float x[CH];
            const uint32_t* ww = (const uint32_t*)&w[u];
            if constexpr (BF) {
                for (int j = 0; j < 4; ++j) {
                    x[2 * j] = bf_lo(ww[j]);
                    x[2 * j + 1] = bf_hi(ww[j]);
                }
            } else {
                for (int j = 0; j < 4; ++j) x[j] = __uint_as_float(ww[j]);
            }
            if constexpr (MODE == 0) {
                if (valid)
                    for (int c = 0; c < CH; ++c) {
                        acc0[c] = fminf(acc0[c], x[c]);
                        acc1[c] = fmaxf(acc1[c], x[c]);
                    }
            } else if constexpr (MODE == 1 || MODE == 3) {
                for (int c = 0; c < CH; ++c) acc0[c] += x[c];  // invalid rows loaded as 0
            } else {
                float ss = 0.f;
                for (int c = 0; c < CH; ++c) ss = fmaf(x[c], x[c], ss);
                ss = group_sum<LPT>(ss);
                const float inv = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
                for (int c = 0; c < CH; ++c) acc0[c] = fmaf(x[c], inv, acc0[c]);
            }
        }
    }

    // fold the row groups (lanes sub, sub + LPT, ...) into lanes 0..LPT-1
    for (int off = LPT; off < 64; off <<= 1) {
        for (int c = 0; c < CH; ++c) {
            const float o0 = __shfl_xor(acc0[c], off);
            const float o1 = __shfl_xor(acc1[c], off);
            if constexpr (MODE == 0) {
                acc0[c] = fminf(acc0[c], o0);
                acc1[c] = fmaxf(acc1[c], o1);
            } else {
                acc0[c] += o0;
            }
        }
    }
    if constexpr (MODE == 1 || MODE == 3) {
        const float invn = 1.0f / (float)nt;
        for (int c = 0; c < CH; ++c) acc0[c] *= invn;
    } else if constexpr (MODE == 2) {
        float ss = 0.f;
        for (int c = 0; c < CH; ++c) ss = fmaf(acc0[c], acc0[c], ss);
        ss = group_sum<LPT>(ss);
        const float inv = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
        for (int c = 0; c < CH; ++c) acc0[c] *= inv;
    }
    if (rg != 0) return;

    const long slab_id = ((long)b * g.Hkv + kvh) * g.max_pages + page;  // by logical page
    if constexpr (MODE == 0) {
        E* out = (E*)a.meta + slab_id * 2 * HD + sub * CH;
        if constexpr (BF) {
            uint4 mn, mx;
            uint32_t* pm = (uint32_t*)&mn;
            uint32_t* px = (uint32_t*)&mx;
            for (int j = 0; j < 4; ++j) {
                // min/max of bf16 values are bf16 values: the top halves are exact
                pm[j] = (__float_as_uint(acc0[2 * j]) >> 16) | (__float_as_uint(acc0[2 * j + 1]) & 0xffff0000u);
                px[j] = (__float_as_uint(acc1[2 * j]) >> 16) | (__float_as_uint(acc1[2 * j + 1]) & 0xffff0000u);
            }
            *(uint4*)out = mn;
            *(uint4*)(out + HD) = mx;
        } else {
            *(float4*)out = make_float4(acc0[0], acc0[1], acc0[2], acc0[3]);
            *(float4*)(out + HD) = make_float4(acc1[0], acc1[1], acc1[2], acc1[3]);
        }
    } else {
        float* out = (float*)a.meta + slab_id * HD + sub * CH;
        for (int c = 0; c < CH; c += 4) *(float4*)(out + c) = make_float4(acc0[c], acc0[c + 1], acc0[c + 2], acc0[c + 3]);
    }
}

template <int HD, bool BF>
hipError_t launch_mode(const MetaArgs& a, dim3 grid, hipStream_t s)
{
    switch (a.mode) {
    case 0: hipLaunchKernelGGL((k_page_meta<HD, BF, 0>), grid, dim3(64 * kWaves), 0, s, a); break;
    case 1: hipLaunchKernelGGL((k_page_meta<HD, BF, 1>), grid, dim3(64 * kWaves), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_page_meta<HD, BF, 2>), grid, dim3(64 * kWaves), 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_page_meta<HD, BF, 3>), grid, dim3(64 * kWaves), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_page_meta(const MetaArgs& a, hipStream_t s)
{
    const long items = (long)a.g.B * (a.page_end - a.page_begin) * a.g.Hkv;
    if (items <= 0) return hipSuccess;
    const dim3 grid((unsigned)((items + kWaves - 1) / kWaves));
    const bool bf = a.g.dtype == 1;
    if (a.g.hd == 128) return bf ? launch_mode<128, true>(a, grid, s) : launch_mode<128, false>(a, grid, s);
    if (a.g.hd == 64) return bf ? launch_mode<64, true>(a, grid, s) : launch_mode<64, false>(a, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace sa
