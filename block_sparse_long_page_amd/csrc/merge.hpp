// Log-sum-exp merge of one output row's split partials by one wave
// (attention-mechanisms article, DeepSeek-V4 section: partial results are
// combined; FlashAttention's running-max rescaling), shared by the combine
// kernel and by the decode kernels that merge in their last workgroup, so
// both give the same bits.  The sums run over the splits in a fixed order,
// so the result does not depend on timing.  A partial with l = 0 is empty
// and its o is not read (past the first eight splits, whose o is fetched
// with the (m, l) pairs); one with l = NaN marks a share that was not
// computed and makes the row's output and lse NaN.
#pragma once

#include "device_common.hpp"

namespace sa {

// COHERENT: the partials were written by other workgroups of the running
// kernel with agent-scope stores; read them with agent-scope loads (coherent
// across the XCDs' L2 caches without a cache invalidation).
template <bool COHERENT>
__device__ __forceinline__ float merge_ld(const float* p)
{
    if constexpr (COHERENT)
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        return *p;
}

template <bool COHERENT>
__device__ __forceinline__ float2 merge_ld2(const float* p)
{
    if constexpr (COHERENT)
        return make_float2(merge_ld<true>(p), merge_ld<true>(p + 1));
    else
        return *(const float2*)p;
}

// ml: the row's n (m, l) pairs; po: its n partial outputs of HD floats; wts
// and later: LDS of at least n entries for this wave; out_bf: bf16 output
// (else fp32) at out + row * HD; lse (nullable) at lse[row].
template <int HD, bool COHERENT>
__device__ __forceinline__ void merge_row(const float* ml, const float* po_row, int n, float* wts, short* later,
                                          bool out_bf, void* out, float* lse, long row)
{
    constexpr int CPL = HD / 64;  // channels per lane
    constexpr int UNROLL = 8;     // split loads in flight
    const int lane = threadIdx.x & 63;
    const float* po = po_row + lane * CPL;

    // the partials of the first splits go out together with the (m, l) pairs
    float v[UNROLL][CPL];
#pragma unroll
    for (int j = 0; j < UNROLL; ++j)
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[j][c] = j < n ? merge_ld<COHERENT>(po + (long)j * HD + c) : 0.f;
    float mx = -INFINITY;
    float2 first = make_float2(0.f, 0.f);  // this lane's pair among the first 64 splits, kept for the weights
    for (int s = lane; s < n; s += 64) {
        const float2 p = merge_ld2<COHERENT>(ml + 2 * s);
        if (s == lane) first = p;
        if (p.y > 0.f) mx = fmaxf(mx, p.x);
    }
    mx = group_max<64>(mx);

    // every split's weight (0 for an empty part; l = NaN marks a share that
    // was not computed and poisons the row), and the later splits that carry
    // one: only their partials are read
    int nlater = 0;
    for (int s0 = 0; s0 < n; s0 += 64) {
        const int s = s0 + lane;
        float w = 0.f;
        if (s < n) {
            const float2 p = s0 == 0 ? first : merge_ld2<COHERENT>(ml + 2 * s);
            w = p.y > 0.f ? expf(p.x - mx) * p.y : (p.y == p.y ? 0.f : p.y);
            wts[s] = w;
        }
        const uint64_t m = __builtin_amdgcn_ballot_w64(s < n && s >= UNROLL && w != 0.f);
        if (s < n && s >= UNROLL && w != 0.f) later[nlater + lanes_below(m)] = (short)s;
        nlater += __builtin_popcountll(m);
    }
    __builtin_amdgcn_wave_barrier();

    // the sums run over the splits in ascending order (the zero weights of
    // empty parts add nothing)
    float tot = 0.f, acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
        if (j >= n) break;
        const float wj = wts[j];
        tot += wj;
        if (wj > 0.f)  // an empty partial (l = 0) contributes nothing, whatever its o holds
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[c] = fmaf(wj, v[j][c], acc[c]);
    }
    for (int u0 = 0; u0 < nlater; u0 += UNROLL) {
#pragma unroll
        for (int j = 0; j < UNROLL; ++j)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                v[j][c] = u0 + j < nlater ? merge_ld<COHERENT>(po + (long)later[u0 + j] * HD + c) : 0.f;
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) {
            if (u0 + j >= nlater) break;
            const float wj = wts[later[u0 + j]];
            tot += wj;
            if (wj > 0.f)
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[c] = fmaf(wj, v[j][c], acc[c]);
        }
    }
    const float inv = tot > 0.f ? 1.0f / tot : (tot == tot ? 0.f : tot);  // NaN stays NaN
    if (out_bf) {
        if constexpr (CPL == 1) {
            uint16_t* o = (uint16_t*)out + row * HD + lane;
            *o = (uint16_t)(pack_bf16(acc[0] * inv, 0.f) & 0xffffu);
        } else {
            uint32_t* o = (uint32_t*)out + (row * HD + lane * CPL) / 2;
#pragma unroll
            for (int c = 0; c < CPL; c += 2) o[c / 2] = pack_bf16(acc[c] * inv, acc[c + 1] * inv);
        }
    } else {
        float* o = (float*)out + row * HD + lane * CPL;
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[c] = acc[c] * inv;
    }
    if (lse && lane == 0) lse[row] = tot > 0.f ? mx + logf(tot) : (tot == tot ? -INFINITY : tot);
}

}  // namespace sa
