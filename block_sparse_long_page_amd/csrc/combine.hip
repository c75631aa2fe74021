// Log-sum-exp merge of split partials (attention-mechanisms article,
// DeepSeek-V4 section: partial results are combined; FlashAttention's
// running-max rescaling).  One wave per output row; the split weights
// e^{m_s - m*} l_s go through LDS, the sums run over s in a fixed order.
#include "device_common.hpp"
#include "kernels.hpp"

namespace sa {

namespace {

constexpr int kMaxSplits = 1024;

template <int HD, bool OUT_BF>
__global__ __launch_bounds__(64) void k_combine(CombineArgs a)
{
    constexpr int CPL = HD / 64;  // channels per lane
    constexpr int UNROLL = 8;     // split loads in flight
    __shared__ float wts[kMaxSplits];
    const int row = blockIdx.x;
    const int lane = threadIdx.x;
    const float* ml = a.part_ml + (long)row * a.splits * 2;

    float mx = -INFINITY;
    for (int s = lane; s < a.splits; s += 64) {
        const float2 v = *(const float2*)(ml + 2 * s);
        if (v.y > 0.f) mx = fmaxf(mx, v.x);
    }
    mx = group_max<64>(mx);
    for (int s = lane; s < a.splits; s += 64) {
        const float2 v = *(const float2*)(ml + 2 * s);
        wts[s] = v.y > 0.f ? expf(v.x - mx) * v.y : 0.f;
    }
    __syncthreads();

    float tot = 0.f, acc[CPL];
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
    const float* po = a.part_o + (long)row * a.splits * HD + lane * CPL;
    for (int s0 = 0; s0 < a.splits; s0 += UNROLL) {
        float v[UNROLL][CPL];
#pragma unroll
        for (int j = 0; j < UNROLL; ++j)
#pragma unroll
            for (int c = 0; c < CPL; ++c) v[j][c] = s0 + j < a.splits ? po[(long)(s0 + j) * HD + c] : 0.f;
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) {
            const float w = s0 + j < a.splits ? wts[s0 + j] : 0.f;
            tot += w;  // the same order in every lane
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[c] = fmaf(w, v[j][c], acc[c]);
        }
    }
    const float inv = tot > 0.f ? 1.0f / tot : 0.f;
    if constexpr (OUT_BF && CPL == 1) {
        uint16_t* out = (uint16_t*)a.out + (long)row * HD + lane;
        *out = (uint16_t)(pack_bf16(acc[0] * inv, 0.f) & 0xffffu);
    } else if constexpr (OUT_BF) {
        uint32_t* out = (uint32_t*)a.out + ((long)row * HD + lane * CPL) / 2;
        for (int c = 0; c < CPL; c += 2) out[c / 2] = pack_bf16(acc[c] * inv, acc[c + 1] * inv);
    } else {
        float* out = (float*)a.out + (long)row * HD + lane * CPL;
        for (int c = 0; c < CPL; ++c) out[c] = acc[c] * inv;
    }
    if (a.lse && lane == 0) a.lse[row] = tot > 0.f ? mx + logf(tot) : -INFINITY;
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s)
{
    if (a.splits < 1 || a.splits > kMaxSplits) return hipErrorInvalidValue;
    const dim3 grid((unsigned)a.rows), block(64);
    const bool bf = a.out_dtype == 1;
    if (a.hd == 128) {
        if (bf) hipLaunchKernelGGL((k_combine<128, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_combine<128, false>), grid, block, 0, s, a);
    } else if (a.hd == 64) {
        if (bf) hipLaunchKernelGGL((k_combine<64, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_combine<64, false>), grid, block, 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sa
