// Log-sum-exp merge of split partials (attention-mechanisms article,
// DeepSeek-V4 section: partial results are combined; FlashAttention's
// running-max rescaling).  One wave per output row; the sums run over the
// splits in a fixed order, so the result does not depend on timing.  A
// partial with l = 0 is empty and its o is not read into the sum; one with
// l = NaN marks a share that was not computed and makes the row's output and
// lse NaN.
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
    const int row = blockIdx.x;
    const int lane = threadIdx.x;
    const int n = a.splits;
    // the step's last kernel appends the next token(s): no kernel of this
    // launch reads the lengths, and the next step's run after it
    if (a.seq_lens && row == 0)
        for (int b = lane; b < a.batch; b += 64) a.seq_lens[b] += a.advance;
    const float* ml = a.part_ml + (long)row * n * 2;
    const float* po = a.part_o + (long)row * n * HD + lane * CPL;

    // the partials of the first splits go out together with the (m, l) pairs
    float v[UNROLL][CPL];
    auto fetch = [&](int s0) {
#pragma unroll
        for (int j = 0; j < UNROLL; ++j)
#pragma unroll
            for (int c = 0; c < CPL; ++c) v[j][c] = s0 + j < n ? po[(long)(s0 + j) * HD + c] : 0.f;
    };
    fetch(0);
    float mx = -INFINITY;
    for (int s = lane; s < n; s += 64) {
        const float2 p = *(const float2*)(ml + 2 * s);
        if (p.y > 0.f) mx = fmaxf(mx, p.x);
    }
    mx = group_max<64>(mx);

    // split s's weight e^{m_s - m*} l_s sits in lane s % 64 of its block of 64
    // splits and is read out uniformly, so the sums run over s in one order
    float tot = 0.f, acc[CPL], w = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
    for (int s0 = 0; s0 < n; s0 += UNROLL) {
        if ((s0 & 63) == 0) {
            const int s = s0 + lane;
            w = 0.f;
            if (s < n) {
                const float2 p = *(const float2*)(ml + 2 * s);
                // l = NaN marks a share that was not computed: it poisons the row
                w = p.y > 0.f ? expf(p.x - mx) * p.y : (p.y == p.y ? 0.f : p.y);
            }
        }
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) {
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), (s0 & 63) + j));
            tot += wj;
            if (wj > 0.f)  // an empty partial (l = 0) contributes nothing, whatever its o holds
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[c] = fmaf(wj, v[j][c], acc[c]);
        }
        if (s0 + UNROLL < n) fetch(s0 + UNROLL);
    }
    const float inv = tot > 0.f ? 1.0f / tot : (tot == tot ? 0.f : tot);  // NaN stays NaN
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
    if (a.lse && lane == 0) a.lse[row] = tot > 0.f ? mx + logf(tot) : (tot == tot ? -INFINITY : tot);
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
