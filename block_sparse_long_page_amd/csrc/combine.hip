// Log-sum-exp merge of split partials (attention-mechanisms article,
// DeepSeek-V4 section: partial results are combined; FlashAttention's
// running-max rescaling).  One wave per output row; the sums run over the
// splits in a fixed order, so the result does not depend on timing.  A
// partial with l = 0 is empty and its o is not read (past the first eight
// splits, whose o is fetched with the (m, l) pairs); one with
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
    __shared__ float wts[kMaxSplits];    // each split's weight e^{m_s - m*} l_s
    __shared__ short later[kMaxSplits];  // the splits past the first UNROLL with a non-zero weight, ascending
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
#pragma unroll
    for (int j = 0; j < UNROLL; ++j)
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[j][c] = j < n ? po[(long)j * HD + c] : 0.f;
    float mx = -INFINITY;
    for (int s = lane; s < n; s += 64) {
        const float2 p = *(const float2*)(ml + 2 * s);
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
            const float2 p = *(const float2*)(ml + 2 * s);
            w = p.y > 0.f ? expf(p.x - mx) * p.y : (p.y == p.y ? 0.f : p.y);
            wts[s] = w;
        }
        const uint64_t m = __builtin_amdgcn_ballot_w64(s < n && s >= UNROLL && w != 0.f);
        if (s < n && s >= UNROLL && w != 0.f) later[nlater + lanes_below(m)] = (short)s;
        nlater += __builtin_popcountll(m);
    }
    __builtin_amdgcn_wave_barrier();

    // the sums run over the splits in ascending order (the zero weights of
    // empty parts add nothing), so the result does not depend on timing
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
            for (int c = 0; c < CPL; ++c) v[j][c] = u0 + j < nlater ? po[(long)later[u0 + j] * HD + c] : 0.f;
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
