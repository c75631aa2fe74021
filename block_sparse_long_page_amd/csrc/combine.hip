// Log-sum-exp merge of split partials, one wave per output row (the merge
// itself, shared with the decode kernels that merge in their last
// workgroup, is merge_row in merge.hpp).
#include "device_common.hpp"
#include "kernels.hpp"
#include "merge.hpp"

namespace sa {

namespace {

constexpr int kMaxSplits = 1024;

template <int HD, bool OUT_BF>
__global__ __launch_bounds__(64) void k_combine(CombineArgs a)
{
    __shared__ float wts[kMaxSplits];    // each split's weight e^{m_s - m*} l_s
    __shared__ short later[kMaxSplits];  // the splits past the first eight with a non-zero weight, ascending
    const int row = blockIdx.x;
    const int lane = threadIdx.x;
    // the step's last kernel appends the next token(s): no kernel of this
    // launch reads the lengths, and the next step's run after it
    if (a.seq_lens && row == 0)
        for (int b = lane; b < a.batch; b += 64) a.seq_lens[b] += a.advance;
    merge_row<HD, false>(a.part_ml + (long)row * a.splits * 2, a.part_o + (long)row * a.splits * HD, a.splits, wts,
                         later, OUT_BF, a.out, a.lse, row);
}

__global__ __launch_bounds__(256) void k_zero_u32(uint32_t* p, long n)
{
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) p[i] = 0u;
}

}  // namespace

hipError_t launch_zero_u32(uint32_t* p, long n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    const long wgs = (n + 255) / 256;
    hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)(wgs < 1024 ? wgs : 1024)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

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
