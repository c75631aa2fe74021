// Load-only reference kernels for the benchmark (not part of the attention
// path; built into libsa_probe.so).  They move bytes and do nothing else, so
// their rate is what the memory system gives an access pattern:
//
//  * k_probe_pages reads exactly the K and V bytes a decode step attends:
//    for every (sequence, KV head) the list of page slabs it attends (a slab
//    is one KV head's rows of one physical page, page_size * head_dim
//    elements), in 16-token tiles of K and V, with the decode's launch
//    shape: `splits` workgroups of 8 waves per (sequence, KV head), each
//    taking a contiguous share of the problem's tiles, tile w of every
//    round of 8 by wave w, three tiles in flight per wave;
//  * k_probe_stream reads one contiguous buffer, 16 bytes per lane, eight
//    loads in flight per lane.
// Both use non-temporal loads, as the attention kernels do for K and V.
//
// Every loaded word is folded into a register that is compared with a
// constant at the end, so no load can be dropped and nothing is written
// (unless the fold happens to equal the constant).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kWaves = 8;
constexpr uint32_t kNever = 0x9e3779b9u;

__device__ __forceinline__ uint32_t fold(uint4 x) { return x.x ^ x.y ^ x.z ^ x.w; }

// non-temporal 16-byte loads, as the attention kernels stream K and V
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const uint4* p)
{
    const u32x4_t w = __builtin_nontemporal_load((const u32x4_t*)p);
    return make_uint4(w.x, w.y, w.z, w.w);
}

// TILE_U4: 16-byte pieces of one 16-token tile of K (or V) per lane
template <int TILE_U4>
__global__ __launch_bounds__(64 * kWaves) void k_probe_pages(const uint4* k, const uint4* v, const int32_t* slabs,
                                                             const int32_t* offsets, int splits, int tiles_per_slab,
                                                             long slab_u4, uint32_t* out)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int prob = blockIdx.x / splits, split = blockIdx.x % splits;
    const int s0 = offsets[prob], ns = offsets[prob + 1] - s0;
    const int n = ns * tiles_per_slab;  // tiles of the problem
    const int t0 = split * (n / splits) + min(split, n % splits);
    const int t1 = t0 + n / splits + (split < n % splits ? 1 : 0);
    if (t0 >= t1) return;  // an empty share (no barriers below)
    uint32_t acc = 0;
    uint4 a[2][TILE_U4], b[2][TILE_U4], c[2][TILE_U4];
    auto load = [&](uint4 (&buf)[2][TILE_U4], int t) {
        const bool ok = t < t1;
        const int tt = ok ? t : t0;  // past the share: re-read the first tile, folded out below
        const int slab = slabs[s0 + tt / tiles_per_slab];
        const long base = (long)slab * slab_u4 + (long)(tt % tiles_per_slab) * (TILE_U4 * 64);
#pragma unroll
        for (int i = 0; i < TILE_U4; ++i) {
            buf[0][i] = ld_nt(k + base + i * 64 + lane);
            buf[1][i] = ld_nt(v + base + i * 64 + lane);
        }
    };
    auto use = [&](const uint4 (&buf)[2][TILE_U4], int t) {
        uint32_t f = 0;
#pragma unroll
        for (int i = 0; i < TILE_U4; ++i) f ^= fold(buf[0][i]) ^ fold(buf[1][i]);
        acc ^= t < t1 ? f : 0u;
    };
    int t = t0 + wave;
    load(a, t);
    load(b, t + kWaves);
    load(c, t + 2 * kWaves);
    for (; t < t1; t += 3 * kWaves) {
        use(a, t);
        load(a, t + 3 * kWaves);
        use(b, t + kWaves);
        load(b, t + 4 * kWaves);
        use(c, t + 2 * kWaves);
        load(c, t + 5 * kWaves);
    }
    if (acc == kNever) out[blockIdx.x] = acc;
}

constexpr int kStreamUnroll = 8;

__global__ __launch_bounds__(256) void k_probe_stream(const uint4* src, long n_u4, uint32_t* out)
{
    const long stride = (long)gridDim.x * 256;
    uint32_t acc = 0;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n_u4; i += stride * kStreamUnroll) {
        uint4 x[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) x[u] = i + u * stride < n_u4 ? ld_nt(src + i + u * stride) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) acc ^= fold(x[u]);
    }
    if (acc == kNever) out[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads the attended page slabs of `problems` (sequence, KV head) pairs:
// slabs[offsets[p] .. offsets[p+1]) are slab indices into k and v (slab s
// starts at element s * page_size * head_dim), bf16 or fp32 elements of
// elem_bytes.  head_dim * elem_bytes must be 256 (one 16-token tile =
// 4 KiB per operand = 4 pieces of 16 bytes per lane) and page_size a
// multiple of 16.  out: at least problems * splits words (normally never
// written).  Returns 0, or 1 for unsupported sizes, 2 for a launch error.
int sa_probe_pages(const void* k, const void* v, const int32_t* slabs, const int32_t* offsets, int problems,
                   int splits, int page_size, int head_dim, int elem_bytes, uint32_t* out, hipStream_t stream)
{
    if (!k || !v || !slabs || !offsets || !out || problems < 1 || splits < 1) return 1;
    if (head_dim * elem_bytes != 256 || page_size < 16 || page_size % 16 != 0) return 1;
    if ((long)problems * splits * 64 * kWaves > 0xffffffffl) return 1;
    const long slab_u4 = (long)page_size * head_dim * elem_bytes / 16;
    hipLaunchKernelGGL((k_probe_pages<4>), dim3((unsigned)(problems * splits)), dim3(64 * kWaves), 0, stream,
                       (const uint4*)k, (const uint4*)v, slabs, offsets, splits, page_size / 16, slab_u4, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Reads `bytes` (a multiple of 16) from src with `workgroups` workgroups of
// 256 lanes; out: at least `workgroups` words.
int sa_probe_stream(const void* src, size_t bytes, int workgroups, uint32_t* out, hipStream_t stream)
{
    if (!src || !out || bytes % 16 != 0 || workgroups < 1 || (long)workgroups * 256 > 0xffffffffl) return 1;
    hipLaunchKernelGGL(k_probe_stream, dim3((unsigned)workgroups), dim3(256), 0, stream, (const uint4*)src,
                       (long)(bytes / 16), out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
