// KeyDiff eviction (course module 14, section 14.4 and exercise 14.2): a
// token's importance is how far its key lies from the mean key of the tokens
// the cache holds; the least distinctive tokens are evicted, the first `sink`
// positions never, and the cache is brought back to its budget after every
// block of new tokens, so it never holds more than budget + block tokens.
//
//  * k_kd_sum: per (sequence, KV head, chunk of kKdChunk tokens) the fp32 sum
//    of the keys (rows in order in each lane, then lanes and waves in a fixed
//    order: bitwise reproducible).
//  * k_kd_dist: every workgroup rebuilds the mean key from the chunk sums, in
//    chunk order, and writes the order key of each candidate's squared
//    distance to it, candidates in reverse position order.
//  * k_kd_topk: one workgroup per (sequence, KV head) keeps the sink and the
//    budget - sink farthest other tokens.  Among equal distances the later
//    position is kept: the candidates are ranked in reverse position order
//    and the block top-k prefers the lower index.  Kept positions ascending.
//  * k_kd_compact: copies the kept tokens' K and V rows, in order, into
//    slots 0 .. count-1 of a destination cache.
// The sum and distance passes stream the keys with 16-byte loads; each wave
// resolves the block-table entries of the pages its rows span once, up front.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "topk_block.hpp"

namespace sa {

namespace {

constexpr int kKdWaves = 4;
constexpr int kKdRowsPerWave = kKdChunk / kKdWaves;
constexpr int kKdU = 16;            // row loads per lane in flight
constexpr int kKdSlots = 64;        // destination slots per compaction workgroup
constexpr int kKdCopyThreads = 256;

__device__ __forceinline__ int kd_len(const Geometry& g, int T, int b)
{
    return imax(0, imin(imin(g.seq_lens[b], T), g.max_pages * g.P));
}

// Physical pages of the logical pages [pg0, pg0 + npg) of one sequence, one
// per lane (npg <= 64), looked up by a lane exchange; with more pages each
// row reads its own entry.  Unmapped pages give -1.
struct WavePages {
    const int32_t* bt;
    int pg0, npg, mine, num_phys;
    __device__ __forceinline__ void init(const int32_t* table, int first, int n, int nphys)
    {
        bt = table;
        pg0 = first;
        npg = n;
        num_phys = nphys;
        const int lane = threadIdx.x & 63;
        mine = n <= 64 && lane < n ? bt[first + lane] : -1;
    }
    __device__ __forceinline__ int phys(int page) const
    {
        const int p = npg <= 64 ? __shfl(mine, page - pg0) : bt[page];
        return p >= 0 && p < num_phys ? p : -1;
    }
};

template <int HD, bool BF>
struct KdLayout {
    typedef typename std::conditional<BF, uint16_t, float>::type E;
    static constexpr int CH = BF ? 8 : 4;      // elements per 16-byte load
    static constexpr int LPT = HD / CH;        // lanes per key row
    static constexpr int RPW = 64 / LPT;       // rows per wave load
    __device__ static __forceinline__ void unpack(const uint4& w, float (&x)[CH])
    {
        const uint32_t* u = (const uint32_t*)&w;
        if constexpr (BF) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] = bf_lo(u[e]);
                x[2 * e + 1] = bf_hi(u[e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(u[e]);
        }
    }
};

// Streams rows [r0, r1) of (b, kvh), kKdU loads per lane in flight, calling
// f(row, x) with this lane's CH channels of each row; rows past r1 and rows
// on unmapped pages read as zeros (a zero key).
template <int HD, bool BF, typename F>
__device__ __forceinline__ void kd_stream(const Geometry& g, const FastDiv& pdiv, int b, int kvh, int r0, int r1, F f)
{
    using Lay = KdLayout<HD, BF>;
    typedef typename Lay::E E;
    const int lane = threadIdx.x & 63;
    const int sub = lane % Lay::LPT, rg = lane / Lay::LPT;
    if (r0 >= r1) return;
    WavePages wp;
    const int pg0 = pdiv.div(r0);
    wp.init(g.block_table + (long)b * g.max_pages, pg0, pdiv.div(r1 - 1) - pg0 + 1, g.num_phys);
    for (int base = r0; base < r1; base += Lay::RPW * kKdU) {
        uint4 w[kKdU];
#pragma unroll
        for (int u = 0; u < kKdU; ++u) {
            const int t = base + u * Lay::RPW + rg;
            const int page = pdiv.div(imin(t, r1 - 1));
            const int ph = wp.phys(page);  // every lane takes part in the exchange
            w[u] = make_uint4(0, 0, 0, 0);
            if (t < r1 && ph >= 0)
                w[u] = *(const uint4*)((const E*)g.k + (((long)ph * g.Hkv + kvh) * g.P + (t - page * g.P)) * HD +
                                       sub * Lay::CH);
        }
#pragma unroll
        for (int u = 0; u < kKdU; ++u) {
            float x[Lay::CH];
            Lay::unpack(w[u], x);
            f(base + u * Lay::RPW + rg, x);
        }
    }
}

template <int HD, bool BF>
__global__ __launch_bounds__(64 * kKdWaves) void k_kd_sum(KeydiffArgs a)
{
    using Lay = KdLayout<HD, BF>;
    __shared__ float wsum[kKdWaves][HD];
    const Geometry& g = a.g;
    const FastDiv pdiv{g.pdiv.d, g.pdiv.magic, g.pdiv.shift};
    const int bh = blockIdx.y, b = bh / g.Hkv, kvh = bh % g.Hkv;
    const int L = kd_len(g, a.T, b);
    const int t0 = blockIdx.x * kKdChunk;
    if (t0 >= L) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % Lay::LPT, rg = lane / Lay::LPT;
    const int r0 = imin(L, t0 + wave * kKdRowsPerWave), r1 = imin(L, r0 + kKdRowsPerWave);

    float acc[Lay::CH];
#pragma unroll
    for (int c = 0; c < Lay::CH; ++c) acc[c] = 0.f;
    kd_stream<HD, BF>(g, pdiv, b, kvh, r0, r1, [&](int, const float (&x)[Lay::CH]) {
#pragma unroll
        for (int c = 0; c < Lay::CH; ++c) acc[c] += x[c];
    });
    // the wave's row groups, then the waves, in a fixed order
#pragma unroll
    for (int off = Lay::LPT; off < 64; off <<= 1)
#pragma unroll
        for (int c = 0; c < Lay::CH; ++c) acc[c] += __shfl_xor(acc[c], off);
    if (rg == 0)
#pragma unroll
        for (int c = 0; c < Lay::CH; ++c) wsum[wave][sub * Lay::CH + c] = acc[c];
    __syncthreads();
    for (int c = threadIdx.x; c < HD; c += 64 * kKdWaves) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kKdWaves; ++w) s += wsum[w][c];
        a.partial[((long)bh * a.nchunks + blockIdx.x) * HD + c] = s;
    }
}

template <int HD, bool BF>
__global__ __launch_bounds__(64 * kKdWaves) void k_kd_dist(KeydiffArgs a)
{
    using Lay = KdLayout<HD, BF>;
    __shared__ float mean[HD];
    const Geometry& g = a.g;
    const FastDiv pdiv{g.pdiv.d, g.pdiv.magic, g.pdiv.shift};
    const int bh = blockIdx.y, b = bh / g.Hkv, kvh = bh % g.Hkv;
    const int L = kd_len(g, a.T, b);
    const int t0 = blockIdx.x * kKdChunk;
    if (t0 >= L) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % Lay::LPT;
    const int nch = (L + kKdChunk - 1) / kKdChunk;
    for (int c = threadIdx.x; c < HD; c += 64 * kKdWaves) {
        float s = 0.f;
        for (int j = 0; j < nch; ++j) s += a.partial[((long)bh * a.nchunks + j) * HD + c];
        mean[c] = s / (float)L;
    }
    __syncthreads();
    float m[Lay::CH];
#pragma unroll
    for (int c = 0; c < Lay::CH; ++c) m[c] = mean[sub * Lay::CH + c];
    const int r0 = imin(L, t0 + wave * kKdRowsPerWave), r1 = imin(L, r0 + kKdRowsPerWave);
    // token t goes to index L-1-t (the sink's indices, past the candidates, are never read)
    uint32_t* okeys = a.okeys + (long)bh * a.Tk + (L - 1);
    kd_stream<HD, BF>(g, pdiv, b, kvh, r0, r1, [&](int t, const float (&x)[Lay::CH]) {
        float d = 0.f;
#pragma unroll
        for (int c = 0; c < Lay::CH; ++c) {
            const float e = x[c] - m[c];
            d = fmaf(e, e, d);
        }
        d = group_sum<Lay::LPT>(d);
        if (sub == 0 && t < r1) okeys[-t] = order_key(d);
    });
}

__global__ __launch_bounds__(kTopkThreads) void k_kd_topk(KeydiffArgs a)
{
    __shared__ __attribute__((aligned(16))) uint32_t keys[kKdMaxCand];
    __shared__ TopkScratch sh;
    const Geometry& g = a.g;
    const int bh = blockIdx.x, b = bh / g.Hkv;
    const int L = kd_len(g, a.T, b);
    const int tid = threadIdx.x;
    int32_t* kept = a.kept + (long)bh * a.budget;
    const int cnt = imin(L, a.budget);
    if (tid == 0) a.count[bh] = cnt;
    for (int i = cnt + tid; i < a.budget; i += kTopkThreads) kept[i] = -1;
    if (L <= a.budget) {
        for (int i = tid; i < L; i += kTopkThreads) kept[i] = i;
        return;
    }
    const int s0 = imin(a.sink, L);
    for (int i = tid; i < s0; i += kTopkThreads) kept[i] = i;
    const int k = a.budget - s0;
    const int m = imin(L - s0, kKdMaxCand);  // the host keeps max_seq_len - sink within the limit
    if (k <= 0 || k >= m) return;
    // candidate j is position L-1-j: later positions get lower indices.  Every
    // thread's 16-byte loads are in flight together (rows are 16-byte aligned
    // and padded to a multiple of 4; keys past m are not used).
    constexpr int NV = kKdMaxCand / (4 * kTopkThreads);
    static_assert(NV * 4 * kTopkThreads == kKdMaxCand, "16-byte loads tile the candidates");
    const uint32_t* src = a.okeys + (long)bh * a.Tk;
    uint4 w[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int j = 4 * (i * kTopkThreads + tid);
        w[i] = j < m ? *(const uint4*)(src + j) : make_uint4(0, 0, 0, 0);
    }
    uint32_t lo = 0xffffffffu, hi = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int j = 4 * (i * kTopkThreads + tid);
        if (j < m) {
            *(uint4*)(keys + j) = w[i];
            const uint32_t* v = (const uint32_t*)&w[i];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j + e < m) {
                    lo = min(lo, v[e]);
                    hi = max(hi, v[e]);
                }
        }
    }
    block_topk_fast(m, k, keys, lo, hi, sh, [&](int pos, int j) { kept[s0 + (k - 1 - pos)] = L - 1 - j; });
}

template <int HD, bool BF>
__global__ __launch_bounds__(kKdCopyThreads) void k_kd_compact(CompactArgs a)
{
    constexpr int PPR = HD * (BF ? 2 : 4) / 16;  // 16-byte pieces per row
    constexpr int ITER = kKdSlots * PPR / kKdCopyThreads;
    static_assert(ITER * kKdCopyThreads == kKdSlots * PPR, "pieces tile the workgroup");
    const Geometry& s = a.src;
    const Geometry& d = a.dst;
    const FastDiv sdiv{s.pdiv.d, s.pdiv.magic, s.pdiv.shift};
    const FastDiv ddiv{d.pdiv.d, d.pdiv.magic, d.pdiv.shift};
    const int bh = blockIdx.y, b = bh / s.Hkv, kvh = bh % s.Hkv;
    const int cnt = imin(a.count[bh], a.budget);
    const int j0 = blockIdx.x * kKdSlots;
    if (j0 >= cnt) return;
    const int32_t* kept = a.kept + (long)bh * a.budget;
    const int span = s.max_pages * s.P;
    uint4 kv[ITER][2];
    long dst_off[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int e = it * kKdCopyThreads + threadIdx.x;
        const int j = j0 + e / PPR, piece = e % PPR;
        dst_off[it] = -1;
        kv[it][0] = kv[it][1] = make_uint4(0, 0, 0, 0);
        if (j >= cnt) continue;
        const int p = kept[j];
        if (p < 0 || p >= span) continue;
        const int sp = sdiv.div(p);
        const int sph = s.block_table[(long)b * s.max_pages + sp];
        const int dp = ddiv.div(j);
        const int dph = d.block_table[(long)b * d.max_pages + dp];
        if (sph < 0 || sph >= s.num_phys || dph < 0 || dph >= d.num_phys) continue;
        const long so = (((long)sph * s.Hkv + kvh) * s.P + (p - sp * s.P)) * PPR + piece;
        kv[it][0] = ((const uint4*)s.k)[so];
        kv[it][1] = ((const uint4*)s.v)[so];
        dst_off[it] = (((long)dph * d.Hkv + kvh) * d.P + (j - dp * d.P)) * PPR + piece;
    }
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        if (dst_off[it] < 0) continue;
        ((uint4*)d.k)[dst_off[it]] = kv[it][0];
        ((uint4*)d.v)[dst_off[it]] = kv[it][1];
    }
}

template <int HD, bool BF>
hipError_t launch_kd(const KeydiffArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)a.nchunks, (unsigned)(a.g.B * a.g.Hkv));
    hipLaunchKernelGGL((k_kd_sum<HD, BF>), grid, dim3(64 * kKdWaves), 0, s, a);
    hipLaunchKernelGGL((k_kd_dist<HD, BF>), grid, dim3(64 * kKdWaves), 0, s, a);
    hipLaunchKernelGGL(k_kd_topk, dim3((unsigned)(a.g.B * a.g.Hkv)), dim3(kTopkThreads), 0, s, a);
    return hipGetLastError();
}

template <int HD, bool BF>
hipError_t launch_compact(const CompactArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)((a.budget + kKdSlots - 1) / kKdSlots), (unsigned)(a.src.B * a.src.Hkv));
    hipLaunchKernelGGL((k_kd_compact<HD, BF>), grid, dim3(kKdCopyThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_keydiff_select(const KeydiffArgs& a, hipStream_t s)
{
    const bool bf = a.g.dtype == 1;
    if (a.g.hd == 128) return bf ? launch_kd<128, true>(a, s) : launch_kd<128, false>(a, s);
    if (a.g.hd == 64) return bf ? launch_kd<64, true>(a, s) : launch_kd<64, false>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_keydiff_compact(const CompactArgs& a, hipStream_t s)
{
    const bool bf = a.src.dtype == 1;
    if (a.src.hd == 128) return bf ? launch_compact<128, true>(a, s) : launch_compact<128, false>(a, s);
    if (a.src.hd == 64) return bf ? launch_compact<64, true>(a, s) : launch_compact<64, false>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace sa
