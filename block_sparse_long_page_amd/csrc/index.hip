// Semantic block index (semantic-blocks page: per request, layer and KV head
// the normalised keys are grouped into semantic blocks by spherical k-means,
// keys and values are laid out again block by block, and a query compares
// itself with the block centres and takes the best blocks up to a token
// budget of L/16).
//
// The build, per (sequence, KV head) over positions [0, N), C blocks:
//   k_idx_norms    1 / |k_t| of every key (0 for a zero key)
//   k_idx_init     centre c = the unit key at position floor(c N / C)
//   then `iters` times, and once more at the end without the update:
//     k_idx_assign   each key's nearest centre (largest dot product, ties to
//                    the lower centre) on the matrix cores:
//                    v_mfma_f32_16x16x32_bf16 with 16 centres (bf16, staged
//                    in LDS) as A and 16 keys as B; the running best stays
//                    in the lane that holds the product
//     k_idx_hist     block counts of each 1024-token chunk
//     k_idx_scan     block offsets, each chunk's first row in every block,
//                    and the centre-update segments (128 rows of a block)
//     k_idx_scatter  stable counting-sort scatter: the position of every row
//                    of the block layout (blocks in order, positions
//                    ascending inside a block)
//     k_idx_seg      sum of the unit keys of one segment, rows in order
//     k_idx_centre   sum of a block's segments in order, normalised (a block
//                    without keys keeps its centre)
//   k_idx_gather   keys and values copied row by row into the block layout.
// Every sum runs in a fixed order, so the build is bitwise reproducible.
//
// k_select_blocks: one workgroup per (sequence, KV head, row): the largest
// q_h . centre_c over the group's heads for every block (a thread per block,
// channels in order), a bitonic sort by
// (score desc, block asc), the running token count in that order, and the
// blocks taken while it stays within the budget (at least one), emitted
// ascending.
#include "device_common.hpp"
#include "kernels.hpp"
#include "topk_block.hpp"

namespace sa {

namespace {

typedef __bf16 ibf16x8_t __attribute__((ext_vector_type(8)));
typedef float if32x4_t __attribute__((ext_vector_type(4)));

// row of token t of (b, kvh) in the paged cache, -1 when its page is unmapped
__device__ __forceinline__ long key_row(const Geometry& g, const FastDiv& pdiv, int b, int kvh, int t)
{
    const int p = pdiv.div(t);
    const int phys = g.block_table[(long)b * g.max_pages + p];
    if (phys < 0 || phys >= g.num_phys) return -1;
    return ((long)phys * g.Hkv + kvh) * g.P + (t - p * g.P);
}

// 8 bf16 -> 8 floats
__device__ __forceinline__ void unpack8(const uint4 w, float* x)
{
    x[0] = bf_lo(w.x), x[1] = bf_hi(w.x), x[2] = bf_lo(w.y), x[3] = bf_hi(w.y);
    x[4] = bf_lo(w.z), x[5] = bf_hi(w.z), x[6] = bf_lo(w.w), x[7] = bf_hi(w.w);
}

// ---- build ---------------------------------------------------------------

template <int HD>
__global__ __launch_bounds__(256) void k_idx_norms(IndexArgs a)
{
    constexpr int LPT = HD / 8;         // lanes per key (16 bytes each)
    constexpr int TPB = 256 / LPT;      // keys per workgroup and round
    constexpr int RK = kIndexRowsPerThread;
    const Geometry& g = a.g;
    const FastDiv pdiv{g.pdiv.d, g.pdiv.magic, g.pdiv.shift};
    const int bk = blockIdx.y, b = bk / g.Hkv, kvh = bk - b * g.Hkv;
    const int part = threadIdx.x % LPT;
    const int32_t* btr = g.block_table + (long)b * g.max_pages;
    // RK keys per lane group: their table entries, then their row loads, all
    // in flight together
    int t[RK], ph[RK];
#pragma unroll
    for (int u = 0; u < RK; ++u) {
        t[u] = (blockIdx.x * RK + u) * TPB + (int)threadIdx.x / LPT;
        ph[u] = t[u] < a.N ? btr[pdiv.div(t[u])] : -1;
    }
    uint4 w[RK];
#pragma unroll
    for (int u = 0; u < RK; ++u) {
        w[u] = make_uint4(0, 0, 0, 0);
        if (ph[u] >= 0 && ph[u] < g.num_phys) {  // as key_row: an unmapped page reads as a zero key
            const long row = ((long)ph[u] * g.Hkv + kvh) * g.P + (t[u] - pdiv.div(t[u]) * g.P);
            w[u] = *(const uint4*)((const uint16_t*)g.k + row * HD + 8 * part);
        }
    }
#pragma unroll
    for (int u = 0; u < RK; ++u) {
        float x[8];
        unpack8(w[u], x);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(x[e], x[e], s);
        s = group_sum<LPT>(s);
        if (t[u] < a.N && part == 0) a.inv_norm[(long)bk * a.N + t[u]] = s > 0.f ? 1.0f / sqrtf(s) : 0.f;
    }
}

template <int HD>
__global__ __launch_bounds__(256) void k_idx_init(IndexArgs a)
{
    constexpr int LPT = HD / 8;
    constexpr int CPB = 256 / LPT;  // centres per workgroup
    const Geometry& g = a.g;
    const FastDiv pdiv{g.pdiv.d, g.pdiv.magic, g.pdiv.shift};
    const int bk = blockIdx.y, b = bk / g.Hkv, kvh = bk - b * g.Hkv;
    const int c = blockIdx.x * CPB + (int)threadIdx.x / LPT, part = threadIdx.x % LPT;
    if (c >= a.C) return;
    const int t = (int)(((long)c * a.N) / a.C);
    const long row = key_row(g, pdiv, b, kvh, t);
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (row >= 0) unpack8(*(const uint4*)((const uint16_t*)g.k + row * HD + 8 * part), x);
    const float inv = a.inv_norm[(long)bk * a.N + t];
    float* cf = a.centres + ((long)bk * a.C + c) * HD + 8 * part;
#pragma unroll
    for (int e = 0; e < 8; ++e) cf[e] = x[e] * inv;
    *(uint4*)(a.cent_bf + ((long)bk * a.C + c) * HD + 8 * part) =
        make_uint4(pack_bf16(x[0] * inv, x[1] * inv), pack_bf16(x[2] * inv, x[3] * inv),
                   pack_bf16(x[4] * inv, x[5] * inv), pack_bf16(x[6] * inv, x[7] * inv));
}

// 256 keys per workgroup (4 waves x 4 tiles of 16); the centres go through
// LDS 128 at a time.  Lane (r, j) of a product holds key r of the tile and
// centres 4j .. 4j+3 of the 16-centre block.
template <int HD>
__global__ __launch_bounds__(256) void k_idx_assign(IndexArgs a)
{
    constexpr int KK = HD / 32;  // products per 16 x 16 block (32 channels each)
    constexpr int TT = 4;        // key tiles per wave
    constexpr int CH = 128;      // centres per LDS round (32 KiB at hd 128: four workgroups per CU)
    __shared__ __attribute__((aligned(16))) uint16_t cl[CH * HD];
    const Geometry& g = a.g;
    const FastDiv pdiv{g.pdiv.d, g.pdiv.magic, g.pdiv.shift};
    const int bk = blockIdx.y, b = bk / g.Hkv, kvh = bk - b * g.Hkv;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, r = lane & 15, j = lane >> 4;
    const int tbase = blockIdx.x * (64 * TT) + wave * 16 * TT;

    // the key rows of the wave's tiles: the block-table entries of all
    // tiles first, then every key load (a table load between two key loads
    // would make each wait for the ones before it)
    const int32_t* btr = g.block_table + (long)b * g.max_pages;
    int ph[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int t = tbase + 16 * tt + r;
        ph[tt] = t < a.N ? btr[pdiv.div(t)] : -1;
    }
    long rows[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {  // as key_row: -1 past the keys or on an unmapped page
        const int t = tbase + 16 * tt + r, p = pdiv.div(t);
        rows[tt] = ph[tt] >= 0 && ph[tt] < g.num_phys ? ((long)ph[tt] * g.Hkv + kvh) * g.P + (t - p * g.P) : -1;
    }
    ibf16x8_t kb[TT][KK];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            uint4 w = make_uint4(0, 0, 0, 0);
            if (rows[tt] >= 0) w = *(const uint4*)((const uint16_t*)g.k + rows[tt] * HD + 32 * kk + 8 * j);
            kb[tt][kk] = __builtin_bit_cast(ibf16x8_t, w);
        }
    float best[TT];
    int bidx[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        best[tt] = -INFINITY;
        bidx[tt] = 0;
    }
    const uint16_t* cb = a.cent_bf + (long)bk * a.C * HD;
    for (int c0 = 0; c0 < a.C; c0 += CH) {
        const int nc = imin(CH, a.C - c0);
        {
            // the round's centres into LDS: every thread's loads in flight
            // together (the first round's with the key loads), then stored
            // once the previous round's centres are no longer read
            constexpr int PER = CH * HD / 8 / 256;
            static_assert(PER * 256 == CH * HD / 8, "16-byte pieces tile the workgroup");
            uint4 w[PER];
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const int e = u * 256 + (int)threadIdx.x;
                w[u] = e < nc * HD / 8 ? ((const uint4*)(cb + (long)c0 * HD))[e] : make_uint4(0, 0, 0, 0);
            }
            __syncthreads();
#pragma unroll
            for (int u = 0; u < PER; ++u)  // rows past nc hold zeros and are not read
                ((uint4*)cl)[u * 256 + (int)threadIdx.x] = w[u];
        }
        __syncthreads();
        for (int blk = 0; blk * 16 < nc; ++blk) {
            const int cr = 16 * blk + r;  // this lane's centre row of the A operand
            ibf16x8_t ca[KK];
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                uint4 w = make_uint4(0, 0, 0, 0);
                if (cr < nc) w = *(const uint4*)(cl + cr * HD + 32 * kk + 8 * j);
                ca[kk] = __builtin_bit_cast(ibf16x8_t, w);
            }
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                if32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca[kk], kb[tt][kk], s, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = c0 + 16 * blk + 4 * j + i;  // centres ascending in this lane
                    if (16 * blk + 4 * j + i < nc && s[i] > best[tt]) {
                        best[tt] = s[i];
                        bidx[tt] = c;
                    }
                }
            }
        }
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        float bv = best[tt];
        int bi = bidx[tt];
#pragma unroll
        for (int m = 16; m <= 32; m *= 2) {  // the four lanes of key r: larger score, then lower centre
            const float ov = __shfl_xor(bv, m);
            const int oi = __shfl_xor(bi, m);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        const int t = tbase + 16 * tt + r;
        if (j == 0 && t < a.N) a.assign[(long)bk * a.N + t] = bi;
    }
}

__global__ __launch_bounds__(256) void k_idx_hist(IndexArgs a)
{
    extern __shared__ int h[];  // [C]
    const int bk = blockIdx.y, chunk = blockIdx.x;
    for (int c = threadIdx.x; c < a.C; c += 256) h[c] = 0;
    __syncthreads();
    const int32_t* as = a.assign + (long)bk * a.N;
    for (int i = threadIdx.x; i < kIndexChunk; i += 256) {
        const int t = chunk * kIndexChunk + i;
        if (t < a.N) atomicAdd(&h[as[t]], 1);
    }
    __syncthreads();
    int32_t* cnt = a.cnt + (long)bk * a.C * a.nchunks + chunk;  // [C][nchunks]
    for (int c = threadIdx.x; c < a.C; c += 256) cnt[(long)c * a.nchunks] = h[c];
}

// One workgroup per (sequence, KV head).  The counts are block-major
// ([C][nchunks]): a wave reduces a block's chunk counts, the workgroup scans
// the block totals (thread i owns blocks 4i .. 4i+3), then a wave turns a
// block's chunk counts into each chunk's first row in the block.
__global__ __launch_bounds__(1024) void k_idx_scan(IndexArgs a)
{
    constexpr int PER = kIndexMaxBlocks / 1024;
    __shared__ int wsum[16];
    __shared__ int tot_l[kIndexMaxBlocks], off_l[kIndexMaxBlocks];
    const int bk = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t* cnt = a.cnt + (long)bk * a.C * a.nchunks;
    constexpr int NL = 8;  // a lane's counts of one block loaded together
    for (int c = wave; c < a.C; c += 16) {
        int s = 0;
        for (int k0 = lane; k0 < a.nchunks; k0 += 64 * NL) {
            int v[NL];
#pragma unroll
            for (int u = 0; u < NL; ++u) v[u] = k0 + 64 * u < a.nchunks ? cnt[(long)c * a.nchunks + k0 + 64 * u] : 0;
#pragma unroll
            for (int u = 0; u < NL; ++u) s += v[u];
        }
        s = __builtin_amdgcn_readlane(wave_inclusive_scan(s), 63);
        if (lane == 0) tot_l[c] = s;
    }
    __syncthreads();
    int tot[PER], nseg[PER];
    int mine = 0, segs = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int c = PER * (int)threadIdx.x + u;
        tot[u] = c < a.C ? tot_l[c] : 0;
        nseg[u] = (tot[u] + kIndexSegment - 1) / kIndexSegment;
        mine += tot[u];
        segs += nseg[u];
    }
    int total, seg_total;
    int off = block_exclusive_scan<1024>(mine, wsum, total);
    int soff = block_exclusive_scan<1024>(segs, wsum, seg_total);
    int32_t* offsets = a.offsets + (long)bk * (a.C + 1);
    int32_t* sb = a.seg_base + (long)bk * (a.C + 1);
    int32_t* sblk = a.seg_block + (long)bk * a.nseg;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int c = PER * (int)threadIdx.x + u;
        if (c < a.C) {
            offsets[c] = off;
            off_l[c] = off;
            sb[c] = soff;
            for (int m = 0; m < nseg[u]; ++m) sblk[soff + m] = c;
        }
        off += tot[u];
        soff += nseg[u];
    }
    if (threadIdx.x == 0) {
        offsets[a.C] = total;
        sb[a.C] = seg_total;
    }
    __syncthreads();
    // each chunk's first row in block c: off[c] + the counts of the earlier chunks
    for (int c = wave; c < a.C; c += 16) {
        int carry = off_l[c];
        for (int k1 = 0; k1 < a.nchunks; k1 += 64 * NL) {
            int v[NL];
#pragma unroll
            for (int u = 0; u < NL; ++u) {
                const int k = k1 + 64 * u + lane;
                v[u] = k < a.nchunks ? cnt[(long)c * a.nchunks + k] : 0;
            }
#pragma unroll
            for (int u = 0; u < NL; ++u) {
                const int k = k1 + 64 * u + lane;
                const int inc = wave_inclusive_scan(v[u]);
                if (k < a.nchunks) cnt[(long)c * a.nchunks + k] = carry + inc - v[u];
                carry += __builtin_amdgcn_readlane(inc, 63);
            }
        }
    }
}

// One wave per chunk: 64 tokens at a time in position order (the chunk's
// assignments all loaded first); a token's row is its block's next free row
// plus the number of earlier lanes with the same block.
__global__ __launch_bounds__(64) void k_idx_scatter(IndexArgs a)
{
    extern __shared__ int cur[];  // [C] next free row of each block for this chunk
    const int bk = blockIdx.y, chunk = blockIdx.x, lane = threadIdx.x;
    const int32_t* base = a.cnt + (long)bk * a.C * a.nchunks + chunk;
    const int32_t* as = a.assign + (long)bk * a.N;
    int32_t* pos = a.positions + (long)bk * a.N;
    // the chunk's assignments, loaded with the blocks' first rows before the
    // ordered scatter
    constexpr int NS = kIndexChunk / 64;
    int cs[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int t = chunk * kIndexChunk + 64 * u + lane;
        cs[u] = t < a.N ? as[t] : -1;
    }
    for (int c = lane; c < a.C; c += 64) cur[c] = base[(long)c * a.nchunks];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int t = chunk * kIndexChunk + 64 * u + lane;
        const int c = cs[u];
        int before = 0, after = 0;
        for (int l = 0; l < 64; ++l) {
            const int cu = __builtin_amdgcn_readlane(c, l);
            before += l < lane && cu == c;
            after += l > lane && cu == c;
        }
        const int at = c >= 0 ? cur[c] + before : 0;
        __builtin_amdgcn_wave_barrier();  // every lane has read its block's counter
        if (c >= 0) {
            pos[at] = t;
            if (after == 0) cur[c] = at + 1;  // the block's last lane of this step
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// One wave per segment: the sum of the unit keys of its rows, rows in order.
// The segment's positions, key rows and 1/|k| are loaded first (two rows per
// lane) and broadcast row by row, so U key rows are in flight at a time.
// Lane l holds channels 2l, 2l+1 (hd 128) or channel l (hd 64).
template <int HD>
__global__ __launch_bounds__(256) void k_idx_seg(IndexArgs a)
{
    constexpr int CPL = HD / 64;  // channels per lane
    constexpr int U = 16;         // rows in flight
    static_assert(kIndexSegment == 128 && kIndexSegment % U == 0, "two rows per lane");
    const Geometry& g = a.g;
    const FastDiv pdiv{g.pdiv.d, g.pdiv.magic, g.pdiv.shift};
    const int bk = blockIdx.y, b = bk / g.Hkv, kvh = bk - b * g.Hkv;
    const int lane = threadIdx.x & 63;
    const int s = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    const int32_t* sb = a.seg_base + (long)bk * (a.C + 1);
    if (s >= sb[a.C]) return;
    const int c = a.seg_block[(long)bk * a.nseg + s];
    const int32_t* offsets = a.offsets + (long)bk * (a.C + 1);
    const int r0 = offsets[c] + (s - sb[c]) * kIndexSegment;
    const int nrows = imin(offsets[c + 1] - r0, kIndexSegment);
    const int32_t* pos = a.positions + (long)bk * a.N;
    const float* inv = a.inv_norm + (long)bk * a.N;
    // row r of the segment: lane r (r < 64) or lane r - 64 of the second
    // pair; both positions, then both block-table entries with both 1/|k|,
    // are loaded together
    const int32_t* btr = g.block_table + (long)b * g.max_pages;
    const int tA = lane < nrows ? pos[r0 + lane] : -1;
    const int tB = 64 + lane < nrows ? pos[r0 + 64 + lane] : -1;
    const int phA = tA >= 0 ? btr[pdiv.div(tA)] : -1, phB = tB >= 0 ? btr[pdiv.div(tB)] : -1;
    const float iA = tA >= 0 ? inv[tA] : 0.f, iB = tB >= 0 ? inv[tB] : 0.f;
    // as key_row: a position on an unmapped page weighs 0 (rows fit 31 bits, checked on the host)
    const bool okA = phA >= 0 && phA < g.num_phys, okB = phB >= 0 && phB < g.num_phys;
    const int rowA = okA ? (int)(((long)phA * g.Hkv + kvh) * g.P + (tA - pdiv.div(tA) * g.P)) : 0;
    const int rowB = okB ? (int)(((long)phB * g.Hkv + kvh) * g.P + (tB - pdiv.div(tB) * g.P)) : 0;
    const float wA = okA ? iA : 0.f, wB = okB ? iB : 0.f;
    float acc[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[e] = 0.f;
    for (int q0 = 0; q0 < nrows; q0 += U) {  // rows past nrows weigh 0
        float x[U][CPL], w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = q0 + u;
            const int rr = r < 64 ? __builtin_amdgcn_readlane(rowA, r) : __builtin_amdgcn_readlane(rowB, r - 64);
            w[u] = __int_as_float(r < 64 ? __builtin_amdgcn_readlane(__float_as_int(wA), r)
                                         : __builtin_amdgcn_readlane(__float_as_int(wB), r - 64));
            if constexpr (CPL == 2) {
                const uint32_t v = *((const uint32_t*)((const uint16_t*)g.k + (long)rr * HD) + lane);
                x[u][0] = bf_lo(v);
                x[u][1] = bf_hi(v);
            } else {
                x[u][0] = __uint_as_float((uint32_t)((const uint16_t*)g.k)[(long)rr * HD + lane] << 16);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < CPL; ++e) acc[e] = fmaf(x[u][e], w[u], acc[e]);
    }
    float* out = a.seg_sum + ((long)bk * a.nseg + s) * HD + CPL * lane;
#pragma unroll
    for (int e = 0; e < CPL; ++e) out[e] = acc[e];
}

template <int HD>
__global__ __launch_bounds__(256) void k_idx_centre(IndexArgs a)
{
    constexpr int CPL = HD / 64;
    const int bk = blockIdx.y, lane = threadIdx.x & 63;
    const int c = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (c >= a.C) return;
    const int32_t* sb = a.seg_base + (long)bk * (a.C + 1);
    float acc[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[e] = 0.f;
    for (int s = sb[c]; s < sb[c + 1]; ++s) {
        const float* x = a.seg_sum + ((long)bk * a.nseg + s) * HD + CPL * lane;
#pragma unroll
        for (int e = 0; e < CPL; ++e) acc[e] += x[e];
    }
    float n2 = 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) n2 = fmaf(acc[e], acc[e], n2);
    n2 = group_sum<64>(n2);
    if (!(n2 > 0.f)) return;  // no keys (or a zero sum): the centre stays
    const float inv = 1.0f / sqrtf(n2);
    float* cf = a.centres + ((long)bk * a.C + c) * HD + CPL * lane;
    uint16_t* cbf = a.cent_bf + ((long)bk * a.C + c) * HD + CPL * lane;
    if constexpr (CPL == 2) {
        cf[0] = acc[0] * inv;
        cf[1] = acc[1] * inv;
        *(uint32_t*)cbf = pack_bf16(acc[0] * inv, acc[1] * inv);
    } else {
        cf[0] = acc[0] * inv;
        cbf[0] = (uint16_t)(pack_bf16(acc[0] * inv, 0.f) & 0xffffu);
    }
}

// 16 bytes of one key row and one value row per thread (the rows are read
// in block order, at random positions: four rows per thread were no faster)
template <int HD>
__global__ __launch_bounds__(256) void k_idx_gather(IndexArgs a)
{
    constexpr int LPT = HD / 8;
    const Geometry& g = a.g;
    const FastDiv pdiv{g.pdiv.d, g.pdiv.magic, g.pdiv.shift};
    const int bk = blockIdx.y, b = bk / g.Hkv, kvh = bk - b * g.Hkv;
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    const int i = (int)(e / LPT), part = (int)(e % LPT);
    if (i >= a.N) return;
    const int t = a.positions[(long)bk * a.N + i];
    const long row = key_row(g, pdiv, b, kvh, t);
    uint4 kw = make_uint4(0, 0, 0, 0), vw = make_uint4(0, 0, 0, 0);
    if (row >= 0) {
        kw = *(const uint4*)((const uint16_t*)g.k + row * HD + 8 * part);
        vw = *(const uint4*)((const uint16_t*)g.v + row * HD + 8 * part);
    }
    const long o = ((long)bk * a.N + i) * HD + 8 * part;
    *(uint4*)((uint16_t*)a.k_blocks + o) = kw;
    *(uint4*)((uint16_t*)a.v_blocks + o) = vw;
}

__global__ __launch_bounds__(256) void k_idx_copy_assign(IndexArgs a, long n)
{
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e < n) a.assign_out[e] = a.assign[e];
}

template <int HD>
hipError_t build_hd(const IndexArgs& a, hipStream_t s)
{
    const int nbk = a.g.B * a.g.Hkv;
    const dim3 b256(256);
    const size_t lds_c = (size_t)a.C * sizeof(int);
    const int keys_wg = 256 / (HD / 8) * kIndexRowsPerThread;  // keys per workgroup of the norms
    hipLaunchKernelGGL((k_idx_norms<HD>), dim3((a.N + keys_wg - 1) / keys_wg, nbk), b256, 0, s, a);
    hipLaunchKernelGGL((k_idx_init<HD>), dim3((a.C + 256 / (HD / 8) - 1) / (256 / (HD / 8)), nbk), b256, 0, s, a);
    for (int it = 0; it <= a.iters; ++it) {
        hipLaunchKernelGGL((k_idx_assign<HD>), dim3((a.N + 255) / 256, nbk), b256, 0, s, a);
        hipLaunchKernelGGL(k_idx_hist, dim3(a.nchunks, nbk), b256, lds_c, s, a);
        hipLaunchKernelGGL(k_idx_scan, dim3(nbk), dim3(1024), 0, s, a);
        hipLaunchKernelGGL(k_idx_scatter, dim3(a.nchunks, nbk), dim3(64), lds_c, s, a);
        if (it == a.iters) break;
        hipLaunchKernelGGL((k_idx_seg<HD>), dim3((a.nseg + 3) / 4, nbk), b256, 0, s, a);
        hipLaunchKernelGGL((k_idx_centre<HD>), dim3((a.C + 3) / 4, nbk), b256, 0, s, a);
    }
    const long cells = (long)a.N * (HD / 8);
    hipLaunchKernelGGL((k_idx_gather<HD>), dim3((unsigned)((cells + 255) / 256), nbk), b256, 0, s, a);
    if (a.assign_out) {
        const long n = (long)nbk * a.N;
        hipLaunchKernelGGL(k_idx_copy_assign, dim3((unsigned)((n + 255) / 256)), b256, 0, s, a, n);
    }
    return hipGetLastError();
}

// ---- block choice ----------------------------------------------------------

template <int HD, int G>
__global__ __launch_bounds__(256) void k_select_blocks(SelectBlocksArgs a)
{
    __shared__ float qs[G][HD];
    __shared__ unsigned long long key[kIndexMaxBlocks];
    __shared__ int wsum[4];
    __shared__ __attribute__((aligned(16))) uint64_t chosen[kIndexMaxBlocks / 64];
    const Geometry& g = a.g;
    int bid = blockIdx.x;
    const int row = bid % a.Q;
    bid /= a.Q;
    const int kvh = bid % g.Hkv, b = bid / g.Hkv;
    const long prob = ((long)b * g.Hkv + kvh) * a.Q + row;
    const int bk = b * g.Hkv + kvh;
    const int wave = threadIdx.x >> 6;

    for (int e = threadIdx.x; e < G * HD; e += 256) {
        const int h = e / HD, d = e - h * HD;
        const uint16_t w = ((const uint16_t*)a.q)[(((long)b * g.Hq + kvh * G + h) * a.Q + row) * HD + d];
        qs[h][d] = __uint_as_float((uint32_t)w << 16);
    }
    int n = 64;  // sort length: a power of two >= C
    while (n < a.C) n *= 2;
    for (int c = threadIdx.x; c < n; c += 256) key[c] = 0ull;
    for (int w = threadIdx.x; w < kIndexMaxBlocks / 64; w += 256) chosen[w] = 0ull;
    __syncthreads();

    // scores: a thread per block, channels in order for every head
    const int32_t* off = a.offsets + (long)bk * (a.C + 1);
    const int32_t* ends = a.ends ? a.ends + (long)bk * a.C : nullptr;
    auto end_of = [&](int c) { return ends ? imax(off[c], imin(ends[c], off[c + 1])) : off[c + 1]; };
    for (int c = threadIdx.x; c < a.C; c += 256) {
        const float4* mu = (const float4*)(a.centres + ((long)bk * a.C + c) * HD);
        float dot[G];
#pragma unroll
        for (int h = 0; h < G; ++h) dot[h] = 0.f;
#pragma unroll 4
        for (int d4 = 0; d4 < HD / 4; ++d4) {
            const float4 m = mu[d4];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                dot[h] = fmaf(qs[h][4 * d4 + 0], m.x, dot[h]);
                dot[h] = fmaf(qs[h][4 * d4 + 1], m.y, dot[h]);
                dot[h] = fmaf(qs[h][4 * d4 + 2], m.z, dot[h]);
                dot[h] = fmaf(qs[h][4 * d4 + 3], m.w, dot[h]);
            }
        }
        float best = dot[0];
#pragma unroll
        for (int h = 1; h < G; ++h) best = fmaxf(best, dot[h]);
        if (end_of(c) > off[c])  // blocks without (visible) tokens are never taken
            key[c] = ((unsigned long long)order_key(best) << 32) | (uint32_t)(0xffffffffu - (uint32_t)c);
    }
    __syncthreads();

    // bitonic sort, descending: larger score first, then the lower block
    for (int size = 2; size <= n; size *= 2) {
        for (int stride = size / 2; stride > 0; stride /= 2) {
            for (int i = threadIdx.x; i < n; i += 256) {
                const int p = i ^ stride;
                if (p > i) {
                    const unsigned long long x = key[i], y = key[p];
                    const bool desc = (i & size) == 0;
                    if (desc ? x < y : x > y) {
                        key[i] = y;
                        key[p] = x;
                    }
                }
            }
            __syncthreads();
        }
    }

    // running token count in sorted order; thread i owns entries per*i ..
    const int per = n / 256 > 0 ? n / 256 : 1;
    auto size_at = [&](int i) {
        const unsigned long long k = i < n ? key[i] : 0ull;
        const int c = (int)(0xffffffffu - (uint32_t)(k & 0xffffffffull));
        return k != 0ull ? end_of(c) - off[c] : 0;
    };
    int mine = 0;
    for (int u = 0; u < per; ++u) mine += size_at(per * (int)threadIdx.x + u);
    int total;
    int run = block_exclusive_scan<256>(mine, wsum, total);
    int take = 0;
    for (int u = 0; u < per; ++u) {
        const int i = per * (int)threadIdx.x + u;
        const int sz = size_at(i);
        run += sz;
        take += sz > 0 && i < a.k_max && run <= a.budget;
    }
    // blocks with a running count within the budget form a prefix of the
    // order; the first nonempty block is always taken
    int unused;
    const int before = block_exclusive_scan<256>(take, wsum, unused);
    const int count_in = before + take;  // the thread of the last entry holds the total
    __shared__ int s_count;
    if (threadIdx.x == 255) s_count = count_in;
    __syncthreads();
    const int count = s_count > 0 ? s_count : (key[0] != 0ull && a.k_max > 0 ? 1 : 0);
    for (int i = threadIdx.x; i < count; i += 256) {
        const int c = (int)(0xffffffffu - (uint32_t)(key[i] & 0xffffffffull));
        atomicOr((unsigned long long*)&chosen[c >> 6], 1ull << (c & 63));
    }
    __syncthreads();
    int32_t* sel = a.sel + prob * a.k_max;
    if (wave == 0) emit_bitmap(a.C, chosen, [&](int p, int c) { sel[p] = c; });
    for (int i = count + (int)threadIdx.x; i < a.k_max; i += 256) sel[i] = -1;
    if (threadIdx.x == 0) a.count[prob] = count;
}

// A thread per (sequence, KV head, block): the first row of the block whose
// position is at or after L - W (binary search; positions ascend in a block).
__global__ __launch_bounds__(256) void k_blocks_visible(VisibleArgs a)
{
    const Geometry& g = a.g;
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)g.B * g.Hkv * a.C) return;
    const int bk = (int)(idx / a.C), c = (int)(idx - (long)bk * a.C);
    const int b = bk / g.Hkv;
    const int L = imax(0, imin(g.seq_lens[b], g.max_pages * g.P));
    const int bound = L - a.W;
    const int32_t* off = a.offsets + (long)bk * (a.C + 1);
    const int32_t* pos = a.positions + (long)bk * a.N;
    int lo = imax(0, imin(off[c], a.N)), hi = imax(lo, imin(off[c + 1], a.N));
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (pos[mid] < bound)
            lo = mid + 1;
        else
            hi = mid;
    }
    a.ends[idx] = lo;
}

}  // namespace

hipError_t launch_blocks_visible(const VisibleArgs& a, hipStream_t s)
{
    const long n = (long)a.g.B * a.g.Hkv * a.C;
    hipLaunchKernelGGL(k_blocks_visible, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_index_build(const IndexArgs& a, hipStream_t s)
{
    if (a.g.dtype != 1 || a.C < 1 || a.C > kIndexMaxBlocks || a.N < 1) return hipErrorInvalidValue;
    if (a.g.hd == 128) return build_hd<128>(a, s);
    if (a.g.hd == 64) return build_hd<64>(a, s);
    return hipErrorInvalidValue;
}

template <int HD>
hipError_t select_blocks_g(const SelectBlocksArgs& a, dim3 grid, hipStream_t s)
{
    switch (a.g.G) {
    case 1: hipLaunchKernelGGL((k_select_blocks<HD, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_select_blocks<HD, 2>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_select_blocks<HD, 4>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_select_blocks<HD, 8>), grid, dim3(256), 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_select_blocks<HD, 16>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_select_blocks(const SelectBlocksArgs& a, hipStream_t s)
{
    if (a.g.dtype != 1 || a.C < 1 || a.C > kIndexMaxBlocks) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((long)a.g.B * a.g.Hkv * a.Q));
    if (a.g.hd == 128) return select_blocks_g<128>(a, grid, s);
    if (a.g.hd == 64) return select_blocks_g<64>(a, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace sa
