// KeyDiff eviction (course module 14, section 14.4 and exercise 14.2): a
// token's importance is how far its key lies from the mean key of the tokens
// the cache holds; the least distinctive tokens are evicted, the first `sink`
// positions never, and the cache is brought back to its budget after every
// block of new tokens, so it never holds more than budget + block tokens.
//
//  * k_kd_sum: per (sequence, KV head, chunk of kKdChunk tokens) the fp32 sum
//    of the keys (rows in order in each lane, then lanes and waves in a fixed
//    order: bitwise reproducible); the last chunks are launched first.  A chunk that the previous eviction's
//    compaction filled takes its sum from the key sums that compaction left
//    (one per group of kKdSlots slots, added in order) instead of reading its
//    keys again: between evictions only the new block's keys are summed.
//  * k_kd_dist: every workgroup rebuilds the mean key from the chunk sums, in
//    chunk order, and writes the order key of each candidate's squared
//    distance to it, candidates in reverse position order.
//  * k_kd_topk: one workgroup per (sequence, KV head) keeps the sink and the
//    budget - sink farthest other tokens.  Among equal distances the later
//    position is kept: the candidates are ranked in reverse position order
//    and the block top-k prefers the lower index.  Kept positions ascending.
//  * k_kd_compact: copies the kept tokens' K and V rows, in order, into
//    slots 0 .. count-1 of a destination cache, and optionally writes the key
//    sum of every group of kKdSlots slots (the next eviction's carried sums).
// The sum and distance passes stream the keys with 16-byte loads; each wave
// resolves the block-table entries of the pages its rows span once, up front.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "topk_block.hpp"

namespace sa {

namespace {

static_assert(kKdChunk % kKdSlots == 0, "a chunk of the sum pass is whole groups of carried sums");

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kKdWaves = 4;
constexpr int kKdRowsPerWave = kKdChunk / kKdWaves;
static_assert(kKdRowsPerWave <= 128, "a wave's rows span at most 128 pages");
constexpr int kKdU = 16;            // row loads per lane in flight
constexpr int kKdCopyThreads = 256;

__device__ __forceinline__ int kd_len(const Geometry& g, int T, int b)
{
    return imax(0, imin(imin(g.seq_lens[b], T), g.max_pages * g.P));
}

// Block-table entries of the logical pages [pg0, pg0 + npg) of one sequence
// (npg <= 128, the pages of one wave's rows), two per lane, looked up by lane
// exchanges.  Entries past npg are -1; every entry is checked against the
// pool before use.
struct WavePages {
    int pg0, npg, lo, hi;  // lo: page pg0 + lane, hi: page pg0 + 64 + lane
    __device__ __forceinline__ void init(const int32_t* table, int first, int n)
    {
        pg0 = first;
        npg = n;
        const int lane = threadIdx.x & 63;
        lo = lane < n ? table[first + lane] : -1;
        hi = 64 + lane < n ? table[first + 64 + lane] : -1;
    }
    // every lane of the wave takes part
    __device__ __forceinline__ int entry(int page) const
    {
        const int i = page - pg0;
        if (npg <= 64) return __shfl(lo, i);
        const int a = __shfl(lo, i & 63), b = __shfl(hi, i & 63);
        return i < 64 ? a : b;
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

// The block-table entries of the pages that rows [w0, w0 + kKdRowsPerWave)
// of sequence b span (clipped to the table), loaded before the sequence's
// length is known, so that this load and the length's are in flight
// together.  The rows a wave streams are a prefix of that range.
__device__ __forceinline__ WavePages kd_wave_pages(const Geometry& g, const FastDiv& pdiv, int b, int w0)
{
    WavePages wp;
    const int cap = g.max_pages * g.P;
    const int hi = imin(w0 + kKdRowsPerWave, cap);
    const int pg0 = pdiv.div(imin(w0, cap - 1));
    wp.init(g.block_table + (long)b * g.max_pages, pg0, w0 < hi ? pdiv.div(hi - 1) - pg0 + 1 : 0);
    return wp;
}

// Streams rows [r0, r1) of (b, kvh) (pages resolved by wp), U loads per lane
// in flight, calling f(row, x) with this lane's CH channels of each row; rows
// past r1 and rows on unmapped pages read as zeros (a zero key).  The pages
// of a round's rows are resolved before any of its loads is issued: a
// block-table load between two row loads would make each row load wait for
// the ones before it.
template <int HD, bool BF, int U, typename F>
__device__ __forceinline__ void kd_stream(const Geometry& g, const FastDiv& pdiv, const WavePages& wp, int kvh,
                                          int r0, int r1, F f)
{
    using Lay = KdLayout<HD, BF>;
    typedef typename Lay::E E;
    const int lane = threadIdx.x & 63;
    const int sub = lane % Lay::LPT, rg = lane / Lay::LPT;
    if (r0 >= r1) return;
    for (int base = r0; base < r1; base += Lay::RPW * U) {
        int ph[U];
#pragma unroll
        for (int u = 0; u < U; ++u) ph[u] = wp.entry(pdiv.div(imin(base + u * Lay::RPW + rg, r1 - 1)));
        uint4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = base + u * Lay::RPW + rg;
            const int page = pdiv.div(imin(t, r1 - 1));
            w[u] = make_uint4(0, 0, 0, 0);
            if (t < r1 && ph[u] >= 0 && ph[u] < g.num_phys)
                w[u] = *(const uint4*)((const E*)g.k + (((long)ph[u] * g.Hkv + kvh) * g.P + (t - page * g.P)) * HD +
                                       sub * Lay::CH);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
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
    // workgroup (i, j) sums chunk nchunks-1-j of pair i: the last chunks,
    // which hold the newest tokens and are never carried, are dispatched first
    const int bh = blockIdx.x, b = bh / g.Hkv, kvh = bh % g.Hkv, chunk = a.nchunks - 1 - (int)blockIdx.y;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t0 = chunk * kKdChunk;
    const int w0 = t0 + wave * kKdRowsPerWave;
    // the length, the carried count and the wave's block-table entries are
    // independent: all three loads are issued before any is waited for
    const int len = g.seq_lens[b];
    const int ccount = a.carried ? a.carried_count[bh] : 0;
    const WavePages wp = kd_wave_pages(g, pdiv, b, w0);
    const int L = imax(0, imin(imin(len, a.T), g.max_pages * g.P));
    if (t0 >= L) return;
    float* const dst = a.partial + ((long)bh * a.nchunks + chunk) * HD;
    if (a.carried && t0 + kKdChunk <= imin(imin(ccount, kKdSlots * a.carried_groups), L)) {
        // a chunk the last compaction filled: the sum of its groups' sums, in order
        const float* cs = a.carried + ((long)bh * a.carried_groups + chunk * (kKdChunk / kKdSlots)) * HD;
        for (int c = threadIdx.x; c < HD; c += 64 * kKdWaves) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < kKdChunk / kKdSlots; ++i) s += cs[i * HD + c];
            dst[c] = s;
        }
        return;
    }
    const int sub = lane % Lay::LPT, rg = lane / Lay::LPT;
    const int r0 = imin(L, w0), r1 = imin(L, r0 + kKdRowsPerWave);

    float acc[Lay::CH];
#pragma unroll
    for (int c = 0; c < Lay::CH; ++c) acc[c] = 0.f;
    // the wave's rows in one round of loads, at most 32 per lane (each lane
    // adds its rows in order)
    constexpr int U = kKdRowsPerWave / Lay::RPW < 32 ? kKdRowsPerWave / Lay::RPW : 32;
    kd_stream<HD, BF, U>(g, pdiv, wp, kvh, r0, r1, [&](int, const float (&x)[Lay::CH]) {
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
        dst[c] = s;
    }
}

template <int HD, bool BF>
__global__ __launch_bounds__(64 * kKdWaves) void k_kd_dist(KeydiffArgs a)
{
    using Lay = KdLayout<HD, BF>;
    constexpr int NT = 64 * kKdWaves;
    constexpr int TPC = NT / HD;  // threads per channel of the mean
    constexpr int MJ = 16;        // chunk sums a thread loads per round
    static_assert(TPC * HD == NT, "threads tile the channels");
    __shared__ float part[TPC][HD];
    const Geometry& g = a.g;
    const FastDiv pdiv{g.pdiv.d, g.pdiv.magic, g.pdiv.shift};
    const int bh = blockIdx.y, b = bh / g.Hkv, kvh = bh % g.Hkv;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane % Lay::LPT;
    const int t0 = blockIdx.x * kKdChunk;
    const int w0 = t0 + wave * kKdRowsPerWave;
    // The mean key: thread (h, c) adds the sums of channel c over its share
    // of the chunks, in chunk order; the TPC shares are then added in order.
    // The first round of chunk-sum loads, the length and the wave's
    // block-table entries are in flight together (chunks past the length
    // were not written and are masked out once it is known).
    const int c = threadIdx.x % HD, h = threadIdx.x / HD;
    const int per = (a.nchunks + TPC - 1) / TPC;
    const int j0 = h * per, j1 = imin(a.nchunks, j0 + per);
    const float* ps = a.partial + (long)bh * a.nchunks * HD + c;
    float v[MJ];
#pragma unroll
    for (int u = 0; u < MJ; ++u) v[u] = j0 + u < j1 ? ps[(long)(j0 + u) * HD] : 0.f;
    const int len = g.seq_lens[b];
    const WavePages wp = kd_wave_pages(g, pdiv, b, w0);
    const int L = imax(0, imin(imin(len, a.T), g.max_pages * g.P));
    if (t0 >= L) return;
    const int nch = (L + kKdChunk - 1) / kKdChunk;
    const int je = imin(j1, nch);
    float s = 0.f;
    for (int jb = j0;;) {
#pragma unroll
        for (int u = 0; u < MJ; ++u)
            if (jb + u < je) s += v[u];
        jb += MJ;
        if (jb >= je) break;
#pragma unroll
        for (int u = 0; u < MJ; ++u) v[u] = jb + u < je ? ps[(long)(jb + u) * HD] : 0.f;
    }
    part[h][c] = s;
    __syncthreads();
    float m[Lay::CH];
#pragma unroll
    for (int e = 0; e < Lay::CH; ++e) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < TPC; ++i) t += part[i][sub * Lay::CH + e];
        m[e] = t / (float)L;
    }
    const int r0 = imin(L, w0), r1 = imin(L, r0 + kKdRowsPerWave);
    // token t goes to index L-1-t (the sink's indices, past the candidates, are never read)
    uint32_t* okeys = a.okeys + (long)bh * a.Tk + (L - 1);
    kd_stream<HD, BF, kKdU>(g, pdiv, wp, kvh, r0, r1, [&](int t, const float (&x)[Lay::CH]) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < Lay::CH; ++e) {
            const float df = x[e] - m[e];
            d = fmaf(df, df, d);
        }
        d = group_sum<Lay::LPT>(d);
        if (sub == 0 && t < r1) okeys[-t] = order_key(d);
    });
}

__global__ __launch_bounds__(kTopkThreads) void k_kd_topk(KeydiffArgs a)
{
    __shared__ __attribute__((aligned(16))) uint32_t keys[kKdMaxCand];
    __shared__ int32_t staged[kKdMaxCand];  // the kept candidates' positions, in order, before one coalesced write
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
    block_topk_fast(m, k, keys, lo, hi, sh, [&](int pos, int j) { staged[k - 1 - pos] = L - 1 - j; });
    __syncthreads();
    for (int i = tid; i < k; i += kTopkThreads) kept[s0 + i] = staged[i];
}

// Past kKdMaxCand candidates the evicted tokens are chosen instead of the
// kept ones (there are fewer of them): candidate i is position sink + i, its
// key the inverted distance key (the nearest to the mean first), and ties go
// to the lower index, i.e. the earlier position is evicted first, as in the
// one-workgroup path.  Stage 1: workgroup (chunk c, sequence and KV head)
// writes the min(e, chunk size) candidates of its chunk to evict first, e =
// the number evicted, ascending.  Every token among the e evicted is among
// its chunk's picks.
__global__ __launch_bounds__(kTopkThreads) void k_kd_evict_chunk(KeydiffArgs a)
{
    __shared__ __attribute__((aligned(16))) uint32_t keys[kTopkChunk];
    __shared__ TopkScratch sh;
    const Geometry& g = a.g;
    const int c = blockIdx.x, bh = blockIdx.y, b = bh / g.Hkv;
    const int L = kd_len(g, a.T, b);
    if (L <= a.budget) return;
    const int s0 = imin(a.sink, L);
    const int m = L - s0, k = a.budget - s0;  // candidates, kept among them
    const int e = m - k;                      // evicted (>= 1)
    const int c0 = c * kTopkChunk;
    const int nc = imin(m - c0, kTopkChunk);
    if (k <= 0 || nc <= 0) return;
    const int ke = imin(e, nc);
    const uint32_t* src = a.okeys + (long)bh * a.Tk;  // candidate i at index m - 1 - i
    uint32_t lo = 0xffffffffu, hi = 0;
    for (int i = threadIdx.x; i < nc; i += kTopkThreads) {
        const uint32_t key = ~src[m - 1 - (c0 + i)];
        keys[i] = key;
        lo = min(lo, key);
        hi = max(hi, key);
    }
    uint32_t* pk = a.part_keys + ((long)bh * a.ecnk + c) * kTopkChunk;
    int32_t* pi = a.part_idx + ((long)bh * a.ecnk + c) * kTopkChunk;
    if (ke == nc) {  // the whole chunk
        for (int i = threadIdx.x; i < nc; i += kTopkThreads) {
            pk[i] = keys[i];
            pi[i] = c0 + i;
        }
        return;
    }
    __syncthreads();
    block_topk_fast(nc, ke, keys, lo, hi, sh, [&](int pos, int i) {
        pk[pos] = keys[i];
        pi[pos] = c0 + i;
    });
}

// Stage 2: one workgroup per (sequence, KV head) picks the e evicted tokens
// among the chunks' picks (laid out chunk after chunk, so ascending
// candidates and ties to the earlier position carry over), marks them in a
// bitmap and writes the sink and every unmarked candidate, ascending.
__global__ __launch_bounds__(kTopkThreads) void k_kd_evict_merge(KeydiffArgs a)
{
    __shared__ __attribute__((aligned(16))) uint32_t keys[kTopkMerge];
    __shared__ TopkScratch sh;
    __shared__ uint32_t evicted[kKdMaxChunks * kTopkChunk / 32];
    __shared__ int off[kKdMaxChunks + 1];
    __shared__ int wsum[kTopkThreads / 64];
    const Geometry& g = a.g;
    const int bh = blockIdx.x, b = bh / g.Hkv;
    const int L = kd_len(g, a.T, b);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
    const int m = L - s0, k = a.budget - s0, e = m - k;
    if (k <= 0) return;  // the sink alone
    const int nch = (m + kTopkChunk - 1) / kTopkChunk;  // <= ecnk
    const int nw = (m + 31) / 32;
    for (int w = tid; w < nw; w += kTopkThreads) evicted[w] = 0u;
    if (tid == 0) {
        int acc = 0;
        for (int c = 0; c < nch; ++c) {
            off[c] = acc;
            acc += imin(e, imin(m - c * kTopkChunk, kTopkChunk));
        }
        off[nch] = acc;
    }
    __syncthreads();
    const int mw = off[nch];  // <= kTopkMerge (host-checked)
    const uint32_t* pk = a.part_keys + (long)bh * a.ecnk * kTopkChunk;
    const int32_t* pi = a.part_idx + (long)bh * a.ecnk * kTopkChunk;
    auto cand_of = [&](int i) {  // candidate index of merged pick i
        int c = 0;
        while (c + 1 < nch && off[c + 1] <= i) ++c;
        return pi[c * kTopkChunk + (i - off[c])];
    };
    if (e >= mw) {  // every pick is evicted
        for (int i = tid; i < mw; i += kTopkThreads) {
            const int ci = cand_of(i);
            atomicOr(&evicted[ci >> 5], 1u << (ci & 31));
        }
    } else {
        uint32_t lo = 0xffffffffu, hi = 0;
        for (int c = 0; c < nch; ++c) {
            const int n = off[c + 1] - off[c];
            for (int i = tid; i < n; i += kTopkThreads) {
                const uint32_t key = pk[c * kTopkChunk + i];
                keys[off[c] + i] = key;
                lo = min(lo, key);
                hi = max(hi, key);
            }
        }
        block_topk_fast(mw, e, keys, lo, hi, sh, [&](int, int i) {
            const int ci = cand_of(i);
            atomicOr(&evicted[ci >> 5], 1u << (ci & 31));
        });
    }
    __syncthreads();
    // the kept candidates in order: a block scan of the per-word counts, 512 words a round
    int base = 0;
    for (int w0 = 0; w0 < nw; w0 += kTopkThreads) {
        const int w = w0 + tid;
        uint32_t keep = 0u;
        if (w < nw) {
            keep = ~evicted[w];
            if (32 * w + 32 > m) keep &= (m - 32 * w >= 32) ? 0xffffffffu : ((1u << (m - 32 * w)) - 1u);
        }
        const int n = __builtin_popcount(keep);
        const int inc = wave_inclusive_scan(n);
        if (lane == 63) wsum[wave] = inc;
        __syncthreads();
        int before = base;
        for (int v = 0; v < wave; ++v) before += wsum[v];
        int total = base;
        for (int v = 0; v < kTopkThreads / 64; ++v) total += wsum[v];
        int r = before + inc - n;
        while (keep) {
            const int bit = __builtin_ctz(keep);
            kept[s0 + r++] = s0 + 32 * w + bit;
            keep &= keep - 1u;
        }
        base = total;
        __syncthreads();
    }
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
        kv[it][0] = ld_stream((const uint4*)s.k + so);
        kv[it][1] = ld_stream((const uint4*)s.v + so);
        dst_off[it] = (((long)dph * d.Hkv + kvh) * d.P + (j - dp * d.P)) * PPR + piece;
    }
    // the copy's stores are non-temporal: the evicted cache is not read again
    // soon, and written back at once they do not land, as dirty lines of the
    // last-level cache, in the next kernels' reads
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        if (dst_off[it] < 0) continue;
        const uint4 k4 = kv[it][0], v4 = kv[it][1];
        __builtin_nontemporal_store(u32x4_t{k4.x, k4.y, k4.z, k4.w}, (u32x4_t*)d.k + dst_off[it]);
        __builtin_nontemporal_store(u32x4_t{v4.x, v4.y, v4.z, v4.w}, (u32x4_t*)d.v + dst_off[it]);
    }
    if (a.slot_sums) {
        // the key sum of this group of slots (a key not copied counts as
        // zero): each thread adds its rows (slots j0 + it * RPI + tid / PPR,
        // in order) for the channels of its piece, then the row groups are
        // added in order
        using Lay = KdLayout<HD, BF>;
        constexpr int RPI = kKdCopyThreads / PPR;  // row groups
        __shared__ float part[RPI][HD];
        float acc[Lay::CH];
#pragma unroll
        for (int c = 0; c < Lay::CH; ++c) acc[c] = 0.f;
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            float x[Lay::CH];
            Lay::unpack(kv[it][0], x);  // zeros when the row was not copied
#pragma unroll
            for (int c = 0; c < Lay::CH; ++c) acc[c] += x[c];
        }
        const int piece = threadIdx.x % PPR;
#pragma unroll
        for (int c = 0; c < Lay::CH; ++c) part[threadIdx.x / PPR][piece * Lay::CH + c] = acc[c];
        __syncthreads();
        float* out = a.slot_sums + ((long)bh * gridDim.x + blockIdx.x) * HD;
        for (int c = threadIdx.x; c < HD; c += kKdCopyThreads) {
            float s = 0.f;
#pragma unroll
            for (int r = 0; r < RPI; ++r) s += part[r][c];
            out[c] = s;
        }
    }
}

template <int HD, bool BF>
hipError_t launch_kd(const KeydiffArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)a.nchunks, (unsigned)(a.g.B * a.g.Hkv));
    hipLaunchKernelGGL((k_kd_sum<HD, BF>), dim3(grid.y, grid.x), dim3(64 * kKdWaves), 0, s, a);
    hipLaunchKernelGGL((k_kd_dist<HD, BF>), grid, dim3(64 * kKdWaves), 0, s, a);
    if (a.ecnk > 0) {  // more candidates than one workgroup holds
        hipLaunchKernelGGL(k_kd_evict_chunk, dim3((unsigned)a.ecnk, (unsigned)(a.g.B * a.g.Hkv)), dim3(kTopkThreads),
                           0, s, a);
        hipLaunchKernelGGL(k_kd_evict_merge, dim3((unsigned)(a.g.B * a.g.Hkv)), dim3(kTopkThreads), 0, s, a);
    } else {
        hipLaunchKernelGGL(k_kd_topk, dim3((unsigned)(a.g.B * a.g.Hkv)), dim3(kTopkThreads), 0, s, a);
    }
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
