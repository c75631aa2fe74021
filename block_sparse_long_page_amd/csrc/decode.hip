// Split-K flash decode over the attended token set (sink + window + the
// middle tokens of the selected pages), exact softmax with a running maximum
// and sum (FlashAttention's online softmax, attention-mechanisms article,
// "FlashAttention does not change what the model looks at").
//
// Workgroup = one (sequence, KV head, query row, split); its four waves each
// stream a contiguous quarter of the split's tokens.  Lane layout inside a
// wave: LPT lanes hold one key/value row with 16-byte loads (8 bf16 or 4 fp32
// channels per lane), so 64/LPT tokens are in flight per load instruction and
// U loads of K and of V per lane per iteration.  Every K/V row is read once
// and shared by the G query heads of the group.
//
// q.k: packed bf16 dot products into fp32 (or fp32 FMAs), summed over the
// LPT lanes with DPP row operations.  Softmax in base 2 with a lazily
// rescaled reference maximum: the accumulators are rescaled only when a
// logit exceeds the reference by more than 2^8, which keeps every weight
// <= 256 and skips most rescales.  p.v accumulates in fp32.  At the end the
// token groups of a wave fold with shuffles and the four waves through LDS;
// the workgroup writes its normalised partial and (m, l).  No atomics.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "merge.hpp"
#include "topk_block.hpp"

namespace sa {

namespace {

#ifndef SA_MFMA_TPS
#define SA_MFMA_TPS 1
#endif
constexpr int kWaves = 4;
constexpr float kRescaleSlack = 8.0f;  // log2 units

template <int HD, int G, bool BF>
__global__ __launch_bounds__(64 * kWaves) void k_decode_generic(DecodeArgs a)
{
    constexpr int CH = BF ? 8 : 4;  // channels per lane
    constexpr int LPT = HD / CH;    // lanes per token
    constexpr int TPW = 64 / LPT;   // tokens per wave load
    constexpr int U = 4;            // loads of K and V in flight per lane
    typedef typename std::conditional<BF, uint16_t, float>::type E;
    const Geometry& g = a.g;

    __shared__ float lds_o[kWaves][G][HD];
    __shared__ float lds_ml[kWaves][G][2];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPT, tg = lane / LPT;

    int bid = blockIdx.x;
    const int split = bid % a.splits;
    bid /= a.splits;
    const int kvh = bid % g.Hkv;
    bid /= g.Hkv;
    const int row = bid % a.Q;
    const int b = bid / a.Q;

    const int L = imax(0, imin(g.seq_lens[b], g.max_pages * g.P));
    const int pos = L - a.Q + row;
    const long prob = ((long)b * g.Hkv + kvh) * a.Q + row;
    TokenSet ts;
    ts.init(L, a.S, a.W, g.P, a.sel ? a.sel + prob * a.k_max : nullptr, a.sel ? a.count[prob] : 0, a.k_max,
            a.parts);
    const FastDiv pdiv{g.pdiv.d, g.pdiv.magic, g.pdiv.shift};

    // this workgroup's slice of the token set, then this wave's
    const int n = ts.total;
    const int f0 = split * (n / a.splits) + imin(split, n % a.splits);
    const int f1 = f0 + n / a.splits + (split < n % a.splits ? 1 : 0);
    const int len = f1 - f0;
    const int w0 = f0 + wave * (len / kWaves) + imin(wave, len % kWaves);
    const int w1 = w0 + len / kWaves + (wave < len % kWaves ? 1 : 0);

    // the group's queries, this lane's channels
    uint32_t qw[G][CH / 2];  // bf16 pairs
    float qf[G][CH];         // fp32
    for (int h = 0; h < G; ++h) {
        const E* qp = (const E*)a.q + (((long)b * g.Hq + kvh * G + h) * a.Q + row) * HD + sub * CH;
        const uint4 w = *(const uint4*)qp;
        if constexpr (BF) {
            qw[h][0] = w.x;
            qw[h][1] = w.y;
            qw[h][2] = w.z;
            qw[h][3] = w.w;
        } else {
            qf[h][0] = __uint_as_float(w.x);
            qf[h][1] = __uint_as_float(w.y);
            qf[h][2] = __uint_as_float(w.z);
            qf[h][3] = __uint_as_float(w.w);
        }
    }

    float m[G], l[G], o[G][CH];
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
        for (int c = 0; c < CH; ++c) o[h][c] = 0.f;
    }

    const E* kbase = (const E*)g.k + (long)kvh * g.P * HD + sub * CH;
    const E* vbase = (const E*)g.v + (long)kvh * g.P * HD + sub * CH;
    const long page_stride = (long)g.Hkv * g.P * HD;
    const int32_t* bt = g.block_table + (long)b * g.max_pages;

    for (int base = w0; base < w1; base += TPW * U) {
        uint4 kw[U], vw[U];
        bool valid[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int f = base + u * TPW + tg;
            int t = f < w1 ? ts.position(f, pdiv) : -1;
            if (t > pos) t = -1;
            long off = 0;
            if (t >= 0) {
                const int pg = pdiv.div(t);
                const int phys = bt[pg];
                if (phys >= 0 && phys < g.num_phys)
                    off = (long)phys * page_stride + (long)(t - pg * g.P) * HD;
                else
                    t = -1;
            }
            valid[u] = t >= 0;
            kw[u] = valid[u] ? *(const uint4*)(kbase + off) : make_uint4(0, 0, 0, 0);
            vw[u] = valid[u] ? *(const uint4*)(vbase + off) : make_uint4(0, 0, 0, 0);
        }

        float z[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t* k32 = (const uint32_t*)&kw[u];
            for (int h = 0; h < G; ++h) {
                float d = 0.f;
                if constexpr (BF) {
                    for (int j = 0; j < 4; ++j) d = dot2_bf16(qw[h][j], k32[j], d);
                } else {
                    for (int j = 0; j < 4; ++j) d = fmaf(qf[h][j], __uint_as_float(k32[j]), d);
                }
                d = group_sum<LPT>(d);
                z[u][h] = valid[u] ? d * a.scale_log2 : -INFINITY;
            }
        }

        for (int h = 0; h < G; ++h) {
            float mx = z[0][h];
            for (int u = 1; u < U; ++u) mx = fmaxf(mx, z[u][h]);
            if (mx > m[h] + kRescaleSlack) {
                const float alpha = __builtin_amdgcn_exp2f(m[h] - mx);  // 0 while m = -inf
                l[h] *= alpha;
                for (int c = 0; c < CH; ++c) o[h][c] *= alpha;
                m[h] = mx;
            }
            const float mref = m[h] == -INFINITY ? 0.f : m[h];
            for (int u = 0; u < U; ++u) z[u][h] = __builtin_amdgcn_exp2f(z[u][h] - mref);  // -inf -> 0
        }

#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t* v32 = (const uint32_t*)&vw[u];
            float v[CH];
            if constexpr (BF) {
                for (int j = 0; j < 4; ++j) {
                    v[2 * j] = bf_lo(v32[j]);
                    v[2 * j + 1] = bf_hi(v32[j]);
                }
            } else {
                for (int j = 0; j < 4; ++j) v[j] = __uint_as_float(v32[j]);
            }
            for (int h = 0; h < G; ++h) {
                const float p = z[u][h];
                l[h] += p;
                for (int c = 0; c < CH; ++c) o[h][c] = fmaf(p, v[c], o[h][c]);
            }
        }
    }

    // fold the token groups of the wave (lanes sub, sub + LPT, ...)
    for (int off = LPT; off < 64; off <<= 1) {
        for (int h = 0; h < G; ++h) {
            const float m2 = __shfl_xor(m[h], off);
            const float l2 = __shfl_xor(l[h], off);
            const float mn = fmaxf(m[h], m2);
            const float a1 = m[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[h] - mn);
            const float a2 = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
            l[h] = l[h] * a1 + l2 * a2;
            for (int c = 0; c < CH; ++c) o[h][c] = o[h][c] * a1 + __shfl_xor(o[h][c], off) * a2;
            m[h] = mn;
        }
    }
    if (tg == 0) {
        for (int h = 0; h < G; ++h) {
            for (int c = 0; c < CH; ++c) lds_o[wave][h][sub * CH + c] = o[h][c];
            if (sub == 0) {
                lds_ml[wave][h][0] = m[h];
                lds_ml[wave][h][1] = l[h];
            }
        }
    }
    __syncthreads();

    // fold the waves and write the partial
    for (int i = threadIdx.x; i < G * HD; i += 64 * kWaves) {
        const int h = i / HD, c = i % HD;
        float ms = -INFINITY;
        for (int w = 0; w < kWaves; ++w) ms = fmaxf(ms, lds_ml[w][h][0]);
        float ls = 0.f, os = 0.f;
        for (int w = 0; w < kWaves; ++w) {
            const float mw = lds_ml[w][h][0];
            const float aw = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - ms);
            ls = fmaf(lds_ml[w][h][1], aw, ls);
            os = fmaf(lds_o[w][h][c], aw, os);
        }
        const long prow = (((long)b * g.Hq + kvh * G + h) * a.Q + row) * a.split_stride + split;
        a.part_o[prow * HD + c] = ls > 0.f ? os / ls : 0.f;
        if (c == 0) {
            a.part_ml[prow * 2 + 0] = ls > 0.f ? ms * kLn2 : -INFINITY;
            a.part_ml[prow * 2 + 1] = ls;
        }
    }
}

constexpr int kPartMiddle = 2;  // the selected pages' middle tokens (TokenSet parts bit)

// ---------------------------------------------------------------------------
// bf16 decode on the matrix cores.  The G query heads of a KV group against a
// tile of 16 tokens are a small dense product, so both products of a tile run
// as MFMAs and the vector ALU only does the softmax:
//  * q.k: v_mfma_f32_16x16x32_bf16 with the tile's keys as A (row = token,
//    8 channels per lane straight from global memory) and the queries as B
//    (column = head; heads past G are zero).  The result leaves, in lane
//    (r, j) = (lane % 16, lane / 16), the logits of head r for tokens 4j..4j+3;
//  * softmax per head with the lazily rescaled reference maximum (base 2, the
//    scale folded into the exponent); the weights of lane (r, j) are exactly
//    the A operand of the next product (row = head r, k = tokens 4j..4j+3);
//  * p.v: v_mfma_f32_16x16x16_bf16 per 16 output channels with the values as
//    B (k = token, column = channel).  The value rows are written to LDS as
//    loaded (row-major, a 32-byte pad per 4 tokens so the column reads below
//    hit distinct banks) and read back one bf16 per token and channel;
//  * the accumulators hold rows = heads 4j..4j+3 and column = channel.
// A workgroup's tokens are listed in a row table in LDS and taken in rounds of
// NW tiles, tile w of each round by wave w, three rounds in flight per wave.
// At the end the waves merge through LDS and the workgroup writes its
// normalised partial and (m, l).
// ---------------------------------------------------------------------------

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int HD, int G>
struct MfmaPlan {
    static constexpr int KK = HD / 32;                 // q.k products per tile (32 channels each)
    static constexpr int NB = HD / 16;                 // p.v products per tile (16 channels each)
    static constexpr int VLD = HD / 32;                // 16-byte value loads per lane per tile
    static constexpr int LPT = HD / 8;                 // lanes per value row
    static constexpr int VROW = HD * 2;                // bytes per value row
    static constexpr int VTILE = 16 * VROW + 4 * 32;   // LDS bytes of one value tile (padded)
    static constexpr int TPS = SA_MFMA_TPS;            // tiles per wave per round
    static constexpr int NW = 8;                       // waves per workgroup: one workgroup fills a CU
    static constexpr int RT = NW * TPS * 16;           // tokens per round
    static constexpr int vbytes() { return NW * TPS * VTILE; }
    static constexpr int obytes() { return NW * G * HD * 4; }
    static constexpr int smem_bytes() { return vbytes() > obytes() ? vbytes() : obytes(); }
    static_assert(kRowsWG % RT == 0 && kRowsWG % (64 * NW) == 0, "rounds tile the row table");
    static_assert(G <= 16, "one MFMA column per head");
    static_assert(NW * 64 == kTopkThreads, "the select-and-decode workgroup runs the block top-k");
};

// LDS byte offset of (token t, byte b) in a value tile
template <int VROW>
__device__ __forceinline__ int vt_off(int t, int b)
{
    return t * VROW + (t >> 2) * 32 + b;
}

// LDS a workgroup of the matrix-core decode shares
template <int HD, int G>
struct MfmaLds {
    using Plan = MfmaPlan<HD, G>;
    __attribute__((aligned(16))) int rows[kRowsWG];
    __attribute__((aligned(16))) unsigned char tiles[Plan::smem_bytes()];  // value tiles, then the waves' outputs
    float wv_m[Plan::NW][G], wv_l[Plan::NW][G];
};

// Per-lane state and tile pipeline of the matrix-core decode.  NT: the K and
// V tiles are loaded non-temporal (a selecting step reads its pages once:
// they give way in the caches to the reused rows, scores and queries); the
// decode of kept pages, which reads the same pages again at the next step,
// loads them normally.
template <int HD, int G, bool NT = false>
struct MfmaCore {
    using Plan = MfmaPlan<HD, G>;
    static constexpr int NW = Plan::NW, KK = Plan::KK, NB = Plan::NB, VLD = Plan::VLD, LPT = Plan::LPT;
    static constexpr int VROW = Plan::VROW, VTILE = Plan::VTILE, TPS = Plan::TPS, RT = Plan::RT;

    struct Buf {
        uint4 k[TPS][KK];
        uint4 v[TPS][VLD];
        int4 rv[TPS];  // rows of tokens 4j .. 4j+3 of each tile (-1: not attended)
    };

    MfmaLds<HD, G>& sm;
    int lane, wave, r, j, vchunk;
    float sl2, slack;
    uint4 qb[KK];
    f32x4_t o[NB];
    float m_run;  // reference maximum of head r (raw q.k units)
    float l_run;  // this lane's share of head r's sum
    const uint16_t* kbase;
    const uint16_t* vbase;
    int nrows;    // entries of the row table in use

    __device__ __forceinline__ MfmaCore(MfmaLds<HD, G>& s, const Geometry& g, float scale_log2)
        : sm(s)
    {
        lane = threadIdx.x & 63;
        wave = wave_index();
        r = lane & 15;
        j = lane >> 4;
        vchunk = lane % LPT;
        sl2 = scale_log2;
        slack = kRescaleSlack / sl2;
        for (int m = 0; m < NB; ++m) o[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m_run = -INFINITY;
        l_run = 0.f;
        kbase = (const uint16_t*)g.k;
        vbase = (const uint16_t*)g.v;
        nrows = 0;
    }

    // B operand of q.k: head r, channels 32 kk + 8 j .. + 8 (heads past G are zero)
    __device__ __forceinline__ void load_queries(const void* q, long qrow0, long head_stride)
    {
        for (int kk = 0; kk < KK; ++kk) {
            qb[kk] = make_uint4(0, 0, 0, 0);
            if (r < G) qb[kk] = *(const uint4*)((const uint16_t*)q + qrow0 + r * head_stride + 32 * kk + 8 * j);
        }
    }

    // value rows: lane (r, j) loads tokens 4j + v (hd 128) or 4j + 2v + r/8 (hd 64), 16 bytes each
    __device__ __forceinline__ int vtok(int v) const { return HD == 128 ? 4 * j + v : 4 * j + 2 * v + (r >> 3); }

    __device__ __forceinline__ bool busy(int rd, int tt) const { return rd * RT + (wave * TPS + tt) * 16 < nrows; }

    // Round rd of the row table.  Every lane issues every load, so the
    // compiler can count the loads in flight and wait for one round only:
    // tokens that are not attended read row 0 instead, their logits are
    // masked to -inf and their value rows written as zeros.
    __device__ __forceinline__ void load(int rd, Buf& B) const { load(rd, B, nrows); }

    // the same with entries at or past `limit` taken as not attended
    __device__ __forceinline__ void load(int rd, Buf& B, int limit) const
    {
#pragma unroll
        for (int tt = 0; tt < TPS; ++tt) load_at(rd * RT + (wave * TPS + tt) * 16, B, tt, limit);
    }

    // the tile of table entries t0 .. t0+15 (t0 a multiple of 16) into slot tt
    __device__ __forceinline__ void load_at(int t0, Buf& B, int tt, int limit) const
    {
        const int* rows = sm.rows;
        const int4 rv = t0 + 4 * j + 3 < limit ? *(const int4*)(rows + t0 + 4 * j)
                                               : make_int4(t0 + 4 * j < limit ? rows[t0 + 4 * j] : -1,
                                                           t0 + 4 * j + 1 < limit ? rows[t0 + 4 * j + 1] : -1,
                                                           t0 + 4 * j + 2 < limit ? rows[t0 + 4 * j + 2] : -1, -1);
        B.rv[tt] = rv;
        const int rk = t0 + r < limit ? imax(rows[t0 + r], 0) : 0;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const uint16_t* kp = kbase + (long)rk * HD + 32 * kk + 8 * j;
            B.k[tt][kk] = NT ? ld_stream(kp) : *(const uint4*)kp;
        }
        const int rows4[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
        for (int v = 0; v < VLD; ++v) {
            const int rr = imax(rows4[HD == 128 ? v : 2 * v + (r >> 3)], 0);
            const uint16_t* vp = vbase + (long)rr * HD + 8 * vchunk;
            B.v[tt][v] = NT ? ld_stream(vp) : *(const uint4*)vp;
        }
    }

    __device__ __forceinline__ void compute(const Buf& B, int tt)
    {
        unsigned char* const vt = sm.tiles + (wave * TPS + tt) * VTILE;  // this wave's value tile
        // q.k
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, B.k[tt][kk]),
                                                        __builtin_bit_cast(bf16x8_t, qb[kk]), s, 0, 0, 0);
        const int4 rv = B.rv[tt];
        const float z[4] = {rv.x >= 0 ? s[0] : -INFINITY, rv.y >= 0 ? s[1] : -INFINITY,
                            rv.z >= 0 ? s[2] : -INFINITY, rv.w >= 0 ? s[3] : -INFINITY};
        // values to LDS as loaded (zeros for tokens that are not attended;
        // selected per component: a select of whole vectors would keep the
        // buffers out of registers)
        const int rows4[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
        for (int v = 0; v < VLD; ++v) {
            const bool ok = rows4[HD == 128 ? v : 2 * v + (r >> 3)] >= 0;
            const uint4 w = B.v[tt][v];
            *(uint4*)(vt + vt_off<VROW>(vtok(v), 16 * vchunk)) =
                make_uint4(ok ? w.x : 0u, ok ? w.y : 0u, ok ? w.z : 0u, ok ? w.w : 0u);
        }
        // softmax: tile maximum of head r over the 4 lanes holding it
        float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
        mx = fmaxf(mx, xor_lanes<16>(mx));
        mx = fmaxf(mx, xor_lanes<32>(mx));
        const bool need = r < G && mx > m_run + slack;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            const float mn = need ? mx : m_run;
            const float alpha = need ? __builtin_amdgcn_exp2f((m_run - mn) * sl2) : 1.f;  // 0 while m = -inf
            l_run *= alpha;
            m_run = mn;
            // accumulator rows are heads 4j + i: fetch their factors
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(alpha, 4 * j + i);
#pragma unroll
                for (int m = 0; m < NB; ++m) o[m][i] *= ai;
            }
        }
        const float mref = m_run == -INFINITY ? 0.f : -m_run * sl2;
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = __builtin_amdgcn_exp2f(fmaf(z[i], sl2, mref));  // -inf -> 0
            l_run += p[i];
        }
        const uint2 pw = make_uint2(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]));
        const i16x4_t pa = __builtin_bit_cast(i16x4_t, pw);
        __builtin_amdgcn_wave_barrier();
        // p.v, 16 channels per product; B operand = values of tokens 4j .. 4j+3 at channel 16m + r
        const unsigned char* vcol = vt + 2 * r;
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            i16x4_t vb;
#pragma unroll
            for (int i = 0; i < 4; ++i) vb[i] = *(const short*)(vcol + vt_off<VROW>(4 * j + i, 32 * m));
            o[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, o[m], 0, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
    }

    // All rounds of the row table, three in flight per wave; the first
    // `loaded` rounds (0 .. 3) may already be loaded into A, B, C.
    // Rounds of the row table, three in flight.  Every step issues its
    // loads (rounds past the end read row 0, masked, from one cached line)
    // and the loop leaves only at the end of a round of three, so the waits
    // count one round each (conditional loads or an exit inside the round
    // made the compiler wait for every load in flight).
    __device__ __forceinline__ void run(Buf& A, Buf& B, Buf& C, int loaded)
    {
        const int nr = (nrows + RT - 1) / RT;
        if (loaded < 1) load(0, A);
        if (loaded < 2) load(1, B);
        if (loaded < 3) load(2, C);
        for (int rd = 0; rd < nr; rd += 3) {
#pragma unroll
            for (int tt = 0; tt < TPS; ++tt)
                if (busy(rd, tt)) compute(A, tt);
            load(rd + 3, A);
#pragma unroll
            for (int tt = 0; tt < TPS; ++tt)
                if (busy(rd + 1, tt)) compute(B, tt);
            load(rd + 4, B);
#pragma unroll
            for (int tt = 0; tt < TPS; ++tt)
                if (busy(rd + 2, tt)) compute(C, tt);
            load(rd + 5, C);
        }
    }

    // The waves' states go to LDS (the output area reuses the value tiles, so
    // every wave first leaves its loop); the workgroup merges them with one
    // exponential per (wave, head) and writes the partial of its G heads:
    // part_o / part_ml rows prow0 + h * prow_step, slot `slot`.
    // coherent: agent-scope stores, for the kernel's own last workgroup to merge
    __device__ __forceinline__ void finish(float* part_o, float* part_ml, long prow0, long prow_step, int stride,
                                           int slot, bool failed = false, bool coherent = false)
    {
        // head r's sum over the 4 lanes holding it
        l_run += xor_lanes<16>(l_run);
        l_run += xor_lanes<32>(l_run);
        lds_barrier();  // the tile loads past the last tile are not waited for
        float* const wv_o = (float*)sm.tiles;  // [NW][G][HD]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = 4 * j + i;
            if (h < G) {
#pragma unroll
                for (int m = 0; m < NB; ++m) wv_o[(wave * G + h) * HD + 16 * m + r] = o[m][i];
            }
        }
        if (j == 0 && r < G) {
            sm.wv_m[wave][r] = m_run * sl2;  // -inf stays -inf
            sm.wv_l[wave][r] = l_run;
        }
        lds_barrier();
        for (int i = threadIdx.x; i < G * HD / 4; i += 64 * NW) {
            const int h = i / (HD / 4), c4 = i % (HD / 4);
            float ms = -INFINITY;
            for (int w = 0; w < NW; ++w) ms = fmaxf(ms, sm.wv_m[w][h]);
            float ls = 0.f;
            float4 os = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int w = 0; w < NW; ++w) {
                const float mw = sm.wv_m[w][h];
                const float wt = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - ms);
                ls = fmaf(sm.wv_l[w][h], wt, ls);
                const float4 ow = *(const float4*)(wv_o + (w * G + h) * HD + 4 * c4);
                os.x = fmaf(ow.x, wt, os.x);
                os.y = fmaf(ow.y, wt, os.y);
                os.z = fmaf(ow.z, wt, os.z);
                os.w = fmaf(ow.w, wt, os.w);
            }
            float inv = ls > 0.f ? 1.0f / ls : 0.f;
            float mo = ls > 0.f ? ms * kLn2 : -INFINITY;
            if (failed) {  // a share was left out: NaN partial, which poisons the row in the combine
                inv = __builtin_nanf("");
                mo = inv;
                ls = inv;
            }
            const long prow = (prow0 + h * prow_step) * stride + slot;
            const float4 ov = make_float4(os.x * inv, os.y * inv, os.z * inv, os.w * inv);
            float* po = part_o + prow * HD + c4 * 4;
            if (coherent) {
                __hip_atomic_store(po + 0, ov.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(po + 1, ov.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(po + 2, ov.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(po + 3, ov.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (c4 == 0) {
                    __hip_atomic_store(part_ml + prow * 2 + 0, mo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(part_ml + prow * 2 + 1, ls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            } else {
                *(float4*)po = ov;
                if (c4 == 0) {
                    part_ml[prow * 2 + 0] = mo;
                    part_ml[prow * 2 + 1] = ls;
                }
            }
        }
    }
};

// The merge of a (sequence b, KV head, row) problem's split partials by the
// last of its `splits` workgroups to finish (MergeArgs): every workgroup
// waits for its own agent-scope partial stores to complete, then counts
// itself in; the last one merges the problem's G output rows, a wave per
// row, with agent-scope loads (merge_row, the combine kernel's arithmetic),
// and clears the counter.  The last problem of a sequence to merge advances
// its length: by then no workgroup of the launch reads it any more.
template <int HD, int G, int NW>
__device__ __forceinline__ void merge_tail(const MergeArgs& m, long prob, int b, int splits, int stride, long prow0,
                                           long prow_step, const float* part_o, const float* part_ml,
                                           int probs_per_batch)
{
    __shared__ int s_last;
    __shared__ float wts[NW][kMergeMaxSplits];
    __shared__ short later[NW][kMergeMaxSplits];
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(m.arrive + prob, 1u) == (unsigned)(splits - 1) ? 1 : 0;
    __syncthreads();
    if (!s_last) return;
    const int wave = threadIdx.x >> 6;
    for (int h = wave; h < G; h += NW) {
        const long prow = prow0 + h * prow_step;
        merge_row<HD, true>(part_ml + prow * stride * 2, part_o + prow * stride * HD, splits, wts[wave], later[wave],
                            m.out_dtype == 1, m.out, m.lse, prow);
    }
    if (threadIdx.x == 0) {
        __hip_atomic_store(m.arrive + prob, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (m.seq_lens && m.advance != 0 && atomicAdd(m.batch_done + b, 1u) == (unsigned)(probs_per_batch - 1)) {
            __hip_atomic_store(m.batch_done + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            m.seq_lens[b] += m.advance;
        }
    }
}

// Row index ((phys * Hkv + kvh) * P + offset) of token t, or -1 when t is past
// the row's position or its page is unmapped.
__device__ __forceinline__ int token_row(int t, int pos, int phys, const Geometry& g, int kvh, const FastDiv& pdiv)
{
    if (t < 0 || t > pos || phys < 0 || phys >= g.num_phys) return -1;
    const int pg = pdiv.div(t);
    return phys * (g.Hkv * g.P) + kvh * g.P + (t - pg * g.P);
}

// Resolves table entries [first, first + cnt) from tokens tok(i), i = 0 ..
// cnt-1, with all block-table loads of a thread in flight together.
template <int NW, typename Tok>
__device__ __forceinline__ void resolve_rows(int* rows, int first, int cnt, Tok tok, int pos, const int32_t* bt,
                                             const Geometry& g, int kvh, const FastDiv& pdiv)
{
    constexpr int PER_T = kRowsWG / (64 * NW);
    int tk[PER_T], ph[PER_T];
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
        const int i = u * 64 * NW + (int)threadIdx.x;
        const int t = i < cnt ? tok(i) : -1;
        tk[u] = t;
        ph[u] = t >= 0 && t <= pos ? bt[pdiv.div(t)] : -1;
    }
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
        const int i = u * 64 * NW + (int)threadIdx.x;
        if (i < cnt) rows[first + i] = token_row(tk[u], pos, ph[u], g, kvh, pdiv);
    }
}

template <int HD, int G>
__global__ __launch_bounds__((64 * MfmaPlan<HD, G>::NW)) void k_decode_mfma(DecodeArgs a)
{
    using Core = MfmaCore<HD, G>;
    constexpr int NW = Core::NW;
    const Geometry& g = a.g;
    __shared__ int sel_lds[kSelCap];
    __shared__ MfmaLds<HD, G> lds;

    int bid = blockIdx.x;
    const int split = bid % a.splits;
    bid /= a.splits;
    const int kvh = bid % g.Hkv;
    bid /= g.Hkv;
    const int row = bid % a.Q;
    const int b = bid / a.Q;
    const long prob = ((long)b * g.Hkv + kvh) * a.Q + row;

    // one round of loads: length, count, page list, the group's queries
    const int L = imax(0, imin(g.seq_lens[b], g.max_pages * g.P));
    const int count = a.sel ? a.count[prob] : 0;
    const int32_t* sel_g = a.sel ? a.sel + prob * a.k_max : nullptr;
    const bool staged = sel_g != nullptr && a.k_max <= kSelCap;
    if (staged)
        for (int i = threadIdx.x; i < a.k_max; i += 64 * NW) sel_lds[i] = sel_g[i];
    Core core(lds, g, a.scale_log2);
    core.load_queries(a.q, (((long)b * g.Hq + kvh * G) * a.Q + row) * HD, (long)a.Q * HD);
    __syncthreads();

    const int pos = L - a.Q + row;
    // the token map reads the page list from LDS when it is staged there
    TokenSetLds tsl;
    TokenSet tsg;
    tsl.init(L, a.S, a.W, g.P, (lds_i32_ptr)sel_lds, staged ? count : 0, a.k_max, a.parts);
    tsg.init(L, a.S, a.W, g.P, staged ? nullptr : sel_g, count, a.k_max, a.parts);
    const FastDiv pdiv{g.pdiv.d, g.pdiv.magic, g.pdiv.shift};
    const int n = staged ? tsl.total : tsg.total;
    const int f0 = split * (n / a.splits) + imin(split, n % a.splits);
    const int f1 = f0 + n / a.splits + (split < n % a.splits ? 1 : 0);
    const int32_t* bt = g.block_table + (long)b * g.max_pages;

    typename Core::Buf A, B, C;
    for (int cb = f0; cb < f1; cb += kRowsWG) {
        const int cnt = imin(f1 - cb, kRowsWG);
        __syncthreads();  // the previous chunk's rows are no longer read
        resolve_rows<NW>(lds.rows, 0, cnt,
                         [&](int i) { return staged ? tsl.position(cb + i, pdiv) : tsg.position(cb + i, pdiv); },
                         pos, bt, g, kvh, pdiv);
        __syncthreads();
        core.nrows = cnt;
        core.run(A, B, C, 0);
    }
    const long prow0 = ((long)b * g.Hq + kvh * G) * a.Q + row;
    core.finish(a.part_o, a.part_ml, prow0, a.Q, a.split_stride, split, false, a.m.out != nullptr);
    if (a.m.out)
        merge_tail<HD, G, NW>(a.m, prob, b, a.splits, a.split_stride, prow0, a.Q, a.part_o, a.part_ml,
                              g.Hkv * a.Q);
}

// Selection and decode in one kernel, for the steps that select.  Every
// workgroup of a (sequence, KV head, row) stages the problem's block-table
// row and page scores in LDS; after that one barrier its waves part.  The
// last wave ranks the pages alone (radix select in one wave), emits the
// ascending page list and publishes it through an LDS flag, while the other
// waves stream the workgroup's share of the sink and window tokens.  Each
// wave then resolves the rows of its own tiles of the selected pages'
// middle tokens and streams them, so no workgroup barrier stands between
// the two shares and the K/V loads keep going while the pages are ranked.
// The workgroup of split 0 also writes the page list and its count.

template <int HD, int G>
__global__ __launch_bounds__((64 * MfmaPlan<HD, G>::NW)) void k_select_decode_mfma(SelectDecodeArgs a)
{
    using Core = MfmaCore<HD, G, true>;
    constexpr int NW = Core::NW;
    constexpr int SW = NW - 1;  // the wave that ranks the pages
    static_assert(Core::TPS == 1, "one tile per wave step");
    static_assert(kFusedMaxCand % 4 == 0 && kFusedMaxCand <= kTopkThreads * kTopkMaxRounds,
                  "the wave top-k reads the keys four at a time and marks them in its bitmap");
    const Geometry& g = a.g;
    __shared__ __attribute__((aligned(16))) uint32_t keys[kFusedMaxCand];
    __shared__ int bt_lds[kFusedMaxCand];
    __shared__ WaveTopkScratch tk;
    __shared__ uint32_t key_range[NW][2];
    __shared__ int sel_lds[kSelCap];
    __shared__ int sel_ready;
    __shared__ int s_failed;  // some wave gave up its wait for the page list
    __shared__ MfmaLds<HD, G> lds;

    int bid = blockIdx.x;
    const int split = bid % a.splits;
    bid /= a.splits;
    const int kvh = bid % g.Hkv;
    bid /= g.Hkv;
    const int row = bid % a.Q;
    const int b = bid / a.Q;
    const long prob = ((long)b * g.Hkv + kvh) * a.Q + row;

    // The first loads do not depend on the sequence length, so they go out
    // with it at entry: the first 2048 entries of the block-table row and of
    // the score row, one 16-byte load each per thread (the host passes
    // 16-byte aligned rows).  Quads past a row's end re-read its last quad
    // and are masked when staged.
    const int32_t* bt_g = g.block_table + (long)b * g.max_pages;
    const float* srow = a.scores + prob * g.max_pages;  // scores of logical pages, candidates from plo
    const int e0 = 4 * (int)threadIdx.x;
    const int ec = imin(e0, g.max_pages - 4);
    const int4 bv = *(const int4*)(bt_g + ec);
    const uint4 sv = *(const uint4*)(srow + ec);

    const int L = imax(0, imin(g.seq_lens[b], g.max_pages * g.P));
    const int pos = L - a.Q + row;
    const int se = imin(a.S, L), ws = imax(se, L - a.W);
    const int plo = se / g.P;
    const int ncand = ws > se ? (ws - 1) / g.P - plo + 1 : 0;
    const int k = imin(a.k_max, ncand);
    Core core(lds, g, a.scale_log2);
    core.load_queries(a.q, (((long)b * g.Hq + kvh * G) * a.Q + row) * HD, (long)a.Q * HD);
    const FastDiv pdiv{g.pdiv.d, g.pdiv.magic, g.pdiv.shift};
    const int lane = threadIdx.x & 63, wave = wave_index();

    // this workgroup's share of the sink and window tokens, first in its
    // table; the middle share starts at the next multiple of 16
    const int nloc = se + (L - ws);
    const int l0 = split * (nloc / a.splits) + imin(split, nloc % a.splits);
    const int nl = nloc / a.splits + (split < nloc % a.splits ? 1 : 0);
    const int nlp = (nl + 15) & ~15;
    auto local_tok = [&](int i) { const int f = l0 + i; return f < se ? f : ws + (f - se); };

    // the block-table row into LDS and the candidates' scores as order keys
    const int npg = imin(g.max_pages, (L + g.P - 1) / g.P);
    const bool rank = k > 0 && k < ncand;
    const int nsc = rank ? plo + ncand : 0;  // score row entries needed
    uint32_t lo = 0xffffffffu, hi = 0;
    auto stage = [&](int e, int btv, float scv) {  // entry e of both rows
        if (e < npg) bt_lds[e] = btv;
        const int i = e - plo;  // candidate index
        if (rank && i >= 0 && i < ncand) {
            const uint32_t key = order_key(scv);
            keys[i] = key;
            lo = min(lo, key);
            hi = max(hi, key);
        }
    };
    stage(e0, bv.x, __uint_as_float(sv.x));
    stage(e0 + 1, bv.y, __uint_as_float(sv.y));
    stage(e0 + 2, bv.z, __uint_as_float(sv.z));
    stage(e0 + 3, bv.w, __uint_as_float(sv.w));
    const int span = imax(npg, nsc);
    for (int e = 4 * 64 * NW + (int)threadIdx.x; e < span; e += 64 * NW)  // longer sequences
        stage(e, e < npg ? bt_g[e] : -1, e < nsc ? srow[e] : 0.f);
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (lane == 0) {
        key_range[wave][0] = lo;
        key_range[wave][1] = hi;
    }
    if (threadIdx.x == 0) {
        sel_ready = 0;
        s_failed = 0;
    }
    __syncthreads();
    const int32_t* bt = bt_lds;

    // Tiles of this wave: local tiles wave, wave + NL, ... (the ranking wave
    // has none), then middle tiles wave, wave + NW, ...  The middle ones
    // become known when the page list is published.
    constexpr int NL = NW - 1;                      // waves that stream the local share
    constexpr int kMidTilesW = kRowsWG / 16 / NW;  // most middle tiles of a wave
    const int nloc_w = wave == SW ? 0 : imax(0, (nlp / 16 - wave + NL - 1) / NL);
    int nt = nloc_w, nm = 0, next = 0;  // tiles known, middle entries, next tile to load
    bool have_mid = false;
    // Takes the page list once the ranking wave has published it (never
    // waits): this wave's middle tiles and their rows, four tiles per step.
    auto poll = [&]() {
        if (have_mid || __hip_atomic_load(&sel_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0) return;
        TokenSetLds tsm;
        tsm.init(L, a.S, a.W, g.P, (lds_i32_ptr)sel_lds, k, a.k_max, kPartMiddle);
        const int nmid = tsm.total;
        const int m0 = split * (nmid / a.splits) + imin(split, nmid % a.splits);
        nm = nmid / a.splits + (split < nmid % a.splits ? 1 : 0);
        const int nmid_w = imax(0, ((nm + 15) / 16 - wave + NW - 1) / NW);
#pragma unroll
        for (int q = 0; q < kMidTilesW; q += 4) {
            const int tq = q + (lane >> 4);
            const int e = 16 * (wave + NW * tq) + (lane & 15);  // entry of the middle share
            if (tq < nmid_w && e < nm) {
                const int t = tsm.position(m0 + e, pdiv);
                lds.rows[nlp + e] = token_row(t, pos, t >= 0 && t <= pos ? bt[pdiv.div(t)] : -1, g, kvh, pdiv);
            }
        }
        __builtin_amdgcn_wave_barrier();
        nt = nloc_w + nmid_w;
        have_mid = true;
    };
    // Loads the next tile into X and returns true, or, when none is known
    // yet or left, loads row 0 masked and returns false: every step issues
    // the same loads, so the waits count one tile each.
    auto issue = [&](typename Core::Buf& X) {
        const bool real = next < nt;
        const bool loc = next < nloc_w;
        const int t0 = loc ? 16 * (wave + NL * next) : 16 * (wave + NW * (next - nloc_w)) + nlp;
        core.load_at(real ? t0 : 0, X, 0, real ? (loc ? nlp : nlp + nm) : 0);
        next += real ? 1 : 0;
        return real;
    };
    // The rows of this wave's local tiles (padding entries are not
    // attended), four tiles per step; the first three tiles' loads go out
    // after the first step.
    auto resolve_local = [&](int q0) {
        const int tq = q0 + (lane >> 4);
        if (tq < nloc_w) {
            const int e = 16 * (wave + NL * tq) + (lane & 15);
            const int t = e < nl ? local_tok(e) : -1;
            lds.rows[e] = token_row(t, pos, t >= 0 && t <= pos ? bt[pdiv.div(t)] : -1, g, kvh, pdiv);
        }
        __builtin_amdgcn_wave_barrier();
    };
    resolve_local(0);

    if (wave == SW) {  // the ranking, while the other waves stream
        auto emit = [&](int p, int i) { sel_lds[p] = plo + i; };
        uint32_t klo = 0xffffffffu, khi = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            klo = min(klo, key_range[w][0]);
            khi = max(khi, key_range[w][1]);
        }
        if (!rank || klo == khi) {  // the list is the lowest k candidates
            for (int i = lane; i < k; i += 64) emit(i, i);
        } else {
            wave_topk(ncand, k, keys, klo, khi, tk, emit);
        }
        __builtin_amdgcn_wave_barrier();
        if (split == 0) {
            int32_t* sel_g = a.sel + prob * a.k_max;
            for (int i = lane; i < a.k_max; i += 64) sel_g[i] = i < k ? sel_lds[i] : -1;
            if (lane == 0) a.count[prob] = k;
        }
        __hip_atomic_store(&sel_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }

    // Three tiles in flight per wave.  Real tiles are computed in tile order
    // whatever the timing of the page list, so results do not depend on it.
    typename Core::Buf A, B, C;
    poll();
    bool ra = issue(A), rb = issue(B), rc = issue(C);
    for (int q0 = 4; q0 < nloc_w; q0 += 4) resolve_local(q0);
    // The only exit is at the end of a round of three, where the loads in
    // flight are in the same order as on the way round, so the waits inside
    // the loop stay at one tile each.
    // The wait for the page list is bounded (its publisher is a wave of this
    // workgroup, so it ends long before the bound); a wave that reaches the
    // bound leaves its share undone, and the workgroup then writes NaN
    // partials and sets the status word instead of a wrong result.
    bool done = false;
    for (int step = 0; step < a.spin_max; ++step) {
        if (!have_mid && next >= nloc_w) poll();
        if (ra) core.compute(A, 0);
        ra = issue(A);
        if (rb) core.compute(B, 0);
        rb = issue(B);
        if (rc) core.compute(C, 0);
        rc = issue(C);
        if (!ra && !rb && !rc) {
            if (have_mid && next >= nt) {
                done = true;
                break;
            }
            __builtin_amdgcn_s_sleep(2);  // waiting for the page list
        }
    }
    if (!done) s_failed = 1;
    lds_barrier();  // (the masked loads of the last round are not waited for)
    const bool failed = s_failed != 0;
    if (failed && threadIdx.x == 0 && a.status) __hip_atomic_store(a.status, kStatusGaveUp, __ATOMIC_RELAXED,
                                                                   __HIP_MEMORY_SCOPE_AGENT);
    const long prow0 = ((long)b * g.Hq + kvh * G) * a.Q + row;
    core.finish(a.part_o, a.part_ml, prow0, a.Q, a.split_stride, split, failed, a.m.out != nullptr);
    if (a.m.out)
        merge_tail<HD, G, NW>(a.m, prob, b, a.splits, a.split_stride, prow0, a.Q, a.part_o, a.part_ml,
                              g.Hkv * a.Q);
}

template <int HD, int G>
hipError_t launch_bf16(const DecodeArgs& a, dim3 grid, hipStream_t s)
{
    hipLaunchKernelGGL((k_decode_mfma<HD, G>), grid, dim3(64 * MfmaPlan<HD, G>::NW), 0, s, a);
    return hipGetLastError();
}

template <int HD, int G>
int bf16_wgs_per_cu()
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_decode_mfma<HD, G>, 64 * MfmaPlan<HD, G>::NW, 0) !=
        hipSuccess)
        return 1;
    return n > 0 ? n : 1;
}

template <int HD, bool BF>
hipError_t launch_g(const DecodeArgs& a, dim3 grid, hipStream_t s)
{
    if constexpr (BF) {
        switch (a.g.G) {
        case 1: return launch_bf16<HD, 1>(a, grid, s);
        case 2: return launch_bf16<HD, 2>(a, grid, s);
        case 4: return launch_bf16<HD, 4>(a, grid, s);
        case 8: return launch_bf16<HD, 8>(a, grid, s);
        case 16: return launch_bf16<HD, 16>(a, grid, s);
        default: return hipErrorInvalidValue;
        }
    } else {
        const dim3 block(64 * kWaves);
        switch (a.g.G) {
        case 1: hipLaunchKernelGGL((k_decode_generic<HD, 1, BF>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((k_decode_generic<HD, 2, BF>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((k_decode_generic<HD, 4, BF>), grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL((k_decode_generic<HD, 8, BF>), grid, block, 0, s, a); break;
        case 16: hipLaunchKernelGGL((k_decode_generic<HD, 16, BF>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

template <int HD, int G>
hipError_t launch_sd(const SelectDecodeArgs& a, dim3 grid, hipStream_t s)
{
    hipLaunchKernelGGL((k_select_decode_mfma<HD, G>), grid, dim3(64 * MfmaPlan<HD, G>::NW), 0, s, a);
    return hipGetLastError();
}

template <int HD>
hipError_t launch_sd_g(const SelectDecodeArgs& a, dim3 grid, hipStream_t s)
{
    switch (a.g.G) {
    case 1: return launch_sd<HD, 1>(a, grid, s);
    case 2: return launch_sd<HD, 2>(a, grid, s);
    case 4: return launch_sd<HD, 4>(a, grid, s);
    case 8: return launch_sd<HD, 8>(a, grid, s);
    case 16: return launch_sd<HD, 16>(a, grid, s);
    default: return hipErrorInvalidValue;
    }
}

template <int HD>
int wgs_per_cu_g(int G)
{
    switch (G) {
    case 1: return bf16_wgs_per_cu<HD, 1>();
    case 2: return bf16_wgs_per_cu<HD, 2>();
    case 4: return bf16_wgs_per_cu<HD, 4>();
    case 8: return bf16_wgs_per_cu<HD, 8>();
    case 16: return bf16_wgs_per_cu<HD, 16>();
    default: return 1;
    }
}

}  // namespace

int decode_wgs_per_cu(int hd, int G, int dtype)
{
    if (dtype != 1) return 2;  // the fp32 kernel: 4 waves, two workgroups per CU
    return hd == 128 ? wgs_per_cu_g<128>(G) : wgs_per_cu_g<64>(G);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s)
{
    const long wgs = (long)a.g.B * a.g.Hkv * a.Q * a.splits;
    const dim3 grid((unsigned)wgs);
    const bool bf = a.g.dtype == 1;
    if (a.g.hd == 128) return bf ? launch_g<128, true>(a, grid, s) : launch_g<128, false>(a, grid, s);
    if (a.g.hd == 64) return bf ? launch_g<64, true>(a, grid, s) : launch_g<64, false>(a, grid, s);
    return hipErrorInvalidValue;
}

hipError_t launch_select_decode(const SelectDecodeArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)((long)a.g.B * a.g.Hkv * a.Q * a.splits));
    if (a.g.dtype != 1) return hipErrorInvalidValue;
    if (a.g.hd == 128) return launch_sd_g<128>(a, grid, s);
    if (a.g.hd == 64) return launch_sd_g<64>(a, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace sa
