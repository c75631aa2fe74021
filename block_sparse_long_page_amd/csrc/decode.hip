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

namespace sa {

namespace {

#ifndef SA_DECODE_U
#define SA_DECODE_U 4
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

// ---------------------------------------------------------------------------
// bf16 kernel.  Same work split as k_decode_generic; per wave:
//  * prologue: the row index ((phys * Hkv + kvh) * P + offset) of each token
//    of the wave's range is resolved once into LDS, so the K/V loads of the
//    main loop never wait on the page list or the block table;
//  * main loop: K/V rows double-buffered in registers (the next U token steps
//    are in flight while the current ones are computed);
//  * q.k: packed bf16 dot products, then a DPP reduce-scatter over the LPT
//    lanes of a token, after which each lane holds the full sum of its own
//    head(s): the exponentials are computed once per (token, head);
//  * p.v: the weights of two tokens are packed as a bf16 pair, broadcast from
//    the lane holding each head, and accumulated with dot2 into fp32.
// ---------------------------------------------------------------------------

template <int HD, int G>
__global__ __launch_bounds__(64 * kWaves) void k_decode_bf16(DecodeArgs a)
{
    constexpr int CH = 8;                  // bf16 channels per lane (one 16-byte load)
    constexpr int LPT = HD / CH;           // lanes per token: 16 (hd 128) or 8 (hd 64)
    constexpr int TPW = 64 / LPT;          // tokens per wave load
    constexpr int U = SA_DECODE_U;         // token steps per buffer (even)
    constexpr int HPL = G > LPT ? G / LPT : 1;  // heads held per lane after the reduce-scatter
    constexpr int DUP = G < LPT ? LPT / G : 1;  // lanes holding the same head
    constexpr int CHUNK = 256;             // tokens resolved per prologue
    static_assert(U % 2 == 0, "tokens are paired for dot2");
    const Geometry& g = a.g;

    constexpr int NGRP = kWaves * TPW;     // token groups of the workgroup, each with its own softmax state
    // q.k partial sums are transposed through LDS when every head's sum fits
    // in one lane group (G <= LPT); rows padded so the writes avoid bank conflicts
    constexpr bool XPOSE = G <= LPT;
    constexpr int XSTRIDE = G * LPT + LPT;
    constexpr int XFLOATS = XPOSE ? kWaves * U * TPW * XSTRIDE : 1;
    constexpr int OFLOATS = NGRP * G * HD;
    __shared__ int rows_lds[kWaves][CHUNK];
    __shared__ float4 smem4[(XFLOATS > OFLOATS ? XFLOATS : OFLOATS) / 4];  // transpose area, then group outputs
    __shared__ float grp_m[NGRP][G], grp_l[NGRP][G];
    float* const xsum = (float*)smem4;
    float4 (*const grp_o)[G][HD / 4] = (float4(*)[G][HD / 4])smem4;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPT, tg = lane / LPT;
    const int head0 = (sub / DUP) * HPL;   // first head this lane holds after the reduce-scatter

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

    const int n = ts.total;
    const int f0 = split * (n / a.splits) + imin(split, n % a.splits);
    const int f1 = f0 + n / a.splits + (split < n % a.splits ? 1 : 0);
    const int len = f1 - f0;
    const int w0 = f0 + wave * (len / kWaves) + imin(wave, len % kWaves);
    const int w1 = w0 + len / kWaves + (wave < len % kWaves ? 1 : 0);

    uint32_t qw[G][4];
    for (int h = 0; h < G; ++h) {
        const uint4 w = *(const uint4*)((const uint16_t*)a.q + (((long)b * g.Hq + kvh * G + h) * a.Q + row) * HD +
                                        sub * CH);
        qw[h][0] = w.x;
        qw[h][1] = w.y;
        qw[h][2] = w.z;
        qw[h][3] = w.w;
    }

    float m_all[G], o[G][CH];
    float m_own[HPL], l_own[HPL];
    for (int h = 0; h < G; ++h) {
        m_all[h] = -INFINITY;
        for (int c = 0; c < CH; ++c) o[h][c] = 0.f;
    }
    for (int j = 0; j < HPL; ++j) {
        m_own[j] = -INFINITY;
        l_own[j] = 0.f;
    }

    const uint16_t* kbase = (const uint16_t*)g.k + sub * CH;
    const uint16_t* vbase = (const uint16_t*)g.v + sub * CH;
    const int32_t* bt = g.block_table + (long)b * g.max_pages;
    const int hkvP = g.Hkv * g.P;
    // logits are kept as raw q.k; the softmax scale (times log2 e) is applied
    // inside the exponentials, and the rescale slack is 2^8 in weight
    const float sl2 = a.scale_log2;
    const float slack = kRescaleSlack / sl2;

    for (int cb = w0; cb < w1; cb += CHUNK) {
        const int ce = imin(w1, cb + CHUNK);
        for (int f = cb + lane; f < ce; f += 64) {
            int t = ts.position(f, pdiv);
            int ri = -1;
            if (t >= 0 && t <= pos) {
                const int pg = pdiv.div(t);
                const int phys = bt[pg];
                if (phys >= 0 && phys < g.num_phys) ri = phys * hkvP + kvh * g.P + (t - pg * g.P);
            }
            rows_lds[wave][f - cb] = ri;
        }
        __builtin_amdgcn_wave_barrier();

        const int nst = (ce - cb + TPW * U - 1) / (TPW * U);

        // Rows of tokens that are not attended are not loaded: their
        // registers keep earlier (finite) data, and their weight is 0.
        auto load = [&](int s, uint4(&kw)[U], uint4(&vw)[U], int(&ri)[U]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = s * (TPW * U) + u * TPW + tg;
                ri[u] = cb + j < ce ? rows_lds[wave][j] : -1;
                if (ri[u] >= 0) {
                    kw[u] = *(const uint4*)(kbase + (long)ri[u] * HD);
                    vw[u] = *(const uint4*)(vbase + (long)ri[u] * HD);
                }
            }
        };

        auto compute = [&](const uint4(&kw)[U], const uint4(&vw)[U], const int(&ri)[U]) {
            float z[U][HPL];
            if constexpr (XPOSE) {
                // each lane writes its partial sums [head][lane-in-group]; the DUP
                // lanes holding a head then add that head's row and share the total
                constexpr int PER = LPT / DUP;  // partials each of them adds
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t* k32 = (const uint32_t*)&kw[u];
                    float* xs = xsum + ((wave * U + u) * TPW + tg) * XSTRIDE;
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        float acc = 0.f;
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc = dot2_bf16(qw[h][j], k32[j], acc);
                        xs[h * LPT + sub] = acc;
                    }
                }
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float* xs = xsum + ((wave * U + u) * TPW + tg) * XSTRIDE + head0 * LPT + (sub % DUP) * PER;
                    float acc = 0.f;
                    if constexpr (PER % 4 == 0) {
#pragma unroll
                        for (int v = 0; v < PER; v += 4) {
                            const float4 t = *(const float4*)(xs + v);
                            acc += (t.x + t.y) + (t.z + t.w);
                        }
                    } else {
#pragma unroll
                        for (int v = 0; v < PER; ++v) acc += xs[v];
                    }
                    acc = group_sum<DUP>(acc);
                    z[u][0] = ri[u] >= 0 ? acc : -INFINITY;  // unscaled q.k
                }
                __builtin_amdgcn_wave_barrier();
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t* k32 = (const uint32_t*)&kw[u];
                    float d[G];
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        float acc = 0.f;
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc = dot2_bf16(qw[h][j], k32[j], acc);
                        d[h] = acc;
                    }
                    reduce_scatter<G, log2c<LPT>() - 1>(d, lane);
#pragma unroll
                    for (int j = 0; j < HPL; ++j) z[u][j] = ri[u] >= 0 ? d[j] : -INFINITY;  // unscaled q.k
                }
            }
            // reference maximum (unscaled q.k units): rescale only when a logit
            // passes it by more than the slack
            bool need = false;
            float mx[HPL];
#pragma unroll
            for (int j = 0; j < HPL; ++j) {
                mx[j] = z[0][j];
#pragma unroll
                for (int u = 1; u < U; ++u) mx[j] = fmaxf(mx[j], z[u][j]);
                need |= mx[j] > m_own[j] + slack;
            }
            if (__builtin_amdgcn_ballot_w64(need) != 0) {
                static_for<0, G>([&](auto hc) {
                    constexpr int h = decltype(hc)::value;
                    const float mh = group_bcast<LPT, (h / HPL) * DUP>(mx[h % HPL], lane);
                    if (mh > m_all[h] + slack) {
                        const float alpha = __builtin_amdgcn_exp2f((m_all[h] - mh) * sl2);  // 0 while m = -inf
#pragma unroll
                        for (int c = 0; c < CH; ++c) o[h][c] *= alpha;
#pragma unroll
                        for (int j = 0; j < HPL; ++j)
                            if (head0 + j == h) {
                                l_own[j] *= alpha;
                                m_own[j] = mh;
                            }
                        m_all[h] = mh;
                    }
                });
            }
            float p[U][HPL];
#pragma unroll
            for (int j = 0; j < HPL; ++j) {
                const float mref = m_own[j] == -INFINITY ? 0.f : -m_own[j] * sl2;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    p[u][j] = __builtin_amdgcn_exp2f(fmaf(z[u][j], sl2, mref));  // -inf -> 0
                    l_own[j] += p[u][j];
                }
            }
#pragma unroll
            for (int u = 0; u < U; u += 2) {
                const uint32_t* va = (const uint32_t*)&vw[u];
                const uint32_t* vb = (const uint32_t*)&vw[u + 1];
                uint32_t vv[CH];  // channel c of tokens u and u+1 as a bf16 pair
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    vv[2 * j] = __builtin_amdgcn_perm(vb[j], va[j], 0x05040100u);      // low halves
                    vv[2 * j + 1] = __builtin_amdgcn_perm(vb[j], va[j], 0x07060302u);  // high halves
                }
                float pk[HPL];
#pragma unroll
                for (int j = 0; j < HPL; ++j) pk[j] = __uint_as_float(pack_bf16(p[u][j], p[u + 1][j]));
                static_for<0, G>([&](auto hc) {
                    constexpr int h = decltype(hc)::value;
                    const uint32_t pp = __float_as_uint(group_bcast<LPT, (h / HPL) * DUP>(pk[h % HPL], lane));
#pragma unroll
                    for (int c = 0; c < CH; ++c) o[h][c] = dot2_bf16(pp, vv[c], o[h][c]);
                });
            }
        };

        uint4 ka[U], va[U], kb[U], vb[U];
        int ra[U], rb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) ka[u] = va[u] = kb[u] = vb[u] = make_uint4(0, 0, 0, 0);
        load(0, ka, va, ra);
        for (int s = 0; s < nst; s += 2) {
            if (s + 1 < nst) load(s + 1, kb, vb, rb);
            compute(ka, va, ra);
            if (s + 1 >= nst) break;
            if (s + 2 < nst) load(s + 2, ka, va, ra);
            compute(kb, vb, rb);
        }
        __builtin_amdgcn_wave_barrier();
    }

    // Every token group writes its state (base-2 reference maximum, sum and
    // unnormalised output) to LDS; the workgroup then merges the groups with
    // one exponential per (group, head) and writes the split's partial.  The
    // output area reuses the transpose area, so all waves first leave the loop.
    __syncthreads();
    const int grp = wave * TPW + tg;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        grp_o[grp][h][sub * 2] = make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
        grp_o[grp][h][sub * 2 + 1] = make_float4(o[h][4], o[h][5], o[h][6], o[h][7]);
    }
#pragma unroll
    for (int j = 0; j < HPL; ++j)
        if (sub % DUP == 0) {
            grp_m[grp][head0 + j] = m_own[j] * sl2;  // -inf stays -inf
            grp_l[grp][head0 + j] = l_own[j];
        }
    __syncthreads();

    for (int i = threadIdx.x; i < G * HD / 4; i += 64 * kWaves) {
        const int h = i / (HD / 4), c4 = i % (HD / 4);
        float ms = -INFINITY;
        for (int gi = 0; gi < NGRP; ++gi) ms = fmaxf(ms, grp_m[gi][h]);
        float ls = 0.f;
        float4 os = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int gi = 0; gi < NGRP; ++gi) {
            const float mg = grp_m[gi][h];
            const float w = mg == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mg - ms);
            ls = fmaf(grp_l[gi][h], w, ls);
            const float4 og = grp_o[gi][h][c4];
            os.x = fmaf(og.x, w, os.x);
            os.y = fmaf(og.y, w, os.y);
            os.z = fmaf(og.z, w, os.z);
            os.w = fmaf(og.w, w, os.w);
        }
        const float inv = ls > 0.f ? 1.0f / ls : 0.f;
        const long prow = (((long)b * g.Hq + kvh * G + h) * a.Q + row) * a.split_stride + split;
        *(float4*)(a.part_o + prow * HD + c4 * 4) = make_float4(os.x * inv, os.y * inv, os.z * inv, os.w * inv);
        if (c4 == 0) {
            a.part_ml[prow * 2 + 0] = ls > 0.f ? ms * kLn2 : -INFINITY;
            a.part_ml[prow * 2 + 1] = ls;
        }
    }
}

template <int HD, bool BF>
hipError_t launch_g(const DecodeArgs& a, dim3 grid, hipStream_t s)
{
    const dim3 block(64 * kWaves);
    if constexpr (BF) {
        switch (a.g.G) {
        case 1: hipLaunchKernelGGL((k_decode_bf16<HD, 1>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((k_decode_bf16<HD, 2>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((k_decode_bf16<HD, 4>), grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL((k_decode_bf16<HD, 8>), grid, block, 0, s, a); break;
        case 16: hipLaunchKernelGGL((k_decode_bf16<HD, 16>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
        }
    } else {
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

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s)
{
    const long wgs = (long)a.g.B * a.g.Hkv * a.Q * a.splits;
    const dim3 grid((unsigned)wgs);
    const bool bf = a.g.dtype == 1;
    if (a.g.hd == 128) return bf ? launch_g<128, true>(a, grid, s) : launch_g<128, false>(a, grid, s);
    if (a.g.hd == 64) return bf ? launch_g<64, true>(a, grid, s) : launch_g<64, false>(a, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace sa
