// The front of one chunk of a sparse prefill over a semantic block index of
// the prompt (semantic-blocks page: one index serves the prompt's
// processing; the rows of a prompt chunk compare themselves with the block
// centres and take the best blocks up to a token budget, among the parts of
// the blocks that precede the chunk's window; the window, the chunk's own
// recent tokens, is attended without selection).
//
// k_prefill_choose: one workgroup per 8 rows of one (chunk, sequence, KV
// head), a wave per row, in one launch with no other kernel before the
// grouped decode (a call may serve several consecutive chunks of the prompt,
// each with its own length and budget):
//  * the visible part of every block (its rows of positions < L - W;
//    positions ascend inside a block, so the part is a prefix): a k-ary
//    search by a team of T lanes per block, T probes a round narrowing the
//    range (T + 1)-fold, every workgroup for itself (a few rounds of loads
//    instead of a launch); the first workgroup of each (sequence, KV head)
//    writes the ends;
//  * the row's block scores, the max over the group's heads of q_h . centre_c
//    in fp32 (a few lanes per block when there are few blocks, their sums
//    added pairwise);
//  * the greedy choice by repeated arg-max over (score desc, block asc):
//    a block is taken while fewer than k_max are taken and the running
//    visible size stays within the budget; the first is always taken;
//    blocks without visible rows are never candidates;
//  * the row's list (ascending) and count, its list index of every block in
//    the grouped decode's slot table ([block][row], -1 where it did not
//    choose the block), and an empty partial (m = -inf, l = 0) for every
//    slot of the list entries it does not use;
//  * per block, how many of the workgroup's 8 rows chose it (the grouped
//    decode sizes its items from these counts without reading the slot
//    table), and the first workgroup of a (sequence, KV head) clears the
//    grouped decode's item counter.
#include "device_common.hpp"
#include "kernels.hpp"
#include "topk_block.hpp"

namespace sa {

namespace {

constexpr int kPfWaves = 8;                    // rows of a workgroup, a wave each
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfRounds = kPfMaxBlocks / 64;   // block keys per lane (one lane per block)
constexpr int kPfProbe = 1;                    // rows a lane reads per round of the visible-end search

template <int HD, int G>
__global__ __launch_bounds__(kPfThreads) void k_prefill_choose(PrefillArgs a)
{
    __shared__ int off_l[kPfMaxBlocks + 1];
    __shared__ int size_l[kPfMaxBlocks];
    __shared__ __attribute__((aligned(16))) float qs[kPfWaves][G][HD];
    __shared__ int nch[kPfMaxBlocks];  // rows of this workgroup that chose each block
    const Geometry& g = a.g;
    const int C = a.C, N = a.N;
    const int ngr = (a.Q + kPfWaves - 1) / kPfWaves;
    const int nbk = g.B * g.Hkv;
    const int grp = blockIdx.x % ngr, vb = blockIdx.x / ngr;  // vb: (chunk, sequence, KV head)
    const int ck = vb / nbk, bk = vb - ck * nbk, b = bk / g.Hkv, kvh = bk - b * g.Hkv;
    const int QS = a.Q * a.nck, row0 = ck * a.Q;  // row stride of q, lists and partials; the chunk's first row
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const int L = imax(0, imin(g.seq_lens[b] + row0, g.max_pages * g.P));
    const int bound = L - a.W;
    const int budget = a.budget[ck];
    const int32_t* off = a.offsets + (long)bk * (C + 1);
    const int32_t* pos = a.positions + (long)bk * N;

    // the rows' queries in fp32, and the block offsets clamped to the layout
    constexpr int QPR = G * HD / 8;  // 16-byte pieces of one row's queries
    for (int e = tid; e < kPfWaves * QPR; e += kPfThreads) {
        const int w = e / QPR, rest = e - w * QPR, h = rest / (HD / 8), d8 = rest - h * (HD / 8);
        const int row = grp * kPfWaves + w;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (row < a.Q)
            u = *(const uint4*)((const uint16_t*)a.q + (((long)b * g.Hq + kvh * G + h) * QS + row0 + row) * HD +
                                8 * d8);
        float4* dst = (float4*)&qs[w][h][8 * d8];
        dst[0] = make_float4(bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y));
        dst[1] = make_float4(bf_lo(u.z), bf_hi(u.z), bf_lo(u.w), bf_hi(u.w));
    }
    for (int c = tid; c <= C; c += kPfThreads) off_l[c] = imax(0, imin(off[c], N));
    for (int c = tid; c < C; c += kPfThreads) nch[c] = 0;
    if (grp == 0 && tid == 0) a.ctr[vb] = 0;  // the grouped decode's item counter
    __syncthreads();

    // Visible ends: block c's rows are [off_l[c], max(off_l[c], off_l[c+1]));
    // the end is the first row whose position is >= bound.  A team of T
    // lanes (T a power of two, T * C <= the workgroup) reads NP = T * kPfProbe
    // rows a round: while more than NP rows remain, rows that split the open
    // range evenly (those below the bound are a prefix, and their count
    // leaves one gap), then the remaining rows themselves, whose count below
    // the bound gives the end.  The first round's loads are issued before
    // the scores below and consumed after them.
    int T = 1;
    while (T < 64 && 2 * T * C <= kPfThreads) T *= 2;
    const int teams = kPfThreads / T, k = tid & (T - 1), NP = T * kPfProbe;
    int probe[kPfProbe];
    auto load_round = [&](int lo, int hi) {
        const long len = hi - lo;
#pragma unroll
        for (int u = 0; u < kPfProbe; ++u) {
            const int i = k * kPfProbe + u;
            const int m = len > NP ? lo + (int)(len * (i + 1) / (NP + 1)) : lo + i;
            probe[u] = m < hi ? pos[m] : 0x7fffffff;  // past the range: never below the bound
        }
    };
    const int c_first = tid / T;
    int lo_first = 0, hi_first = 0;
    if (c_first < C) {
        lo_first = off_l[c_first];
        hi_first = imax(lo_first, off_l[c_first + 1]);
        load_round(lo_first, hi_first);
    }

    const int r = grp * kPfWaves + wave;
    const bool row_ok = r < a.Q;

    // Scores: LPB lanes per block, each over HD / LPB channels; block
    // cl + per * i in round i.  Lane = part * per + cl.
    const int LPB = C <= 16 ? 4 : C <= 32 ? 2 : 1;
    const int per = 64 / LPB, part = lane / per, cl = lane - part * per;
    const int D = HD / LPB;
    const int R = (C + per - 1) / per;  // rounds (<= kPfRounds)
    uint64_t kk[kPfRounds];
#pragma unroll
    for (int i = 0; i < kPfRounds; ++i) {
        kk[i] = 0ull;
        if (i < R) {
            const int c = cl + per * i;
            const bool valid = c < C;
            const float4* mu = (const float4*)(a.centres + ((long)bk * C + (valid ? c : 0)) * HD + part * D);
            float dot[G];
#pragma unroll
            for (int h = 0; h < G; ++h) dot[h] = 0.f;
            for (int d4 = 0; d4 < D / 4; ++d4) {
                const float4 m = mu[d4];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float4 x = *(const float4*)&qs[wave][h][part * D + 4 * d4];
                    dot[h] = fmaf(x.x, m.x, dot[h]);
                    dot[h] = fmaf(x.y, m.y, dot[h]);
                    dot[h] = fmaf(x.z, m.z, dot[h]);
                    dot[h] = fmaf(x.w, m.w, dot[h]);
                }
            }
            // the parts of a block differ in lane bits 4 and 5
#pragma unroll
            for (int h = 0; h < G; ++h) {
                if (per <= 16) dot[h] += xor_lanes<16>(dot[h]);
                if (per <= 32) dot[h] += xor_lanes<32>(dot[h]);
            }
            float best = dot[0];
#pragma unroll
            for (int h = 1; h < G; ++h) best = fmaxf(best, dot[h]);
            if (valid) kk[i] = ((uint64_t)order_key(best) << 32) | (uint32_t)(0xffffffffu - (uint32_t)c);
        }
    }

    // complete the search (the first round's probes are in `probe`)
    for (int c = c_first; c < C; c += teams) {
        int lo = lo_first, hi = hi_first;
        if (c != c_first) {
            lo = off_l[c];
            hi = imax(lo, off_l[c + 1]);
            load_round(lo, hi);
        }
        int end;
        for (;;) {  // the same for every lane of the team
            int nb = 0;
#pragma unroll
            for (int u = 0; u < kPfProbe; ++u) nb += probe[u] < bound;
            for (int o = 1; o < T; o <<= 1) nb += __shfl_xor(nb, o);
            const long len = hi - lo;
            if (len <= NP) {
                end = lo + nb;
                break;
            }
            const int nlo = nb > 0 ? lo + (int)(len * nb / (NP + 1)) + 1 : lo;
            hi = nb < NP ? lo + (int)(len * (nb + 1) / (NP + 1)) : hi;
            lo = nlo;
            load_round(lo, hi);
        }
        if (k == 0) {
            size_l[c] = end - off_l[c];
            if (grp == 0) a.ends[(long)vb * C + c] = end;
        }
    }
    __syncthreads();

    if (row_ok) {
        // blocks without visible rows are not candidates
    #pragma unroll
        for (int i = 0; i < kPfRounds; ++i) {
            const int c = cl + per * i;
            if (i < R && c < C && size_l[c] <= 0) kk[i] = 0ull;
        }

        // Greedy choice by repeated arg-max (a key is 0 once taken, or for a
        // block without visible rows).  The first block is taken whatever its
        // size; then blocks while fewer than k_max are taken and the running
        // size stays within the budget; the first that does not fit ends it.
        uint32_t mine = 0;  // bit i: this lane's block of round i is taken
        int count = 0;
        long run = 0;
        for (;;) {
            uint64_t best = 0ull;
    #pragma unroll
            for (int i = 0; i < kPfRounds; ++i) best = kk[i] > best ? kk[i] : best;
            const uint32_t bh = (uint32_t)(best >> 32);
            const uint32_t mh = wave_max_u32(bh);
            if (mh == 0u) break;  // no candidate left
            const uint32_t ml = wave_max_u32(bh == mh ? (uint32_t)best : 0u);
            const int c = (int)(0xffffffffu - ml);
            const int sz = size_l[c];
            if (count > 0 && (count >= a.k_max || run + sz > budget)) break;
            run += sz;
            ++count;
    #pragma unroll
            for (int i = 0; i < kPfRounds; ++i)
                if (cl + per * i == c) {
                    kk[i] = 0ull;
                    mine |= 1u << i;
                }
        }

        // the list in block order, the slot table, the unused slots
        int32_t* sel = a.sel + ((long)bk * QS + row0 + r) * a.k_max;
        int16_t* slots = a.slots + (long)vb * C * kGroupMaxRows + r;
        int base = 0;
    #pragma unroll
        for (int i = 0; i < kPfRounds; ++i) {
            if (i < R) {
                const int c = cl + per * i;
                const bool t = ((mine >> i) & 1u) != 0u && part == 0;
                const uint64_t bal = __builtin_amdgcn_ballot_w64(t);  // part-0 lanes are 0 .. per-1, blocks ascending
                const int j = base + lanes_below(bal);
                if (part == 0 && c < C) {
                    if (t) {
                        sel[j] = c;
                        atomicAdd(&nch[c], 1);
                    }
                    slots[(long)c * kGroupMaxRows] = t ? (int16_t)j : (int16_t)-1;
                }
                base += __builtin_popcountll(bal);
            }
        }
        for (int j = count + lane; j < a.k_max; j += 64) sel[j] = -1;
        if (lane == 0) a.count[(long)bk * QS + row0 + r] = count;
        const int nempty = (a.k_max - count) * a.tsplit * G;
        for (int e = lane; e < nempty; e += 64) {
            const int h = e % G, rest = e / G, s = rest % a.tsplit, j = count + rest / a.tsplit;
            const long prow = ((long)b * g.Hq + kvh * G + h) * QS + row0 + r;
            const long slot = prow * a.split_stride + (long)j * a.tsplit + s;
            *(float2*)(a.part_ml + slot * 2) = make_float2(-INFINITY, 0.f);
        }
    }

    // rows of this group of 8 that chose each block (the decode's passes);
    // the first group also zeroes the entries past the last group
    __syncthreads();
    for (int c = tid; c < C; c += kPfThreads) {
        unsigned char* rc = a.rows + ((long)vb * C + c) * 16;
        rc[grp] = (unsigned char)nch[c];
        if (grp == 0)
            for (int q8 = ngr; q8 < 16; ++q8) rc[q8] = 0;
    }
}

template <int HD>
hipError_t choose_g(const PrefillArgs& a, dim3 grid, hipStream_t s)
{
    const dim3 block(kPfThreads);
    switch (a.g.G) {
    case 1: hipLaunchKernelGGL((k_prefill_choose<HD, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_prefill_choose<HD, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_prefill_choose<HD, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_prefill_choose<HD, 8>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_prefill_choose<HD, 16>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_choose(const PrefillArgs& a, hipStream_t s)
{
    if (a.g.dtype != 1 || a.C < 1 || a.C > kPfMaxBlocks || a.Q < 1 || a.Q > kGroupMaxRows || a.k_max < 1 ||
        a.nck < 1 || a.nck > kPfMaxChunks)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)((long)a.nck * a.g.B * a.g.Hkv * ((a.Q + kPfWaves - 1) / kPfWaves)));
    if (a.g.hd == 128) return choose_g<128>(a, grid, s);
    if (a.g.hd == 64) return choose_g<64>(a, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace sa
