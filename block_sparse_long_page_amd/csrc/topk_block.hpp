// Block-wide top-k of the page scores of one (sequence, KV head, row), for
// 512-thread workgroups: used by the selection kernel and by the decode kernel
// that selects its own pages.
#pragma once

#include "device_common.hpp"

namespace sa {

// order-preserving float -> uint32 (larger float, larger key); -0 maps to +0
__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    u = u == 0x80000000u ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopkThreads = 512;
constexpr int kTopkMaxRounds = 24;  // keys per thread: up to 12288 candidate pages

constexpr int kCntChunks = (kTopkMaxRounds * (kTopkThreads / 64) + 63) / 64;

// Exclusive prefix sums of cnt[0 .. n) held across the wave: entry e's prefix
// is lane e % 64 of ex[e / 64].
__device__ __forceinline__ void scan_counts(const int* cnt, int n, int lane, int (&ex)[kCntChunks])
{
    int carry = 0;
#pragma unroll
    for (int c = 0; c < kCntChunks; ++c) {
        const int e = c * 64 + lane;
        const int v = e < n ? cnt[e] : 0;
        const int inc = wave_inclusive_scan(v);
        ex[c] = inc - v + carry;
        carry += __builtin_amdgcn_readlane(inc, 63);
    }
}

// the prefix of entry e (wave-uniform)
__device__ __forceinline__ int pick_count(const int (&ex)[kCntChunks], int e)
{
    const int c = e >> 6, l = e & 63;
    int v = __builtin_amdgcn_readlane(ex[0], l);
#pragma unroll
    for (int i = 1; i < kCntChunks; ++i)
        if (c == i) v = __builtin_amdgcn_readlane(ex[i], l);
    return v;
}

constexpr int kTopkPasses = 4;  // 32 key bits, 8 per pass

constexpr int kTopkBoundMax = 64;  // keys of the boundary digit ranked directly by one wave, one per lane

struct TopkScratch {
    int hist[kTopkPasses][256];
    uint32_t mm[kTopkThreads / 64][2];
    int cnt_eq[kTopkMaxRounds * (kTopkThreads / 64)];  // round-major: flat (round, wave) order is page order
    int cnt_in[kTopkMaxRounds * (kTopkThreads / 64)];
    int gts[kTopkThreads / 64];
    // one-pass path: the boundary digit's keys, then a bitmap of the chosen indices
    int nb;
    uint32_t b_key[kTopkBoundMax];
    int b_idx[kTopkBoundMax];
    uint64_t chosen[kTopkMaxRounds * kTopkThreads / 64];
};

// The k largest of the n scores sc[0 .. n) (1 <= k < n <= kTopkThreads *
// kTopkMaxRounds), ties to the lower index, in ascending index order:
// emit(position, index) once per chosen index.  Called by all 512 threads
// with the n order keys in keys[] (LDS) and each thread's min and max key.
//  1. min and max of the keys give the bits every key shares;
//  2. radix select, 8 bits at a time from the highest differing bit: an LDS
//     histogram of the digit among the keys that match the prefix decided so
//     far; every wave then scans the histogram itself and finds the digit
//     where the count from the top reaches k;
//  3. compaction in ascending index order: every key above the k-th, then the
//     lowest indices among those equal to it, placed by wave scans of the
//     per-wave counts.
// Loops over the keys stay rolled (unrolled by four) so the code fits the
// instruction cache.
// Loads the order keys of sc[0 .. n) into keys[] (all of a thread's loads in
// flight together) and returns this thread's min and max key.
__device__ __forceinline__ void topk_load_keys(const float* sc, int n, uint32_t* keys, uint32_t& lo, uint32_t& hi)
{
    const int tid = threadIdx.x;
    lo = 0xffffffffu;
    hi = 0;
    for (int base = 0; base < n; base += 4 * kTopkThreads) {
        float v[4];  // four loads in flight per thread
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = base + u * kTopkThreads + tid;
            v[u] = i < n ? sc[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = base + u * kTopkThreads + tid;
            if (i < n) {
                const uint32_t key = order_key(v[u]);
                keys[i] = key;
                lo = min(lo, key);
                hi = max(hi, key);
            }
        }
    }
}

template <typename Emit>
__device__ __forceinline__ void block_topk_keys(int n, int k, const uint32_t* keys, uint32_t lo, uint32_t hi,
                                                TopkScratch& sh, Emit emit)
{
    constexpr int NW = kTopkThreads / 64;
    constexpr int kPasses = kTopkPasses;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < kPasses * 256; i += kTopkThreads) (&sh.hist[0][0])[i] = 0;
    const int rounds = (n + kTopkThreads - 1) / kTopkThreads;  // <= kTopkMaxRounds (host-checked)
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (lane == 0) {
        sh.mm[wave][0] = lo;
        sh.mm[wave][1] = hi;
    }
    __syncthreads();
    for (int w = 0; w < NW; ++w) {
        lo = min(lo, sh.mm[w][0]);
        hi = max(hi, sh.mm[w][1]);
    }

    uint32_t kth = hi;  // the k-th largest key
    if (lo != hi) {
        int top = 31 - __builtin_clz(lo ^ hi);  // highest bit that differs
        uint32_t prefix = top == 31 ? 0u : (hi & ~((2u << top) - 1u));
        int need = k;  // keys still to take among those matching the prefix
        for (int pass = 0; top >= 0; ++pass) {
            const int width = top + 1 < 8 ? top + 1 : 8;
            const int shift = top + 1 - width;
            const uint32_t dmask = (1u << width) - 1u;
            const int up = shift + width;  // bits >= up are decided
            const uint32_t hmask = up >= 32 ? 0u : ~((1u << up) - 1u);
#pragma unroll 4
            for (int i = tid; i < n; i += kTopkThreads) {
                const uint32_t key = keys[i];
                if ((key & hmask) == prefix) atomicAdd(&sh.hist[pass][(key >> shift) & dmask], 1);
            }
            __syncthreads();
            // lane j owns digits 255-4j .. 252-4j, so lane order is digit order from the top
            const int4 c = *(const int4*)&sh.hist[pass][252 - 4 * lane];  // digits 252-4j .. 255-4j
            const int s = c.x + c.y + c.z + c.w;
            const int above = wave_inclusive_scan(s) - s;  // keys with a larger digit than this lane's
            const uint64_t hit = __builtin_amdgcn_ballot_w64(above < need && above + s >= need);
            const int hl = (int)__builtin_ctzll(hit);
            int acc = __builtin_amdgcn_readlane(above, hl);
            const int cw = __builtin_amdgcn_readlane(c.w, hl), cz = __builtin_amdgcn_readlane(c.z, hl);
            const int cy = __builtin_amdgcn_readlane(c.y, hl);
            int digit;
            if (acc + cw >= need) {
                digit = 255 - 4 * hl;
            } else if (acc + cw + cz >= need) {
                digit = 254 - 4 * hl;
                acc += cw;
            } else if (acc + cw + cz + cy >= need) {
                digit = 253 - 4 * hl;
                acc += cw + cz;
            } else {
                digit = 252 - 4 * hl;
                acc += cw + cz + cy;
            }
            prefix |= (uint32_t)digit << shift;
            need -= acc;
            top = shift - 1;
        }
        kth = prefix;
    }

    // per-wave counts of keys equal to kth and above it, round by round
    int gt_local = 0;
#pragma unroll 4
    for (int r = 0; r < rounds; ++r) {
        const int i = r * kTopkThreads + tid;
        const uint32_t key = i < n ? keys[i] : 0u;
        const int ne = __builtin_popcountll(__builtin_amdgcn_ballot_w64(i < n && key == kth));
        gt_local += __builtin_popcountll(__builtin_amdgcn_ballot_w64(i < n && key > kth));
        if (lane == 0) sh.cnt_eq[r * NW + wave] = ne;
    }
    if (lane == 0) sh.gts[wave] = gt_local;
    __syncthreads();
    int gt = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) gt += sh.gts[w];
    const int need = k - gt;  // equal keys to take, lowest pages first
    const int ncnt = rounds * NW;

    // chosen: above kth, or equal to it and among the first `need` equal keys
    // in page order (round, wave, lane); the rank of a wave's first equal key
    // is the exclusive prefix of the counts in (round, wave) order
    int ex[kCntChunks];
    scan_counts(sh.cnt_eq, ncnt, lane, ex);
    uint32_t mine = 0;  // bit r: this thread's key of round r is chosen
#pragma unroll 4
    for (int r = 0; r < rounds; ++r) {
        const int i = r * kTopkThreads + tid;
        const uint32_t key = i < n ? keys[i] : 0u;
        const bool eq = i < n && key == kth;
        const int rank = pick_count(ex, r * NW + wave);
        const bool in = i < n && (key > kth || (eq && rank + lanes_below(__builtin_amdgcn_ballot_w64(eq)) < need));
        const int cc = __builtin_popcountll(__builtin_amdgcn_ballot_w64(in));
        if (lane == 0) sh.cnt_in[r * NW + wave] = cc;
        mine |= (uint32_t)in << r;
    }
    __syncthreads();
    int ox[kCntChunks];
    scan_counts(sh.cnt_in, ncnt, lane, ox);
    for (int r = 0; r < rounds; ++r) {
        const int i = r * kTopkThreads + tid;
        const bool in = (mine >> r) & 1u;
        const uint64_t inm = __builtin_amdgcn_ballot_w64(in);
        const int here = pick_count(ox, r * NW + wave);
        if (in) emit(here + lanes_below(inm), i);
    }
}

// ---------------------------------------------------------------------------
// The same selection with one radix pass in the common case.  After the bits
// every key shares, one 8-bit digit histogram gives the boundary digit d (the
// count of keys with a larger digit is below k, with d included it reaches
// k): keys with a larger digit are chosen outright (set in a bitmap by wave
// ballots), and when at most 64 keys carry digit d they are gathered and one
// wave ranks them by direct comparison of (key, lower index first), taking
// the best k - (count above).  When more keys carry d, the next 8 bits of
// just those keys are histogrammed, and so on, until the boundary bucket
// (the keys matching every decided bit) holds at most 64 keys; only a bucket
// of more than 64 equal keys falls back to the multi-pass select above (same
// result).  The workgroup then emits the bitmap in ascending index order, a
// word per thread placed by a block scan.
//
// The steps:
//   topk_begin          every thread, before the barrier that publishes the keys
//   topk_digits         every thread after it (histogram), then a barrier
//   topk_boundary       every wave: the boundary digit, its count, the count above
//   topk_refine         every thread, while the bucket holds more than 64 keys
//   topk_collect_block  every thread: the bitmap of keys above the bucket and
//                       the bucket's keys, then a barrier
//   take_boundary       one wave: ranks the bucket's keys into the bitmap
//   emit_bitmap_block   every thread, after a barrier
// ---------------------------------------------------------------------------

struct TopkPlan {
    uint32_t lo, hi;  // smallest and largest key
    int shift;        // the digit is (key >> shift) & dmask
    uint32_t dmask;
    int d, nd, above;  // boundary digit, its key count, keys with a larger digit
    // the decided bits: the boundary bucket is the keys with (key & hmask) ==
    // prefix, the keys above it those with (key & hmask) > prefix
    uint32_t hmask, prefix;
};

// Every thread, with its min and max key: clears the histograms and publishes
// the wave's key range.
__device__ __forceinline__ void topk_begin(TopkScratch& sh, uint32_t lo, uint32_t hi)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < kTopkPasses * 256; i += kTopkThreads) (&sh.hist[0][0])[i] = 0;
    if (tid == 0) sh.nb = 0;
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (lane == 0) {
        sh.mm[wave][0] = lo;
        sh.mm[wave][1] = hi;
    }
}

// Every thread, after the barrier that follows topk_begin: the key range and
// the digit below the bits every key shares; unless every key is equal, the
// thread's keys go into the digit histogram (a barrier must follow).
__device__ __forceinline__ TopkPlan topk_digits(TopkScratch& sh, int n, const uint32_t* keys)
{
    constexpr int NW = kTopkThreads / 64;
    TopkPlan t;
    t.lo = 0xffffffffu;
    t.hi = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        t.lo = min(t.lo, sh.mm[w][0]);
        t.hi = max(t.hi, sh.mm[w][1]);
    }
    t.shift = 0;
    t.dmask = 0;
    t.d = -1;
    t.nd = 0;
    t.above = 0;
    if (t.lo == t.hi) return t;
    const int top = 31 - __builtin_clz(t.lo ^ t.hi);  // highest bit that differs
    const int width = top + 1 < 8 ? top + 1 : 8;
    t.shift = top + 1 - width;
    t.dmask = (1u << width) - 1u;
    t.hmask = ~((1u << t.shift) - 1u);
    t.prefix = t.hi & ~((2u << top) - 1u);  // the bits every key shares (none when top = 31)
#pragma unroll 4
    for (int i = threadIdx.x; i < n; i += kTopkThreads) atomicAdd(&sh.hist[0][(keys[i] >> t.shift) & t.dmask], 1);
    return t;
}

// Any wave: in a 256-entry digit histogram, the digit where the count of
// keys from the top reaches need (1 <= need <= the histogram's total), its
// count, and the count of keys with a larger digit.
__device__ __forceinline__ void boundary_digit(const int* hist, int need, int& d, int& nd, int& above)
{
    const int lane = threadIdx.x & 63;
    // lane j owns digits 255-4j .. 252-4j, so lane order is digit order from the top
    const int4 c = *(const int4*)&hist[252 - 4 * lane];
    const int s4 = c.x + c.y + c.z + c.w;
    const int above4 = wave_inclusive_scan(s4) - s4;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(above4 < need && above4 + s4 >= need);
    const int hl = (int)__builtin_ctzll(hit);
    above = __builtin_amdgcn_readlane(above4, hl);
    const int cw = __builtin_amdgcn_readlane(c.w, hl), cz = __builtin_amdgcn_readlane(c.z, hl);
    const int cy = __builtin_amdgcn_readlane(c.y, hl), cx = __builtin_amdgcn_readlane(c.x, hl);
    if (above + cw >= need) {
        d = 255 - 4 * hl;
        nd = cw;
    } else if (above + cw + cz >= need) {
        d = 254 - 4 * hl;
        nd = cz;
        above += cw;
    } else if (above + cw + cz + cy >= need) {
        d = 253 - 4 * hl;
        nd = cy;
        above += cw + cz;
    } else {
        d = 252 - 4 * hl;
        nd = cx;
        above += cw + cz + cy;
    }
}

// Any wave, after the histogram's barrier (and only when lo != hi): the
// digit where the count of keys from the top reaches k.
__device__ __forceinline__ void topk_boundary(const TopkScratch& sh, int k, TopkPlan& t)
{
    boundary_digit(sh.hist[0], k, t.d, t.nd, t.above);
    t.prefix |= (uint32_t)t.d << t.shift;
}

// Every thread, after topk_boundary, while the boundary bucket holds more
// than kTopkBoundMax keys: the next 8 bits of the bucket's keys (the
// histograms topk_begin cleared, one per pass; every thread reads every key,
// only the bucket's are counted), until the bucket holds at most
// kTopkBoundMax keys or every bit is decided.  Returns whether it does (else
// its keys are all equal).
__device__ __forceinline__ bool topk_refine(TopkScratch& sh, int n, int k, const uint32_t* keys, TopkPlan& t)
{
    int pass = 1;
    while (t.nd > kTopkBoundMax && t.shift > 0 && pass < kTopkPasses) {
        const int width = t.shift < 8 ? t.shift : 8;
        const int shift = t.shift - width;
        const uint32_t dmask = (1u << width) - 1u;
        int* hist = sh.hist[pass];
#pragma unroll 4
        for (int i = threadIdx.x; i < n; i += kTopkThreads) {
            const uint32_t key = keys[i];
            if ((key & t.hmask) == t.prefix) atomicAdd(&hist[(key >> shift) & dmask], 1);
        }
        __syncthreads();
        int d, nd, above;
        boundary_digit(hist, k - t.above, d, nd, above);
        t.above += above;
        t.d = d;
        t.nd = nd;
        t.shift = shift;
        t.dmask = dmask;
        t.hmask |= dmask << shift;
        t.prefix |= (uint32_t)d << shift;
        ++pass;
    }
    return t.nd <= kTopkBoundMax;
}

// Every thread (a barrier must follow): keys above the boundary bucket into
// the bitmap (word w holds indices 64w .. 64w+63), the bucket's keys into
// the boundary list (t.nd <= kTopkBoundMax).
__device__ __forceinline__ void topk_collect_block(int n, const uint32_t* keys, const TopkPlan& t, TopkScratch& sh)
{
    constexpr int NW = kTopkThreads / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rounds = (n + kTopkThreads - 1) / kTopkThreads;
    for (int r = 0; r < rounds; ++r) {
        const int i = r * kTopkThreads + tid;
        const uint32_t mk = (i < n ? keys[i] : 0u) & t.hmask;
        const uint64_t up = __builtin_amdgcn_ballot_w64(i < n && mk > t.prefix);
        if (lane == 0) sh.chosen[r * NW + wave] = up;
        if (i < n && mk == t.prefix) {
            const uint32_t key = keys[i];
            const int slot = atomicAdd(&sh.nb, 1);
            sh.b_key[slot] = key;
            sh.b_idx[slot] = i;
        }
    }
}

// One wave: ranks the nd <= 64 boundary keys b_key/b_idx (larger key first,
// then lower index) by lane reads from registers and sets the best `need`
// of them in the bitmap.
__device__ __forceinline__ void take_boundary(int nd, int need, const uint32_t* b_key, const int* b_idx,
                                              uint64_t* chosen)
{
    const int lane = threadIdx.x & 63;
    const bool mine = lane < nd;
    const uint32_t bk = mine ? b_key[lane] : 0u;
    const int bi = mine ? b_idx[lane] : 0;
    int rank = 0;
    for (int u = 0; u < nd; ++u) {
        const uint32_t ku = (uint32_t)__builtin_amdgcn_readlane((int)bk, u);
        const int iu = __builtin_amdgcn_readlane(bi, u);
        rank += ku > bk || (ku == bk && iu < bi);
    }
    if (mine && rank < need) atomicOr((unsigned long long*)&chosen[bi >> 6], 1ull << (bi & 63));
}

// One wave: emits the set bits of the bitmap of n indices in ascending order.
template <typename Emit>
__device__ __forceinline__ void emit_bitmap(int n, const uint64_t* chosen, Emit emit)
{
    const int lane = threadIdx.x & 63;
    const int nwords = (n + 63) / 64;
    int base = 0;
    for (int w0 = 0; w0 < nwords; w0 += 64) {
        const int w = w0 + lane;
        uint64_t bits = w < nwords ? chosen[w] : 0ull;
        const int cnt = __builtin_popcountll(bits);
        const int inc = wave_inclusive_scan(cnt);
        int pos = base + inc - cnt;
        while (bits) {
            const int b = __builtin_ctzll(bits);
            emit(pos++, 64 * w + b);
            bits &= bits - 1;
        }
        base += __builtin_amdgcn_readlane(inc, 63);
    }
}

// Every thread: emits the set bits of the bitmap of n <= 64 * kTopkThreads
// indices in ascending order, a word per thread placed by a block scan of
// the words' counts (wsum: kTopkThreads / 64 ints of LDS).
template <typename Emit>
__device__ __forceinline__ void emit_bitmap_block(int n, const uint64_t* chosen, int* wsum, Emit emit)
{
    const int w = threadIdx.x;
    uint64_t bits = w < (n + 63) / 64 ? chosen[w] : 0ull;
    int total;
    int pos = block_exclusive_scan<kTopkThreads>(__builtin_popcountll(bits), wsum, total);
    while (bits) {
        emit(pos++, 64 * w + __builtin_ctzll(bits));
        bits &= bits - 1;
    }
}

// The whole selection by the block (all 512 threads), keys already in LDS
// and each thread's min and max key given.
template <typename Emit>
__device__ __forceinline__ void block_topk_fast(int n, int k, const uint32_t* keys, uint32_t lo, uint32_t hi,
                                                TopkScratch& sh, Emit emit)
{
    const int tid = threadIdx.x;
    topk_begin(sh, lo, hi);
    __syncthreads();
    TopkPlan t = topk_digits(sh, n, keys);
    if (t.lo == t.hi) {  // every key equal: the lowest k indices
        for (int i = tid; i < k; i += kTopkThreads) emit(i, i);
        return;
    }
    __syncthreads();
    topk_boundary(sh, k, t);
    // uniform: every wave read the same histograms
    if (t.nd > kTopkBoundMax && !topk_refine(sh, n, k, keys, t)) {
        __syncthreads();  // more equal keys at the boundary than one wave ranks: the multi-pass select
        block_topk_keys(n, k, keys, t.lo, t.hi, sh, emit);
        return;
    }
    topk_collect_block(n, keys, t, sh);
    __syncthreads();
    if ((tid >> 6) == 0) take_boundary(t.nd, k - t.above, sh.b_key, sh.b_idx, sh.chosen);
    __syncthreads();
    emit_bitmap_block(n, sh.chosen, sh.gts, emit);
}

// ---------------------------------------------------------------------------
// The same selection by one wave alone, so that a workgroup's other waves can
// go on with other work once the keys are in LDS.  Radix select 8 bits at a
// time from the highest bit where the smallest and largest key differ: each
// pass histograms the digit of the keys that match the bits decided so far
// and finds the digit where the count from the top reaches the keys still
// needed.  The passes stop once the boundary bucket (the keys that match
// every decided bit) holds at most 64 keys, or when every bit is decided
// (the bucket's keys are then all equal).  One pass over the keys in index
// order then sets the bitmap of the keys above the bucket and either
// gathers the bucket (ranked by key, then lower index) or, for equal keys,
// takes the lowest indices; the bitmap is emitted in ascending order.
// ---------------------------------------------------------------------------

struct WaveTopkScratch {
    alignas(16) int hist[256];
    uint32_t b_key[kTopkBoundMax];
    int b_idx[kTopkBoundMax];
    uint64_t chosen[kTopkMaxRounds * kTopkThreads / 64];
};

// The k largest of the n keys keys[0 .. n) (1 <= k < n <= kTopkThreads *
// kTopkMaxRounds; lo < hi the smallest and largest key; the array 16-byte
// aligned and readable up to the next multiple of 4), ties to the lower
// index: emit(position, index) once per chosen index, ascending.  One wave.
template <typename Emit>
__device__ __forceinline__ void wave_topk(int n, int k, const uint32_t* keys, uint32_t lo, uint32_t hi,
                                          WaveTopkScratch& sh, Emit emit)
{
    const int lane = threadIdx.x & 63;
    int top = 31 - __builtin_clz(lo ^ hi);  // highest bit that differs
    uint32_t hmask = top == 31 ? 0u : ~((2u << top) - 1u);  // the bits decided
    uint32_t prefix = hi & hmask;
    int need = k;  // keys still to take among those matching the prefix
    int nb;        // keys matching the prefix
    for (;;) {
        const int width = top + 1 < 8 ? top + 1 : 8;
        const int shift = top + 1 - width;
        const uint32_t dmask = (1u << width) - 1u;
        *(int4*)&sh.hist[4 * lane] = make_int4(0, 0, 0, 0);
        __builtin_amdgcn_wave_barrier();
        for (int i = 4 * lane; i < n; i += 256) {  // four keys per lane and step
            const uint4 kv = *(const uint4*)(keys + i);
            const uint32_t kq[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (i + u < n && (kq[u] & hmask) == prefix) atomicAdd(&sh.hist[(kq[u] >> shift) & dmask], 1);
        }
        __builtin_amdgcn_wave_barrier();
        // lane j owns digits 255-4j .. 252-4j, so lane order is digit order from the top
        const int4 c = *(const int4*)&sh.hist[252 - 4 * lane];
        const int s4 = c.x + c.y + c.z + c.w;
        const int above4 = wave_inclusive_scan(s4) - s4;
        const uint64_t hit = __builtin_amdgcn_ballot_w64(above4 < need && above4 + s4 >= need);
        const int hl = (int)__builtin_ctzll(hit);
        int above = __builtin_amdgcn_readlane(above4, hl);
        const int cw = __builtin_amdgcn_readlane(c.w, hl), cz = __builtin_amdgcn_readlane(c.z, hl);
        const int cy = __builtin_amdgcn_readlane(c.y, hl), cx = __builtin_amdgcn_readlane(c.x, hl);
        int d;
        if (above + cw >= need) {
            d = 255 - 4 * hl;
            nb = cw;
        } else if (above + cw + cz >= need) {
            d = 254 - 4 * hl;
            nb = cz;
            above += cw;
        } else if (above + cw + cz + cy >= need) {
            d = 253 - 4 * hl;
            nb = cy;
            above += cw + cz;
        } else {
            d = 252 - 4 * hl;
            nb = cx;
            above += cw + cz + cy;
        }
        need -= above;
        prefix |= (uint32_t)d << shift;
        hmask |= dmask << shift;
        if (nb <= kTopkBoundMax || shift == 0) break;
        top = shift - 1;
    }

    // keys above the bucket: (key & hmask) > prefix; in it: == prefix
    const bool gather = nb <= kTopkBoundMax;  // otherwise every bucket key is equal
    int seen = 0;                             // bucket keys at lower indices
    for (int w = 0; 64 * w < n; ++w) {
        const int i = 64 * w + lane;
        const uint32_t hk = (i < n ? keys[i] : 0u) & hmask;
        const bool in = i < n && hk == prefix;
        const uint64_t inm = __builtin_amdgcn_ballot_w64(in);
        const int below = seen + lanes_below(inm);
        const uint64_t up = __builtin_amdgcn_ballot_w64(i < n && (hk > prefix || (!gather && in && below < need)));
        if (gather && in) {
            sh.b_key[below] = keys[i];
            sh.b_idx[below] = i;
        }
        seen += __builtin_popcountll(inm);
        if (lane == 0) sh.chosen[w] = up;
    }
    __builtin_amdgcn_wave_barrier();
    if (gather) {
        take_boundary(nb, need, sh.b_key, sh.b_idx, sh.chosen);
        __builtin_amdgcn_wave_barrier();
    }
    emit_bitmap(n, sh.chosen, emit);
}

}  // namespace sa
