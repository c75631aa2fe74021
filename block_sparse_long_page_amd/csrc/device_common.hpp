// Device-side helpers shared by the gfx950 kernels: bf16 unpacking, packed
// bf16 dot products, DPP row reductions and the token map of an attended set.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sa {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- bf16 ---------------------------------------------------------------

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// acc + a.lo*b.lo + a.hi*b.hi with bf16 inputs and an fp32 accumulator
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc,
                                           false);
}

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ---- cross-lane -----------------------------------------------------------

// DPP move for controls whose every lane reads a valid source lane (quad
// permutes, row mirrors and rotations, row broadcasts): no "old" value needed.
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of N lanes (N = 2..64); every lane of a group
// receives the group total.  Groups of up to 16 stay inside a DPP row.
template <int N>
__device__ __forceinline__ float group_sum(float x)
{
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
    if constexpr (N >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: partner lane ^1
    if constexpr (N >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: partner lane ^2
    if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror: the other quad of the 8
    if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror: the other 8 of the row
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    if constexpr (N >= 64) x += __shfl_xor(x, 32);
    return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x)
{
    if constexpr (N >= 2) x = fmaxf(x, dpp<0xB1>(x));
    if constexpr (N >= 4) x = fmaxf(x, dpp<0x4E>(x));
    if constexpr (N >= 8) x = fmaxf(x, dpp<0x141>(x));
    if constexpr (N >= 16) x = fmaxf(x, dpp<0x140>(x));
    if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16));
    if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

// Exchange with the lane whose index differs in bit BIT (and, for BIT 3 and
// 2, in the lower bits too: row_mirror / row_half_mirror are involutions that
// stay inside a 16- or 8-lane group).
template <int BIT>
__device__ __forceinline__ float flip(float x)
{
    if constexpr (BIT == 3) return dpp<0x140>(x);  // row_mirror
    else if constexpr (BIT == 2) return dpp<0x141>(x);  // row_half_mirror
    else if constexpr (BIT == 1) return dpp<0x4E>(x);  // quad_perm [2,3,0,1]
    else return dpp<0xB1>(x);  // quad_perm [1,0,3,2]
}

// Reduce-scatter of C partial sums over the lanes of a group (bits BIT..0):
// at each bit the lane keeps the lower or upper half of its values (by that
// lane bit) and adds the partner's copy of that half; once one value is
// left the remaining bits all-reduce it.
template <int C, int BIT>
__device__ __forceinline__ void reduce_scatter(float* d, int lane)
{
    if constexpr (BIT >= 0) {
        if constexpr (C > 1) {
            constexpr int H = C / 2;
            const bool up = (lane >> BIT) & 1;
#pragma unroll
            for (int i = 0; i < H; ++i) {
                const float send = up ? d[i] : d[i + H];
                const float keep = up ? d[i + H] : d[i];
                d[i] = keep + flip<BIT>(send);
            }
            reduce_scatter<H, BIT - 1>(d, lane);
        } else {
            d[0] += flip<BIT>(d[0]);
            reduce_scatter<1, BIT - 1>(d, lane);
        }
    }
}

template <int N>
constexpr int log2c() { return N <= 1 ? 0 : 1 + log2c<N / 2>(); }

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Broadcast lane SRC of each group of N lanes (N = 16: DPP row_newbcast;
// N = 8: a bpermute inside the 8-lane half).
template <int N, int SRC>
__device__ __forceinline__ float group_bcast(float x, int lane)
{
    if constexpr (N == 16)
        return dpp<0x150 + SRC>(x);  // row_newbcast
    else
        return __shfl(x, (lane & ~(N - 1)) + SRC);
}

// The value held by lane ^ OFF (OFF = 8, 16 or 32), without LDS: a DPP row
// rotation by 8 inside a 16-lane row, or the gfx950 permlane swaps, which
// exchange 16-lane rows (odd with even) or 32-lane halves of a register.
template <int OFF>
__device__ __forceinline__ float xor_lanes(float x)
{
    static_assert(OFF == 8 || OFF == 16 || OFF == 32, "lane offset");
    if constexpr (OFF == 8) {
        return dpp<0x128>(x);  // row_ror:8
    } else {
        const uint32_t u = __float_as_uint(x);
        const int lane = __lane_id();
        if constexpr (OFF == 16) {
            const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
            return __uint_as_float((lane & 16) ? r[0] : r[1]);
        } else {
            const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
            return __uint_as_float((lane & 32) ? r[0] : r[1]);
        }
    }
}

// ---- wave-wide integer primitives (DPP inside 16-lane rows, readlane across rows) ----

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x)
{
    return __builtin_amdgcn_mov_dpp(x, CTRL, 0xf, 0xf, false);
}

// the row shifts leave lanes whose source is outside the row at 0
template <int CTRL>
__device__ __forceinline__ int dpp_shr0(int x)
{
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}

// the wave's index in its workgroup, in a scalar register (the compiler does
// not infer that threadIdx.x / 64 is the same across a wave)
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

// Number of lanes of this wave below the calling lane whose bit is set in m.
__device__ __forceinline__ int lanes_below(uint64_t m)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x)
{
    x = min(x, (uint32_t)dpp_i<0xB1>((int)x));
    x = min(x, (uint32_t)dpp_i<0x4E>((int)x));
    x = min(x, (uint32_t)dpp_i<0x141>((int)x));
    x = min(x, (uint32_t)dpp_i<0x140>((int)x));
    const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
    const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
    return min(min(a, b), min(c, d));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x)
{
    x = max(x, (uint32_t)dpp_i<0xB1>((int)x));
    x = max(x, (uint32_t)dpp_i<0x4E>((int)x));
    x = max(x, (uint32_t)dpp_i<0x141>((int)x));
    x = max(x, (uint32_t)dpp_i<0x140>((int)x));
    const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
    const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
    return max(max(a, b), max(c, d));
}

// Inclusive prefix sum over the 64 lanes in lane order: row shifts by 1, 2,
// 4, 8 inside each 16-lane row, then the totals of the lower rows.
__device__ __forceinline__ int wave_inclusive_scan(int x)
{
    x += dpp_shr0<0x111>(x);  // row_shr:1
    x += dpp_shr0<0x112>(x);  // row_shr:2
    x += dpp_shr0<0x114>(x);  // row_shr:4
    x += dpp_shr0<0x118>(x);  // row_shr:8
    const int t0 = __builtin_amdgcn_readlane(x, 15), t1 = __builtin_amdgcn_readlane(x, 31);
    const int t2 = __builtin_amdgcn_readlane(x, 47);
    const int lane = __lane_id();
    return x + (lane < 16 ? 0 : lane < 32 ? t0 : lane < 48 ? t0 + t1 : t0 + t1 + t2);
}

// Exclusive scan of one int per thread over a workgroup of NT threads (NT/64
// waves); `wsum` holds NT/64 ints of LDS.  Every thread gets the total too.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int& total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int inc = wave_inclusive_scan(v);
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        before += w < wave ? wsum[w] : 0;
        total += wsum[w];
    }
    __syncthreads();  // wsum may be reused
    return before + inc - v;
}

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }

// A 16-byte load marked non-temporal, for what a kernel streams once (the K
// and V rows of a selecting step, the rows a copy moves): the streamed lines
// leave the caches to the data that is reused (block-table rows, scores,
// queries, partials).
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const void* p)
{
    const nt_u32x4 w = __builtin_nontemporal_load((const nt_u32x4*)p);
    return make_uint4(w.x, w.y, w.z, w.w);
}

// A workgroup barrier that orders LDS accesses only.  Global loads still in
// flight (those of a tile pipeline that ran past its last tile, whose
// results are not used) are not waited for, as __syncthreads would: on this
// chip one counter covers global loads and stores, and its release waits
// for all of them.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }

// n / d for 0 <= n < 2^31 with a host-computed magic pair (Granlund and
// Montgomery's round-up method): q = (umulhi(n, magic) + n) >> shift.
struct FastDiv {
    uint32_t d, magic, shift;
    __device__ __forceinline__ int div(int n) const
    {
        uint32_t hi = __umulhi((uint32_t)n, magic);
        return (int)((hi + (uint32_t)n) >> shift);
    }
};

// ---- the attended token set of one (sequence, KV head, row) ---------------
//
// Tokens in ascending position: the sink [0, se), the middle-region part of
// each selected page (pages ascending), then the window [ws, L).  Flat index
// f in [0, total) maps to a position.  Only the first and the last selected
// page can be cut by the region edges; interior candidates are whole pages.
// `parts` keeps the sink and window (bit 0) and/or the middle (bit 1).
template <typename SelPtr>
struct TokenSetT {
    int L, se, ws, P;
    int nsel;         // selected pages in use; -1 means every middle page (dense)
    int first_start;  // position of the first middle token of sel[0]
    int len0;         // middle tokens of sel[0]
    int mid_total;    // middle tokens attended
    int n_sink, n_mid;
    int total;
    SelPtr sel;

    __device__ __forceinline__ void init(int L_, int S, int W, int P_, SelPtr sel_, int count, int k_max,
                                         int parts)
    {
        L = L_;
        P = P_;
        se = imin(S, L);
        ws = imax(se, L - W);
        sel = sel_;
        nsel = 0;
        first_start = se;
        len0 = 0;
        mid_total = 0;
        if (ws > se) {
            if (sel_ == nullptr) {
                nsel = -1;
                mid_total = ws - se;
            } else {
                const int plo = se / P, phi = (ws - 1) / P;
                nsel = imax(0, imin(count, imin(k_max, phi - plo + 1)));
                if (nsel > 0) {
                    const int p0 = sel_[0];
                    first_start = imax(p0 * P, se);
                    len0 = imax(0, imin((p0 + 1) * P, ws) - first_start);
                    mid_total = len0;
                    if (nsel > 1) {
                        const int pl = sel_[nsel - 1];
                        const int lenl = imax(0, imin((pl + 1) * P, ws) - pl * P);
                        mid_total += (nsel - 2) * P + lenl;
                    }
                }
            }
        }
        n_sink = (parts & 1) ? se : 0;
        n_mid = (parts & 2) ? mid_total : 0;
        total = n_sink + n_mid + ((parts & 1) ? L - ws : 0);
    }

    // Position of flat index f; -1 when the entry does not name a middle
    // token (a bad selected page), so the caller skips it.
    __device__ __forceinline__ int position(int f, const FastDiv& pdiv) const
    {
        if (f < n_sink) return f;
        f -= n_sink;
        if (f >= n_mid) return ws + (f - n_mid);
        if (nsel < 0) return se + f;
        int t;
        if (f < len0) {
            t = first_start + f;
        } else {
            f -= len0;
            const int j = pdiv.div(f);
            t = sel[1 + j] * P + (f - j * P);
        }
        return (t >= se && t < ws) ? t : -1;
    }
};

typedef const __attribute__((address_space(3))) int32_t* lds_i32_ptr;
using TokenSet = TokenSetT<const int32_t*>;       // page list in global memory
using TokenSetLds = TokenSetT<lds_i32_ptr>;       // page list staged in LDS

}  // namespace sa
