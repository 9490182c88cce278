// exact_norm.hpp -- device helpers for the exact sum of squares of the
// gradient partition and its overflow test, shared by the standalone
// reductions (norm.hip) and the flattens that compute the sum while they
// copy (flatten.hip).
//
// The sum is an integer count of 2^-48 units.  Each thread keeps a few
// binary64 accumulators that cannot round under a per-thread bound of
// kNormMaxPerThread = 2^12 elements:
//
//   binary16 gradients: every square is a multiple of 2^-48 below 2^32, and
//   exact in binary32 (22 significant bits), where one mixed-precision fma
//   forms it from the binary16 value.
//     h = x^2 rounded to a multiple of 2^-8   ((x^2 + C) - C, C = 1.5*2^44)
//     l = x^2 - h, exactly                     (|l| <= 2^-9)
//     sum(h) stays a multiple of 2^-8 below 2^44, sum(l) a multiple of 2^-48
//     below 2^3.  An inf or NaN input leaves h or l non-finite, and finite
//     inputs cannot: that is the overflow test (no look at exponent fields).
//
//   binary32 gradients (the accumulation form): on the fast path every value
//   is a multiple of 2^-24 below 2^24 in magnitude (any binary32 sum of at
//   most 256 binary16 values is), so x^2 is a multiple of 2^-48 below 2^48.
//     a = x^2 rounded to a multiple of 2^16   (fma(x, x, C1) - C1, C1 = 1.5*2^68)
//     r = x^2 - a, exactly, |r| <= 2^15       (fma(x, x, -a))
//     b = r rounded to a multiple of 2^-16    ((r + C2) - C2, C2 = 1.5*2^36)
//     c = r - b, a multiple of 2^-48 on the fast path: ((. + C3) - C3,
//         C3 = 24) leaves it unchanged, and a value it changes marks a square
//         off the 2^-48 grid
//     sum(a) < 2^60 in steps of 2^16, sum(b) < 2^27 in steps of 2^-16,
//     sum(c) < 2^-5 in steps of 2^-48: 44 significant bits at most.
//   A value off the fast path (|x| >= 2^24, or a square off the grid) makes
//   the partial ask for the wide pass (wide_sum.hpp), which sums the squares
//   of any binary32 values exactly; an inf or NaN is an overflow.

// The sums become signed base-2^32 limbs that threads, workgroups and the
// grid add without carries.  A workgroup's partial is stored carried (each
// limb below 2^32, the top one below 2^30), so any number of partials up to
// 2^30 adds inside int64.
// At the end one thread carries the total into 128 bits and converts it to
// binary64 with a single round-to-nearest-even: the exactly rounded sum,
// independent of grid shape and schedule.  A total of 2^128 units or more
// (2^80; only binary32 values can get there) also asks for the wide pass.
#pragma once

#include <math.h>

#include "zero_internal.hpp"

namespace zero {
namespace exact {

// Status bits of a thread, a workgroup partial and a whole reduction.
constexpr uint32_t kOvf = 1u;       // an inf or NaN: the step is skipped
constexpr uint32_t kWide = 2u;      // the fast sum does not hold: the wide pass sums exactly

// ---- binary16 gradients ------------------------------------------------------------

constexpr double kSplit16 = 0x1.8p44;          // 1.5 * 2^44: its ulp is 2^-8

// Signed base-2^32 limbs of an integer count of 2^-48 units:
// l0 + l1*2^32 + l2*2^64 + l3*2^96.
struct Limbs {
    int64_t l0, l1, l2, l3;
};

struct Acc16 {
    double h = 0.0, l = 0.0;

    __device__ __forceinline__ void square(_Float16 v)
    {
        // x^2 exact in binary32; written as an fma with a zero addend so that
        // gfx950 forms it from the binary16 operand in one v_fma_mix_f32
        // (a plain product keeps a separate binary16 -> binary32 conversion)
        const float xf = float(v);
        const double s = double(__builtin_fmaf(xf, xf, 0.0f));
        const double hh = (s + kSplit16) - kSplit16;               // x^2 to a multiple of 2^-8
        h += hh;
        l += s - hh;                                               // x^2 - hh, exact
    }
    // Eight binary16 values in one 16-byte vector.
    __device__ __forceinline__ void vec(u32x4 v)
    {
        const f16x8 e = __builtin_bit_cast(f16x8, v);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            square(e[k]);
    }
    // One element given as its bit pattern.
    __device__ __forceinline__ void bits(uint16_t b) { square(__builtin_bit_cast(_Float16, b)); }
    // An inf or NaN among the values leaves a non-finite h or l (x = +-inf:
    // hh = inf, l gets inf - inf; NaN propagates), and finite values keep
    // both finite (h < 2^44, |l| < 2^3): the overflow test needs no
    // separate look at the exponent fields.
    __device__ __forceinline__ uint32_t status() const
    {
        return (__builtin_isfinite(h) && __builtin_isfinite(l)) ? 0u : kOvf;
    }
    // The thread's sum as limbs; an inf/NaN seen by the thread voids it
    // (the overflow flag makes the sum irrelevant anyway).
    __device__ __forceinline__ Limbs limbs() const
    {
        const bool bad = status() != 0;
        const int64_t hu = bad ? 0 : int64_t(h * 256.0);    // sum(h) / 2^-8, < 2^52
        const int64_t lu = bad ? 0 : int64_t(l * 0x1p48);   // sum(l) / 2^-48, |.| < 2^51
        const int64_t hs = hu << 8;                         // hu * 2^40 = hs * 2^32
        return Limbs{lu & 0xFFFFFFFFll, (hs & 0xFFFFFFFFll) + (lu >> 32), hs >> 32, 0};
    }
};

// ---- binary32 gradients ------------------------------------------------------------

constexpr double kSplit32Hi = 0x1.8p68;        // ulp 2^16
constexpr double kSplit32Mid = 0x1.8p36;       // ulp 2^-16
constexpr double kSplit32Lo = 0x1.8p4;         // ulp 2^-48

struct Acc32 {
    double a = 0.0, b = 0.0, c = 0.0;
    uint32_t big = 0;            // bit 31: some |x| >= 2^24 (0x4B800000), inf and NaN included
    uint32_t infnan = 0;         // bit 31: some inf or NaN (0x7F800000)
    bool off = false;            // some square off the 2^-48 grid

    __device__ __forceinline__ void add(float v)
    {
        const uint32_t u = __builtin_bit_cast(uint32_t, v) & 0x7FFFFFFFu;
        big |= u + 0x34800000u;
        infnan |= u + 0x00800000u;
        const double x = double(v);
        const double ha = __builtin_fma(x, x, kSplit32Hi) - kSplit32Hi;  // to a multiple of 2^16
        const double r = __builtin_fma(x, x, -ha);                        // exact, |r| <= 2^15
        const double hb = (r + kSplit32Mid) - kSplit32Mid;                // to a multiple of 2^-16
        const double d = r - hb;                                          // exact
        const double hc = (d + kSplit32Lo) - kSplit32Lo;                  // d itself on the fast path
        off |= hc != d;
        a += ha;
        b += hb;
        c += hc;
    }
    __device__ __forceinline__ void vec(f32x4 v)
    {
        add(v.x);
        add(v.y);
        add(v.z);
        add(v.w);
    }
    __device__ __forceinline__ uint32_t status() const
    {
        if (infnan & 0x80000000u)
            return kOvf;
        return ((big & 0x80000000u) || off) ? kWide : 0u;
    }
    __device__ __forceinline__ Limbs limbs() const
    {
        const bool bad = status() != 0;
        const int64_t la = bad ? 0 : int64_t(a * 0x1p-16);   // units of 2^16 = 2^64 * 2^-48, < 2^44
        const int64_t lb = bad ? 0 : int64_t(b * 0x1p16);    // units of 2^-16 = 2^32 * 2^-48, |.| < 2^43
        const int64_t lc = bad ? 0 : int64_t(c * 0x1p48);    // units of 2^-48, |.| < 2^43
        return Limbs{lc, lb, la, 0};
    }
};

// ---- limbs -------------------------------------------------------------------------

// Carries l0, l1, l2 into [0, 2^32); the value is unchanged and >= 0, so l3
// ends up >= 0.
__host__ __device__ __forceinline__ Limbs carry(Limbs s)
{
    s.l1 += s.l0 >> 32;
    s.l0 &= 0xFFFFFFFFll;
    s.l2 += s.l1 >> 32;
    s.l1 &= 0xFFFFFFFFll;
    s.l3 += s.l2 >> 32;
    s.l2 &= 0xFFFFFFFFll;
    return s;
}

// Adds a stored partial as four 32-bit limbs and ORs in its status bits.
__host__ __device__ __forceinline__ void fold_partial(Limbs& s, uint32_t& flag, const NormPartial& p)
{
    s.l0 += int64_t(p.w0 & 0xFFFFFFFFull);
    s.l1 += int64_t(p.w0 >> 32);
    s.l2 += int64_t(p.w1 & 0xFFFFFFFFull);
    s.l3 += int64_t((p.w1 >> 32) & 0x3FFFFFFFull);
    flag |= uint32_t(p.w1 >> kPartialStatusShift);
}

// The total as an unsigned 128-bit value; false if it is 2^128 or more.
__host__ __device__ __forceinline__ bool limbs_to_u128(Limbs s, uint64_t& hi, uint64_t& lo)
{
    s = carry(s);
    lo = uint64_t(s.l0) | (uint64_t(s.l1) << 32);
    hi = uint64_t(s.l2) | (uint64_t(s.l3) << 32);
    return (s.l3 >> 32) == 0;
}

// Sums limbs and ORs flags over BLOCK threads (every one of them must call
// it); the result is valid in thread 0.  BLOCK = 64 is one wave: lane
// shuffles only, no LDS and no barrier, so the other waves of the workgroup
// may have exited.  A larger BLOCK is the whole workgroup and ends with a
// barrier, so the LDS it uses may be reused right after.
template <int BLOCK>
__device__ __forceinline__ void block_fold(Limbs& s, uint32_t& flag)
{
    __shared__ int64_t s0[BLOCK / 64], s1[BLOCK / 64], s2[BLOCK / 64], s3[BLOCK / 64];
    __shared__ uint32_t sf[BLOCK / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        s.l0 += __shfl_xor(s.l0, off, 64);
        s.l1 += __shfl_xor(s.l1, off, 64);
        s.l2 += __shfl_xor(s.l2, off, 64);
        s.l3 += __shfl_xor(s.l3, off, 64);
        flag |= __shfl_xor(flag, off, 64);
    }
    if (BLOCK > 64) {
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) {
            s0[wave] = s.l0;
            s1[wave] = s.l1;
            s2[wave] = s.l2;
            s3[wave] = s.l3;
            sf[wave] = flag;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int w = 1; w < BLOCK / 64; ++w) {
                s.l0 += s0[w];
                s.l1 += s1[w];
                s.l2 += s2[w];
                s.l3 += s3[w];
                flag |= sf[w];
            }
        }
        __syncthreads();
    }
}

// A workgroup's partial: the carried sum and the status bits (kOvf, kWide
// fit the two bits); a sum of 2^126 units or more asks for the wide pass,
// and then its value is not used.
__host__ __device__ __forceinline__ NormPartial make_partial(Limbs s, uint32_t status)
{
    static_assert((kOvf | kWide) < 4u, "status bits");
    s = carry(s);
    if (s.l3 >> 30)
        status |= kWide;
    NormPartial p;
    p.w0 = uint64_t(s.l0) | (uint64_t(s.l1) << 32);
    p.w1 = uint64_t(s.l2) | (uint64_t(s.l3 & 0x3FFFFFFFll) << 32) | (uint64_t(status) << kPartialStatusShift);
    return p;
}

}  // namespace exact
}  // namespace zero
