// exact_norm.hpp -- device helpers for the exact sum of squares of binary16
// gradients and the step decision, shared by the standalone reduction
// (norm.hip) and the flatten that computes the sum while it copies
// (flatten.hip).
//
// Every square of a finite binary16 value is an integer multiple of 2^-48
// below 2^32.  Each thread keeps two binary64 accumulators that stay exact by
// construction:
//   hh = x^2 rounded to a multiple of 2^-8   (fma(x, x, C) - C, C = 1.5*2^44)
//   lo = x^2 - hh, exactly                    (fma(x, x, -hh), |lo| <= 2^-9)
// With at most kNormMaxPerThread = 2^12 elements per thread, sum(hh) stays a
// multiple of 2^-8 below 2^44 and sum(lo) a multiple of 2^-48 below 2^3, so
// neither addition ever rounds.  The two sums become integers of 2^-48 units,
// split into signed base-2^32 limbs that workgroups and the grid add without
// carries; one thread propagates the carries at the end and converts the
// 128-bit total to binary64 with a single round-to-nearest-even.  The result
// is the exactly rounded sum, independent of grid shape and schedule.
#pragma once

#include <math.h>

#include "zero_internal.hpp"

namespace zero {
namespace exact {

constexpr double kSplit = 0x1.8p44;           // 1.5 * 2^44: its ulp is 2^-8

// The exponent test adds 0x0400 to each masked exponent field of a word that
// holds two binary16 values: only an all-ones field carries into bit 15
// (resp. 31), and the low half never carries into the high half.
__device__ __forceinline__ uint32_t exp_test(uint32_t w) { return (w & 0x7C007C00u) + 0x04000400u; }

__device__ __forceinline__ uint32_t exp_test(u32x4 v)
{
    return exp_test(v.x) | exp_test(v.y) | exp_test(v.z) | exp_test(v.w);
}

constexpr uint32_t kOverflowBits = 0x80008000u;

__device__ __forceinline__ void acc_square(_Float16 h, double& ah, double& al)
{
    const double x = double(float(h));                       // exact
    const double hh = __builtin_fma(x, x, kSplit) - kSplit;  // x^2 to a multiple of 2^-8
    ah += hh;
    al += __builtin_fma(x, x, -hh);                          // x^2 - hh, exact
}

__device__ __forceinline__ void acc_vec(u32x4 v, double& ah, double& al, uint32_t& flag)
{
    flag |= exp_test(v);
    const f16x8 h = __builtin_bit_cast(f16x8, v);
#pragma unroll
    for (int k = 0; k < 8; ++k)
        acc_square(h[k], ah, al);
}

// One binary16 element given as its bit pattern.
__device__ __forceinline__ void acc_bits(uint16_t b, double& ah, double& al, uint32_t& flag)
{
    flag |= (uint32_t(b) & 0x7C00u) + 0x0400u;
    acc_square(__builtin_bit_cast(_Float16, b), ah, al);
}

// Signed base-2^32 limbs of an integer count of 2^-48 units.
struct Limbs {
    int64_t l0, l1, l2;
};

// A thread's exact accumulators as limbs; an inf/NaN seen by the thread
// (flag) voids its sum, which the overflow flag makes irrelevant anyway.
__device__ __forceinline__ Limbs to_limbs(double ah, double al, uint32_t flag)
{
    if (flag & kOverflowBits) {
        ah = 0.0;
        al = 0.0;
    }
    const int64_t hu = int64_t(ah * 256.0);       // sum(hh) / 2^-8, < 2^52
    const int64_t lu = int64_t(al * 0x1p48);      // sum(lo) / 2^-48, |.| < 2^51
    const int64_t hs = hu << 8;                   // hu * 2^40 = hs * 2^32
    return Limbs{lu & 0xFFFFFFFFll, (hs & 0xFFFFFFFFll) + (lu >> 32), hs >> 32};
}

// Carries l0 and l1 into [0, 2^32) (the value is unchanged and >= 0, so l2
// ends up >= 0).  Stored partials are normalised, so any number of them up
// to 2^30 can be added in int64.
__device__ __forceinline__ Limbs normalize(Limbs s)
{
    const int64_t c0 = s.l0 >> 32;
    s.l0 &= 0xFFFFFFFFll;
    s.l1 += c0;
    const int64_t c1 = s.l1 >> 32;
    s.l1 &= 0xFFFFFFFFll;
    s.l2 += c1;
    return s;
}

// Carries the limbs into an unsigned 128-bit value (the total is >= 0).
__device__ __forceinline__ void limbs_to_u128(Limbs s, uint64_t& hi, uint64_t& lo)
{
    const int64_t c0 = s.l0 >> 32;
    const uint64_t w0 = uint64_t(s.l0) & 0xFFFFFFFFull;
    const int64_t t1 = s.l1 + c0;
    const uint64_t w1 = uint64_t(t1) & 0xFFFFFFFFull;
    const int64_t t2 = s.l2 + (t1 >> 32);        // limbs 2 and up, < 2^63
    lo = w0 | (w1 << 32);
    hi = uint64_t(t2);
}

// Sums limbs and ORs flags over a workgroup of BLOCK threads (every thread
// must call it); the result is valid in thread 0.  Ends with a barrier, so
// the LDS it uses may be reused right after.
template <int BLOCK>
__device__ __forceinline__ void block_fold(Limbs& s, uint32_t& flag)
{
    __shared__ int64_t s0[BLOCK / 64], s1[BLOCK / 64], s2[BLOCK / 64];
    __shared__ uint32_t sf[BLOCK / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        s.l0 += __shfl_xor(s.l0, off, 64);
        s.l1 += __shfl_xor(s.l1, off, 64);
        s.l2 += __shfl_xor(s.l2, off, 64);
        flag |= __shfl_xor(flag, off, 64);
    }
    if (BLOCK > 64) {
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) {
            s0[wave] = s.l0;
            s1[wave] = s.l1;
            s2[wave] = s.l2;
            sf[wave] = flag;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int w = 1; w < BLOCK / 64; ++w) {
                s.l0 += s0[w];
                s.l1 += s1[w];
                s.l2 += s2[w];
                flag |= sf[w];
            }
        }
        __syncthreads();
    }
}

__device__ __forceinline__ NormPartial make_partial(Limbs s, uint32_t flag)
{
    s = normalize(s);
    NormPartial p;
    p.l0 = s.l0;
    p.l1 = s.l1;
    p.l2 = s.l2;
    p.flag = flag;
    p.pad = 0;
    return p;
}

}  // namespace exact
}  // namespace zero
