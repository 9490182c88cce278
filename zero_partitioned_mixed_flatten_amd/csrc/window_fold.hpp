// window_fold.hpp -- the integer core of the 1-bit stage's scale folds
// (onebit.hip): a workgroup's window sum read back from its carried partial,
// moved onto a coarser window with rounding, and the test of whether the
// error interval around the folded integer can change its binary64 rounding.
// Host and device code, so that the same functions also run on the CPU
// against exact Python integers (tests/sanitize/window_driver.cpp).
#pragma once

#include "decide.hpp"
#include "exact_norm.hpp"

namespace zero {
namespace window {

// A carried partial as a 128-bit integer (its status bits are zero here).
__host__ __device__ __forceinline__ unsigned __int128 partial_value(const NormPartial& p)
{
    return ((unsigned __int128)(p.w1 & ((uint64_t(1) << kPartialStatusShift) - 1)) << 64) | p.w0;
}

// Adds v * 2^-d rounded to the nearest integer (ties up) to the limbs; v is
// below 2^126 and d >= 0.
__host__ __device__ __forceinline__ void add_moved(exact::Limbs& s, unsigned __int128 v, int d)
{
    if (d >= 127)
        return;                                               // below half a unit
    if (d > 0)
        v = (v + ((unsigned __int128)1 << (d - 1))) >> d;
    s.l0 += int64_t(uint64_t(v) & 0xFFFFFFFFull);
    s.l1 += int64_t(uint64_t(v) >> 32);
    s.l2 += int64_t(uint64_t(v >> 64) & 0xFFFFFFFFull);
    s.l3 += int64_t(uint64_t(v >> 96));
}

// W = hi*2^64 + lo lies within half/2 units of the exact sum.  Rounding to
// binary64 is monotonic: when W - half/2 and W + half/2 round to the same
// value, every sum between them does, and that is the exactly rounded sum.
// (The 1-bit folds have W >= 2^79 whenever a value is nonzero and half below
// 2^42, so 2W - half > 0.)  Otherwise the wide pass decides.
__host__ __device__ __forceinline__ bool decides(uint64_t hi, uint64_t lo, uint64_t half)
{
    const unsigned __int128 w2 = ((unsigned __int128)hi << 65) | ((unsigned __int128)lo << 1);   // 2W < 2^124
    const unsigned __int128 a = w2 - half, b = w2 + half;
    return u128_to_f64(uint64_t(a >> 64), uint64_t(a)) == u128_to_f64(uint64_t(b >> 64), uint64_t(b));
}

}  // namespace window
}  // namespace zero
