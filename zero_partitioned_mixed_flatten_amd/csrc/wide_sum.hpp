// wide_sum.hpp -- the exact sum of squares of ANY finite binary32 values,
// rounded once to binary64: the pass that completes a reduction whose fast
// form (exact_norm.hpp for the fp32 gradient, the 1-bit scales' windowed
// sums) cannot vouch for its own result.
//
// Every finite binary32 value is x = M * 2^e with M an integer below 2^24
// and e >= -149 (IEEE-754 binary32), so x^2 = M^2 * 2^(2e) is a whole
// number of 2^-298 units below 2^256.  A workgroup adds the squares of its
// elements into kDigits base-2^32 digits of such units, each held in a 64-bit
// LDS word (one ds_add_u64 per nonzero digit, at most three per element), so
// no digit carries until the workgroup is done: every addition is below
// 2^32 and a workgroup adds at most 2^31 elements.  The workgroup then
// carries its digits and stores them as one partial; the last workgroup to
// arrive adds the partials digit by digit, carries, and rounds the integer
// to binary64 to nearest with ties to even.  The result does not depend on
// the grid or the order of the additions.
//
// The pass is launched after every fast reduction that may need it and reads
// a pending flag that the fast reduction left in device memory: when it is
// clear (always, on real shards of summed binary16 gradients) every
// workgroup returns at once.  The digit additions are LDS atomics, so the
// pass is bound by the LDS atomic rate, not by HBM; it runs only for inputs
// off the fast path.
#pragma once

#include <math.h>

#include "zero_internal.hpp"

namespace zero {
namespace wide {

constexpr int kDigits = 20;          // 640 bits: 2^256 * 2^298 times up to 2^86 elements
constexpr int kUnitExp = -298;       // units of 2^-298
constexpr int kBlock = 256;
constexpr uint64_t kMaxBlocks = 512;

struct alignas(16) WidePartial {
    uint64_t d[kDigits];
};
static_assert(sizeof(WidePartial) == 160, "wide partial layout");

// Workgroups of the wide pass for n elements: at least 2^16 elements each,
// at most kMaxBlocks of them (so at most 2^31 elements each for n <= 2^40).
__host__ __device__ inline uint64_t grid(uint64_t n)
{
    uint64_t g = (n + 65535) >> 16;
    if (g < 1) g = 1;
    if (g > kMaxBlocks) g = kMaxBlocks;
    return g;
}

// x^2 (x finite) as three base-2^32 digits d0, d1, d2 of weights 2^(32k),
// 2^(32(k+1)), 2^(32(k+2)) units; k = -1 for x = 0.
struct SquareDigits {
    int k;
    uint64_t d0, d1, d2;
};

__host__ __device__ inline SquareDigits square_digits(float x)
{
    const uint32_t b = __builtin_bit_cast(uint32_t, x);
    const uint32_t field = (b >> 23) & 0xFFu;
    uint64_t M = b & 0x7FFFFFu;
    int e = -149;                                   // subnormal or zero
    if (field) {
        M |= 0x800000u;                             // normal: hidden bit
        e = int(field) - 150;
    }
    if (M == 0)
        return SquareDigits{-1, 0, 0, 0};
    const int pos = 2 * e - kUnitExp;               // x^2 = M^2 * 2^pos units, 0 <= pos <= 508
    const int sh = pos & 31;
    const uint64_t sq = M * M;                      // below 2^48
    const uint64_t lo = sq << sh;                   // bits 0..63 of sq * 2^sh
    const uint64_t hi = sh ? (sq >> (64 - sh)) : 0; // bits 64..79
    return SquareDigits{pos >> 5, lo & 0xFFFFFFFFull, lo >> 32, hi};
}

// Adds x^2 (x finite) into the workgroup's LDS digits.
__device__ __forceinline__ void add_square(uint64_t* acc, float x)
{
    const SquareDigits s = square_digits(x);
    if (s.k < 0)
        return;
    if (s.d0)
        atomicAdd(reinterpret_cast<unsigned long long*>(acc + s.k), (unsigned long long)s.d0);
    if (s.d1)
        atomicAdd(reinterpret_cast<unsigned long long*>(acc + s.k + 1), (unsigned long long)s.d1);
    if (s.d2)
        atomicAdd(reinterpret_cast<unsigned long long*>(acc + s.k + 2), (unsigned long long)s.d2);
}

// Brings every digit below 2^32 (the top one keeps the rest).
__host__ __device__ inline void carry(uint64_t* d)
{
    for (int j = 0; j < kDigits - 1; ++j) {
        d[j + 1] += d[j] >> 32;
        d[j] &= 0xFFFFFFFFull;
    }
}

// The carried integer times 2^-298, rounded once to binary64 (nearest, ties
// to even): the top 64 bits go through the correctly rounded 64-bit
// conversion with every lower nonzero bit folded into bit 0 as a sticky bit,
// far below the rounding position.  The result is at least 2^-298 when the
// integer is nonzero: a normal binary64, so the final scaling is exact.
__host__ __device__ inline double to_f64(const uint64_t* d)
{
    int t = kDigits - 1;
    while (t > 0 && d[t] == 0)
        --t;
    if (t == 0)
        return ldexp(double(d[0]), kUnitExp);       // below 2^32: exact
    uint64_t w = (d[t] << 32) | d[t - 1];
    const int lz = __builtin_clzll(w);              // < 32: d[t] != 0
    bool sticky = false;
    for (int j = 0; j + 2 < t; ++j)
        sticky |= d[j] != 0;
    const uint64_t below = t >= 2 ? d[t - 2] : 0;
    if (lz) {
        w = (w << lz) | (below >> (32 - lz));
        sticky |= (below & ((uint64_t(1) << (32 - lz)) - 1)) != 0;
    } else {
        sticky |= below != 0;
    }
    return ldexp(double(w | (sticky ? 1u : 0u)), 32 * (t - 1) - lz + kUnitExp);
}

// The sum in units of 2^-48 as (hi, lo) when it is a whole number of them
// below 2^128; otherwise false.  2^-48 is 2^250 units of 2^-298.
__host__ __device__ inline bool to_units48(const uint64_t* d, uint64_t& hi, uint64_t& lo)
{
    for (int j = 0; j < 7; ++j)                     // bits 0..223
        if (d[j])
            return false;
    if (d[7] & 0x3FFFFFFull)                        // bits 224..249
        return false;
    if (d[11] >> 26)                                // bits 378..383
        return false;
    for (int j = 12; j < kDigits; ++j)
        if (d[j])
            return false;
    // bits 250..377 = digits 7..11 shifted right by 26
    lo = (d[7] >> 26) | (d[8] << 6) | (d[9] << 38);
    hi = (d[9] >> 26) | (d[10] << 6) | ((d[11] & 0x3FFFFFFull) << 38);
    return true;
}

// The pass.  Src has `float at(uint64_t i) const`, the i-th value whose
// square is summed; Fin has `bool pending() const` (the fast reduction asked
// for this pass), `uint32_t* counter() const` (an arrival counter that is 0
// between calls) and `void finish(const uint64_t* digits) const`, which the
// last workgroup's thread 0 calls with the carried total (it clears the
// pending flag).
template <typename Src, typename Fin>
__global__ __launch_bounds__(kBlock) void wide_sum_kernel(Src src, uint64_t n, Fin fin,
                                                          WidePartial* __restrict__ ws)
{
    if (!fin.pending())                             // the same answer for every workgroup
        return;
    __shared__ uint64_t acc[kDigits];
    if (threadIdx.x < kDigits)
        acc[threadIdx.x] = 0;
    __syncthreads();
    const uint64_t stride = uint64_t(gridDim.x) * kBlock;
    for (uint64_t i = uint64_t(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride)
        add_square(acc, src.at(i));
    __syncthreads();

    __shared__ uint32_t s_last;
    if (threadIdx.x == 0) {
        WidePartial p;
        for (int j = 0; j < kDigits; ++j)
            p.d[j] = acc[j];
        carry(p.d);
        ws[blockIdx.x] = p;
        // release this workgroup's partial; the last workgroup acquires everyone's
        const uint32_t prev = __hip_atomic_fetch_add(fin.counter(), 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = prev == gridDim.x - 1;
        if (last)
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_last = last ? 1u : 0u;
    }
    __syncthreads();
    if (!s_last)
        return;
    __shared__ uint64_t tot[kDigits];
    if (threadIdx.x < kDigits) {
        uint64_t t = 0;                             // at most 512 digits below 2^32
        for (uint32_t b = 0; b < gridDim.x; ++b)
            t += ws[b].d[threadIdx.x];
        tot[threadIdx.x] = t;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        carry(tot);
        fin.finish(tot);
        *fin.counter() = 0;                         // re-arm for the next call
    }
}

}  // namespace wide
}  // namespace zero
