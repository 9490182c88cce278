// norm.hip -- exact squared L2 norm + inf/NaN test of a rank's flat fp16
// gradient partition, and the step decision that follows from them (dynamic
// loss scaling with skip-step, Micikevicius et al. 2018; global-norm
// clipping, Pascanu et al. 2013; Adam's bias corrections, Kingma & Ba 2015).
// The pages fix the gradient as fp16 and the optimizer state as fp32 (ZeRO
// paper card, "Bottleneck"); the rest of this step is the published methods.
//
// Exactness instead of a floating-point sum.  A finite binary16 value is
// M * 2^(E'-25) with an 11-bit integer M and E' = max(E, 1), so its square is
// M^2 * 2^(2E'-2) units of 2^-48: an integer below 2^80.  Each thread adds
// these integers into a 96-bit accumulator, workgroups fold them into 128
// bits, and the last workgroup converts the total to binary64 with a single
// round-to-nearest-even.  The result is therefore the exactly rounded sum,
// independent of the grid, the wavefront schedule and the device -- which is
// what lets the clip factor derived from it be bitwise reproducible.
//
// Pass structure (one launch, no host synchronisation):
//   every workgroup: grid-stride over 16-byte vectors (8 elements), integer
//     square-accumulate + exponent test, wavefront shuffle reduction, then an
//     LDS fold across the 4 wavefronts; thread 0 stores the block partial and
//     increments an arrival counter with agent-scope acquire/release;
//   the last workgroup to arrive folds all partials (integer addition, so
//     the order is irrelevant), converts, takes the decision in binary64 on one
//     thread and writes it to the step state, then re-arms the counter.
// Pure streaming (2 bytes per element read): no MFMA.
#include <math.h>

#include "zero_internal.hpp"

namespace zero {
namespace {

struct DecideArgs {
    double lr, beta1, beta2, eps, wd, clip, backoff, growth, min_scale;
    int32_t growth_interval;
};

struct U128 {
    uint64_t lo, hi;
};

__device__ __forceinline__ U128 add128(U128 a, U128 b)
{
    U128 r;
    r.lo = a.lo + b.lo;
    r.hi = a.hi + b.hi + (r.lo < a.lo ? 1 : 0);
    return r;
}

// Adds the square of the binary16 value in the low 16 bits of h, in units
// of 2^-48, to the 96-bit (lo, hi) accumulator.  Exponent 31 (inf/NaN)
// contributes an arbitrary finite amount; the flag makes the sum irrelevant.
__device__ __forceinline__ void acc_square(uint32_t h, uint64_t& lo, uint32_t& hi)
{
    const uint32_t e = (h >> 10) & 31u;
    const uint32_t m = (h & 1023u) | (e ? 1024u : 0u);
    const uint32_t s = e ? 2u * e - 2u : 0u;                 // 2*max(e,1) - 2, 0..60
    const uint64_t sq = uint64_t(m * m);                     // < 2^22
    const uint64_t l = sq << s;                              // bits 0..63
    const uint32_t h2 = uint32_t((sq << (s > 32u ? s - 32u : 0u)) >> 32);  // bits 64..95
    const uint64_t nl = lo + l;
    hi += h2 + (nl < l ? 1u : 0u);
    lo = nl;
}

// Two binary16 values per 32-bit word.  The exponent test adds 0x0400 to
// each masked exponent field: only an all-ones field carries into bit 15
// (resp. 31), and the low half never carries into the high half.
__device__ __forceinline__ void acc_word(uint32_t w, uint64_t& lo, uint32_t& hi, uint32_t& flag)
{
    flag |= (w & 0x7C007C00u) + 0x04000400u;
    acc_square(w & 0xFFFFu, lo, hi);
    acc_square(w >> 16, lo, hi);
}

__device__ __forceinline__ void acc_vec(u32x4 v, uint64_t& lo, uint32_t& hi, uint32_t& flag)
{
    acc_word(v.x, lo, hi, flag);
    acc_word(v.y, lo, hi, flag);
    acc_word(v.z, lo, hi, flag);
    acc_word(v.w, lo, hi, flag);
}

// Exact unsigned 128-bit integer -> binary64, round to nearest even.  The
// top 64 significant bits go through the (correctly rounded) 64-bit
// conversion with every lower nonzero bit folded into bit 0 as a sticky bit;
// bit 0 lies far below the rounding position, so the rounding is exact.
__device__ double u128_to_f64(uint64_t hi, uint64_t lo)
{
    if (hi == 0)
        return double(lo);
    const int lz = __clzll(hi);
    const uint64_t top = lz ? ((hi << lz) | (lo >> (64 - lz))) : hi;
    const uint64_t rest = lz ? (lo << lz) : lo;
    return ldexp(double(top | (rest != 0 ? 1u : 0u)), 64 - lz);
}

__device__ void decide(zero_step_state_t* st, const DecideArgs& d, U128 units, bool ovf)
{
    const double S = st->loss_scale;
    st->sumsq_units[0] = units.lo;
    st->sumsq_units[1] = units.hi;
    st->overflow = ovf ? 1 : 0;
    if (ovf) {
        const double s2 = S * d.backoff;
        st->loss_scale = s2 < d.min_scale ? d.min_scale : s2;
        st->good_steps = 0;
        st->skipped_total += 1;
        st->skip = 1;
        st->sumsq = INFINITY;
        st->grad_norm = INFINITY;
        st->gmul = 0.0f;
        return;
    }
    const double sumsq = ldexp(u128_to_f64(units.hi, units.lo), -48);
    const double norm = sqrt(sumsq) / S;
    st->skip = 0;
    st->sumsq = sumsq;
    st->grad_norm = norm;
    st->step += 1;
    const double b1p = st->beta1_pow * d.beta1;
    const double b2p = st->beta2_pow * d.beta2;
    st->beta1_pow = b1p;
    st->beta2_pow = b2p;
    const double coef = (d.clip > 0.0 && norm > d.clip) ? d.clip / norm : 1.0;
    st->gmul = float(coef / S);
    st->bc1 = float(1.0 - b1p);
    st->bc2 = float(1.0 - b2p);
    st->lr = float(d.lr);
    st->beta1 = float(d.beta1);
    st->beta2 = float(d.beta2);
    st->omb1 = float(1.0 - d.beta1);
    st->omb2 = float(1.0 - d.beta2);
    st->eps = float(d.eps);
    st->wd = float(d.wd);
    int32_t good = st->good_steps + 1;
    if (d.growth_interval > 0 && good >= d.growth_interval) {
        st->loss_scale = S * d.growth;
        good = 0;
    }
    st->good_steps = good;
}

// Folds (lo, hi, flag) over the workgroup; the result is valid in thread 0.
__device__ __forceinline__ void block_fold(U128& acc, uint32_t& flag)
{
    __shared__ uint64_t s_lo[kNormBlock / 64], s_hi[kNormBlock / 64];
    __shared__ uint32_t s_flag[kNormBlock / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        U128 o;
        o.lo = __shfl_xor(acc.lo, off, 64);
        o.hi = __shfl_xor(acc.hi, off, 64);
        flag |= __shfl_xor(flag, off, 64);
        acc = add128(acc, o);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s_lo[wave] = acc.lo;
        s_hi[wave] = acc.hi;
        s_flag[wave] = flag;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kNormBlock / 64; ++w) {
            acc = add128(acc, U128{s_lo[w], s_hi[w]});
            flag |= s_flag[w];
        }
    }
}

__global__ __launch_bounds__(kNormBlock) void norm_overflow_kernel(const uint16_t* __restrict__ g, uint64_t n,
                                                                   zero_step_state_t* __restrict__ st,
                                                                   NormPartial* __restrict__ ws, DecideArgs d)
{
    uint64_t lo = 0;
    uint32_t hi = 0, flag = 0;
    const uint64_t nvec = n >> 3;
    const u32x4* __restrict__ gv = reinterpret_cast<const u32x4*>(g);
    const uint64_t stride = uint64_t(gridDim.x) * kNormBlock;
    uint64_t j = uint64_t(blockIdx.x) * kNormBlock + threadIdx.x;
    for (; j + 3 * stride < nvec; j += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(gv + j);
        const u32x4 b = __builtin_nontemporal_load(gv + j + stride);
        const u32x4 c = __builtin_nontemporal_load(gv + j + 2 * stride);
        const u32x4 e = __builtin_nontemporal_load(gv + j + 3 * stride);
        acc_vec(a, lo, hi, flag);
        acc_vec(b, lo, hi, flag);
        acc_vec(c, lo, hi, flag);
        acc_vec(e, lo, hi, flag);
    }
    for (; j < nvec; j += stride)
        acc_vec(__builtin_nontemporal_load(gv + j), lo, hi, flag);
    if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {        // the last n % 8 elements
        const uint32_t h = g[(nvec << 3) + threadIdx.x];
        flag |= (h & 0x7C00u) + 0x0400u;
        acc_square(h, lo, hi);
    }

    U128 acc{lo, hi};
    block_fold(acc, flag);

    __shared__ uint32_t s_last;
    if (threadIdx.x == 0) {
        NormPartial p;
        p.lo = acc.lo;
        p.hi = acc.hi;
        p.flag = flag;
        p.pad[0] = p.pad[1] = p.pad[2] = 0;
        ws[blockIdx.x] = p;
        // release this block's partial / acquire everyone else's
        const uint32_t prev = __hip_atomic_fetch_add(&st->done_blocks, 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == gridDim.x - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (!s_last)
        return;

    // Last workgroup: fold every partial.
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");      // acquire for every thread of this block
    U128 tot{0, 0};
    uint32_t tflag = 0;
    for (uint32_t b = threadIdx.x; b < gridDim.x; b += kNormBlock) {
        const NormPartial p = ws[b];
        tot = add128(tot, U128{p.lo, p.hi});
        tflag |= p.flag;
    }
    block_fold(tot, tflag);
    if (threadIdx.x == 0) {
        decide(st, d, tot, (tflag & 0x80008000u) != 0);
        st->done_blocks = 0;                                 // re-arm for the next call
    }
}

bool finite_all(const zero_hparams_t* hp)
{
    const double v[] = {hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->max_grad_norm,
                        hp->backoff, hp->growth, hp->min_scale};
    for (double x : v)
        if (!isfinite(x))
            return false;
    return true;
}

}  // namespace
}  // namespace zero

using namespace zero;

extern "C" int zero_shard_norm_overflow(const uint16_t* grad16, uint64_t n, const zero_hparams_t* hp,
                                        zero_step_state_t* dev_state, void* workspace,
                                        size_t workspace_bytes, void* stream)
{
    if (!hp || !dev_state || !workspace || (n && !grad16))
        return ZERO_EINVAL;
    if (!finite_all(hp) || hp->lr < 0 || hp->beta1 < 0 || hp->beta1 >= 1 || hp->beta2 < 0 ||
        hp->beta2 >= 1 || hp->eps <= 0 || hp->weight_decay < 0 || hp->backoff <= 0 ||
        hp->backoff > 1 || hp->growth < 1 || hp->min_scale <= 0)
        return ZERO_EINVAL;
    if ((n && !is_aligned(grad16, 16)) || !is_aligned(dev_state, 8) || !is_aligned(workspace, 16))
        return ZERO_EALIGN;
    if (n > kNormMaxElems)
        return ZERO_ERANGE;
    const uint64_t grid = norm_grid(n);
    if (workspace_bytes < grid * sizeof(NormPartial))
        return ZERO_ERANGE;
    DecideArgs d;
    d.lr = hp->lr;
    d.beta1 = hp->beta1;
    d.beta2 = hp->beta2;
    d.eps = hp->eps;
    d.wd = hp->weight_decay;
    d.clip = hp->max_grad_norm;
    d.backoff = hp->backoff;
    d.growth = hp->growth;
    d.min_scale = hp->min_scale;
    d.growth_interval = hp->growth_interval;
    hipLaunchKernelGGL(norm_overflow_kernel, dim3(uint32_t(grid)), dim3(kNormBlock), 0, (hipStream_t)stream,
                       grad16, n, dev_state, static_cast<NormPartial*>(workspace), d);
    return launch_status();
}
