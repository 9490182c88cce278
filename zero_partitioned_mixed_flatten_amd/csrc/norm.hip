// norm.hip -- exact squared L2 norm + inf/NaN test of a rank's flat fp16
// gradient partition, and the step decision that follows from them (dynamic
// loss scaling with skip-step, Micikevicius et al. 2018; global-norm
// clipping, Pascanu et al. 2013; Adam's bias corrections, Kingma & Ba 2015).
// The pages fix the gradient as fp16 and the optimizer state as fp32 (ZeRO
// paper card, "Bottleneck"); the rest of this step is the published methods.
//
// Exactness instead of a rounded floating-point sum.  Every square of a
// finite binary16 value is an integer multiple of 2^-48 below 2^32.  Each
// thread keeps two binary64 accumulators that stay exact by construction:
//   hh = x^2 rounded to a multiple of 2^-8   (fma(x, x, C) - C, C = 1.5*2^44)
//   lo = x^2 - hh, exactly                    (fma(x, x, -hh), |lo| <= 2^-9)
// With at most kNormMaxPerThread = 2^12 elements per thread, sum(hh) stays a
// multiple of 2^-8 below 2^44 and sum(lo) a multiple of 2^-48 below 2^3, so
// neither addition ever rounds.  The two sums become integers of 2^-48 units,
// split into signed base-2^32 limbs that workgroups and the grid add without
// carries; one thread propagates the carries at the end and converts the
// 128-bit total to binary64 with a single round-to-nearest-even.  The result
// is the exactly rounded sum, independent of grid shape and schedule, so the
// clip factor derived from it is bitwise reproducible.
//
// Shape for gfx950: 1024-thread workgroups, at most one per CU (256), each
// thread streaming 16-byte vectors (8 elements) with four nontemporal loads
// in flight; about 8 VALU operations per element.  The last workgroup to arrive
// (agent-scope acq_rel counter, one increment per workgroup) folds the
// partials, takes the decision in binary64 on one thread and writes it into
// the step state.  Pure streaming (2 bytes per element read): no MFMA.
#include <math.h>

#include "zero_internal.hpp"

namespace zero {
namespace {

struct DecideArgs {
    double lr, beta1, beta2, eps, wd, clip, backoff, growth, min_scale;
    int32_t growth_interval;
};

constexpr double kSplit = 0x1.8p44;           // 1.5 * 2^44: its ulp is 2^-8

// The exponent test adds 0x0400 to each masked exponent field of a word that
// holds two binary16 values: only an all-ones field carries into bit 15
// (resp. 31), and the low half never carries into the high half.
__device__ __forceinline__ uint32_t exp_test(u32x4 v)
{
    return ((v.x & 0x7C007C00u) + 0x04000400u) | ((v.y & 0x7C007C00u) + 0x04000400u) |
           ((v.z & 0x7C007C00u) + 0x04000400u) | ((v.w & 0x7C007C00u) + 0x04000400u);
}

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

// Signed base-2^32 limbs of an integer count of 2^-48 units.
struct Limbs {
    int64_t l0, l1, l2;
};

__device__ __forceinline__ Limbs to_limbs(double ah, double al)
{
    const int64_t hu = int64_t(ah * 256.0);       // sum(hh) / 2^-8, < 2^52
    const int64_t lu = int64_t(al * 0x1p48);      // sum(lo) / 2^-48, |.| < 2^51
    const int64_t hs = hu << 8;                   // hu * 2^40 = hs * 2^32
    return Limbs{lu & 0xFFFFFFFFll, (hs & 0xFFFFFFFFll) + (lu >> 32), hs >> 32};
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

// Exact unsigned 128-bit integer -> binary64, round to nearest even: the top
// 64 significant bits go through the (correctly rounded) 64-bit conversion
// with every lower nonzero bit folded into bit 0 as a sticky bit, far below
// the rounding position.
__device__ double u128_to_f64(uint64_t hi, uint64_t lo)
{
    if (hi == 0)
        return double(lo);
    const int lz = __clzll(hi);
    const uint64_t top = lz ? ((hi << lz) | (lo >> (64 - lz))) : hi;
    const uint64_t rest = lz ? (lo << lz) : lo;
    return ldexp(double(top | (rest != 0 ? 1u : 0u)), 64 - lz);
}

__device__ void decide(zero_step_state_t* st, const DecideArgs& d, uint64_t hi, uint64_t lo, bool ovf)
{
    const double S = st->loss_scale;
    st->sumsq_units[0] = lo;
    st->sumsq_units[1] = hi;
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
    const double sumsq = ldexp(u128_to_f64(hi, lo), -48);
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

// Sums limbs and ORs flags over the workgroup; the result is valid in thread 0.
__device__ __forceinline__ void block_fold(Limbs& s, uint32_t& flag)
{
    __shared__ int64_t s0[kNormBlock / 64], s1[kNormBlock / 64], s2[kNormBlock / 64];
    __shared__ uint32_t sf[kNormBlock / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        s.l0 += __shfl_xor(s.l0, off, 64);
        s.l1 += __shfl_xor(s.l1, off, 64);
        s.l2 += __shfl_xor(s.l2, off, 64);
        flag |= __shfl_xor(flag, off, 64);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s0[wave] = s.l0;
        s1[wave] = s.l1;
        s2[wave] = s.l2;
        sf[wave] = flag;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kNormBlock / 64; ++w) {
            s.l0 += s0[w];
            s.l1 += s1[w];
            s.l2 += s2[w];
            flag |= sf[w];
        }
    }
    __syncthreads();                               // the arrays are reused by the last workgroup
}

__global__ __launch_bounds__(kNormBlock) void norm_overflow_kernel(const uint16_t* __restrict__ g, uint64_t n,
                                                                   zero_step_state_t* __restrict__ st,
                                                                   NormPartial* __restrict__ ws, DecideArgs d)
{
    double ah = 0.0, al = 0.0;
    uint32_t flag = 0;
    const uint64_t nvec = n >> 3;
    const u32x4* __restrict__ gv = reinterpret_cast<const u32x4*>(g);
    const uint64_t stride = uint64_t(gridDim.x) * kNormBlock;
    uint64_t j = uint64_t(blockIdx.x) * kNormBlock + threadIdx.x;
    for (; j + 3 * stride < nvec; j += 4 * stride) {      // four 16-byte loads in flight
        const u32x4 a = __builtin_nontemporal_load(gv + j);
        const u32x4 b = __builtin_nontemporal_load(gv + j + stride);
        const u32x4 c = __builtin_nontemporal_load(gv + j + 2 * stride);
        const u32x4 e = __builtin_nontemporal_load(gv + j + 3 * stride);
        acc_vec(a, ah, al, flag);
        acc_vec(b, ah, al, flag);
        acc_vec(c, ah, al, flag);
        acc_vec(e, ah, al, flag);
    }
    for (; j < nvec; j += stride)
        acc_vec(__builtin_nontemporal_load(gv + j), ah, al, flag);
    if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {         // the last n % 8 elements
        const uint16_t h = g[(nvec << 3) + threadIdx.x];
        flag |= (h & 0x7C00u) + 0x0400u;
        acc_square(__builtin_bit_cast(_Float16, h), ah, al);
    }
    if (flag & 0x80008000u) {                              // an inf/NaN: the sum is void
        ah = 0.0;
        al = 0.0;
    }

    Limbs s = to_limbs(ah, al);
    block_fold(s, flag);

    __shared__ uint32_t s_last;
    if (threadIdx.x == 0) {
        NormPartial p;
        p.l0 = s.l0;
        p.l1 = s.l1;
        p.l2 = s.l2;
        p.flag = flag;
        p.pad = 0;
        ws[blockIdx.x] = p;
        // release this block's partial / acquire everyone else's
        const uint32_t prev = __hip_atomic_fetch_add(&st->done_blocks, 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == gridDim.x - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (!s_last)
        return;

    // Last workgroup: fold every partial (integer limbs: order is irrelevant).
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    Limbs t{0, 0, 0};
    uint32_t tflag = 0;
    for (uint32_t b = threadIdx.x; b < gridDim.x; b += kNormBlock) {
        const NormPartial p = ws[b];
        t.l0 += p.l0;
        t.l1 += p.l1;
        t.l2 += p.l2;
        tflag |= p.flag;
    }
    block_fold(t, tflag);
    if (threadIdx.x == 0) {
        uint64_t hi, lo;
        limbs_to_u128(t, hi, lo);
        decide(st, d, hi, lo, (tflag & 0x80008000u) != 0);
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
