// decide.hpp -- the step decision, one source for the GPU reductions
// (norm.hip) and the host step (host_step.cpp): dynamic loss scaling with
// skip-step (Micikevicius et al. 2018), clipping by the global norm (Pascanu
// et al. 2013) and Adam's bias corrections (Kingma & Ba 2015), from the exact
// sum of squares.  All scalar arithmetic is binary64, each value rounded once
// to binary32 where it enters the element update.
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "zero_mi355x.h"

namespace zero {

struct DecideArgs {
    double lr, beta1, beta2, eps, wd, clip, backoff, growth, min_scale;
    int32_t growth_interval;
};

// Exact unsigned 128-bit integer -> binary64, round to nearest even: the top
// 64 significant bits go through the (correctly rounded) 64-bit conversion
// with every lower nonzero bit folded into bit 0 as a sticky bit, far below
// the rounding position.
__host__ __device__ inline double u128_to_f64(uint64_t hi, uint64_t lo)
{
    if (hi == 0)
        return double(lo);
    const int lz = __builtin_clzll(hi);
    const uint64_t top = lz ? ((hi << lz) | (lo >> (64 - lz))) : hi;
    const uint64_t rest = lz ? (lo << lz) : lo;
    return ldexp(double(top | (rest != 0 ? 1u : 0u)), 64 - lz);
}

// The decision from the exactly rounded sum of squares and the overflow flag,
// written into the step state (sumsq_units is the caller's business).
__host__ __device__ inline void decide_sum(zero_step_state_t* st, const DecideArgs& d, double sumsq, bool ovf)
{
    const double S = st->loss_scale;
    st->overflow = ovf ? 1 : 0;
    st->wide_pending = 0;
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

// The decision from the exact sum as a count of 2^-48 units (hi:lo).
__host__ __device__ inline void decide_state(zero_step_state_t* st, const DecideArgs& d, uint64_t hi, uint64_t lo,
                                             bool ovf)
{
    st->sumsq_units[0] = lo;
    st->sumsq_units[1] = hi;
    decide_sum(st, d, ovf ? 0.0 : ldexp(u128_to_f64(hi, lo), -48), ovf);
}

// A fast fp32 reduction that cannot vouch for its sum leaves the step
// undecided for the wide pass: skipped until then, loss scale and counters
// untouched.
__host__ __device__ inline void defer_to_wide(zero_step_state_t* st)
{
    st->wide_pending = 1;
    st->overflow = 0;
    st->skip = 1;
    st->gmul = 0.0f;
}

inline bool hparams_ok(const zero_hparams_t* hp)
{
    const double v[] = {hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->max_grad_norm,
                        hp->backoff, hp->growth, hp->min_scale};
    for (double x : v)
        if (!isfinite(x))
            return false;
    return !(hp->lr < 0 || hp->beta1 < 0 || hp->beta1 >= 1 || hp->beta2 < 0 || hp->beta2 >= 1 ||
             hp->eps <= 0 || hp->weight_decay < 0 || hp->backoff <= 0 || hp->backoff > 1 || hp->growth < 1 ||
             hp->min_scale <= 0);
}

inline DecideArgs decide_args(const zero_hparams_t* hp)
{
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
    return d;
}

}  // namespace zero
