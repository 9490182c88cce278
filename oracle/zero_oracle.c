/*
 * zero_oracle.c -- reference oracle for the ZeRO partitioned mixed-precision
 * Adam step on one data-parallel rank's flat shard.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load or call this library.  It
 * shares no source, header, table or helper with the HIP library; the two
 * only see the same seeded inputs.
 *
 * Plain and slow on purpose: one thread, one element at a time, each
 * floating-point operator is one IEEE-754 round-to-nearest-even operation
 * (built with -O2 -ffp-contract=off, no fast-math; on x86-64 float and
 * double arithmetic is SSE, so there is no excess precision).
 *
 * What the pages fix (ZeRO paper card, sections "Bottleneck" and "Evidence";
 * ZeRO-2 article, "model state memory"):
 *   - mixed-precision Adam keeps fp16 parameters and fp16 gradients plus fp32
 *     master parameters, fp32 momentum and fp32 variance: 2+2+12 = 16 bytes
 *     per parameter (1.5B parameters -> at least 24 GB);
 *   - stage 1 partitions the optimizer state, stage 2 adds the gradients,
 *     stage 3 adds the parameters, each across the Nd data-parallel ranks
 *     ("Method" section: 4x, 8x and Nd-proportional reductions);
 *   - model state lives in contiguous, defragmented buffers ("Method",
 *     ZeRO-R paragraph; ZeRO-2 article, fragmented memory).
 * Everything the pages leave open is taken from the published methods the
 * step is made of, and each such reading is stated where it is used:
 *   - Adam: Kingma & Ba 2015, Algorithm 1 (bias-corrected moments);
 *   - decoupled weight decay: Loshchilov & Hutter 2019, Algorithm 2;
 *   - dynamic loss scaling with skipped steps: Micikevicius et al. 2018;
 *   - clipping by the global L2 norm: Pascanu et al. 2013.
 *
 * Every function here is pinned by a CPU test against something other than
 * itself (page figures, closed forms, numpy's binary16 routines, exact
 * rational sums, math.fsum).  No function is "parity unpinned".
 *
 * The sums of squares are the plain definition: every square exact, the
 * sum exact, one rounding to binary64 at the end (wide_t below).  No
 * window, grid or domain bound enters them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if defined(__FAST_MATH__)
#error "the oracle must be built without fast-math"
#endif

/* ------------------------------------------------------------------ */
/* IEEE-754 binary16 <-> binary32, written from the format definition.  */
/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.   */
/* ------------------------------------------------------------------ */

/* Exact widening: every binary16 value is a binary32 value. */
float oracle_f32_from_f16(uint16_t h)
{
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu;
    uint32_t f = h & 0x3ffu;
    uint32_t bits;
    float out;
    if (e == 0x1fu) {                       /* infinity or NaN */
        bits = sign | 0x7f800000u | (f << 13);
    } else if (e == 0) {                    /* zero or subnormal: f * 2^-24 */
        out = (float)f * 0x1p-24f;          /* exact: f < 2^10 */
        return sign ? -out : out;
    } else {                                /* normal: rebias 15 -> 127 */
        bits = sign | ((e - 15u + 127u) << 23) | (f << 13);
    }
    memcpy(&out, &bits, sizeof out);
    return out;
}

/* Round-to-nearest, ties-to-even narrowing.  Subnormal results are kept,
 * values at or beyond 65520 (the midpoint above the largest finite binary16,
 * 65504) become infinity, a NaN stays a quiet NaN. */
uint16_t oracle_f16_from_f32(float x)
{
    uint32_t b;
    memcpy(&b, &x, sizeof b);
    uint16_t sign = (uint16_t)((b >> 16) & 0x8000u);
    uint32_t e = (b >> 23) & 0xffu;
    uint32_t f = b & 0x7fffffu;

    if (e == 0xffu)                          /* infinity, or NaN kept quiet */
        return (uint16_t)(sign | 0x7c00u | (f ? (0x200u | (f >> 13)) : 0u));
    if (e == 0)                              /* |x| < 2^-126: far below 2^-25 */
        return sign;

    int32_t E = (int32_t)e - 127;            /* x = M * 2^(E-23), M has 24 bits */
    uint32_t M = f | 0x800000u;

    if (E > 15)                              /* |x| >= 2^16 */
        return (uint16_t)(sign | 0x7c00u);

    if (E >= -14) {                          /* normal binary16 range */
        uint32_t q = M >> 13;                /* 11-bit significand, 1024..2047 */
        uint32_t r = M & 0x1fffu;            /* the 13 discarded bits */
        if (r > 0x1000u || (r == 0x1000u && (q & 1u)))
            q += 1;
        if (q == 2048u) {                    /* carried into the next binade */
            q = 1024u;
            E += 1;
        }
        if (E > 15)
            return (uint16_t)(sign | 0x7c00u);
        return (uint16_t)(sign | (uint32_t)((E + 15) << 10) | (q - 1024u));
    }

    /* subnormal binary16: result is q * 2^-24 with q = round(M * 2^(E+1)) */
    int32_t shift = -(E + 1);                /* >= 14 here */
    if (shift > 24)                          /* |x| < 2^-25: rounds to zero */
        return sign;
    uint32_t q = M >> shift;
    uint32_t r = M & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (r > half || (r == half && (q & 1u)))
        q += 1;                              /* q == 1024 encodes 2^-14 itself */
    return (uint16_t)(sign | q);
}

void oracle_f16_from_f32_array(const float* x, uint16_t* out, uint64_t n)
{
    for (uint64_t i = 0; i < n; ++i)
        out[i] = oracle_f16_from_f32(x[i]);
}

void oracle_f32_from_f16_array(const uint16_t* h, float* out, uint64_t n)
{
    for (uint64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_from_f16(h[i]);
}

/* ------------------------------------------------------------------ */
/* Model-state bytes per data-parallel rank (ZeRO paper card, sections  */
/* "Bottleneck" and "Method"; ZeRO-2 article, model state memory).      */
/* Each rank owns P = ceil(psi / nd) parameters of the flat state.      */
/*   stage 0 (plain DP): (2 + 2 + K) * psi                              */
/*   stage 1 (P_os):     2 psi + 2 psi + K * P                          */
/*   stage 2 (P_os+g):   2 psi + (2 + K) * P                            */
/*   stage 3 (P_os+g+p): (2 + 2 + K) * P                                */
/* Returns 0, or -1 for a bad stage / nd == 0 / overflow of 64 bits.    */
/* ------------------------------------------------------------------ */
int oracle_state_bytes(uint64_t psi, uint32_t nd, uint32_t k, int stage, uint64_t* out)
{
    if (nd == 0 || out == 0)
        return -1;
    unsigned __int128 P = ((unsigned __int128)psi + nd - 1) / nd;
    unsigned __int128 Psi = psi;
    unsigned __int128 bytes;
    switch (stage) {
    case 0: bytes = (2 + 2 + (unsigned __int128)k) * Psi; break;
    case 1: bytes = 2 * Psi + 2 * Psi + (unsigned __int128)k * P; break;
    case 2: bytes = 2 * Psi + (2 + (unsigned __int128)k) * P; break;
    case 3: bytes = (2 + 2 + (unsigned __int128)k) * P; break;
    default: return -1;
    }
    if (bytes > (unsigned __int128)UINT64_MAX)
        return -1;
    *out = (uint64_t)bytes;
    return 0;
}

/* ------------------------------------------------------------------ */
/* Flatten (ZeRO paper card, "Method": contiguous buffers against       */
/* fragmentation; DeepSpeed article: gradient accumulation is managed   */
/* by the library).  Each segment copies `count` binary16 elements from */
/* src[src_off ...] to dst[dst_off ...].                                */
/*   dst binary16, no accumulate:  bit copy                            */
/*   dst binary16, accumulate:     dst = f16(f32(dst) + f32(src))      */
/*   dst binary32, no accumulate:  dst = f32(src)                      */
/*   dst binary32, accumulate:     dst = dst + f32(src)                */
/* Destination elements no segment covers are left alone.               */
/* ------------------------------------------------------------------ */
typedef struct {
    const uint16_t* src;
    uint64_t src_off;
    uint64_t dst_off;
    uint64_t count;
} oracle_segment_t;

void oracle_flatten(const oracle_segment_t* segs, uint32_t nsegs, void* dst,
                    int dst_is_f32, int accumulate)
{
    for (uint32_t s = 0; s < nsegs; ++s) {
        const uint16_t* src = segs[s].src + segs[s].src_off;
        for (uint64_t i = 0; i < segs[s].count; ++i) {
            uint64_t d = segs[s].dst_off + i;
            if (dst_is_f32) {
                float* out = (float*)dst;
                float g = oracle_f32_from_f16(src[i]);
                out[d] = accumulate ? out[d] + g : g;
            } else {
                uint16_t* out = (uint16_t*)dst;
                if (accumulate)
                    out[d] = oracle_f16_from_f32(oracle_f32_from_f16(out[d]) +
                                                 oracle_f32_from_f16(src[i]));
                else
                    out[d] = src[i];
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* Exact sum of squares, rounded once.  Every binary32 value (and so    */
/* every binary16 value) is x = M * 2^e with M an integer below 2^24   */
/* and e >= -149, so x^2 = M^2 * 2^(2e) is an integer number of units   */
/* of 2^-298 (the square of the smallest subnormal), below 2^256.  The  */
/* sum is kept as that integer, in base-2^32 digits (one per 64-bit    */
/* word, carried every 2^31 additions), converted to binary64 once,   */
/* rounding to nearest with ties to even.  640 bits hold the sum of    */
/* more than 2^80 squares of the largest binary32, so the integer never */
/* wraps on any input this oracle can be given.                        */
/* ------------------------------------------------------------------ */
#define WIDE_DIGITS 20
#define WIDE_UNIT_EXP (-298)

typedef struct {
    uint64_t d[WIDE_DIGITS];                 /* digit k weighs 2^(32k) units */
    uint64_t adds;                           /* additions since the last carry */
} wide_t;

/* Brings every digit back below 2^32 (the value is unchanged). */
static void wide_carry(wide_t* w)
{
    for (int j = 0; j < WIDE_DIGITS - 1; ++j) {
        w->d[j + 1] += w->d[j] >> 32;
        w->d[j] &= 0xffffffffu;
    }
    w->adds = 0;
}

static void wide_add_square(wide_t* w, float x)
{
    uint32_t b;
    memcpy(&b, &x, sizeof b);
    uint32_t field = (b >> 23) & 0xffu;      /* the caller passes finite values only */
    uint64_t M = b & 0x7fffffu;              /* |x| = M * 2^e (IEEE-754 binary32): */
    int e = -149;                            /*   subnormal or zero: e = -149 */
    if (field != 0) {                        /*   normal: hidden bit, e = field - 150 */
        M |= 0x800000u;
        e = (int)field - 150;
    }
    int pos = 2 * e - WIDE_UNIT_EXP;         /* x^2 = M^2 * 2^pos units, pos >= 0 */
    unsigned __int128 v = (unsigned __int128)(M * M) << (pos % 32);   /* below 2^80 */
    int k = pos / 32;
    /* Each digit gets less than 2^32 per addition, so 2^31 additions fit in
     * its 64-bit word before the carry. */
    w->d[k] += (uint64_t)v & 0xffffffffu;
    w->d[k + 1] += (uint64_t)(v >> 32) & 0xffffffffu;
    w->d[k + 2] += (uint64_t)(v >> 64);
    if (++w->adds == (1u << 31))
        wide_carry(w);
}

static int wide_bit(const wide_t* w, int i)
{
    return (int)((w->d[i / 32] >> (i % 32)) & 1u);
}

/* The integer times 2^-298, rounded to the nearest binary64, ties to even. */
static double wide_to_double(wide_t* w)
{
    wide_carry(w);
    int top = -1;                            /* index of the highest set bit */
    for (int i = 32 * WIDE_DIGITS - 1; i >= 0 && top < 0; --i)
        if (wide_bit(w, i))
            top = i;
    if (top < 0)
        return 0.0;
    int low = top - 52;                      /* the lowest bit a binary64 significand keeps */
    if (low < 0)
        low = 0;
    uint64_t m = 0;                          /* bits top..low: at most 53 of them */
    for (int i = top; i >= low; --i)
        m = (m << 1) | (uint64_t)wide_bit(w, i);
    if (low > 0) {
        int round = wide_bit(w, low - 1);
        int sticky = 0;
        for (int i = low - 2; i >= 0; --i)
            sticky |= wide_bit(w, i);
        if (round && (sticky || (m & 1u)))
            m += 1;                          /* may reach 2^53: still exact in binary64 */
    }
    return ldexp((double)m, low + WIDE_UNIT_EXP);
}

/* ------------------------------------------------------------------ */
/* Squared L2 norm and the inf/NaN test of the flat binary16 gradient.  */
/* overflow = some element has an all-ones exponent (inf or NaN).       */
/* sumsq    = sum over i of g_i^2, exact, rounded once to binary64.    */
/* When overflow is set the sum has no meaning and is +inf.            */
/* ------------------------------------------------------------------ */
void oracle_norm_overflow(const uint16_t* g, uint64_t n, double* sumsq, int32_t* overflow)
{
    wide_t w;
    memset(&w, 0, sizeof w);
    for (uint64_t i = 0; i < n; ++i) {
        if ((g[i] & 0x7c00u) == 0x7c00u) {
            *overflow = 1;
            *sumsq = INFINITY;
            return;
        }
        wide_add_square(&w, oracle_f32_from_f16(g[i]));
    }
    *overflow = 0;
    *sumsq = wide_to_double(&w);
}

/* ------------------------------------------------------------------ */
/* The same reduction over an fp32 gradient partition (the gradient-    */
/* accumulation form: micro-batch fp16 gradients summed in fp32; the    */
/* DeepSpeed article leaves gradient accumulation to the library).      */
/* overflow = some element is inf or NaN.                               */
/* sumsq    = sum over i of x_i^2, exact, rounded once to binary64     */
/*            (never infinite: every square is below 2^256).           */
/* ------------------------------------------------------------------ */
void oracle_norm_overflow_f32(const float* g, uint64_t n, double* sumsq, int32_t* overflow)
{
    wide_t w;
    memset(&w, 0, sizeof w);
    for (uint64_t i = 0; i < n; ++i) {
        if (!isfinite(g[i])) {
            *overflow = 1;
            *sumsq = INFINITY;
            return;
        }
        wide_add_square(&w, g[i]);
    }
    *overflow = 0;
    *sumsq = wide_to_double(&w);
}

/* ------------------------------------------------------------------ */
/* Step decision: dynamic loss scaling, skip-step, clipping, bias       */
/* correction.  Scalars are binary64; the per-element factors are each  */
/* rounded once to binary32.                                            */
/* ------------------------------------------------------------------ */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
    double max_grad_norm;        /* clip threshold on the unscaled norm; <= 0: no clipping */
    double backoff;              /* loss-scale factor after an overflow (0.5) */
    double growth;               /* loss-scale factor after growth_interval clean steps (2) */
    double min_scale;            /* the loss scale never drops below this (1) */
    int32_t growth_interval;     /* consecutive clean steps before growth (20); <= 0: never */
    int32_t reserved;
} oracle_hparams_t;

typedef struct {
    /* carried from step to step */
    double loss_scale;           /* S: the gradients arrive multiplied by S */
    double beta1_pow, beta2_pow; /* beta^t as running binary64 products */
    int64_t step;                /* t: applied (not skipped) steps so far */
    int32_t good_steps;          /* clean steps since the last scale change */
    int32_t skipped_total;
    /* written by the last decision */
    double sumsq;                /* sum of squares of the scaled gradient */
    double grad_norm;            /* sqrt(sumsq) / S, +inf on overflow */
    int32_t overflow, skip;
    float gmul;                  /* f32(coef / S): unscale and clip in one factor */
    float bc1, bc2;              /* f32(1 - beta1^t), f32(1 - beta2^t) */
    float lr, beta1, beta2, omb1, omb2, eps, wd;
} oracle_state_t;

void oracle_state_init(oracle_state_t* st, double initial_scale)
{
    memset(st, 0, sizeof *st);
    st->loss_scale = initial_scale;
    st->beta1_pow = 1.0;
    st->beta2_pow = 1.0;
}

void oracle_decide(oracle_state_t* st, const oracle_hparams_t* hp, double sumsq, int32_t overflow)
{
    double S = st->loss_scale;
    st->sumsq = sumsq;
    st->overflow = overflow ? 1 : 0;

    if (overflow) {
        /* Micikevicius et al.: skip the update, shrink the scale, restart the count. */
        double s2 = S * hp->backoff;
        st->loss_scale = s2 < hp->min_scale ? hp->min_scale : s2;
        st->good_steps = 0;
        st->skipped_total += 1;
        st->skip = 1;
        st->grad_norm = INFINITY;
        st->gmul = 0.0f;
        return;
    }

    st->skip = 0;
    double norm = sqrt(sumsq) / S;                 /* norm of the unscaled gradient */
    st->grad_norm = norm;

    /* Kingma & Ba: t counts applied steps; beta^t kept as running products. */
    st->step += 1;
    st->beta1_pow *= hp->beta1;
    st->beta2_pow *= hp->beta2;

    /* Pascanu et al.: rescale to the threshold when the norm exceeds it. */
    double coef = (hp->max_grad_norm > 0.0 && norm > hp->max_grad_norm)
                      ? hp->max_grad_norm / norm : 1.0;
    st->gmul = (float)(coef / S);
    st->bc1 = (float)(1.0 - st->beta1_pow);
    st->bc2 = (float)(1.0 - st->beta2_pow);
    st->lr = (float)hp->lr;
    st->beta1 = (float)hp->beta1;
    st->beta2 = (float)hp->beta2;
    st->omb1 = (float)(1.0 - hp->beta1);
    st->omb2 = (float)(1.0 - hp->beta2);
    st->eps = (float)hp->eps;
    st->wd = (float)hp->weight_decay;

    /* Grow the scale after growth_interval consecutive clean steps; the
     * gradients of this step were scaled by the old S, used above. */
    st->good_steps += 1;
    if (hp->growth_interval > 0 && st->good_steps >= hp->growth_interval) {
        st->loss_scale = S * hp->growth;
        st->good_steps = 0;
    }
}

/* ------------------------------------------------------------------ */
/* Element update, binary32 throughout, one rounding per operator:      */
/*   g  = g16 * gmul                        (unscale + clip)            */
/*   m  = beta1*m + (1-beta1)*g             (Kingma & Ba, Alg. 1)       */
/*   v  = beta2*v + (1-beta2)*(g*g)                                      */
/*   mh = m / (1-beta1^t),  vh = v / (1-beta2^t)                        */
/*   u  = mh / (sqrt(vh) + eps) + wd*p      (Loshchilov & Hutter, Alg. 2 */
/*   p  = p - lr*u                           with schedule multiplier lr) */
/*   p16 = f16(p)                                                       */
/* A skipped step changes nothing.                                       */
/* ------------------------------------------------------------------ */
void oracle_adam_update(const oracle_state_t* st, uint16_t* p16, float* p32, float* m32,
                        float* v32, const uint16_t* g16, uint64_t n)
{
    if (st->skip)
        return;
    for (uint64_t i = 0; i < n; ++i) {
        float g = oracle_f32_from_f16(g16[i]) * st->gmul;
        float m = st->beta1 * m32[i] + st->omb1 * g;
        float v = st->beta2 * v32[i] + st->omb2 * (g * g);
        float mh = m / st->bc1;
        float vh = v / st->bc2;
        float u = mh / (sqrtf(vh) + st->eps) + st->wd * p32[i];
        float p = p32[i] - st->lr * u;
        m32[i] = m;
        v32[i] = v;
        p32[i] = p;
        p16[i] = oracle_f16_from_f32(p);
    }
}

/* The element update with an fp32 gradient (the accumulation form): the
 * same operations in the same order, with g = grad32[i] * gmul. */
void oracle_adam_update_f32(const oracle_state_t* st, uint16_t* p16, float* p32, float* m32,
                            float* v32, const float* g32, uint64_t n)
{
    if (st->skip)
        return;
    for (uint64_t i = 0; i < n; ++i) {
        float g = g32[i] * st->gmul;
        float m = st->beta1 * m32[i] + st->omb1 * g;
        float v = st->beta2 * v32[i] + st->omb2 * (g * g);
        float mh = m / st->bc1;
        float vh = v / st->bc2;
        float u = mh / (sqrtf(vh) + st->eps) + st->wd * p32[i];
        float p = p32[i] - st->lr * u;
        m32[i] = m;
        v32[i] = v;
        p32[i] = p;
        p16[i] = oracle_f16_from_f32(p);
    }
}

/* One whole step: flatten the segments into grad16 (bit copy), reduce,
 * decide, update. */
void oracle_step(const oracle_hparams_t* hp, oracle_state_t* st,
                 const oracle_segment_t* segs, uint32_t nsegs, uint16_t* grad16,
                 uint16_t* p16, float* p32, float* m32, float* v32, uint64_t n)
{
    double sumsq;
    int32_t overflow;
    oracle_flatten(segs, nsegs, grad16, 0, 0);
    oracle_norm_overflow(grad16, n, &sumsq, &overflow);
    oracle_decide(st, hp, sumsq, overflow);
    oracle_adam_update(st, p16, p32, m32, v32, grad16, n);
}

/* ------------------------------------------------------------------ */
/* 1-bit Adam, compression stage (DeepSpeed article: 1-bit Adam cuts    */
/* communication up to 5x with Adam-like convergence; the algorithm is  */
/* Tang et al. 2021, "1-bit Adam", Algorithm 1).  After a warm-up of    */
/* ordinary Adam steps the variance v is frozen; each step then         */
/*   m  = beta1*m + (1-beta1)*g                (local momentum)          */
/*   x  = m + ew;  cw = C[x];  ew = x - cw     (worker error feedback)   */
/*   u  = avg_workers(cw) + es; m = C[u]; es = u - m   (server side)     */
/*   p  = p - lr*(m/(sqrt(v)+eps) + wd*p)      (frozen v; decoupled wd)  */
/* With one data-parallel rank the rank is its own server and the       */
/* average is its own cw.                                               */
/*                                                                      */
/* The compressor C[x] = s * sgn(x), one bit per element plus one       */
/* scale per vector: sgn(x) = +1 for x >= 0 (zeros included) and -1     */
/* otherwise; s = ||x||_2 / sqrt(d) in fp32, so that C[x] keeps the L2  */
/* norm of x.  S = sum of x_i^2 exactly, rounded once to binary64 (the  */
/* same exact sum as the gradient norm), then s = fp32(sqrt(S / d))     */
/* with correctly rounded binary64 division and square root.            */
/* ------------------------------------------------------------------ */
float oracle_onebit_scale(const float* x, uint64_t n, double* sumsq_out)
{
    /* A non-finite element (possible only when the stage's own binary32
     * arithmetic overflows) makes the sum of squares what IEEE arithmetic
     * over the squares gives: NaN if some element is NaN, else +inf. */
    int inf = 0, nan = 0;
    for (uint64_t i = 0; i < n; ++i) {
        nan |= isnan(x[i]);
        inf |= isinf(x[i]);
    }
    wide_t w;
    memset(&w, 0, sizeof w);
    if (!inf && !nan)
        for (uint64_t i = 0; i < n; ++i)
            wide_add_square(&w, x[i]);
    double S = nan ? (double)NAN : inf ? INFINITY : wide_to_double(&w);
    if (sumsq_out)
        *sumsq_out = S;
    return n ? (float)sqrt(S / (double)n) : 0.0f;
}

/* Sign bits, little-endian within each byte: bit k of byte j is element 8j+k,
 * 1 for x >= 0 (sgn = +1), 0 for x < 0. */
void oracle_onebit_pack(const float* x, uint64_t n, uint8_t* bits)
{
    for (uint64_t j = 0; j < (n + 7) / 8; ++j)
        bits[j] = 0;
    for (uint64_t i = 0; i < n; ++i)
        if (!(x[i] < 0.0f))
            bits[i / 8] |= (uint8_t)(1u << (i % 8));
}

/* x -> the compressed vector s*sgn(x) and the new error x - s*sgn(x). */
static void compress(const float* x, uint64_t n, float s, float* c, float* err)
{
    for (uint64_t i = 0; i < n; ++i) {
        c[i] = x[i] < 0.0f ? -s : s;
        err[i] = x[i] - c[i];
    }
}

/* One compression-stage step; scales[0] = worker scale, scales[1] = server
 * scale.  Nothing changes when the decision skipped the step. */
int oracle_onebit_step(const oracle_state_t* st, uint16_t* p16, float* p32, float* m32, const float* v32,
                       float* err_w, float* err_s, const uint16_t* g16, uint64_t n,
                       uint8_t* bits_w, uint8_t* bits_s, float* scales)
{
    if (st->skip)
        return 0;
    float* x = (float*)calloc(n ? n : 1, sizeof(float));
    float* c = (float*)calloc(n ? n : 1, sizeof(float));
    if (!x || !c) {
        free(x);
        free(c);
        return -1;
    }
    for (uint64_t i = 0; i < n; ++i) {                  /* local momentum, then the worker's error */
        float g = oracle_f32_from_f16(g16[i]) * st->gmul;
        m32[i] = st->beta1 * m32[i] + st->omb1 * g;
        x[i] = m32[i] + err_w[i];
    }
    scales[0] = oracle_onebit_scale(x, n, 0);
    oracle_onebit_pack(x, n, bits_w);
    compress(x, n, scales[0], c, err_w);
    for (uint64_t i = 0; i < n; ++i)                    /* server: one worker's average is its own */
        x[i] = c[i] + err_s[i];
    scales[1] = oracle_onebit_scale(x, n, 0);
    oracle_onebit_pack(x, n, bits_s);
    compress(x, n, scales[1], m32, err_s);              /* the momentum becomes the server's output */
    for (uint64_t i = 0; i < n; ++i) {
        float u = m32[i] / (sqrtf(v32[i]) + st->eps) + st->wd * p32[i];
        p32[i] = p32[i] - st->lr * u;
        p16[i] = oracle_f16_from_f32(p32[i]);
    }
    free(x);
    free(c);
    return 0;
}
