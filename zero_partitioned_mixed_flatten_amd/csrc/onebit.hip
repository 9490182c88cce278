// onebit.hip -- the compression stage of 1-bit Adam on one rank's flat shard
// (the DeepSpeed article: 1-bit Adam cuts communication up to 5x with
// Adam-like convergence; the algorithm is Tang et al. 2021, Algorithm 1).
// After a warm-up of ordinary Adam steps the variance is frozen; each step
//   m = beta1*m + (1-beta1)*g;  x = m + ew;  cw = s_w*sgn(x);  ew = x - cw
//   u = cw + es;  m = s_s*sgn(u);  es = u - m      (one rank is its own server)
//   p = p - lr*(m/(sqrt(v)+eps) + wd*p),  p16 = fp16(p)
// with sgn(x) = +1 for x >= 0, -1 otherwise, and s = ||x||_2/sqrt(d) in fp32
// from the EXACT sum of squares rounded once to binary64.  The fast sum works in
// windows: the kernel that produces x (or u) sums, per workgroup b, its squares
// rounded to the nearest multiple of 2^(2E_b-80), E_b the binary exponent of
// that workgroup's max|x| (never a tie), as an exact integer W_b.  A fold
// kernel takes E, the largest E_b, and adds every W_b moved onto the window of
// E and rounded to the nearest unit: W.  Each square is then off by at most
// half a unit of 2^(2E-80) and each moved W_b by half a unit more, so the
// exact sum lies within (n + blocks)/2 units of W (the fold's own two levels
// add half a unit per group), and when the ends of that interval round to
// the same binary64 value, that value is the exactly rounded sum.  When they
// do not, the wide pass (wide_sum.hpp) sums the squares with no window and
// sets the scale.
// The sign bits (one byte per 8 elements, element 8j+k in bit k of byte j)
// are what a multi-rank run would exchange.  The device picks the stage:
// while the applied-step count is at most the warm-up length, these kernels
// return before any load and the ordinary update runs instead.
//
// Five kernels, because two global scales sit on the data path:
//   A  momentum; per workgroup max|x| and window sum of x^2     one-shot, 16 elements per thread
//   B  fold of A's window sums: s_w                             a few workgroups, one round of loads
//   C  worker compression: sign byte, ew, u = cw + es; per workgroup max|u| and window sum of u^2
//   D  fold of C's window sums: s_s                             as B
//   E  server compression + update: m, es, bits, p, p16
// (a wide pass follows B and D; it returns at once unless the window could
// not vouch for its sum).  Per-block maxima go to memory (no same-address
// atomics, which serialise).  Summing in A and C, from the values already in
// registers, saves the two passes that read x and u back (12.125 bytes per
// element).
// Element layout of the one-shot kernels: the whole bytes of the sign payload
// cover groups of 4 elements, g < 2*floor(n/8); thread t of workgroup b of E
// owns groups 512b+t and 512b+t+256, of A and C groups 1024b+t+256k (k < 4),
// so every vector load and store of a wave is one contiguous span.  A thread's 4 sign bits of a group are a nibble; the
// two lanes of an even/odd pair hold the two nibbles of one byte and join
// them with a lane shuffle.  The elements past the last whole byte (fewer
// than 8) are done one by one.
// The exact windowed square: z = x * 2^(40-E_b) (exact, |z| < 2^41),
//   a = fma(z, z, C1) - C1       z^2 to a multiple of 2^41 (C1 = 1.5*2^93)
//   b = (fma(z, z, -a) + C2) - C2   the rest, to the nearest integer (C2 = 1.5*2^52)
// so z^2 rounded to an integer is a + b.  A lane adds at most 23 squares (16,
// and 7 of the ragged end), so a wave's sum(a) < 2^93 in steps of 2^41 and
// |sum(b)| < 2^51 fold across the wave in binary64 without rounding; each
// wave's sums then become limbs.
#include <math.h>

#include "decide.hpp"
#include "exact_norm.hpp"
#include "wide_sum.hpp"
#include "window_fold.hpp"

namespace zero {
namespace {

constexpr int kBlock = 256;                  // one-shot kernels A, C, E
// The one-shot kernels run at most kOneShotCap (E) or kOneShotCapAC (A, C)
// workgroups per CU, enforced by a dynamic-LDS reservation they never touch
// (as the Adam kernel).  Measured on MI355X: E 1.6% faster at 2 than at full
// occupancy.  A and C were too (4.7% and 3.2%) until they took over the window
// sums: with the workgroup max and the sum's fold at the end of every
// workgroup, 4 per CU made the stage 949-952 -> 901-909 us (full occupancy
// 906-913, 6 per CU 900-903).  A and C also hold a few static LDS bytes,
// which the reservation leaves room for.
constexpr int kOneShotCap = 2;
constexpr int kOneShotCapAC = 4;
// Groups of 4 elements per thread in A and C (E: 2).  Each of their
// workgroups ends with a max, a window sum and a partial, paid once per
// kGroupsAC * 1024 elements, and the folds read half as many partials as
// with 2.  Measured on MI355X (gpt2 shard, one compression step, same box):
// 2 groups 904 us, 3 908, 4 891-896 (kept), 8 920.
constexpr int kGroupsAC = 4;
static_assert(4 * kGroupsAC + 7 <= 64, "the binary64 wave fold of the window sums needs at most 64 squares per lane");
constexpr double kWinHi = 0x1.8p93;          // ulp 2^41
constexpr double kWinLo = 0x1.8p52;          // ulp 1

struct Coef {
    float gmul, b1, omb1, eps, wd, lr;
};

__device__ __forceinline__ Coef coef_of(const zero_step_state_t* st)
{
    return Coef{st->gmul, st->beta1, st->omb1, st->eps, st->wd, st->lr};
}

__device__ __forceinline__ float sgn_scale(float x, float s) { return x < 0.0f ? -s : s; }
__device__ __forceinline__ uint32_t abs_bits(float x) { return __builtin_bit_cast(uint32_t, x) & 0x7FFFFFFFu; }

// Max over a workgroup of BLOCK threads; valid in thread 0.
template <int BLOCK>
__device__ __forceinline__ uint32_t block_max(uint32_t v)
{
    __shared__ uint32_t sm[BLOCK / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    if (BLOCK > 64) {
        if ((threadIdx.x & 63) == 0)
            sm[threadIdx.x >> 6] = v;
        __syncthreads();
        if (threadIdx.x == 0)
            for (int w = 1; w < BLOCK / 64; ++w)
                v = sm[w] > v ? sm[w] : v;
        __syncthreads();
    }
    return v;
}

// Binary exponent E of a positive binary32 given as bits: 2^E <= x < 2^(E+1).
__device__ __forceinline__ int exponent_of(uint32_t bits)
{
    const int e = int(bits >> 23);
    if (e)
        return e - 127;
    return (31 - __builtin_clz(bits)) - 149;                 // subnormal: highest mantissa bit
}

struct AccWin {
    double a = 0.0, b = 0.0;
    __device__ __forceinline__ void add(float x, double w)
    {
        const double z = double(x) * w;                       // exact
        const double hi = __builtin_fma(z, z, kWinHi) - kWinHi;
        a += hi;
        b += (__builtin_fma(z, z, -hi) + kWinLo) - kWinLo;
    }
    __device__ __forceinline__ exact::Limbs limbs() const
    {
        // an inf or NaN input leaves a or b non-finite; the fold then sets the
        // scale from the maxima alone, so the sum is not needed
        if (!__builtin_isfinite(a) || !__builtin_isfinite(b))
            return exact::Limbs{0, 0, 0, 0};
        const int64_t au = int64_t(a * 0x1p-41);              // < 2^53
        const int64_t bu = int64_t(b);                         // |.| <= 2^52
        const int64_t hs = au << 9;                            // au * 2^41 = hs * 2^32
        return exact::Limbs{bu & 0xFFFFFFFFll, (hs & 0xFFFFFFFFll) + (bu >> 32), hs >> 32, 0};
    }
};

// Every thread: the max of v over the workgroup (one barrier).
__device__ __forceinline__ uint32_t block_max_all(uint32_t v)
{
    __shared__ uint32_t sm[kBlock / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    if ((threadIdx.x & 63) == 0)
        sm[threadIdx.x >> 6] = v;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w)
        v = sm[w] > v ? sm[w] : v;
    return v;
}

// The workgroup's window sum as a carried partial, valid in thread 0 (every
// thread calls it).  A lane holds at most 4 * kGroupsAC + 7 squares (at most
// 64 keep it exact), so each wave folds its binary64 sums exactly (header
// note) before lane 0 turns them into limbs.
__device__ __forceinline__ NormPartial window_partial(AccWin acc)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        acc.a += __shfl_xor(acc.a, off, 64);
        acc.b += __shfl_xor(acc.b, off, 64);
    }
    __shared__ exact::Limbs s_w[kBlock / 64];
    if ((threadIdx.x & 63) == 0)
        s_w[threadIdx.x >> 6] = acc.limbs();
    __syncthreads();
    NormPartial p{0, 0};
    if (threadIdx.x == 0) {
        exact::Limbs t{0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < kBlock / 64; ++w) {
            t.l0 += s_w[w].l0;
            t.l1 += s_w[w].l1;
            t.l2 += s_w[w].l2;
            t.l3 += s_w[w].l3;
        }
        p = exact::make_partial(t, 0);
    }
    return p;
}

// The window of a block maximum given as bits: 2^(40-E).
__device__ __forceinline__ double window_of(uint32_t mx) { return ldexp(1.0, 40 - exponent_of(mx)); }

// The two groups of 4 elements a thread of E owns (see the layout note
// above; A and C take GroupsN), out of ng = 2*floor(n/8); ragged0 = 4*ng is
// the first element done one by one.
struct Groups {
    uint64_t ng, ja, jb, ragged0;
    __device__ explicit Groups(uint64_t n)
        : ng((n >> 3) * 2), ja(uint64_t(blockIdx.x) * (2 * kBlock) + threadIdx.x), jb(ja + kBlock),
          ragged0((n >> 3) * 8)
    {
    }
    __device__ bool both() const { return jb < ng; }
    __device__ bool first() const { return ja < ng; }
};

// The G groups of 4 elements a thread of A or C owns: j(k) = j0 + k * kBlock
// (k < G), out of ng = 2*floor(n/8), so each load and store instruction of a
// wave covers one contiguous span; the workgroup spans G * kBlock groups.
template <int G>
struct GroupsN {
    uint64_t ng, j0;
    __device__ explicit GroupsN(uint64_t n) : ng((n >> 3) * 2), j0(uint64_t(blockIdx.x) * (G * kBlock) + threadIdx.x) {}
    __device__ uint64_t j(int k) const { return j0 + uint64_t(k) * kBlock; }
    __device__ bool has(int k) const { return j(k) < ng; }
    __device__ bool all() const { return has(G - 1); }
};

// Joins the sign nibbles of an even/odd lane pair into the byte of group j
// (j even on the even lane); the even lane stores it.  Called by all lanes.
__device__ __forceinline__ void store_byte_pair(uint8_t* bits, uint64_t j, uint32_t nib, bool valid)
{
    const uint32_t other = uint32_t(__shfl_xor(int(nib), 1, 64));
    if (valid && (threadIdx.x & 1) == 0)
        bits[j >> 1] = uint8_t(nib | (other << 4));
}

// The sign nibble of group j from a byte payload.
__device__ __forceinline__ uint32_t nibble_of(const uint8_t* bits, uint64_t j)
{
    return (uint32_t(bits[j >> 1]) >> (4 * (j & 1))) & 15u;
}

// ---- A: momentum + block max of |m + ew| ----------------------------------------

// m -> beta1*m + (1-beta1)*g*gmul; x = m + ew into x, and the max of |x|.
__device__ __forceinline__ void momentum4(f16x4 g, f32x4& m, f32x4 e, const Coef& c, f32x4& x, uint32_t& mx)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma clang fp contract(off)
        const float gk = float(g[k]) * c.gmul;
        m[k] = c.b1 * m[k] + c.omb1 * gk;
        x[k] = m[k] + e[k];
        const uint32_t a = abs_bits(x[k]);
        mx = a > mx ? a : mx;
    }
}

__global__ __launch_bounds__(kBlock) void onebit_momentum_kernel(float* __restrict__ m32, const float* __restrict__ ew,
                                                                 const uint16_t* __restrict__ g16, uint64_t n,
                                                                 const zero_step_state_t* __restrict__ st,
                                                                 int64_t warmup, uint32_t* __restrict__ blockmax,
                                                                 NormPartial* __restrict__ part)
{
    if (st->step <= warmup)                      // a warm-up step: the Adam update runs instead
        return;
    extern __shared__ char occupancy_reserve[];  // see kOneShotCap
    if (n == UINT64_MAX)
        occupancy_reserve[threadIdx.x] = 0;
    constexpr int G = kGroupsAC;
    const GroupsN<G> gr(n);
    f32x4* __restrict__ M = reinterpret_cast<f32x4*>(m32);
    const f32x4* __restrict__ EW = reinterpret_cast<const f32x4*>(ew);
    const u32x2* __restrict__ GV = reinterpret_cast<const u32x2*>(g16);
    uint32_t mx = 0;
    f32x4 x[G] = {};
    float xr = 0.0f;
    if (gr.all()) {
        // Every stream here is read once and m is written back in place:
        // nontemporal loads and stores throughout (the gradient alone: 5%
        // faster; m and e_w as well: the 1-bit stage 2.6% faster).
        u32x2 g[G];
        f32x4 m[G], e[G];
#pragma unroll
        for (int k = 0; k < G; ++k) {
            g[k] = __builtin_nontemporal_load(GV + gr.j(k));
            m[k] = __builtin_nontemporal_load(M + gr.j(k));
            e[k] = __builtin_nontemporal_load(EW + gr.j(k));
        }
        __builtin_amdgcn_sched_barrier(0);
        // the loads are out before the skip flag is read (see loads_first_use)
        if (st->skip) {
            if (n == UINT64_MAX) {
                f32x4 t{};
#pragma unroll
                for (int k = 0; k < G; ++k)
                    t += m[k] + e[k] + bits_of(g[k]);
                M[gr.j(0)] = t;
            }
            return;
        }
        const Coef c = coef_of(st);
#pragma unroll
        for (int k = 0; k < G; ++k)
            momentum4(__builtin_bit_cast(f16x4, g[k]), m[k], e[k], c, x[k], mx);
#pragma unroll
        for (int k = 0; k < G; ++k)
            __builtin_nontemporal_store(m[k], M + gr.j(k));
    } else {
        if (st->skip)
            return;
        const Coef c = coef_of(st);
#pragma unroll
        for (int k = 0; k < G; ++k)
            if (gr.has(k)) {
                f32x4 mk = M[gr.j(k)];
                momentum4(__builtin_bit_cast(f16x4, GV[gr.j(k)]), mk, EW[gr.j(k)], c, x[k], mx);
                M[gr.j(k)] = mk;
            }
    }
    const bool ragged = blockIdx.x == 0 && threadIdx.x < (n & 7);
    if (ragged) {
#pragma clang fp contract(off)
        const Coef c = coef_of(st);
        const uint64_t i = ((n >> 3) << 3) + threadIdx.x;
        const float gk = float(__builtin_bit_cast(_Float16, g16[i])) * c.gmul;
        const float mi = c.b1 * m32[i] + c.omb1 * gk;
        m32[i] = mi;
        xr = mi + ew[i];
        const uint32_t a = abs_bits(xr);
        mx = a > mx ? a : mx;
    }
    // the workgroup's window (E_b from its max |x|) and its exact window sum
    mx = block_max_all(mx);
    AccWin acc;
    if (mx) {
        const double w = window_of(mx);
#pragma unroll
        for (int k = 0; k < G; ++k)
            if (gr.has(k))
                for (int q = 0; q < 4; ++q)
                    acc.add(x[k][q], w);
        if (ragged)
            acc.add(xr, w);
    }
    const NormPartial p = window_partial(acc);
    if (threadIdx.x == 0) {
        blockmax[blockIdx.x] = mx;
        part[blockIdx.x] = p;
    }
}

// ---- B / D: the fold of the window sums, and the scale ------------------------------------

// Which scale a fold writes.
enum Which { kWorker = 0, kServer = 1 };

// The scale from the exactly rounded sum of squares S of n values.
template <int WHICH>
__device__ __forceinline__ void set_scale(zero_onebit_state_t* ob, double S, uint64_t n)
{
    const float scale = n ? float(sqrt(S / double(n))) : 0.0f;
    if (WHICH == kWorker) {
        ob->scale_w = scale;
        ob->sumsq_w = S;
    } else {
        ob->scale_s = scale;
        ob->sumsq_s = S;
    }
}

// Window sums moved onto the window of the largest of their maxima: every
// thread takes its entries j = first, first + stride, ... (of count), eight
// loads in flight per round; returns the workgroup max in every thread and
// the moved sum (exact limbs of rounded moves) in thread 0.
__device__ __forceinline__ uint32_t fold_windows(const uint32_t* __restrict__ mxs, const NormPartial* __restrict__ parts,
                                                 uint64_t count, uint64_t first, uint64_t stride, exact::Limbs& t)
{
    // the largest maximum of this workgroup's entries
    uint32_t mx = 0;
    for (uint64_t j = first; j < count; j += 8 * stride) {
        uint32_t v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            v[q] = j + q * stride < count ? mxs[j + q * stride] : 0u;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            mx = v[q] > mx ? v[q] : mx;
    }
    __shared__ uint32_t s_mx;
    mx = block_max<kNormBlock>(mx);
    if (threadIdx.x == 0)
        s_mx = mx;
    __syncthreads();
    mx = s_mx;
    t = exact::Limbs{0, 0, 0, 0};
    if (mx) {
        const int E = exponent_of(mx);
        for (uint64_t j = first; j < count; j += 8 * stride) {
            uint32_t v[8];
            NormPartial q8[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const bool in = j + q * stride < count;
                v[q] = in ? mxs[j + q * stride] : 0u;
                q8[q] = in ? parts[j + q * stride] : NormPartial{0, 0};
            }
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (v[q])
                    window::add_moved(t, window::partial_value(q8[q]), 2 * (E - exponent_of(v[q])));
        }
    }
    uint32_t flag = 0;
    exact::block_fold<kNormBlock>(t, flag);
    return mx;
}

// B (WHICH = kWorker) and D (kServer): the scale from the nb window sums of
// A or C.  Each workgroup moves its share onto the window of its own largest
// maximum; with several workgroups the last to arrive moves their sums onto
// the window of the largest of all (half a unit each).
template <int WHICH>
__global__ __launch_bounds__(kNormBlock) void onebit_scale_kernel(const uint32_t* __restrict__ blockmax,
                                                                  const NormPartial* __restrict__ part, uint64_t nb,
                                                                  uint64_t n, const zero_step_state_t* __restrict__ st,
                                                                  int64_t warmup,
                                                                  zero_onebit_state_t* __restrict__ ob,
                                                                  uint32_t* __restrict__ gmax,
                                                                  NormPartial* __restrict__ gpart)
{
    if (st->skip || st->step <= warmup)
        return;
    const uint64_t stride = uint64_t(gridDim.x) * kNormBlock;
    exact::Limbs t;
    uint32_t mx = fold_windows(blockmax, part, nb, uint64_t(blockIdx.x) * kNormBlock + threadIdx.x, stride, t);
    uint64_t half = n + nb;                                   // twice the error bound, in units of the window
    if (gridDim.x > 1) {
        __shared__ uint32_t s_last;
        if (threadIdx.x == 0) {
            gmax[blockIdx.x] = mx;
            gpart[blockIdx.x] = exact::make_partial(t, 0);
            // release this workgroup's sum; the last one acquires everyone's
            const uint32_t prev = __hip_atomic_fetch_add(&ob->done_blocks, 1u, __ATOMIC_RELEASE,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            const bool last = prev == gridDim.x - 1;
            if (last)
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            s_last = last ? 1u : 0u;
        }
        __syncthreads();
        if (!s_last)
            return;
        mx = fold_windows(gmax, gpart, gridDim.x, threadIdx.x, kNormBlock, t);
        half += gridDim.x;
    }
    if (threadIdx.x == 0) {
        uint64_t hi = 0, lo = 0;
        exact::limbs_to_u128(t, hi, lo);                        // < (n + nb) * 2^82: always fits
        const int qexp = mx ? 2 * exponent_of(mx) - 80 : 0;
        if (WHICH == kWorker) {
            ob->qexp_w = qexp;
            ob->units_w[0] = lo;
            ob->units_w[1] = hi;
        } else {
            ob->qexp_s = qexp;
            ob->units_s[0] = lo;
            ob->units_s[1] = hi;
        }
        if (mx >= 0x7F800000u) {
            // an inf or NaN (binary32 overflow in the stage's own adds): the sum
            // of squares IEEE arithmetic gives, NaN if any NaN (its bits are the
            // larger), else +inf
            set_scale<WHICH>(ob, mx > 0x7F800000u ? double(NAN) : double(INFINITY), n);
        } else if (!mx || window::decides(hi, lo, half)) {
            const double S = mx ? ldexp(u128_to_f64(hi, lo), qexp) : 0.0;
            set_scale<WHICH>(ob, S, n);
        } else {
            ob->wide_pending |= 1u << WHICH;                    // the wide pass sets the scale
        }
        ob->done_blocks = 0;                                    // re-arm for the next fold
    }
}

// ---- C: worker compression ----------------------------------------------------------

// x = m + ew -> sign nibble, ew = x - s_w*sgn(x), u = s_w*sgn(x) + es into u,
// and the max of |u|.
__device__ __forceinline__ uint32_t compress4(f32x4 m, f32x4& e, f32x4 s, float sw, f32x4& u, uint32_t& mx)
{
    uint32_t nib = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float x = m[k] + e[k];
        const float cw = sgn_scale(x, sw);
        nib |= (x < 0.0f ? 0u : 1u) << k;
        e[k] = x - cw;
        u[k] = cw + s[k];
        const uint32_t a = abs_bits(u[k]);
        mx = a > mx ? a : mx;
    }
    return nib;
}

__global__ __launch_bounds__(kBlock) void onebit_compress_worker_kernel(const float* __restrict__ m32,
                                                                        float* __restrict__ ew,
                                                                        const float* __restrict__ es,
                                                                        uint8_t* __restrict__ bits_w, uint64_t n,
                                                                        const zero_step_state_t* __restrict__ st,
                                                                        int64_t warmup,
                                                                        const zero_onebit_state_t* __restrict__ ob,
                                                                        uint32_t* __restrict__ blockmax,
                                                                        NormPartial* __restrict__ part)
{
    if (st->step <= warmup)
        return;
    extern __shared__ char occupancy_reserve[];  // see kOneShotCap
    if (n == UINT64_MAX)
        occupancy_reserve[threadIdx.x] = 0;
    constexpr int G = kGroupsAC;
    const GroupsN<G> gr(n);
    const f32x4* __restrict__ M = reinterpret_cast<const f32x4*>(m32);
    f32x4* __restrict__ EW = reinterpret_cast<f32x4*>(ew);
    const f32x4* __restrict__ ES = reinterpret_cast<const f32x4*>(es);
    uint32_t mx = 0, nib[G] = {};
    f32x4 u[G] = {};
    if (gr.all()) {
        // nontemporal throughout: e_w is rewritten in place, and a plain load
        // ahead of an in-place nontemporal store is the slow pattern
        f32x4 m[G], e[G], sv[G];
#pragma unroll
        for (int k = 0; k < G; ++k) {
            m[k] = __builtin_nontemporal_load(M + gr.j(k));
            e[k] = __builtin_nontemporal_load(EW + gr.j(k));
            sv[k] = __builtin_nontemporal_load(ES + gr.j(k));
        }
        __builtin_amdgcn_sched_barrier(0);
        if (st->skip) {                          // loads first (see loads_first_use)
            if (n == UINT64_MAX) {
                f32x4 t{};
#pragma unroll
                for (int k = 0; k < G; ++k)
                    t += m[k] + e[k] + sv[k];
                EW[gr.j(0)] = t;
            }
            return;
        }
        const float sw = ob->scale_w;
#pragma unroll
        for (int k = 0; k < G; ++k)
            nib[k] = compress4(m[k], e[k], sv[k], sw, u[k], mx);
#pragma unroll
        for (int k = 0; k < G; ++k)
            __builtin_nontemporal_store(e[k], EW + gr.j(k));
    } else {
        if (st->skip)
            return;
        const float sw = ob->scale_w;
#pragma unroll
        for (int k = 0; k < G; ++k)
            if (gr.has(k)) {
                f32x4 ek = EW[gr.j(k)];
                nib[k] = compress4(M[gr.j(k)], ek, ES[gr.j(k)], sw, u[k], mx);
                EW[gr.j(k)] = ek;
            }
    }
#pragma unroll
    for (int k = 0; k < G; ++k)
        store_byte_pair(bits_w, gr.j(k), nib[k], gr.has(k));
    // the ragged last byte (fewer than 8 elements, one thread)
    const bool ragged = blockIdx.x == 0 && threadIdx.x == 0 && (n & 7);
    float ur[7] = {};
    if (ragged) {
        const uint64_t nvec = n >> 3;
        const float sw = ob->scale_w;
        uint32_t byte = 0;
#pragma unroll
        for (int k = 0; k < 7; ++k) {                     // fixed indices: ur stays in registers
            const uint64_t i = (nvec << 3) + k;
            if (i < n) {
                const float x = m32[i] + ew[i];
                const float cw = sgn_scale(x, sw);
                byte |= (x < 0.0f ? 0u : 1u) << k;
                ew[i] = x - cw;
                ur[k] = cw + es[i];
                const uint32_t a = abs_bits(ur[k]);
                mx = a > mx ? a : mx;
            }
        }
        bits_w[nvec] = uint8_t(byte);
    }
    // the workgroup's window (from its max |u|) and its exact window sum
    mx = block_max_all(mx);
    AccWin acc;
    if (mx) {
        const double w = window_of(mx);
#pragma unroll
        for (int k = 0; k < G; ++k)
            if (gr.has(k))
                for (int q = 0; q < 4; ++q)
                    acc.add(u[k][q], w);
        if (ragged)
#pragma unroll
            for (int k = 0; k < 7; ++k)
                if (uint64_t(k) < (n & 7))
                    acc.add(ur[k], w);
    }
    const NormPartial p = window_partial(acc);
    if (threadIdx.x == 0) {
        blockmax[blockIdx.x] = mx;
        part[blockIdx.x] = p;
    }
}

// ---- E: server compression + update ----------------------------------------------------

__device__ __forceinline__ void update(float m, float& p, float v, const Coef& c)
{
#pragma clang fp contract(off)
    const float u = m / (__builtin_sqrtf(v) + c.eps) + c.wd * p;
    p = p - c.lr * u;
}

// One group: u = s_w*sgn_w + es -> server sign nibble (returned), m = s_s*sgn(u),
// es = u - m, the parameter update and its fp16 copy h.
__device__ __forceinline__ uint32_t server_update4(uint32_t wnib, f32x4& s, f32x4& p, f32x4 v, f32x4& m, u32x2& h,
                                                   float sw, float ss, const Coef& c)
{
    uint32_t nib = 0;
    f16x4 h16;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float u = (((wnib >> k) & 1) ? sw : -sw) + s[k];
        const float mi = sgn_scale(u, ss);
        nib |= (u < 0.0f ? 0u : 1u) << k;
        s[k] = u - mi;
        m[k] = mi;
        float pk = p[k];
        update(mi, pk, v[k], c);
        p[k] = pk;
        h16[k] = _Float16(pk);
    }
    h = __builtin_bit_cast(u32x2, h16);
    return nib;
}

__global__ __launch_bounds__(kBlock) void onebit_update_kernel(uint16_t* __restrict__ p16, float* __restrict__ p32,
                                                               float* __restrict__ m32, const float* __restrict__ v32,
                                                               float* __restrict__ es,
                                                               const uint8_t* __restrict__ bits_w,
                                                               uint8_t* __restrict__ bits_s, uint64_t n,
                                                               const zero_step_state_t* __restrict__ st,
                                                               int64_t warmup,
                                                               const zero_onebit_state_t* __restrict__ ob)
{
    if (st->step <= warmup)
        return;
    extern __shared__ char occupancy_reserve[];  // see kOneShotCap
    if (n == UINT64_MAX)
        occupancy_reserve[threadIdx.x] = 0;
    const Groups gr(n);
    f32x4* __restrict__ ES = reinterpret_cast<f32x4*>(es);
    f32x4* __restrict__ P = reinterpret_cast<f32x4*>(p32);
    f32x4* __restrict__ M = reinterpret_cast<f32x4*>(m32);
    const f32x4* __restrict__ V = reinterpret_cast<const f32x4*>(v32);
    u32x2* __restrict__ H = reinterpret_cast<u32x2*>(p16);
    uint32_t nib_a = 0, nib_b = 0;
    if (gr.both()) {
        // the payload bytes are loaded as they are; picking the nibble waits
        // for them, so it comes after every load is out
        const uint32_t ba = bits_w[gr.ja >> 1], bb = bits_w[gr.jb >> 1];
        // v is frozen (read only) and p is read once: nontemporal loads of both
        // made this kernel 5% faster, and the next momentum pass 1.4% slower;
        // the same hint on e_s makes the stage about 2% slower (kept plain)
        f32x4 sa = ES[gr.ja], sb = ES[gr.jb];
        f32x4 pa = __builtin_nontemporal_load(P + gr.ja), pb = __builtin_nontemporal_load(P + gr.jb);
        const f32x4 va = __builtin_nontemporal_load(V + gr.ja), vb = __builtin_nontemporal_load(V + gr.jb);
        __builtin_amdgcn_sched_barrier(0);
        if (st->skip) {                          // loads first (see loads_first_use)
            if (n == UINT64_MAX)
                P[gr.ja] = sa + sb + pa + pb + va + vb + float(ba + bb);
            return;
        }
        const Coef c = coef_of(st);
        const float sw = ob->scale_w, ss = ob->scale_s;
        const uint32_t wa = (ba >> (4 * (gr.ja & 1))) & 15u, wb = (bb >> (4 * (gr.jb & 1))) & 15u;
        f32x4 ma, mb;
        u32x2 ha, hb;
        nib_a = server_update4(wa, sa, pa, va, ma, ha, sw, ss, c);
        nib_b = server_update4(wb, sb, pb, vb, mb, hb, sw, ss, c);
        __builtin_nontemporal_store(sa, ES + gr.ja);
        __builtin_nontemporal_store(sb, ES + gr.jb);
        __builtin_nontemporal_store(ma, M + gr.ja);
        __builtin_nontemporal_store(mb, M + gr.jb);
        __builtin_nontemporal_store(pa, P + gr.ja);
        __builtin_nontemporal_store(pb, P + gr.jb);
        __builtin_nontemporal_store(ha, H + gr.ja);
        __builtin_nontemporal_store(hb, H + gr.jb);
    } else {
        if (st->skip)
            return;
        if (gr.first()) {
            f32x4 sa = ES[gr.ja], pa = P[gr.ja], ma;
            u32x2 ha;
            nib_a = server_update4(nibble_of(bits_w, gr.ja), sa, pa, V[gr.ja], ma, ha, ob->scale_w, ob->scale_s,
                                   coef_of(st));
            ES[gr.ja] = sa;
            M[gr.ja] = ma;
            P[gr.ja] = pa;
            H[gr.ja] = ha;
        }
    }
    store_byte_pair(bits_s, gr.ja, nib_a, gr.first());
    store_byte_pair(bits_s, gr.jb, nib_b, gr.both());
    if (blockIdx.x == 0 && threadIdx.x == 0 && (n & 7)) {
        const uint64_t nvec = n >> 3;
        const uint32_t bw = bits_w[nvec];
        const Coef c = coef_of(st);
        const float sw = ob->scale_w, ss = ob->scale_s;
        uint32_t bs = 0;
        for (uint64_t i = nvec << 3; i < n; ++i) {
            const float u = (((bw >> (i & 7)) & 1) ? sw : -sw) + es[i];
            const float mi = sgn_scale(u, ss);
            bs |= (u < 0.0f ? 0u : 1u) << (i & 7);
            es[i] = u - mi;
            m32[i] = mi;
            float p = p32[i];
            update(mi, p, v32[i], c);
            p32[i] = p;
            p16[i] = __builtin_bit_cast(uint16_t, _Float16(p));
        }
        bits_s[nvec] = uint8_t(bs);
    }
}

// ---- the wide pass for a scale the window could not round (wide_sum.hpp) --------------

struct WorkerValues {
    const float* m;
    const float* ew;
    __device__ float at(uint64_t i) const { return m[i] + ew[i]; }
};

// u = s_w*sgn(x) + es, rebuilt from the worker's sign bits as the D kernel does
struct ServerValues {
    const uint8_t* bits;
    const float* es;
    const zero_onebit_state_t* ob;
    __device__ float at(uint64_t i) const
    {
        const float sw = ob->scale_w;
        return (((bits[i >> 3] >> (i & 7)) & 1) ? sw : -sw) + es[i];
    }
};

template <int WHICH>
struct ScaleFinish {
    zero_onebit_state_t* ob;
    uint64_t n;
    __device__ bool pending() const { return ((ob->wide_pending >> WHICH) & 1u) != 0; }
    __device__ uint32_t* counter() const { return &ob->done_blocks; }
    __device__ void finish(const uint64_t* digits) const
    {
        set_scale<WHICH>(ob, wide::to_f64(digits), n);
        ob->wide_pending &= ~(1u << WHICH);
    }
};

__global__ void onebit_state_init_kernel(zero_onebit_state_t* ob)
{
    zero_onebit_state_t s;
    memset(&s, 0, sizeof s);
    *ob = s;
}

// Workspace: the per-workgroup maxima and window sums of A and of C, the
// fold's per-workgroup maxima and sums, and the wide pass's partials.
struct Plan {
    uint64_t grid1;                 // one-shot kernel E (2 groups of 4 per thread)
    uint64_t grid_ac;               // one-shot kernels A and C (kGroupsAC groups of 4 per thread)
    uint64_t gridf;                 // the folds (B, D)
    uint64_t off_max_a, off_part_a, off_max_c, off_part_c, off_fmax, off_fpart, off_wide, bytes;
};

Plan plan(uint64_t n)
{
    Plan p;
    const uint64_t nvec = n >> 3;
    p.grid1 = (nvec + kBlock - 1) / kBlock;
    if (p.grid1 < 1) p.grid1 = 1;
    const uint64_t ng = 2 * nvec, per_ac = uint64_t(kGroupsAC) * kBlock;
    p.grid_ac = (ng + per_ac - 1) / per_ac;
    if (p.grid_ac < 1) p.grid_ac = 1;
    // two window sums per thread (one round of loads) where that takes at most
    // 256 workgroups; eight per thread measured 1 us slower on the gpt2 shard
    const uint64_t per = uint64_t(kNormBlock) * 2;
    p.gridf = (p.grid_ac + per - 1) / per;
    if (p.gridf > kNormMaxBlocks) p.gridf = kNormMaxBlocks;
    auto up = [](uint64_t b) { return (b + 255) / 256 * 256; };
    p.off_max_a = 0;
    p.off_part_a = p.off_max_a + up(p.grid_ac * 4);
    p.off_max_c = p.off_part_a + up(p.grid_ac * sizeof(NormPartial));
    p.off_part_c = p.off_max_c + up(p.grid_ac * 4);
    p.off_fmax = p.off_part_c + up(p.grid_ac * sizeof(NormPartial));
    p.off_fpart = p.off_fmax + up(p.gridf * 4);
    p.off_wide = p.off_fpart + up(p.gridf * sizeof(NormPartial));
    p.bytes = p.off_wide + up(wide::grid(n) * sizeof(wide::WidePartial));
    return p;
}

}  // namespace
}  // namespace zero

using namespace zero;

extern "C" size_t zero_onebit_workspace_bytes(uint64_t n) { return size_t(plan(n).bytes); }

extern "C" int zero_onebit_state_init(zero_onebit_state_t* dev_onebit, void* stream)
{
    if (!dev_onebit)
        return ZERO_EINVAL;
    if (!is_aligned(dev_onebit, 8))
        return ZERO_EALIGN;
    hipLaunchKernelGGL(onebit_state_init_kernel, dim3(1), dim3(1), 0, (hipStream_t)stream, dev_onebit);
    return launch_status();
}

extern "C" int zero_onebit_step(uint16_t* p16, float* p32, float* m32, float* v32, float* err_w,
                                float* err_s, const uint16_t* grad16, uint64_t n, uint8_t* bits_w, uint8_t* bits_s,
                                const zero_step_state_t* dev_state, zero_onebit_state_t* dev_onebit,
                                int64_t warmup, void* workspace, size_t workspace_bytes, void* stream)
{
    if (warmup < 0)
        return ZERO_EINVAL;
    if (!dev_state || !dev_onebit || !workspace ||
        (n && (!p16 || !p32 || !m32 || !v32 || !err_w || !err_s || !grad16 || !bits_w || !bits_s)))
        return ZERO_EINVAL;
    if (!is_aligned(dev_state, 8) || !is_aligned(dev_onebit, 8) || !is_aligned(workspace, 256))
        return ZERO_EALIGN;
    if (n && (!is_aligned(p16, 16) || !is_aligned(p32, 16) || !is_aligned(m32, 16) || !is_aligned(v32, 16) ||
              !is_aligned(err_w, 16) || !is_aligned(err_s, 16) || !is_aligned(grad16, 16)))
        return ZERO_EALIGN;
    if (n > kNormMaxElems)
        return ZERO_ERANGE;
    const Plan pl = plan(n);
    if (workspace_bytes < pl.bytes || pl.grid1 > 0x7fffffffull)
        return ZERO_ERANGE;
    char* ws = static_cast<char*>(workspace);
    uint32_t* max_a = reinterpret_cast<uint32_t*>(ws + pl.off_max_a);
    NormPartial* part_a = reinterpret_cast<NormPartial*>(ws + pl.off_part_a);
    uint32_t* max_c = reinterpret_cast<uint32_t*>(ws + pl.off_max_c);
    NormPartial* part_c = reinterpret_cast<NormPartial*>(ws + pl.off_part_c);
    uint32_t* fmax = reinterpret_cast<uint32_t*>(ws + pl.off_fmax);
    NormPartial* fpart = reinterpret_cast<NormPartial*>(ws + pl.off_fpart);
    wide::WidePartial* part_w = reinterpret_cast<wide::WidePartial*>(ws + pl.off_wide);
    const dim3 gw(uint32_t(wide::grid(n)));
    hipStream_t s = (hipStream_t)stream;
    const dim3 g1(uint32_t(pl.grid1)), gac(uint32_t(pl.grid_ac)), gf(uint32_t(pl.gridf));
    const uint32_t cap = lds_reservation(kOneShotCap);
    const uint32_t cap_ac0 = lds_reservation(kOneShotCapAC);
    const uint32_t cap_ac = cap_ac0 > 512 ? cap_ac0 - 512 : 0;   // room for A's and C's static LDS
    // a warm-up step: the ordinary update (it returns at once in the compression stage)
    int rc = adam_step_gated(p16, p32, m32, v32, grad16, n, dev_state, stream, warmup);
    if (rc != ZERO_OK)
        return rc;
    hipLaunchKernelGGL(onebit_momentum_kernel, gac, dim3(kBlock), cap_ac, s, m32, err_w, grad16, n, dev_state,
                       warmup, max_a, part_a);
    if ((rc = launch_status()) != ZERO_OK)
        return rc;
    hipLaunchKernelGGL(onebit_scale_kernel<kWorker>, gf, dim3(kNormBlock), 0, s, max_a, part_a, pl.grid_ac, n,
                       dev_state, warmup, dev_onebit, fmax, fpart);
    if ((rc = launch_status()) != ZERO_OK)
        return rc;
    hipLaunchKernelGGL((wide::wide_sum_kernel<WorkerValues, ScaleFinish<kWorker>>), gw, dim3(wide::kBlock), 0, s,
                       WorkerValues{m32, err_w}, n, ScaleFinish<kWorker>{dev_onebit, n}, part_w);
    if ((rc = launch_status()) != ZERO_OK)
        return rc;
    hipLaunchKernelGGL(onebit_compress_worker_kernel, gac, dim3(kBlock), cap_ac, s, m32, err_w, err_s, bits_w, n,
                       dev_state, warmup, dev_onebit, max_c, part_c);
    if ((rc = launch_status()) != ZERO_OK)
        return rc;
    hipLaunchKernelGGL(onebit_scale_kernel<kServer>, gf, dim3(kNormBlock), 0, s, max_c, part_c, pl.grid_ac, n,
                       dev_state, warmup, dev_onebit, fmax, fpart);
    if ((rc = launch_status()) != ZERO_OK)
        return rc;
    hipLaunchKernelGGL((wide::wide_sum_kernel<ServerValues, ScaleFinish<kServer>>), gw, dim3(wide::kBlock), 0, s,
                       ServerValues{bits_w, err_s, dev_onebit}, n, ScaleFinish<kServer>{dev_onebit, n}, part_w);
    if ((rc = launch_status()) != ZERO_OK)
        return rc;
    hipLaunchKernelGGL(onebit_update_kernel, g1, dim3(kBlock), cap, s, p16, p32, m32, v32, err_s,
                       bits_w, bits_s, n, dev_state, warmup, dev_onebit);
    return launch_status();
}
