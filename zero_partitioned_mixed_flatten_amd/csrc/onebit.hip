// onebit.hip -- the compression stage of 1-bit Adam on one rank's flat shard
// (the DeepSpeed article: 1-bit Adam cuts communication up to 5x with
// Adam-like convergence; the algorithm is Tang et al. 2021, Algorithm 1).
// After a warm-up of ordinary Adam steps the variance is frozen; each step
//   m = beta1*m + (1-beta1)*g;  x = m + ew;  cw = s_w*sgn(x);  ew = x - cw
//   u = cw + es;  m = s_s*sgn(u);  es = u - m      (one rank is its own server)
//   p = p - lr*(m/(sqrt(v)+eps) + wd*p),  p16 = fp16(p)
// with sgn(x) = +1 for x >= 0, -1 otherwise, and s = ||x||_2/sqrt(d) in fp32
// from the EXACT sum of squares rounded once to binary64.  The fast sum
// works in a window: with E the binary exponent of max|x|, each square is
// rounded to the nearest multiple of 2^(2E-80) (never a tie) and the
// integers are summed exactly; the exact sum then lies within n/2 units of
// that integer W, and when W - n/2 and W + n/2 round to the same binary64
// value that value is the exactly rounded sum.  When they do not, the wide
// pass (wide_sum.hpp) sums the squares with no window and sets the scale.
// The sign bits (one byte per 8 elements, element 8j+k in bit k of byte j)
// are what a multi-rank run would exchange.  The device picks the stage:
// while the applied-step count is at most the warm-up length, these kernels
// return before any load and the ordinary update runs instead.
//
// Five kernels, because two global scales sit on the data path:
//   A  momentum + per-block max|x|           one-shot, 8 elements per thread
//   B  exact sum of x^2 in the window, s_w   <= 256 workgroups x 1024, grid-stride
//      with eight 4-element groups' loads in flight; every workgroup first folds A's
//      block maxima (L2-resident), the last one to arrive folds the limbs and
//      writes s_w
//   C  worker compression: sign byte, ew, u = cw + es, per-block max|u|
//   D  exact sum of u^2, s_s                  as B (u is recomputed from the bits)
//   E  server compression + update: m, es, bits, p, p16
// (a wide pass follows B and D; it returns at once unless the window could
// not vouch for its sum).  Per-block maxima go to memory (no same-address atomics, which serialise).
// Element layout of the one-shot kernels: the whole bytes of the sign payload
// cover groups of 4 elements, g < 2*floor(n/8); thread t of workgroup b owns
// groups 512b+t and 512b+t+256, so every vector load and store of a wave is
// one contiguous span.  A thread's 4 sign bits of a group are a nibble; the
// two lanes of an even/odd pair hold the two nibbles of one byte and join
// them with a lane shuffle.  The elements past the last whole byte (fewer
// than 8) are done one by one.
// The exact windowed square: z = x * 2^(40-E) (exact, |z| < 2^41),
//   a = fma(z, z, C1) - C1       z^2 to a multiple of 2^41 (C1 = 1.5*2^93)
//   b = (fma(z, z, -a) + C2) - C2   the rest, to the nearest integer (C2 = 1.5*2^52)
// so z^2 rounded to an integer is a + b; with at most 2^11 elements per
// thread, sum(a) <= 2^93 in steps of 2^41 and |sum(b)| <= 2^51 stay exact.
#include <math.h>

#include "decide.hpp"
#include "exact_norm.hpp"
#include "wide_sum.hpp"

namespace zero {
namespace {

constexpr int kBlock = 256;                  // one-shot kernels A, C, E
// The one-shot kernels run at most kOneShotCap workgroups per CU, enforced by
// a dynamic-LDS reservation they never touch (as the Adam kernel): measured on
// MI355X, momentum 4.7%, compression 3.2% and the update after it 1.6% faster
// than at full occupancy.  A and C also hold block_max's few static LDS bytes,
// which the reservation leaves room for.
constexpr int kOneShotCap = 2;
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
        const int64_t au = int64_t(a * 0x1p-41);              // < 2^53
        const int64_t bu = int64_t(b);                         // |.| <= 2^52
        const int64_t hs = au << 9;                            // au * 2^41 = hs * 2^32
        return exact::Limbs{bu & 0xFFFFFFFFll, (hs & 0xFFFFFFFFll) + (bu >> 32), hs >> 32, 0};
    }
};

// The two groups of 4 elements a thread of a one-shot kernel owns (see the
// layout note above), out of ng = 2*floor(n/8); ragged0 = 4*ng is the first
// element done one by one.
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

__device__ __forceinline__ void momentum4(f16x4 g, f32x4& m, f32x4 e, const Coef& c, uint32_t& mx)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma clang fp contract(off)
        const float gk = float(g[k]) * c.gmul;
        m[k] = c.b1 * m[k] + c.omb1 * gk;
        const uint32_t a = abs_bits(m[k] + e[k]);
        mx = a > mx ? a : mx;
    }
}

__global__ __launch_bounds__(kBlock) void onebit_momentum_kernel(float* __restrict__ m32, const float* __restrict__ ew,
                                                                 const uint16_t* __restrict__ g16, uint64_t n,
                                                                 const zero_step_state_t* __restrict__ st,
                                                                 int64_t warmup, uint32_t* __restrict__ blockmax)
{
    if (st->step <= warmup)                      // a warm-up step: the Adam update runs instead
        return;
    extern __shared__ char occupancy_reserve[];  // see kOneShotCap
    if (n == UINT64_MAX)
        occupancy_reserve[threadIdx.x] = 0;
    const Groups gr(n);
    f32x4* __restrict__ M = reinterpret_cast<f32x4*>(m32);
    const f32x4* __restrict__ EW = reinterpret_cast<const f32x4*>(ew);
    const u32x2* __restrict__ G = reinterpret_cast<const u32x2*>(g16);
    uint32_t mx = 0;
    if (gr.both()) {
        // Every stream here is read once and m is written back in place:
        // nontemporal loads and stores throughout (the gradient alone: 5%
        // faster; m and e_w as well: the 1-bit stage 2.6% faster).
        const u32x2 ga = __builtin_nontemporal_load(G + gr.ja), gb = __builtin_nontemporal_load(G + gr.jb);
        f32x4 ma = __builtin_nontemporal_load(M + gr.ja), mb = __builtin_nontemporal_load(M + gr.jb);
        const f32x4 ea = __builtin_nontemporal_load(EW + gr.ja), eb = __builtin_nontemporal_load(EW + gr.jb);
        __builtin_amdgcn_sched_barrier(0);
        // the loads are out before the skip flag is read (see loads_first_use)
        if (st->skip) {
            if (n == UINT64_MAX)
                M[gr.ja] = ma + mb + ea + eb + bits_of(ga) + bits_of(gb);
            return;
        }
        const Coef c = coef_of(st);
        momentum4(__builtin_bit_cast(f16x4, ga), ma, ea, c, mx);
        momentum4(__builtin_bit_cast(f16x4, gb), mb, eb, c, mx);
        __builtin_nontemporal_store(ma, M + gr.ja);
        __builtin_nontemporal_store(mb, M + gr.jb);
    } else {
        if (st->skip)
            return;
        if (gr.first()) {
            f32x4 ma = M[gr.ja];
            momentum4(__builtin_bit_cast(f16x4, G[gr.ja]), ma, EW[gr.ja], coef_of(st), mx);
            M[gr.ja] = ma;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
#pragma clang fp contract(off)
        const Coef c = coef_of(st);
        const uint64_t i = gr.ragged0 + threadIdx.x;
        const float gk = float(__builtin_bit_cast(_Float16, g16[i])) * c.gmul;
        const float mi = c.b1 * m32[i] + c.omb1 * gk;
        m32[i] = mi;
        const uint32_t a = abs_bits(mi + ew[i]);
        mx = a > mx ? a : mx;
    }
    mx = block_max<kBlock>(mx);
    if (threadIdx.x == 0)
        blockmax[blockIdx.x] = mx;
}

// ---- B / D: the exact windowed sum and the scale ------------------------------------

// The vector whose scale is taken: x = m + ew (worker), or u = s_w*sgn + es (server).
struct WorkerX {
    const float* m;
    const float* ew;
    __device__ __forceinline__ float at(uint64_t i) const { return m[i] + ew[i]; }
    // group j: elements 4j..4j+3
    __device__ __forceinline__ void vec(uint64_t j, float (&x)[4]) const
    {
        const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(m) + j);
        const f32x4 c = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(ew) + j);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            x[k] = a[k] + c[k];
    }
};

struct ServerU {
    const uint8_t* bits;
    const float* es;
    float sw;
    __device__ __forceinline__ float at(uint64_t i) const
    {
        const float c = ((bits[i >> 3] >> (i & 7)) & 1) ? sw : -sw;
        return c + es[i];
    }
    __device__ __forceinline__ void vec(uint64_t j, float (&x)[4]) const
    {
        const uint32_t nib = nibble_of(bits, j);
        const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(es) + j);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            x[k] = (((nib >> k) & 1) ? sw : -sw) + a[k];
    }
};

// Which scale a sum kernel writes.
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

// The window rounds each of the n squares to a whole number of units (off by
// at most half a unit each), so the exact sum lies within n/2 units of the
// window's integer W.  Rounding to binary64 is monotonic: when W - n/2 and
// W + n/2 round to the same value, every sum between them does, and RNE(W)
// is the exactly rounded sum.  (W >= 2^80 whenever a value is nonzero, so
// 2W - n > 0.)  Otherwise the wide pass decides.
__device__ __forceinline__ bool window_decides(uint64_t hi, uint64_t lo, uint64_t n)
{
    const unsigned __int128 w2 = ((unsigned __int128)hi << 65) | ((unsigned __int128)lo << 1);   // 2W < 2^124
    const unsigned __int128 a = w2 - n, b = w2 + n;
    return u128_to_f64(uint64_t(a >> 64), uint64_t(a)) == u128_to_f64(uint64_t(b >> 64), uint64_t(b));
}

template <int WHICH, typename V>
__device__ void sum_and_scale(const V& vsrc, uint64_t n, const uint32_t* __restrict__ blockmax, uint64_t nmax,
                              const zero_step_state_t* __restrict__ st, zero_onebit_state_t* __restrict__ ob,
                              NormPartial* __restrict__ ws)
{
    // the window: max over the previous kernel's block maxima (L2-resident;
    // eight loads in flight per thread, or the fold is a chain of latencies)
    uint32_t mx = 0;
    uint64_t b = threadIdx.x;
    for (; b + 7 * kNormBlock < nmax; b += 8 * kNormBlock) {
        uint32_t v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            v[q] = blockmax[b + q * kNormBlock];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            mx = v[q] > mx ? v[q] : mx;
    }
    for (; b < nmax; b += kNormBlock)
        mx = blockmax[b] > mx ? blockmax[b] : mx;
    __shared__ uint32_t s_mx;
    mx = block_max<kNormBlock>(mx);
    if (threadIdx.x == 0)
        s_mx = mx;
    __syncthreads();
    mx = s_mx;
    const int E = mx ? exponent_of(mx) : 0;
    const double w = ldexp(1.0, 40 - E);

    AccWin acc;
    if (mx) {
        const uint64_t ng = (n >> 3) * 2;                     // groups of 4 in whole payload bytes
        const uint64_t stride = uint64_t(gridDim.x) * kNormBlock;
        // a round: each wave reads 512 consecutive groups (its eight loads
        // 64 groups apart), the grid 8 * stride groups
        const uint64_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        uint64_t j = (uint64_t(blockIdx.x) * (kNormBlock / 64) + wave) * 512 + lane;
        for (; j + 448 < ng; j += 8 * stride) {               // eight groups' loads in flight
            float x[8][4];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                vsrc.vec(j + 64 * q, x[q]);
#pragma unroll
            for (int q = 0; q < 8; ++q)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    acc.add(x[q][k], w);
        }
        for (int q = 0; q < 8; ++q, j += 64) {                // the grid's last, partial round
            if (j < ng) {
                float x[4];
                vsrc.vec(j, x);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    acc.add(x[k], w);
            }
        }
        if (blockIdx.x == 0 && threadIdx.x < (n & 7))
            acc.add(vsrc.at(4 * ng + threadIdx.x), w);   // elements past the last whole byte
    }
    exact::Limbs s = acc.limbs();
    uint32_t flag = 0;
    exact::block_fold<kNormBlock>(s, flag);

    __shared__ uint32_t s_last;
    if (threadIdx.x == 0) {
        ws[blockIdx.x] = exact::make_partial(s, 0);
        // release this partial; the last workgroup acquires everyone's
        const uint32_t prev = __hip_atomic_fetch_add(&ob->done_blocks, 1u, __ATOMIC_RELEASE,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        const bool last = prev == gridDim.x - 1;
        if (last)
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_last = last ? 1u : 0u;
    }
    __syncthreads();
    if (!s_last || threadIdx.x >= 64)
        return;
    // the last workgroup's first wave folds the partials, four loads per lane
    // in flight per batch of 256, then a shuffle fold with no barrier
    exact::Limbs t{0, 0, 0, 0};
    uint32_t tflag = 0;
    for (uint32_t b0 = 0; b0 < gridDim.x; b0 += 256) {
        NormPartial q[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t b = b0 + threadIdx.x + 64 * k;
            q[k] = b < gridDim.x ? ws[b] : NormPartial{0, 0};
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
            exact::fold_partial(t, tflag, q[k]);
    }
    exact::block_fold<64>(t, tflag);
    if (threadIdx.x == 0) {
        uint64_t hi = 0, lo = 0;
        exact::limbs_to_u128(t, hi, lo);                        // < n * 2^82: always fits
        const int qexp = 2 * E - 80;
        if (WHICH == kWorker) {
            ob->qexp_w = mx ? qexp : 0;
            ob->units_w[0] = lo;
            ob->units_w[1] = hi;
        } else {
            ob->qexp_s = mx ? qexp : 0;
            ob->units_s[0] = lo;
            ob->units_s[1] = hi;
        }
        if (!mx || window_decides(hi, lo, n)) {
            const double S = mx ? ldexp(u128_to_f64(hi, lo), qexp) : 0.0;
            set_scale<WHICH>(ob, S, n);
        } else {
            ob->wide_pending |= 1u << WHICH;                    // the wide pass sets the scale
        }
        ob->done_blocks = 0;                                    // re-arm for the next sum
    }
}

__global__ __launch_bounds__(kNormBlock) void onebit_sum_worker_kernel(const float* __restrict__ m32,
                                                                       const float* __restrict__ ew, uint64_t n,
                                                                       const uint32_t* __restrict__ blockmax,
                                                                       uint64_t nmax,
                                                                       const zero_step_state_t* __restrict__ st,
                                                                       int64_t warmup,
                                                                       zero_onebit_state_t* __restrict__ ob,
                                                                       NormPartial* __restrict__ ws)
{
    if (st->skip || st->step <= warmup)
        return;
    sum_and_scale<kWorker>(WorkerX{m32, ew}, n, blockmax, nmax, st, ob, ws);
}

__global__ __launch_bounds__(kNormBlock) void onebit_sum_server_kernel(const uint8_t* __restrict__ bits_w,
                                                                       const float* __restrict__ es, uint64_t n,
                                                                       const uint32_t* __restrict__ blockmax,
                                                                       uint64_t nmax,
                                                                       const zero_step_state_t* __restrict__ st,
                                                                       int64_t warmup,
                                                                       zero_onebit_state_t* __restrict__ ob,
                                                                       NormPartial* __restrict__ ws)
{
    if (st->skip || st->step <= warmup)
        return;
    sum_and_scale<kServer>(ServerU{bits_w, es, ob->scale_w}, n, blockmax, nmax, st, ob, ws);
}

// ---- C: worker compression ----------------------------------------------------------

// x = m + ew -> sign nibble, ew = x - s_w*sgn(x), and the max of |s_w*sgn(x) + es|.
__device__ __forceinline__ uint32_t compress4(f32x4 m, f32x4& e, f32x4 s, float sw, uint32_t& mx)
{
    uint32_t nib = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float x = m[k] + e[k];
        const float cw = sgn_scale(x, sw);
        nib |= (x < 0.0f ? 0u : 1u) << k;
        e[k] = x - cw;
        const uint32_t a = abs_bits(cw + s[k]);
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
                                                                        uint32_t* __restrict__ blockmax)
{
    if (st->step <= warmup)
        return;
    extern __shared__ char occupancy_reserve[];  // see kOneShotCap
    if (n == UINT64_MAX)
        occupancy_reserve[threadIdx.x] = 0;
    const Groups gr(n);
    const f32x4* __restrict__ M = reinterpret_cast<const f32x4*>(m32);
    f32x4* __restrict__ EW = reinterpret_cast<f32x4*>(ew);
    const f32x4* __restrict__ ES = reinterpret_cast<const f32x4*>(es);
    uint32_t mx = 0, nib_a = 0, nib_b = 0;
    if (gr.both()) {
        // nontemporal throughout: e_w is rewritten in place, and a plain load
        // ahead of an in-place nontemporal store is the slow pattern
        const f32x4 ma = __builtin_nontemporal_load(M + gr.ja), mb = __builtin_nontemporal_load(M + gr.jb);
        f32x4 ea = __builtin_nontemporal_load(EW + gr.ja), eb = __builtin_nontemporal_load(EW + gr.jb);
        const f32x4 sa = __builtin_nontemporal_load(ES + gr.ja), sb = __builtin_nontemporal_load(ES + gr.jb);
        __builtin_amdgcn_sched_barrier(0);
        if (st->skip) {                          // loads first (see loads_first_use)
            if (n == UINT64_MAX)
                EW[gr.ja] = ma + mb + ea + eb + sa + sb;
            return;
        }
        const float sw = ob->scale_w;
        nib_a = compress4(ma, ea, sa, sw, mx);
        nib_b = compress4(mb, eb, sb, sw, mx);
        __builtin_nontemporal_store(ea, EW + gr.ja);
        __builtin_nontemporal_store(eb, EW + gr.jb);
    } else {
        if (st->skip)
            return;
        if (gr.first()) {
            f32x4 ea = EW[gr.ja];
            nib_a = compress4(M[gr.ja], ea, ES[gr.ja], ob->scale_w, mx);
            EW[gr.ja] = ea;
        }
    }
    store_byte_pair(bits_w, gr.ja, nib_a, gr.first());
    store_byte_pair(bits_w, gr.jb, nib_b, gr.both());
    if (blockIdx.x == 0 && threadIdx.x == 0 && (n & 7)) {     // the ragged last byte
        const uint64_t nvec = n >> 3;
        const float sw = ob->scale_w;
        uint32_t byte = 0;
        for (uint64_t i = nvec << 3; i < n; ++i) {
            const float x = m32[i] + ew[i];
            const float cw = sgn_scale(x, sw);
            byte |= (x < 0.0f ? 0u : 1u) << (i & 7);
            ew[i] = x - cw;
            const uint32_t a = abs_bits(cw + es[i]);
            mx = a > mx ? a : mx;
        }
        bits_w[nvec] = uint8_t(byte);
    }
    mx = block_max<kBlock>(mx);
    if (threadIdx.x == 0)
        blockmax[blockIdx.x] = mx;
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

// Workspace: block maxima of A and C, then the partials of B and D.
struct Plan {
    uint64_t grid1;                 // one-shot kernels (A, C, E)
    uint64_t grid2;                 // sums (B, D)
    uint64_t off_max_a, off_max_c, off_part_b, off_part_d, off_wide, bytes;
};

Plan plan(uint64_t n)
{
    Plan p;
    const uint64_t nvec = n >> 3;
    p.grid1 = (nvec + kBlock - 1) / kBlock;
    if (p.grid1 < 1) p.grid1 = 1;
    // at most 2^11 elements per thread, so the binary64 window sums stay exact
    p.grid2 = norm_grid(n);
    const uint64_t per = uint64_t(kNormBlock) * 2048;
    if ((n + p.grid2 * kNormBlock - 1) / (p.grid2 * kNormBlock) > 2048)
        p.grid2 = (n + per - 1) / per;
    auto up = [](uint64_t b) { return (b + 255) / 256 * 256; };
    p.off_max_a = 0;
    p.off_max_c = up(p.grid1 * 4);
    p.off_part_b = p.off_max_c + up(p.grid1 * 4);
    p.off_part_d = p.off_part_b + up(p.grid2 * sizeof(NormPartial));
    p.off_wide = p.off_part_d + up(p.grid2 * sizeof(NormPartial));
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
    uint32_t* max_c = reinterpret_cast<uint32_t*>(ws + pl.off_max_c);
    NormPartial* part_b = reinterpret_cast<NormPartial*>(ws + pl.off_part_b);
    NormPartial* part_d = reinterpret_cast<NormPartial*>(ws + pl.off_part_d);
    wide::WidePartial* part_w = reinterpret_cast<wide::WidePartial*>(ws + pl.off_wide);
    const dim3 gw(uint32_t(wide::grid(n)));
    hipStream_t s = (hipStream_t)stream;
    const dim3 g1(uint32_t(pl.grid1)), g2(uint32_t(pl.grid2));
    const uint32_t cap = lds_reservation(kOneShotCap);
    const uint32_t cap_ac = cap > 256 ? cap - 256 : 0;     // room for block_max's static LDS
    // a warm-up step: the ordinary update (it returns at once in the compression stage)
    int rc = adam_step_gated(p16, p32, m32, v32, grad16, n, dev_state, stream, warmup);
    if (rc != ZERO_OK)
        return rc;
    hipLaunchKernelGGL(onebit_momentum_kernel, g1, dim3(kBlock), cap_ac, s, m32, err_w, grad16, n, dev_state,
                       warmup, max_a);
    if ((rc = launch_status()) != ZERO_OK)
        return rc;
    hipLaunchKernelGGL(onebit_sum_worker_kernel, g2, dim3(kNormBlock), 0, s, m32, err_w, n, max_a, pl.grid1,
                       dev_state, warmup, dev_onebit, part_b);
    if ((rc = launch_status()) != ZERO_OK)
        return rc;
    hipLaunchKernelGGL((wide::wide_sum_kernel<WorkerValues, ScaleFinish<kWorker>>), gw, dim3(wide::kBlock), 0, s,
                       WorkerValues{m32, err_w}, n, ScaleFinish<kWorker>{dev_onebit, n}, part_w);
    if ((rc = launch_status()) != ZERO_OK)
        return rc;
    hipLaunchKernelGGL(onebit_compress_worker_kernel, g1, dim3(kBlock), cap_ac, s, m32, err_w, err_s, bits_w, n,
                       dev_state, warmup, dev_onebit, max_c);
    if ((rc = launch_status()) != ZERO_OK)
        return rc;
    hipLaunchKernelGGL(onebit_sum_server_kernel, g2, dim3(kNormBlock), 0, s, bits_w, err_s, n, max_c, pl.grid1,
                       dev_state, warmup, dev_onebit, part_d);
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
