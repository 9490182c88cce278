// host_step.cpp -- the ZeRO-Offload form of the shard step: the fp32 master
// parameters, momentum and variance stay in host memory and the CPU steps
// them, while the GPU keeps only what the forward and backward passes need
// (the DeepSpeed article's ZeRO-Offload paragraph: ZeRO-2 plus CPU memory,
// 13B parameters on one V100).  Per step the fp16 gradient partition comes
// down over PCIe, the CPU computes the exact norm, the decision and the
// AdamW update, and the fp16 parameters go back up.
//
// Host design (x86-64 with AVX-512F/BW/VL/DQ, F16C and FMA; both CPUs this
// library targets have them, and zero_host_create refuses a CPU without):
//   * a persistent pool of worker threads owned by a caller-created context;
//     every parallel phase splits its range into contiguous per-worker slices
//     aligned to 64 elements, and the calling thread works as worker 0;
//   * the update: 16 parameters per AVX-512 iteration, masked loads/stores at
//     the slice edges; in the body (arrays 64-byte aligned) plain stores of the
//     fp32 p, m, v, which go back to the lines just loaded (no
//     read-for-ownership; a nontemporal store to a line the core holds was
//     8-28% slower on the two CPUs measured), and a nontemporal store of the
//     fp16 copy, whose staging buffer is not read here (28 bytes of DRAM
//     traffic per parameter); every operation is one binary32
//     round-to-nearest-even operation in the order of the device kernel, and
//     the fp16 copy is VCVTPS2PH with round-to-nearest-even;
//   * the exact norm: the device's binary64 split (h = fma(x,x,C) - C,
//     l = fma(x,x,-h)) in 8-lane registers, each lane summing at most 2^12
//     squares before it is flushed into a 128-bit integer per worker, so the
//     sum is exact and the decision bit-identical to the GPU's;
//   * the offload step pipelines: the D2H copy of the gradient is split into
//     chunks, each followed by an event.  When the device has already taken
//     the decision (its exact reduction is bit-identical to this one), the
//     128-byte state comes down first and the workers update chunk i while
//     chunk i+1 is in flight; otherwise they reduce chunk i while chunk i+1 is
//     in flight, decide, then update.  Either way the H2D copy of each chunk
//     of fp16 parameters is enqueued as soon as the workers have updated it.
#include <hip/hip_runtime.h>
#include <immintrin.h>
#include <sched.h>
#include <string.h>

#include <algorithm>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include "decide.hpp"
#include "zero_internal.hpp"

#define ZERO_HOST_ISA __attribute__((target("avx512f,avx512bw,avx512vl,avx512dq,f16c,fma")))

namespace zero {
namespace {

// ---- worker pool ---------------------------------------------------------------------

class Pool {
public:
    explicit Pool(int threads) : threads_(threads)
    {
        for (int w = 1; w < threads_; ++w)
            workers_.emplace_back([this, w] { loop(w); });
    }
    ~Pool()
    {
        {
            std::lock_guard<std::mutex> g(mu_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto& t : workers_)
            t.join();
    }
    int size() const { return threads_; }

    // Runs f(worker) on every worker (the caller is worker 0) and returns when
    // all have finished.
    void run(const std::function<void(int)>& f)
    {
        std::unique_lock<std::mutex> g(run_mu_);
        if (threads_ == 1) {
            f(0);
            return;
        }
        {
            std::lock_guard<std::mutex> l(mu_);
            job_ = &f;
            pending_ = threads_ - 1;
            ++generation_;
        }
        cv_.notify_all();
        f(0);
        std::unique_lock<std::mutex> l(mu_);
        done_cv_.wait(l, [this] { return pending_ == 0; });
        job_ = nullptr;
    }

private:
    void loop(int w)
    {
        uint64_t seen = 0;
        for (;;) {
            const std::function<void(int)>* job;
            {
                std::unique_lock<std::mutex> l(mu_);
                cv_.wait(l, [&] { return stop_ || generation_ != seen; });
                if (stop_)
                    return;
                seen = generation_;
                job = job_;
            }
            (*job)(w);
            {
                std::lock_guard<std::mutex> l(mu_);
                if (--pending_ == 0)
                    done_cv_.notify_one();
            }
        }
    }

    int threads_;
    std::vector<std::thread> workers_;
    std::mutex mu_, run_mu_;
    std::condition_variable cv_, done_cv_;
    const std::function<void(int)>* job_ = nullptr;
    uint64_t generation_ = 0;
    int pending_ = 0;
    bool stop_ = false;
};

// Slice [begin, end) of [lo, hi) for worker w of `workers`, with interior
// boundaries on multiples of 64 elements.
inline void slice(uint64_t lo, uint64_t hi, int w, int workers, uint64_t& begin, uint64_t& end)
{
    const uint64_t units = (hi - lo + 63) / 64;
    const uint64_t per = units / workers, extra = units % workers;
    const uint64_t u0 = w * per + (uint64_t(w) < extra ? w : extra);
    const uint64_t u1 = u0 + per + (uint64_t(w) < extra ? 1 : 0);
    begin = lo + u0 * 64 < hi ? lo + u0 * 64 : hi;
    end = lo + u1 * 64 < hi ? lo + u1 * 64 : hi;
}

struct alignas(64) NormAcc {
    unsigned __int128 units;     // exact sum of squares, 2^-48 units
    bool bad;                    // an inf/NaN was seen
};

// ---- exact norm (AVX-512) --------------------------------------------------------

constexpr double kSplit16 = 0x1.8p44;            // ulp 2^-8: h is x^2 to a multiple of 2^-8
constexpr int kFlushIters = 4096;                // squares per lane between flushes (<= 2^12)

ZERO_HOST_ISA inline void square_acc(__m512d x, __m512d& h, __m512d& l)
{
    const __m512d c = _mm512_set1_pd(kSplit16);
    const __m512d t = _mm512_sub_pd(_mm512_fmadd_pd(x, x, c), c);
    h = _mm512_add_pd(h, t);
    l = _mm512_add_pd(l, _mm512_fmsub_pd(x, x, t));
}

// Adds the lanes of the accumulators (sum(h) < 2^44 in steps of 2^-8,
// |sum(l)| < 2^3 in steps of 2^-48 per lane) to the 128-bit total.
ZERO_HOST_ISA inline void flush(__m512d (&h)[4], __m512d (&l)[4], unsigned __int128& units)
{
    alignas(64) int64_t hv[8], lv[8];
    __int128 t = 0;
    for (int k = 0; k < 4; ++k) {
        _mm512_store_si512(hv, _mm512_cvtpd_epi64(_mm512_mul_pd(h[k], _mm512_set1_pd(256.0))));
        _mm512_store_si512(lv, _mm512_cvtpd_epi64(_mm512_mul_pd(l[k], _mm512_set1_pd(0x1p48))));
        for (int j = 0; j < 8; ++j)
            t += (__int128(hv[j]) << 40) + lv[j];
        h[k] = _mm512_setzero_pd();
        l[k] = _mm512_setzero_pd();
    }
    units += (unsigned __int128)t;               // a sum of squares: never negative
}

ZERO_HOST_ISA void norm_range(const uint16_t* g, uint64_t a, uint64_t b, NormAcc& acc)
{
    const __m512i expo = _mm512_set1_epi16(0x7C00);
    __m512d h[4] = {_mm512_setzero_pd(), _mm512_setzero_pd(), _mm512_setzero_pd(), _mm512_setzero_pd()};
    __m512d l[4] = {h[0], h[0], h[0], h[0]};
    __mmask32 bad = 0;
    int iters = 0;
    for (uint64_t i = a; i < b; i += 32) {
        const uint64_t left = b - i;
        const __mmask32 m = left >= 32 ? ~__mmask32(0) : __mmask32((1u << left) - 1);
        const __m512i v = _mm512_maskz_loadu_epi16(m, g + i);
        bad |= _mm512_mask_cmpeq_epi16_mask(m, _mm512_and_si512(v, expo), expo);
        const __m512 f0 = _mm512_cvtph_ps(_mm512_castsi512_si256(v));
        const __m512 f1 = _mm512_cvtph_ps(_mm512_extracti64x4_epi64(v, 1));
        square_acc(_mm512_cvtps_pd(_mm512_castps512_ps256(f0)), h[0], l[0]);
        square_acc(_mm512_cvtps_pd(_mm256_castpd_ps(_mm512_extractf64x4_pd(_mm512_castps_pd(f0), 1))), h[1], l[1]);
        square_acc(_mm512_cvtps_pd(_mm512_castps512_ps256(f1)), h[2], l[2]);
        square_acc(_mm512_cvtps_pd(_mm256_castpd_ps(_mm512_extractf64x4_pd(_mm512_castps_pd(f1), 1))), h[3], l[3]);
        if (++iters == kFlushIters) {
            if (!bad)
                flush(h, l, acc.units);
            iters = 0;
        }
    }
    if (bad)
        acc.bad = true;                          // the sum is void; the step is skipped
    else
        flush(h, l, acc.units);
}

// ---- AdamW update (AVX-512) -------------------------------------------------------

struct Coef {
    float gmul, b1, b2, omb1, omb2, bc1, bc2, eps, wd, lr;
};

template <bool NT>
ZERO_HOST_ISA inline void adam16(uint16_t* p16, float* p32, float* m32, float* v32, const uint16_t* g16,
                                 __mmask16 mk, const Coef& c)
{
    const __m512 g = _mm512_mul_ps(_mm512_cvtph_ps(_mm256_maskz_loadu_epi16(mk, g16)), _mm512_set1_ps(c.gmul));
    const __m512 p = _mm512_maskz_loadu_ps(mk, p32);
    const __m512 m = _mm512_maskz_loadu_ps(mk, m32);
    const __m512 v = _mm512_maskz_loadu_ps(mk, v32);
    const __m512 mn = _mm512_add_ps(_mm512_mul_ps(_mm512_set1_ps(c.b1), m), _mm512_mul_ps(_mm512_set1_ps(c.omb1), g));
    const __m512 vn = _mm512_add_ps(_mm512_mul_ps(_mm512_set1_ps(c.b2), v),
                                    _mm512_mul_ps(_mm512_set1_ps(c.omb2), _mm512_mul_ps(g, g)));
    const __m512 mh = _mm512_div_ps(mn, _mm512_set1_ps(c.bc1));
    const __m512 vh = _mm512_div_ps(vn, _mm512_set1_ps(c.bc2));
    const __m512 u = _mm512_add_ps(_mm512_div_ps(mh, _mm512_add_ps(_mm512_sqrt_ps(vh), _mm512_set1_ps(c.eps))),
                                   _mm512_mul_ps(_mm512_set1_ps(c.wd), p));
    const __m512 pn = _mm512_sub_ps(p, _mm512_mul_ps(_mm512_set1_ps(c.lr), u));
    const __m256i h = _mm512_cvtps_ph(pn, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
    if (NT) {                                    // aligned body: only the fp16 copy bypasses the caches
        _mm512_store_ps(p32, pn);
        _mm512_store_ps(m32, mn);
        _mm512_store_ps(v32, vn);
        _mm256_stream_si256(reinterpret_cast<__m256i*>(p16), h);
    } else {
        _mm512_mask_storeu_ps(p32, mk, pn);
        _mm512_mask_storeu_ps(m32, mk, mn);
        _mm512_mask_storeu_ps(v32, mk, vn);
        _mm256_mask_storeu_epi16(p16, mk, h);
    }
}

ZERO_HOST_ISA void adam_range(uint16_t* p16, float* p32, float* m32, float* v32, const uint16_t* g16, uint64_t a,
                              uint64_t b, const Coef& c)
{
    uint64_t i = a;
    // masked elements up to the first index where every stream is 64-byte aligned
    // (the fp16 copy then is 32-byte aligned), if the arrays share that phase
    const uintptr_t pa = reinterpret_cast<uintptr_t>(p32 + a);
    const uint64_t body = (pa & 3) ? b : a + ((64 - (pa & 63)) & 63) / 4;
    const bool nt = body < b && !(reinterpret_cast<uintptr_t>(m32 + body) & 63) &&
                    !(reinterpret_cast<uintptr_t>(v32 + body) & 63) &&
                    !(reinterpret_cast<uintptr_t>(p16 + body) & 31);
    if (nt) {
        for (; i < body; i += 16) {
            const uint64_t left = body - i;
            const __mmask16 mk = left >= 16 ? __mmask16(0xFFFF) : __mmask16((1u << left) - 1);
            adam16<false>(p16 + i, p32 + i, m32 + i, v32 + i, g16 + i, mk, c);
        }
        i = body;
        for (; i + 16 <= b; i += 16)
            adam16<true>(p16 + i, p32 + i, m32 + i, v32 + i, g16 + i, 0xFFFF, c);
        _mm_sfence();                            // the fp16 copy's nontemporal stores visible before the pool returns
    }
    for (; i < b; i += 16) {
        const uint64_t left = b - i;
        const __mmask16 mk = left >= 16 ? __mmask16(0xFFFF) : __mmask16((1u << left) - 1);
        adam16<false>(p16 + i, p32 + i, m32 + i, v32 + i, g16 + i, mk, c);
    }
}

// ---- streaming copy (the host bandwidth reference) ---------------------------------

ZERO_HOST_ISA void copy_range(uint8_t* dst, const uint8_t* src, uint64_t a, uint64_t b)
{
    for (uint64_t i = a; i < b; i += 64)
        _mm512_stream_si512(reinterpret_cast<__m512i*>(dst + i),
                            _mm512_stream_load_si512(reinterpret_cast<const void*>(src + i)));
    _mm_sfence();
}

bool cpu_ok()
{
    __builtin_cpu_init();
    return __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
           __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("avx512dq") &&
           __builtin_cpu_supports("f16c") && __builtin_cpu_supports("fma");
}

int online_cpus()
{
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof set, &set) == 0)
        return CPU_COUNT(&set);
    const unsigned n = std::thread::hardware_concurrency();
    return n ? int(n) : 1;
}

Coef coef_of(const zero_step_state_t* st)
{
    return Coef{st->gmul, st->beta1, st->beta2, st->omb1, st->omb2, st->bc1, st->bc2, st->eps, st->wd, st->lr};
}

}  // namespace
}  // namespace zero

using namespace zero;

struct zero_host_ctx {
    explicit zero_host_ctx(int threads) : pool(threads), acc(threads) {}
    Pool pool;
    std::vector<NormAcc> acc;
    std::vector<hipEvent_t> events;
    std::vector<uint64_t> bounds;                // chunk boundaries of the last offloaded step
    int event_device = -1;
};

namespace {

void norm_reset(zero_host_ctx_t* ctx)
{
    for (auto& a : ctx->acc) {
        a.units = 0;
        a.bad = false;
    }
}

void norm_chunk(zero_host_ctx_t* ctx, const uint16_t* g, uint64_t lo, uint64_t hi)
{
    const int T = ctx->pool.size();
    ctx->pool.run([&](int w) {
        uint64_t a, b;
        slice(lo, hi, w, T, a, b);
        if (a < b)
            norm_range(g, a, b, ctx->acc[w]);
    });
}

// Folds the workers' exact sums and takes the decision.
void norm_decide(zero_host_ctx_t* ctx, const zero_hparams_t* hp, zero_step_state_t* st)
{
    unsigned __int128 total = 0;
    bool bad = false, too_large = false;
    for (const auto& a : ctx->acc) {
        bad |= a.bad;
        too_large |= __builtin_add_overflow(total, a.units, &total);
    }
    decide_state(st, decide_args(hp), uint64_t(total >> 64), uint64_t(total), bad || too_large);
}

void adam_chunk(zero_host_ctx_t* ctx, uint16_t* p16, float* p32, float* m32, float* v32, const uint16_t* g16,
                uint64_t lo, uint64_t hi, const Coef& c)
{
    const int T = ctx->pool.size();
    ctx->pool.run([&](int w) {
        uint64_t a, b;
        slice(lo, hi, w, T, a, b);
        if (a < b)
            adam_range(p16, p32, m32, v32, g16, a, b, c);
    });
}

}  // namespace

extern "C" int zero_host_create(int threads, zero_host_ctx_t** out)
{
    if (!out)
        return ZERO_EINVAL;
    *out = nullptr;
    if (!cpu_ok())
        return ZERO_ENOTSUP;
    if (threads <= 0)
        threads = online_cpus();
    if (threads > 1024)
        return ZERO_ERANGE;
    zero_host_ctx_t* ctx = new (std::nothrow) zero_host_ctx_t(threads);
    if (!ctx)
        return ZERO_ENOMEM;
    *out = ctx;
    return ZERO_OK;
}

extern "C" void zero_host_destroy(zero_host_ctx_t* ctx)
{
    if (!ctx)
        return;
    for (hipEvent_t e : ctx->events)
        (void)hipEventDestroy(e);
    delete ctx;
}

extern "C" int zero_host_threads(const zero_host_ctx_t* ctx) { return ctx ? ctx->pool.size() : 0; }

extern "C" int zero_host_state_init(zero_step_state_t* state, double initial_scale)
{
    if (!state || !(initial_scale > 0) || !isfinite(initial_scale))
        return ZERO_EINVAL;
    memset(state, 0, sizeof *state);
    state->loss_scale = initial_scale;
    state->beta1_pow = 1.0;
    state->beta2_pow = 1.0;
    return ZERO_OK;
}

extern "C" int zero_host_norm_overflow(zero_host_ctx_t* ctx, const uint16_t* grad16, uint64_t n,
                                       const zero_hparams_t* hp, zero_step_state_t* state)
{
    if (!ctx || !hp || !state || (n && !grad16))
        return ZERO_EINVAL;
    if (!hparams_ok(hp))
        return ZERO_EINVAL;
    norm_reset(ctx);
    if (n)
        norm_chunk(ctx, grad16, 0, n);
    norm_decide(ctx, hp, state);
    return ZERO_OK;
}

extern "C" int zero_host_adam_step(zero_host_ctx_t* ctx, uint16_t* p16, float* p32, float* m32, float* v32,
                                   const uint16_t* grad16, uint64_t n, const zero_step_state_t* state)
{
    if (!ctx || !state || (n && (!p16 || !p32 || !m32 || !v32 || !grad16)))
        return ZERO_EINVAL;
    if (state->skip || n == 0)
        return ZERO_OK;
    adam_chunk(ctx, p16, p32, m32, v32, grad16, 0, n, coef_of(state));
    return ZERO_OK;
}

extern "C" int zero_host_stream_copy(zero_host_ctx_t* ctx, void* dst, const void* src, uint64_t bytes)
{
    if (!ctx || ((!dst || !src) && bytes))
        return ZERO_EINVAL;
    if (!is_aligned(dst, 64) || !is_aligned(src, 64) || (bytes & 63))
        return ZERO_EALIGN;
    const int T = ctx->pool.size();
    ctx->pool.run([&](int w) {
        uint64_t a, b;
        slice(0, bytes / 64, w, T, a, b);        // in 64-byte lines
        if (a < b)
            copy_range(static_cast<uint8_t*>(dst), static_cast<const uint8_t*>(src), a * 64, b * 64);
    });
    return ZERO_OK;
}

namespace {

// Chunk boundaries of an offloaded step over n elements, chunks at most
// `largest` (a multiple of 64) elements long.  The first chunks ramp up from
// largest/16 by doubling and the last ones ramp down the same way, so the CPU
// starts updating once a small first chunk has landed and the last
// parameters go up right after their update: the copy of a full chunk is
// neither waited for at the start nor left over at the end.  Every boundary
// but n is a multiple of 64.
void chunk_bounds(uint64_t n, uint64_t largest, std::vector<uint64_t>& b)
{
    b.clear();
    b.push_back(0);
    if (n == 0)
        return;
    uint64_t m = (largest / 16) & ~uint64_t(63);
    if (m < 64) m = 64;
    std::vector<uint64_t> ramp;                  // m, 2m, 4m, ... below `largest`
    uint64_t r = 0;
    for (uint64_t s = m; s < largest; s *= 2) {
        ramp.push_back(s);
        r += s;
    }
    const uint64_t n64 = n & ~uint64_t(63);
    auto add = [&](uint64_t len) { b.push_back(b.back() + len); };
    if (n64 >= 2 * r + largest) {
        for (uint64_t s : ramp) add(s);
        const uint64_t mid = n64 - 2 * r;
        if (mid % largest) add(mid % largest);
        for (uint64_t q = mid / largest; q; --q) add(largest);
        for (auto it = ramp.rbegin(); it != ramp.rend(); ++it) add(*it);
    } else {                                     // too short for both ramps: ramp up only
        uint64_t s = m;
        while (b.back() < n64) {
            add(std::min(s, n64 - b.back()));
            s = std::min(2 * s, largest);
        }
    }
    if (b.back() == 0)
        b.push_back(n);                          // fewer than 64 elements: one chunk
    else
        b.back() = n;                            // the last chunk takes the ragged end
}

}  // namespace

extern "C" int zero_offload_step(zero_host_ctx_t* ctx, const uint16_t* dev_grad16, uint16_t* dev_p16,
                                 uint16_t* host_grad16, uint16_t* host_p16, float* p32, float* m32, float* v32,
                                 uint64_t n, const zero_hparams_t* hp, zero_step_state_t* state,
                                 const zero_step_state_t* dev_state, uint64_t chunk_elems, void* stream)
{
    if (!ctx || !state || (!dev_state && !hp) ||
        (n && (!dev_grad16 || !dev_p16 || !host_grad16 || !host_p16 || !p32 || !m32 || !v32)))
        return ZERO_EINVAL;
    if (!dev_state && !hparams_ok(hp))
        return ZERO_EINVAL;
    if (dev_state && !is_aligned(dev_state, 8))
        return ZERO_EALIGN;
    if (chunk_elems == 0 || (chunk_elems & 63))
        return ZERO_EALIGN;
    hipStream_t s = (hipStream_t)stream;
    if ((n + chunk_elems - 1) / chunk_elems > 4096)
        return ZERO_ERANGE;
    chunk_bounds(n, chunk_elems, ctx->bounds);   // the two ramps add at most 8 chunks
    const uint64_t chunks = ctx->bounds.size() - 1;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return hip_fail(hipGetLastError());
    if (ctx->event_device != dev) {              // events belong to the device they were made on
        for (hipEvent_t e : ctx->events)
            (void)hipEventDestroy(e);
        ctx->events.clear();
        ctx->event_device = dev;
    }
    while (ctx->events.size() < chunks + 1) {
        hipEvent_t e;
        const hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableTiming);
        if (err != hipSuccess)
            return hip_fail(err);
        ctx->events.push_back(e);
    }
    hipEvent_t* ev = ctx->events.data();         // ev[0]: the state, ev[1 + c]: gradient chunk c
    const uint64_t* bnd = ctx->bounds.data();
    auto lo_of = [&](uint64_t c) { return bnd[c]; };
    auto hi_of = [&](uint64_t c) { return bnd[c + 1]; };
    // the decision first (when the device has made it), then the gradient, chunk by chunk
    if (dev_state) {
        hipError_t err = hipMemcpyAsync(state, dev_state, sizeof *state, hipMemcpyDeviceToHost, s);
        if (err == hipSuccess)
            err = hipEventRecord(ev[0], s);
        if (err != hipSuccess)
            return hip_fail(err);
    }
    for (uint64_t c = 0; c < chunks; ++c) {
        hipError_t err = hipMemcpyAsync(host_grad16 + lo_of(c), dev_grad16 + lo_of(c), (hi_of(c) - lo_of(c)) * 2,
                                        hipMemcpyDeviceToHost, s);
        if (err == hipSuccess)
            err = hipEventRecord(ev[1 + c], s);
        if (err != hipSuccess)
            return hip_fail(err);
    }
    if (dev_state) {
        const hipError_t err = hipEventSynchronize(ev[0]);
        if (err != hipSuccess)
            return hip_fail(err);
    } else {                                     // reduce each chunk as it lands, then decide here
        norm_reset(ctx);
        for (uint64_t c = 0; c < chunks; ++c) {
            const hipError_t err = hipEventSynchronize(ev[1 + c]);
            if (err != hipSuccess)
                return hip_fail(err);
            norm_chunk(ctx, host_grad16, lo_of(c), hi_of(c));
        }
        norm_decide(ctx, hp, state);
    }
    if (state->skip)
        return ZERO_OK;                          // nothing changes, nothing goes back up
    // update chunk by chunk as the gradient lands; send each chunk of fp16 parameters up when ready
    const Coef co = coef_of(state);
    for (uint64_t c = 0; c < chunks; ++c) {
        hipError_t err = dev_state ? hipEventSynchronize(ev[1 + c]) : hipSuccess;
        if (err != hipSuccess)
            return hip_fail(err);
        adam_chunk(ctx, host_p16, p32, m32, v32, host_grad16, lo_of(c), hi_of(c), co);
        err = hipMemcpyAsync(dev_p16 + lo_of(c), host_p16 + lo_of(c), (hi_of(c) - lo_of(c)) * 2,
                             hipMemcpyHostToDevice, s);
        if (err != hipSuccess)
            return hip_fail(err);
    }
    return ZERO_OK;
}
