// host.hip -- host-side entry points of the C ABI (status text, model-state
// arithmetic, bucket planning), the step-state initialiser and the streaming
// copy used as the bandwidth reference.
#include <math.h>
#include <string.h>

#include <atomic>

#include "wide_sum.hpp"
#include "zero_internal.hpp"

namespace zero {

static thread_local hipError_t g_last_hip_error = hipSuccess;

int hip_fail(hipError_t e)
{
    g_last_hip_error = e;
    return ZERO_EHIP;
}

int launch_status()
{
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? ZERO_OK : hip_fail(e);
}

uint64_t norm_grid(uint64_t n)
{
    // At least two 8-element vectors per thread, at most one workgroup per
    // CU, unless a thread would then sum more than kNormMaxPerThread elements.
    // A function of n alone, so workspace sizes are stable.
    const uint64_t per_block = uint64_t(kNormBlock) * 8 * 2;
    uint64_t g = (n + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > kNormMaxBlocks) g = kNormMaxBlocks;
    const uint64_t threads = g * kNormBlock;
    if ((n + threads - 1) / threads > kNormMaxPerThread)
        g = (n + uint64_t(kNormBlock) * kNormMaxPerThread - 1) / (uint64_t(kNormBlock) * kNormMaxPerThread);
    return g;
}

// ---- step-state initialiser --------------------------------------------------

__global__ void state_init_kernel(zero_step_state_t* st, double scale)
{
    zero_step_state_t s;
    memset(&s, 0, sizeof s);
    s.loss_scale = scale;
    s.beta1_pow = 1.0;
    s.beta2_pow = 1.0;
    *st = s;
}

uint64_t decide_grid(uint64_t count)
{
    // Up to 2^15 partials (1 MiB, L2-resident after the flatten) one workgroup
    // folds faster than several that must meet at an agent-scope arrival
    // counter; beyond that, two partials per thread (a workgroup's loads are
    // then all in flight at once) and at most one workgroup per CU.
    if (count <= (uint64_t(1) << 15))
        return 1;
    const uint64_t per_block = uint64_t(kNormBlock) * 2;
    uint64_t g = (count + per_block - 1) / per_block;
    if (g < 2) g = 2;
    if (g > kNormMaxBlocks) g = kNormMaxBlocks;
    return g;
}

// ---- occupancy cap ----------------------------------------------------------------

uint32_t lds_reservation(int blocks_per_cu)
{
    // Per-device LDS bytes per CU, looked up once (160 KiB on gfx950).
    static std::atomic<int> lds_per_cu[64];
    static std::atomic<bool> init[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64 || blocks_per_cu < 1)
        return 0;
    if (!init[dev].load(std::memory_order_acquire)) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess)
            v = 0;
        lds_per_cu[dev].store(v, std::memory_order_relaxed);
        init[dev].store(true, std::memory_order_release);
    }
    uint32_t r = uint32_t(lds_per_cu[dev].load(std::memory_order_relaxed)) / uint32_t(blocks_per_cu);
    if (r > 65536) r = 65536;
    return r & ~255u;
}

// ---- streaming copy (bandwidth reference) --------------------------------------

// One 16-byte vector per thread, one-shot grid, nontemporal both ways: the
// fastest plain copy shape measured on MI355X.
__global__ __launch_bounds__(256) void stream_copy_kernel(u32x4* __restrict__ dst,
                                                          const u32x4* __restrict__ src, uint64_t nvec)
{
    const uint64_t i = uint64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i < nvec)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace zero

using namespace zero;

extern "C" const char* zero_status_string(int code)
{
    switch (code) {
    case ZERO_OK: return "ok";
    case ZERO_EINVAL: return "invalid argument (null pointer, bad dtype/stage or hyperparameter)";
    case ZERO_EALIGN: return "buffer not aligned as required";
    case ZERO_ERANGE: return "size or segment out of range";
    case ZERO_EHIP: return hipGetErrorString(g_last_hip_error);
    case ZERO_ENOTSUP: return "the host CPU lacks AVX-512 (F, BW, VL, DQ), F16C or FMA";
    case ZERO_ENOMEM: return "out of host memory";
    default: return "unknown status code";
    }
}

extern "C" int zero_state_bytes(uint64_t psi, uint32_t nd, uint32_t k, int stage, uint64_t* out_bytes)
{
    if (!out_bytes || nd == 0 || stage < 0 || stage > 3)
        return ZERO_EINVAL;
    typedef unsigned __int128 u128;
    const u128 owned = (u128(psi) + nd - 1) / nd;       // parameters this rank owns
    const u128 full = psi;
    u128 fp16_params = 2 * full, fp16_grads = 2 * full, opt = u128(k) * full;
    if (stage >= 1) opt = u128(k) * owned;              // P_os
    if (stage >= 2) fp16_grads = 2 * owned;             // P_g
    if (stage >= 3) fp16_params = 2 * owned;            // P_p
    const u128 total = fp16_params + fp16_grads + opt;
    if (total > u128(UINT64_MAX))
        return ZERO_ERANGE;
    *out_bytes = uint64_t(total);
    return ZERO_OK;
}

extern "C" int zero_bucket_segments(const zero_segment_t* segs, uint32_t nsegs, uint64_t begin,
                                    uint64_t end, zero_segment_t* out, uint32_t cap, uint32_t* out_n)
{
    if ((!segs && nsegs) || !out_n || begin > end || (!out && cap))
        return ZERO_EINVAL;
    uint32_t k = 0;
    for (uint32_t i = 0; i < nsegs; ++i) {
        const uint64_t d0 = segs[i].dst_off, d1 = segs[i].dst_off + segs[i].count;
        const uint64_t lo = d0 > begin ? d0 : begin, hi = d1 < end ? d1 : end;
        if (lo >= hi)
            continue;
        if (k < cap) {
            out[k].src = segs[i].src;
            out[k].src_off = segs[i].src_off + (lo - d0);
            out[k].dst_off = lo;
            out[k].count = hi - lo;
        }
        ++k;
    }
    *out_n = k;
    return k > cap ? ZERO_ERANGE : ZERO_OK;
}

// The fast reductions' partials and, for the fp32 forms, the wide pass's
// partials (the two passes run one after the other and share the space).
extern "C" size_t zero_norm_workspace_bytes(uint64_t n)
{
    const uint64_t fast = norm_grid(n) * sizeof(NormPartial);
    const uint64_t wide = wide::grid(n) * sizeof(wide::WidePartial);
    return size_t(fast > wide ? fast : wide);
}

extern "C" size_t zero_decide_workspace_bytes(uint64_t count)
{
    const uint64_t fast = decide_grid(count) * sizeof(NormPartial);
    const uint64_t wide = wide::kMaxBlocks * sizeof(wide::WidePartial);
    return size_t(fast > wide ? fast : wide);
}

extern "C" int zero_step_state_init(zero_step_state_t* dev_state, double initial_scale, void* stream)
{
    if (!dev_state || !(initial_scale > 0.0) || !isfinite(initial_scale))
        return ZERO_EINVAL;
    if (!is_aligned(dev_state, 8))
        return ZERO_EALIGN;
    hipLaunchKernelGGL(state_init_kernel, dim3(1), dim3(1), 0, (hipStream_t)stream, dev_state,
                       initial_scale);
    return launch_status();
}

extern "C" int zero_stream_copy(void* dst, const void* src, uint64_t bytes, void* stream)
{
    if (!dst || !src)
        return ZERO_EINVAL;
    if (!is_aligned(dst, 16) || !is_aligned(src, 16) || (bytes & 15))
        return ZERO_EALIGN;
    const uint64_t nvec = bytes / 16;
    if (nvec == 0)
        return ZERO_OK;
    const uint64_t grid = (nvec + 255) / 256;
    if (grid > 0x7fffffffull)
        return ZERO_ERANGE;
    hipLaunchKernelGGL(stream_copy_kernel, dim3(uint32_t(grid)), dim3(256), 0, (hipStream_t)stream,
                       (u32x4*)dst, (const u32x4*)src, nvec);
    return launch_status();
}
