// norm.hip -- exact squared L2 norm + overflow test of a rank's flat gradient
// partition, and the step decision that follows from them (dynamic loss
// scaling with skip-step, Micikevicius et al. 2018; global-norm clipping,
// Pascanu et al. 2013; Adam's bias corrections, Kingma & Ba 2015).  The pages
// fix the gradient as fp16 and the optimizer state as fp32 (ZeRO paper card,
// "Bottleneck"); the fp32 form is the gradient-accumulation partition (the
// DeepSpeed article leaves gradient accumulation to the library).  The rest
// of this step is the published methods.
//
// The sum is exact (exact_norm.hpp): binary64 accumulators that cannot round
// under a per-thread element bound, integer limbs across the grid, one
// round-to-nearest-even at the end.  The result is the exactly rounded sum,
// independent of grid shape and schedule, so the clip factor derived from it
// is bitwise reproducible.  An fp32 partition holding a value the fast sum
// cannot take exactly (off the 2^-24 grid, or 2^24 or more in magnitude)
// leaves the decision pending, and the wide pass launched right after
// (wide_sum.hpp) sums it exactly and decides; otherwise that pass returns at
// once.
//
// Two kernels share the tail:
//   norm_overflow_kernel  reads the partition itself: 1024-thread workgroups,
//                         at most one per CU (256), each thread streaming
//                         16-byte vectors with four nontemporal loads in
//                         flight; about 8 VALU operations per fp16 element,
//                         about 12 binary64 operations per fp32 element;
//   decide_kernel         folds the per-workgroup partials a fused flatten
//                         (flatten.hip) already computed while copying
//                         (one wave up to 512 partials; decide_grid: a
//                         single workgroup, which then decides without an
//                         arrival counter or fence, up to 2^15 partials;
//                         more take two per thread over up to 256
//                         workgroups).
// With several workgroups, each stores its carried partial and bumps an
// agent-scope arrival counter once with release order; the last one to
// arrive acquires, and its first wave folds all partials, takes the decision
// in binary64 on one thread, writes it into the step state and re-arms the
// counter.  No MFMA: 2 or 4 bytes per element.
#include <math.h>

#include <mutex>

#include "decide.hpp"
#include "exact_norm.hpp"
#include "wide_sum.hpp"

namespace zero {
namespace {

using exact::Limbs;

// The reduction's end, on one thread: overflow -> the skip decision; a sum
// the fast form cannot vouch for -> left to the wide pass; else the decision.
__device__ __forceinline__ void conclude(zero_step_state_t* st, const DecideArgs& d, Limbs t, uint32_t status)
{
    uint64_t hi, lo;
    const bool fits = exact::limbs_to_u128(t, hi, lo);
    if (status & exact::kOvf)
        decide_state(st, d, hi, lo, true);
    else if (!fits || (status & exact::kWide))
        defer_to_wide(st);
    else
        decide_state(st, d, hi, lo, false);
}

// Called by every thread of every workgroup with that workgroup's limbs and
// status (valid in thread 0): publish, and let the last workgroup decide.
__device__ __forceinline__ void publish_and_decide(Limbs s, uint32_t flag, zero_step_state_t* st,
                                                   NormPartial* ws, const DecideArgs& d)
{
    if (gridDim.x == 1) {          // one workgroup holds the whole sum: no arrival counter, no fence
        if (threadIdx.x == 0)
            conclude(st, d, s, flag);
        return;
    }
    __shared__ uint32_t s_last;
    if (threadIdx.x == 0) {
        ws[blockIdx.x] = exact::make_partial(s, flag);
        // Release this workgroup's partial.  Only the last workgroup acquires
        // the others' (its increment ends the release sequence of every
        // earlier one), so the rest skip the acquire's cache invalidation.
        const uint32_t prev = __hip_atomic_fetch_add(&st->done_blocks, 1u, __ATOMIC_RELEASE,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        const bool last = prev == gridDim.x - 1;
        if (last)
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_last = last ? 1u : 0u;
    }
    __syncthreads();
    if (!s_last || threadIdx.x >= 64)
        return;

    // Last workgroup: its first wave folds every partial (integer limbs:
    // order is irrelevant), four per lane per batch with the loads in
    // flight together (one batch for up to 256 workgroups, the usual grid),
    // then a shuffle fold with no barrier.
    Limbs t{0, 0, 0, 0};
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
        conclude(st, d, t, tflag);
        st->done_blocks = 0;                                 // re-arm for the next call
    }
}

// The wide pass over an fp32 partition (wide_sum.hpp), and how it ends: the
// exact sum of squares rounded once, then the decision.
struct F32Values {
    const float* g;
    __device__ float at(uint64_t i) const { return g[i]; }
};

struct NormFinish {
    zero_step_state_t* st;
    DecideArgs d;
    __device__ bool pending() const { return st->wide_pending != 0; }
    __device__ uint32_t* counter() const { return &st->done_blocks; }
    __device__ void finish(const uint64_t* digits) const
    {
        uint64_t hi, lo;
        if (!wide::to_units48(digits, hi, lo))
            hi = lo = ~uint64_t(0);
        st->sumsq_units[0] = lo;
        st->sumsq_units[1] = hi;
        decide_sum(st, d, wide::to_f64(digits), false);
    }
};

int launch_wide(const float* grad, uint64_t n, zero_step_state_t* st, const DecideArgs& d, void* workspace,
                hipStream_t s)
{
    hipLaunchKernelGGL((wide::wide_sum_kernel<F32Values, NormFinish>), dim3(uint32_t(wide::grid(n))),
                       dim3(wide::kBlock), 0, s, F32Values{grad}, n, NormFinish{st, d},
                       static_cast<wide::WidePartial*>(workspace));
    return launch_status();
}

// Element type of the partition: 16-byte vectors, the exact accumulator, and
// a scalar load of one element for the tail.
template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {
    static constexpr int kPerVec = 8;
    using Acc = exact::Acc16;
    __device__ static void one(Acc& acc, const uint16_t* g, uint64_t i) { acc.bits(g[i]); }
};
template <>
struct Elem<float> {
    static constexpr int kPerVec = 4;
    using Acc = exact::Acc32;
    __device__ static void one(Acc& acc, const float* g, uint64_t i) { acc.add(g[i]); }
};

__device__ __forceinline__ void acc_vec(exact::Acc16& acc, u32x4 v) { acc.vec(v); }
__device__ __forceinline__ void acc_vec(exact::Acc32& acc, u32x4 v) { acc.vec(__builtin_bit_cast(f32x4, v)); }

template <typename T>
__global__ __launch_bounds__(kNormBlock) void norm_overflow_kernel(const T* __restrict__ g, uint64_t n,
                                                                   zero_step_state_t* __restrict__ st,
                                                                   NormPartial* __restrict__ ws, DecideArgs d)
{
    using E = Elem<T>;
    typename E::Acc acc;
    const uint64_t nvec = n / E::kPerVec;
    const u32x4* __restrict__ gv = reinterpret_cast<const u32x4*>(g);
    const uint64_t stride = uint64_t(gridDim.x) * kNormBlock;
    // a round: each wave reads one contiguous 4 KiB block (its four load
    // instructions 1 KiB apart), the grid 4 * stride vectors
    const uint64_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t j = (uint64_t(blockIdx.x) * (kNormBlock / 64) + wave) * 256 + lane;
    for (; j + 192 < nvec; j += 4 * stride) {             // four 16-byte loads in flight
        const u32x4 a = __builtin_nontemporal_load(gv + j);
        const u32x4 b = __builtin_nontemporal_load(gv + j + 64);
        const u32x4 c = __builtin_nontemporal_load(gv + j + 128);
        const u32x4 e = __builtin_nontemporal_load(gv + j + 192);
        acc_vec(acc, a);
        acc_vec(acc, b);
        acc_vec(acc, c);
        acc_vec(acc, e);
    }
    for (int k = 0; k < 4; ++k, j += 64)                  // the grid's last, partial round
        if (j < nvec)
            acc_vec(acc, __builtin_nontemporal_load(gv + j));
    if (blockIdx.x == 0 && threadIdx.x < n - nvec * E::kPerVec)   // the last n % kPerVec elements
        E::one(acc, g, nvec * E::kPerVec + threadIdx.x);

    uint32_t flag = acc.status();
    Limbs s = acc.limbs();
    exact::block_fold<kNormBlock>(s, flag);
    publish_and_decide(s, flag, st, ws, d);
}

// Folds `count` carried partials (from a fused flatten) and decides.  BLOCK
// = 64 for a few partials: one wave (eight per lane, loads in flight
// together) folds them with lane shuffles, no LDS and no barrier.
constexpr uint64_t kOneWavePartials = 512;

template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void decide_kernel(const NormPartial* __restrict__ in, uint64_t count,
                                                       zero_step_state_t* __restrict__ st,
                                                       NormPartial* __restrict__ ws, DecideArgs d)
{
    Limbs s{0, 0, 0, 0};
    uint32_t flag = 0;
    const uint64_t stride = uint64_t(gridDim.x) * BLOCK;
    uint64_t i = uint64_t(blockIdx.x) * BLOCK + threadIdx.x;
    // eight partials' loads in flight per round, the last round guarded (so a
    // thread's few left-over partials cost one load latency, not one each)
    for (; i < count; i += 8 * stride) {
        NormPartial q[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            q[k] = i + k * stride < count ? in[i + k * stride] : NormPartial{0, 0};
#pragma unroll
        for (int k = 0; k < 8; ++k)
            exact::fold_partial(s, flag, q[k]);
    }
    exact::block_fold<BLOCK>(s, flag);
    publish_and_decide(s, flag, st, ws, d);
}

// `workspace_bytes` must cover what this call uses: the fast reduction's
// partials and, for fp32, the wide pass's (the public entry points ask for
// zero_norm_workspace_bytes(n), which covers both forms).
template <typename T>
int norm_overflow(const T* grad, uint64_t n, const zero_hparams_t* hp, zero_step_state_t* dev_state,
                  void* workspace, size_t workspace_bytes, void* stream)
{
    if (!hp || !dev_state || !workspace || (n && !grad))
        return ZERO_EINVAL;
    if (!hparams_ok(hp))
        return ZERO_EINVAL;
    if ((n && !is_aligned(grad, 16)) || !is_aligned(dev_state, 8) || !is_aligned(workspace, 16))
        return ZERO_EALIGN;
    if (n > kNormMaxElems)
        return ZERO_ERANGE;
    const uint64_t grid = norm_grid(n);
    uint64_t need = grid * sizeof(NormPartial);
    if (sizeof(T) == 4 && need < wide::grid(n) * sizeof(wide::WidePartial))
        need = wide::grid(n) * sizeof(wide::WidePartial);
    if (workspace_bytes < need)
        return ZERO_ERANGE;
    const DecideArgs d = decide_args(hp);
    hipLaunchKernelGGL(norm_overflow_kernel<T>, dim3(uint32_t(grid)), dim3(kNormBlock), 0, (hipStream_t)stream,
                       grad, n, dev_state, static_cast<NormPartial*>(workspace), d);
    int rc = launch_status();
    if (rc == ZERO_OK && sizeof(T) == 4)       // fp32: the wide pass, a no-op unless the fast sum asked for it
        rc = launch_wide(reinterpret_cast<const float*>(grad), n, dev_state, d, workspace, (hipStream_t)stream);
    return rc;
}

}  // namespace
}  // namespace zero

using namespace zero;

extern "C" int zero_shard_norm_overflow(const uint16_t* grad16, uint64_t n, const zero_hparams_t* hp,
                                        zero_step_state_t* dev_state, void* workspace,
                                        size_t workspace_bytes, void* stream)
{
    if (n <= kNormMaxElems && workspace_bytes < zero_norm_workspace_bytes(n))
        return (!hp || !dev_state || !workspace || (n && !grad16)) ? ZERO_EINVAL : ZERO_ERANGE;
    return norm_overflow(grad16, n, hp, dev_state, workspace, workspace_bytes, stream);
}

extern "C" int zero_shard_norm_overflow_f32(const float* grad32, uint64_t n, const zero_hparams_t* hp,
                                            zero_step_state_t* dev_state, void* workspace,
                                            size_t workspace_bytes, void* stream)
{
    return norm_overflow(grad32, n, hp, dev_state, workspace, workspace_bytes, stream);
}

// ---- the fp16 reduction without a workspace argument ------------------------------

namespace zero {
namespace {

// Scratch of zero_shard_norm_overflow_noalloc: the per-workgroup partials of
// the standalone fp16 reduction, one per workgroup of its grid.  The array is
// a host-side stand-in in host code; kernels get its device address from
// scratch_address(), never its name.
constexpr uint64_t kScratchPartials = kNormMaxBlocks;
static __device__ __align__(256) NormPartial scratch[kScratchPartials];

// The largest n whose grid fits the scratch array (norm_grid(n) <= 256: at
// most 4096 elements per thread of 256 workgroups of 1024).
constexpr uint64_t kNoAllocMaxElems = kScratchPartials * kNormBlock * kNormMaxPerThread;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];

// The device address of `scratch` on the current device, looked up once per
// device (each GPU holds its own copy of the array).
int scratch_address(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices)
        return ZERO_ERANGE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return hip_fail(e);
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return ZERO_OK;
}

}  // namespace
}  // namespace zero

extern "C" int zero_shard_norm_overflow_noalloc(const uint16_t* grad16, uint64_t n, const zero_hparams_t* hp,
                                                zero_step_state_t* dev_state, void* stream)
{
    if (!hp || !dev_state || (n && !grad16))
        return ZERO_EINVAL;
    if (!hparams_ok(hp))
        return ZERO_EINVAL;
    if ((n && !is_aligned(grad16, 16)) || !is_aligned(dev_state, 8))
        return ZERO_EALIGN;
    if (n > kNoAllocMaxElems)
        return ZERO_ERANGE;
    void* ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc != ZERO_OK)
        return rc;
    // Every workgroup writes its own partial before the last one reads them,
    // so nothing in the scratch array has to start at zero.
    return norm_overflow(grad16, n, hp, dev_state, ws, kScratchPartials * sizeof(NormPartial), stream);
}

namespace zero {
namespace {

int decide(const void* partials, uint64_t count, const float* grad32, uint64_t n, const zero_hparams_t* hp,
           zero_step_state_t* dev_state, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!hp || !dev_state || !workspace || (count && !partials))
        return ZERO_EINVAL;
    if (!hparams_ok(hp))
        return ZERO_EINVAL;
    if ((count && !is_aligned(partials, 16)) || !is_aligned(dev_state, 8) || !is_aligned(workspace, 16))
        return ZERO_EALIGN;
    if (count > kMaxPartials || (grad32 && n > kNormMaxElems))
        return ZERO_ERANGE;
    if (workspace_bytes < zero_decide_workspace_bytes(count))     // covers both passes
        return ZERO_ERANGE;
    const uint64_t grid = decide_grid(count);
    const DecideArgs d = decide_args(hp);
    if (count <= kOneWavePartials)              // one wave, one round of loads, a shuffle fold
        hipLaunchKernelGGL(decide_kernel<64>, dim3(1), dim3(64), 0, (hipStream_t)stream,
                           static_cast<const NormPartial*>(partials), count, dev_state,
                           static_cast<NormPartial*>(workspace), d);
    else
        hipLaunchKernelGGL(decide_kernel<kNormBlock>, dim3(uint32_t(grid)), dim3(kNormBlock), 0, (hipStream_t)stream,
                           static_cast<const NormPartial*>(partials), count, dev_state,
                           static_cast<NormPartial*>(workspace), d);
    int rc = launch_status();
    if (rc == ZERO_OK && grad32)
        rc = launch_wide(grad32, n, dev_state, d, workspace, (hipStream_t)stream);
    return rc;
}

}  // namespace
}  // namespace zero

extern "C" int zero_shard_decide(const void* partials, uint64_t count, const zero_hparams_t* hp,
                                 zero_step_state_t* dev_state, void* workspace, size_t workspace_bytes,
                                 void* stream)
{
    return decide(partials, count, nullptr, 0, hp, dev_state, workspace, workspace_bytes, stream);
}

extern "C" int zero_shard_decide_f32(const void* partials, uint64_t count, const float* grad32, uint64_t n,
                                     const zero_hparams_t* hp, zero_step_state_t* dev_state, void* workspace,
                                     size_t workspace_bytes, void* stream)
{
    if (n && !grad32)
        return ZERO_EINVAL;
    if (n && !is_aligned(grad32, 4))
        return ZERO_EALIGN;
    // n == 0: an empty partition needs no wide pass (its fast sum is exact)
    return decide(partials, count, n ? grad32 : nullptr, n, hp, dev_state, workspace, workspace_bytes, stream);
}
