// adam.hip -- the fused shard update: unscale + clip + Adam with bias
// correction and decoupled weight decay, writing the fp32 master parameter,
// momentum and variance and the fp16 parameter copy in one pass.
//
// State per parameter as the pages fix it (ZeRO paper card, "Bottleneck"):
// fp16 parameter and gradient, fp32 master parameter, momentum and variance.
// The update is Kingma & Ba 2015 (Algorithm 1, bias-corrected moments) with
// Loshchilov & Hutter 2019 decoupled weight decay (Algorithm 2, schedule
// multiplier = lr); the clip factor and the loss-scale reciprocal arrive as
// one fp32 multiplier from the decision in the step state.
//
// Memory traffic per parameter: read fp16 g (2) + fp32 p, m, v (12); write
// fp32 p, m, v (12) + fp16 p (2) = 28 bytes, about 20 flops -- far below the
// fp32 ridge point, so this is an HBM-streaming kernel: no LDS traffic, no
// MFMA.  The gradient-accumulation form reads an fp32 gradient instead
// (30 bytes per parameter) and is otherwise the same kernel.
// Shape, chosen by measurement on MI355X:
//   * one-shot grid: each workgroup owns 2048 consecutive parameters and each
//     thread two groups of 4 of them, 1024 apart (an 8-byte load of fp16 g or
//     a 16-byte load of fp32 g, and a 16-byte load of each of p, m, v, per
//     group; the matching stores), so every load and store instruction of a
//     wave covers one contiguous span and the wave front of resident
//     workgroups sweeps memory once, in order (giving each thread 8 adjacent
//     parameters instead, with two 16-byte accesses 32 bytes apart across the
//     lanes, was about 1% slower);
//   * nontemporal loads (every input is read once) and nontemporal stores
//     (nothing written here is read again by this kernel); all eight loads
//     of a thread are issued before the step state is read, so the skip
//     test does not delay the streams;
//   * at most kBlocksPerCU workgroups resident per CU, enforced by reserving
//     LDS the kernel never touches: with all 8 waves per SIMD resident the
//     8 concurrent read/write streams thrash HBM pages, and 2 waves per SIMD
//     sustain more bandwidth.
// Every operation below is one binary32 round-to-nearest-even operation
// (built without contraction, with correctly rounded division and square
// root, denormals kept).
#include "zero_internal.hpp"

namespace zero {
namespace {

constexpr int kBlock = 256;
constexpr int kBlocksPerCU = 2;

struct Coef {
    float gmul, b1, b2, omb1, omb2, bc1, bc2, eps, wd, lr;
};

__device__ __forceinline__ void update(float gh, float& p, float& m, float& v, const Coef& c)
{
#pragma clang fp contract(off)
    const float g = gh * c.gmul;
    const float mn = c.b1 * m + c.omb1 * g;
    const float vn = c.b2 * v + c.omb2 * (g * g);
    const float mh = mn / c.bc1;
    const float vh = vn / c.bc2;
    const float u = mh / (__builtin_sqrtf(vh) + c.eps) + c.wd * p;
    p = p - c.lr * u;
    m = mn;
    v = vn;
}

// Gradient group j (parameters 4j..4j+3) as loaded: four fp16 bit patterns
// (8 bytes) or four fp32 values (16 bytes).  The gradient is read once and
// never again this step: nontemporal loads.  Widening waits for the load, so
// it is a separate step, done after every load of the thread is in flight.
__device__ __forceinline__ u32x2 load_grad_raw(const uint16_t* g, uint64_t j)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(g) + j);
}

__device__ __forceinline__ f32x4 load_grad_raw(const float* g, uint64_t j)
{
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g) + j);
}

// Widened to fp32 (exact for fp16).
__device__ __forceinline__ void widen(u32x2 r, float* out)
{
    const f16x4 h = __builtin_bit_cast(f16x4, r);
#pragma unroll
    for (int k = 0; k < 4; ++k)
        out[k] = float(h[k]);
}

__device__ __forceinline__ void widen(f32x4 r, float* out)
{
    out[0] = r.x; out[1] = r.y; out[2] = r.z; out[3] = r.w;
}

// fp32 master parameter, momentum or variance group j, read once per step:
// nontemporal like the gradient.  With the contiguous per-instruction mapping
// this measured 1-2% faster than plain loads (an in-place copy with plain
// loads and nontemporal stores ran 14% slower than with nontemporal loads).
__device__ __forceinline__ f32x4 load_state4(const f32x4* q) { return __builtin_nontemporal_load(q); }

__device__ __forceinline__ Coef coef(const zero_step_state_t* st)
{
    Coef c;
    c.gmul = st->gmul;
    c.b1 = st->beta1;
    c.b2 = st->beta2;
    c.omb1 = st->omb1;
    c.omb2 = st->omb2;
    c.bc1 = st->bc1;
    c.bc2 = st->bc2;
    c.eps = st->eps;
    c.wd = st->wd;
    c.lr = st->lr;
    return c;
}

__device__ __forceinline__ u32x2 to_f16x4(const float* p)
{
    f16x4 h;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        h[k] = _Float16(p[k]);                    // round to nearest even
    return __builtin_bit_cast(u32x2, h);
}

__device__ __forceinline__ float grad_at(const uint16_t* g, uint64_t i) { return float(__builtin_bit_cast(_Float16, g[i])); }
__device__ __forceinline__ float grad_at(const float* g, uint64_t i) { return g[i]; }

// GATED (the warm-up steps of 1-bit Adam, zero_onebit_step): the update
// runs only while st->step <= gate, tested before any load, so a step of the
// compression stage pays no traffic here.
template <typename G, bool GATED>
__global__ __launch_bounds__(kBlock) void adam_step_kernel(uint16_t* __restrict__ p16, float* __restrict__ p32,
                                                           float* __restrict__ m32, float* __restrict__ v32,
                                                           const G* __restrict__ grad, uint64_t n,
                                                           const zero_step_state_t* __restrict__ st, int64_t gate)
{
    if (GATED && st->step > gate)
        return;
    // The occupancy cap: the launch reserves dynamic LDS that no thread
    // touches (the store below is unreachable for any real n); referencing it
    // keeps the reservation part of the kernel's declared resources.
    extern __shared__ char occupancy_reserve[];
    if (n == UINT64_MAX)
        occupancy_reserve[threadIdx.x] = 0;

    // groups of 4 parameters: this thread's are ja and jb = ja + kBlock
    const uint64_t ng = n >> 2;
    const uint64_t ja = uint64_t(blockIdx.x) * (2 * kBlock) + threadIdx.x;
    const uint64_t jb = ja + kBlock;
    f32x4* __restrict__ P = reinterpret_cast<f32x4*>(p32);
    f32x4* __restrict__ M = reinterpret_cast<f32x4*>(m32);
    f32x4* __restrict__ V = reinterpret_cast<f32x4*>(v32);
    u32x2* __restrict__ H = reinterpret_cast<u32x2*>(p16);
    if (jb < ng) {                                // both groups: all loads first
        // The eight loads go out before the step state is read
        // (loads_first_use in zero_internal.hpp).
        const auto ga = load_grad_raw(grad, ja), gb = load_grad_raw(grad, jb);
        const f32x4 pa = load_state4(P + ja), pb = load_state4(P + jb), ma = load_state4(M + ja),
                    mb = load_state4(M + jb), va = load_state4(V + ja), vb = load_state4(V + jb);
        __builtin_amdgcn_sched_barrier(0);
        if (st->skip) {                          // overflow: this step changes nothing
            if (n == UINT64_MAX)                 // never true: keeps the loads ahead of the test
                P[ja] = pa + pb + ma + mb + va + vb + bits_of(ga) + bits_of(gb);
            return;
        }
        const Coef c = coef(st);
        float g[8];
        widen(ga, g);
        widen(gb, g + 4);
        float p[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
        float m[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
        float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
        for (int k = 0; k < 8; ++k)
            update(g[k], p[k], m[k], v[k], c);
        __builtin_nontemporal_store(f32x4{p[0], p[1], p[2], p[3]}, P + ja);
        __builtin_nontemporal_store(f32x4{p[4], p[5], p[6], p[7]}, P + jb);
        __builtin_nontemporal_store(f32x4{m[0], m[1], m[2], m[3]}, M + ja);
        __builtin_nontemporal_store(f32x4{m[4], m[5], m[6], m[7]}, M + jb);
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, V + ja);
        __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, V + jb);
        __builtin_nontemporal_store(to_f16x4(p), H + ja);
        __builtin_nontemporal_store(to_f16x4(p + 4), H + jb);
    } else {
        if (st->skip)
            return;
        const Coef c = coef(st);
        if (ja < ng) {                            // the last workgroup: group ja only
            float g[4];
            widen(load_grad_raw(grad, ja), g);
            const f32x4 pa = P[ja], ma = M[ja], va = V[ja];
            float p[4] = {pa.x, pa.y, pa.z, pa.w};
            float m[4] = {ma.x, ma.y, ma.z, ma.w};
            float v[4] = {va.x, va.y, va.z, va.w};
#pragma unroll
            for (int k = 0; k < 4; ++k)
                update(g[k], p[k], m[k], v[k], c);
            P[ja] = f32x4{p[0], p[1], p[2], p[3]};
            M[ja] = f32x4{m[0], m[1], m[2], m[3]};
            V[ja] = f32x4{v[0], v[1], v[2], v[3]};
            H[ja] = to_f16x4(p);
        }
    }

    // the last n % 4 parameters, one per thread of the first workgroup
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
        const Coef c = coef(st);
        const uint64_t i = (ng << 2) + threadIdx.x;
        float p = p32[i], m = m32[i], v = v32[i];
        update(grad_at(grad, i), p, m, v, c);
        p32[i] = p;
        m32[i] = m;
        v32[i] = v;
        p16[i] = __builtin_bit_cast(uint16_t, _Float16(p));
    }
}

}  // namespace

template <typename G, bool GATED>
int adam_step(uint16_t* p16, float* p32, float* m32, float* v32, const G* grad, uint64_t n,
              const zero_step_state_t* dev_state, void* stream, int64_t gate)
{
    if (!dev_state || (n && (!p16 || !p32 || !m32 || !v32 || !grad)))
        return ZERO_EINVAL;
    if (!is_aligned(dev_state, 8))
        return ZERO_EALIGN;
    if (n == 0)
        return ZERO_OK;
    if (!is_aligned(p16, 16) || !is_aligned(p32, 16) || !is_aligned(m32, 16) || !is_aligned(v32, 16) ||
        !is_aligned(grad, 16))
        return ZERO_EALIGN;
    const uint64_t ng = n >> 2;
    uint64_t grid = (ng + 2 * kBlock - 1) / (2 * kBlock);
    if (grid < 1) grid = 1;
    if (grid > 0x7fffffffull)
        return ZERO_ERANGE;
    hipLaunchKernelGGL((adam_step_kernel<G, GATED>), dim3(uint32_t(grid)), dim3(kBlock),
                       lds_reservation(kBlocksPerCU), (hipStream_t)stream, p16, p32, m32, v32, grad, n, dev_state,
                       gate);
    return launch_status();
}

int adam_step_gated(uint16_t* p16, float* p32, float* m32, float* v32, const uint16_t* grad16, uint64_t n,
                    const zero_step_state_t* dev_state, void* stream, int64_t gate)
{
    return adam_step<uint16_t, true>(p16, p32, m32, v32, grad16, n, dev_state, stream, gate);
}

}  // namespace zero

using namespace zero;

extern "C" int zero_shard_adam_step(uint16_t* p16, float* p32, float* m32, float* v32, const uint16_t* grad16,
                                    uint64_t n, const zero_step_state_t* dev_state, void* stream)
{
    return adam_step<uint16_t, false>(p16, p32, m32, v32, grad16, n, dev_state, stream, 0);
}

extern "C" int zero_shard_adam_step_f32(uint16_t* p16, float* p32, float* m32, float* v32, const float* grad32,
                                        uint64_t n, const zero_step_state_t* dev_state, void* stream)
{
    return adam_step<float, false>(p16, p32, m32, v32, grad32, n, dev_state, stream, 0);
}
