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
// fp32 ridge point, so this is an HBM-streaming kernel: no LDS, no MFMA.
// Each thread-iteration takes 8 consecutive parameters: one 16-byte load of
// g, two 16-byte loads each of p, m, v, and the matching 16-byte stores,
// nontemporal because nothing is reused.  Every operation below is one
// binary32 round-to-nearest-even operation (built without contraction, with
// correctly rounded division and square root, denormals kept).
#include "zero_internal.hpp"

namespace zero {
namespace {

constexpr int kBlock = 256;
constexpr uint64_t kMaxBlocks = 8192;

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

__global__ __launch_bounds__(kBlock) void adam_step_kernel(uint16_t* __restrict__ p16, float* __restrict__ p32,
                                                           float* __restrict__ m32, float* __restrict__ v32,
                                                           const uint16_t* __restrict__ g16, uint64_t n,
                                                           const zero_step_state_t* __restrict__ st)
{
    if (st->skip)
        return;                                  // overflow: this step changes nothing
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

    const uint64_t nvec = n >> 3;
    const uint64_t stride = uint64_t(gridDim.x) * kBlock;
    const u32x4* __restrict__ gv = reinterpret_cast<const u32x4*>(g16);
    u32x4* __restrict__ hv = reinterpret_cast<u32x4*>(p16);
    f32x4* __restrict__ pv = reinterpret_cast<f32x4*>(p32);
    f32x4* __restrict__ mv = reinterpret_cast<f32x4*>(m32);
    f32x4* __restrict__ vv = reinterpret_cast<f32x4*>(v32);

    for (uint64_t j = uint64_t(blockIdx.x) * kBlock + threadIdx.x; j < nvec; j += stride) {
        const f16x8 g = __builtin_bit_cast(f16x8, __builtin_nontemporal_load(gv + j));
        f32x4 pa = __builtin_nontemporal_load(pv + 2 * j), pb = __builtin_nontemporal_load(pv + 2 * j + 1);
        f32x4 ma = __builtin_nontemporal_load(mv + 2 * j), mb = __builtin_nontemporal_load(mv + 2 * j + 1);
        f32x4 va = __builtin_nontemporal_load(vv + 2 * j), vb = __builtin_nontemporal_load(vv + 2 * j + 1);
        float p[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
        float m[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
        float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
        f16x8 h;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            update(float(g[k]), p[k], m[k], v[k], c);
            h[k] = _Float16(p[k]);                // round to nearest even
        }
        __builtin_nontemporal_store(f32x4{p[0], p[1], p[2], p[3]}, pv + 2 * j);
        __builtin_nontemporal_store(f32x4{p[4], p[5], p[6], p[7]}, pv + 2 * j + 1);
        __builtin_nontemporal_store(f32x4{m[0], m[1], m[2], m[3]}, mv + 2 * j);
        __builtin_nontemporal_store(f32x4{m[4], m[5], m[6], m[7]}, mv + 2 * j + 1);
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, vv + 2 * j);
        __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, vv + 2 * j + 1);
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, h), hv + j);
    }

    // the last n % 8 parameters, one per thread of the first workgroup
    if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
        const uint64_t i = (nvec << 3) + threadIdx.x;
        float p = p32[i], m = m32[i], v = v32[i];
        update(float(__builtin_bit_cast(_Float16, g16[i])), p, m, v, c);
        p32[i] = p;
        m32[i] = m;
        v32[i] = v;
        p16[i] = __builtin_bit_cast(uint16_t, _Float16(p));
    }
}

}  // namespace
}  // namespace zero

using namespace zero;

extern "C" int zero_shard_adam_step(uint16_t* p16, float* p32, float* m32, float* v32, const uint16_t* grad16,
                                    uint64_t n, const zero_step_state_t* dev_state, void* stream)
{
    if (!dev_state || (n && (!p16 || !p32 || !m32 || !v32 || !grad16)))
        return ZERO_EINVAL;
    if (!is_aligned(dev_state, 8))
        return ZERO_EALIGN;
    if (n == 0)
        return ZERO_OK;
    if (!is_aligned(p16, 16) || !is_aligned(p32, 16) || !is_aligned(m32, 16) || !is_aligned(v32, 16) ||
        !is_aligned(grad16, 16))
        return ZERO_EALIGN;
    const uint64_t nvec = n >> 3;
    uint64_t grid = (nvec + kBlock - 1) / kBlock;
    if (grid < 1) grid = 1;
    if (grid > kMaxBlocks) grid = kMaxBlocks;
    hipLaunchKernelGGL(adam_step_kernel, dim3(uint32_t(grid)), dim3(kBlock), 0, (hipStream_t)stream, p16, p32,
                       m32, v32, grad16, n, dev_state);
    return launch_status();
}
