// flatten.hip -- pack per-layer fp16 gradient tensors into a rank's contiguous
// partition (ZeRO paper card, "Method": ZeRO-R keeps contiguous buffers
// against fragmentation and sizes its temporary buffers; the DeepSpeed
// article notes the library owns gradient accumulation, hence the
// accumulating forms).
//
// Design for gfx950.  Segments ride in the kernel-argument block (up to
// kMaxSegs per launch), so there is no device-side table to build or upload;
// each workgroup finds its segment by a uniform binary search over a prefix
// of block counts held in that block.  Within a segment the destination is
// split into a scalar head that reaches 16-byte alignment, a body of aligned
// 8-element vectors (one 16-byte fp16 store or two 16-byte fp32 stores per
// thread-vector) and a scalar tail.  When the source shares the destination's
// 16-byte phase the body loads are 16-byte vector loads; otherwise each
// thread gathers its 8 source elements with 2-byte loads (still coalesced
// across the wavefront).  The work is pure streaming: 4 bytes per element
// for the fp16 copy, so no LDS and no MFMA.  Measured on MI355X inside the
// whole step: one 16-byte vector per thread; nontemporal loads (the per-layer
// sources are read once); plain stores, so the fresh partition is still in
// the 256 MB Infinity Cache when the norm reads it next.
#include "zero_internal.hpp"

namespace zero {
namespace {

constexpr uint32_t kMaxSegs = 64;
constexpr int kBlock = 256;
constexpr int kVecsPerThread = 1;
constexpr uint64_t kVecsPerBlock = uint64_t(kBlock) * kVecsPerThread;

enum Mode { kCopy16 = 0, kAcc16 = 1, kTo32 = 2, kAcc32 = 3 };

struct FlatArgs {
    const uint16_t* src[kMaxSegs];      // element 0 of each segment (src + src_off)
    uint64_t dst_off[kMaxSegs];
    uint64_t count[kMaxSegs];
    uint32_t first_block[kMaxSegs + 1]; // prefix sum of blocks per segment
    uint32_t nsegs;
};

__device__ __forceinline__ uint64_t head_len(uint64_t dst_off, uint64_t count)
{
    const uint64_t h = (8 - (dst_off & 7)) & 7;
    return h < count ? h : count;
}

template <int MODE>
__device__ __forceinline__ void put_scalar(void* dst, uint64_t i, uint16_t s)
{
    if (MODE == kCopy16) {
        static_cast<uint16_t*>(dst)[i] = s;
    } else if (MODE == kAcc16) {
        _Float16* d = static_cast<_Float16*>(dst);
        d[i] = d[i] + __builtin_bit_cast(_Float16, s);        // correctly rounded binary16 add
    } else if (MODE == kTo32) {
        static_cast<float*>(dst)[i] = float(__builtin_bit_cast(_Float16, s));
    } else {
        float* d = static_cast<float*>(dst);
        d[i] = d[i] + float(__builtin_bit_cast(_Float16, s));
    }
}

// dst index i is a multiple of 8.
template <int MODE>
__device__ __forceinline__ void put_vector(void* dst, uint64_t i, u32x4 s)
{
    if (MODE == kCopy16) {
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(dst) + i) = s;
    } else if (MODE == kAcc16) {
        u32x4* d = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(dst) + i);
        f16x8 a = __builtin_bit_cast(f16x8, *d);
        f16x8 b = __builtin_bit_cast(f16x8, s);
        *d = __builtin_bit_cast(u32x4, a + b);
    } else {
        f16x8 h = __builtin_bit_cast(f16x8, s);
        f32x4* d = reinterpret_cast<f32x4*>(static_cast<float*>(dst) + i);
        f32x4 lo = {float(h[0]), float(h[1]), float(h[2]), float(h[3])};
        f32x4 hi = {float(h[4]), float(h[5]), float(h[6]), float(h[7])};
        if (MODE == kAcc32) {
            lo = d[0] + lo;
            hi = d[1] + hi;
        }
        d[0] = lo;
        d[1] = hi;
    }
}

template <int MODE>
__global__ __launch_bounds__(kBlock) void flatten_kernel(FlatArgs a, void* __restrict__ dst)
{
    // Segment of this workgroup: the last s with first_block[s] <= blockIdx.x.
    const uint32_t b = blockIdx.x;
    uint32_t lo = 0, hi = a.nsegs;
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (a.first_block[mid] <= b) lo = mid; else hi = mid;
    }
    const uint16_t* __restrict__ src = a.src[lo];
    const uint64_t doff = a.dst_off[lo];
    const uint64_t cnt = a.count[lo];
    const uint64_t head = head_len(doff, cnt);
    const uint64_t nv = (cnt - head) >> 3;
    const uint64_t local = b - a.first_block[lo];
    const bool vec_src = is_aligned(src + head, 16);

    // body: vectors [v0, v1) of this segment
    const uint64_t v0 = local * kVecsPerBlock;
    const uint64_t v1 = v0 + kVecsPerBlock < nv ? v0 + kVecsPerBlock : nv;
    const uint16_t* __restrict__ sbody = src + head;
    const uint64_t dbody = doff + head;
    if (vec_src) {
        u32x4 r[kVecsPerThread];
#pragma unroll
        for (int k = 0; k < kVecsPerThread; ++k) {
            const uint64_t v = v0 + threadIdx.x + uint64_t(k) * kBlock;
            if (v < v1)
                r[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sbody) + v);
        }
#pragma unroll
        for (int k = 0; k < kVecsPerThread; ++k) {
            const uint64_t v = v0 + threadIdx.x + uint64_t(k) * kBlock;
            if (v < v1)
                put_vector<MODE>(dst, dbody + 8 * v, r[k]);
        }
    } else {
        for (uint64_t v = v0 + threadIdx.x; v < v1; v += kBlock) {
            const uint16_t* s = sbody + 8 * v;
            u32x4 r;
            r.x = uint32_t(s[0]) | (uint32_t(s[1]) << 16);
            r.y = uint32_t(s[2]) | (uint32_t(s[3]) << 16);
            r.z = uint32_t(s[4]) | (uint32_t(s[5]) << 16);
            r.w = uint32_t(s[6]) | (uint32_t(s[7]) << 16);
            put_vector<MODE>(dst, dbody + 8 * v, r);
        }
    }

    // head and tail: fewer than 8 elements each, done by the segment's first block
    if (local == 0) {
        const uint64_t t0 = head + 8 * nv;
        const uint64_t t = threadIdx.x;
        if (t < head)
            put_scalar<MODE>(dst, doff + t, src[t]);
        if (t < cnt - t0)
            put_scalar<MODE>(dst, doff + t0 + t, src[t0 + t]);
    }
}

int launch(const FlatArgs& a, uint32_t blocks, int mode, void* dst, hipStream_t s)
{
    switch (mode) {
    case kCopy16: hipLaunchKernelGGL(flatten_kernel<kCopy16>, dim3(blocks), dim3(kBlock), 0, s, a, dst); break;
    case kAcc16: hipLaunchKernelGGL(flatten_kernel<kAcc16>, dim3(blocks), dim3(kBlock), 0, s, a, dst); break;
    case kTo32: hipLaunchKernelGGL(flatten_kernel<kTo32>, dim3(blocks), dim3(kBlock), 0, s, a, dst); break;
    default: hipLaunchKernelGGL(flatten_kernel<kAcc32>, dim3(blocks), dim3(kBlock), 0, s, a, dst); break;
    }
    return launch_status();
}

}  // namespace
}  // namespace zero

using namespace zero;

extern "C" int zero_flatten_bucket(const zero_segment_t* segs, uint32_t nsegs, void* dst, uint64_t dst_len,
                                   int dst_dtype, int accumulate, void* stream)
{
    if ((dst_dtype != ZERO_F16 && dst_dtype != ZERO_F32) || (nsegs && (!segs || !dst)))
        return ZERO_EINVAL;
    if (nsegs == 0)
        return ZERO_OK;
    if (!is_aligned(dst, 16))
        return ZERO_EALIGN;
    for (uint32_t i = 0; i < nsegs; ++i) {
        if (segs[i].count == 0)
            continue;
        if (!segs[i].src)
            return ZERO_EINVAL;
        if (!is_aligned(segs[i].src, 2))
            return ZERO_EALIGN;
        if (segs[i].dst_off > dst_len || segs[i].count > dst_len - segs[i].dst_off)
            return ZERO_ERANGE;
        if (segs[i].src_off > (UINT64_MAX >> 2) - segs[i].count)
            return ZERO_ERANGE;
    }
    const int mode = (dst_dtype == ZERO_F16 ? kCopy16 : kTo32) + (accumulate ? 1 : 0);
    hipStream_t s = (hipStream_t)stream;

    FlatArgs a;
    uint32_t k = 0;
    uint64_t blocks = 0;
    for (uint32_t i = 0; i <= nsegs; ++i) {
        uint64_t need = 0;
        if (i < nsegs && segs[i].count) {
            const uint64_t head = (8 - (segs[i].dst_off & 7)) & 7;
            const uint64_t nv = segs[i].count > head ? (segs[i].count - head) / 8 : 0;
            need = nv ? (nv + kVecsPerBlock - 1) / kVecsPerBlock : 1;
            if (need > 0x7fffffffull)
                return ZERO_ERANGE;
        }
        // flush the batch when it is full, would overflow the grid, or at the end
        if (k && (i == nsegs || k == kMaxSegs || blocks + need > 0x7fffffffull)) {
            a.first_block[k] = uint32_t(blocks);
            a.nsegs = k;
            int rc = launch(a, uint32_t(blocks), mode, dst, s);
            if (rc != ZERO_OK)
                return rc;
            k = 0;
            blocks = 0;
        }
        if (i == nsegs || need == 0)
            continue;
        a.src[k] = segs[i].src + segs[i].src_off;
        a.dst_off[k] = segs[i].dst_off;
        a.count[k] = segs[i].count;
        a.first_block[k] = uint32_t(blocks);
        blocks += need;
        ++k;
    }
    return ZERO_OK;
}
