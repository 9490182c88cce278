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
// 8-element vectors (one 16-byte fp16 store per thread-vector; an fp32
// destination takes the body in 4-element units instead, one 16-byte store
// each, so every store instruction of a wave stays contiguous) and a scalar
// tail.  When the source shares the destination's
// 16-byte phase the body loads are 16-byte vector loads; otherwise each
// thread gathers its 8 source elements with 2-byte loads (still coalesced
// across the wavefront).  The work is pure streaming: 4 bytes per element
// for the fp16 copy, so no LDS and no MFMA.  Measured on MI355X inside the
// whole step: one 16-byte vector per thread; nontemporal loads (the per-layer
// sources are read once); plain stores, so the fresh partition is still in
// the 256 MB Infinity Cache when the norm pass reads it next.
//
// The fused form (NORM) also accumulates the exact sum of squares and the
// inf/NaN test of every value it stores (exact_norm.hpp) and writes one
// partial per workgroup, so the norm needs no second pass over the
// partition: zero_shard_decide folds the partials and takes the decision.
// It takes three vectors per thread (the fold is amortised over 6144
// elements, and a 25M-element bucket is 4069 workgroups, two full
// generations of 2048 resident ones, where four vectors left a half-empty
// second generation) and nontemporal stores (nothing reads the partition before
// the Adam pass, and draining dirty cache lines during it costs more).
#include <hip/hip_ext.h>

#include <algorithm>
#include <type_traits>
#include <utility>
#include <vector>

#include "exact_norm.hpp"

namespace zero {
namespace {

constexpr uint32_t kMaxSegs = 64;
constexpr int kBlock = 256;

// 16-byte vectors per thread: 1 for the plain flatten, 3 for the fused one.
template <bool NORM>
struct Geometry {
    static constexpr int kVecsPerThread = NORM ? 3 : 1;
    static constexpr uint64_t kVecsPerBlock = uint64_t(kBlock) * kVecsPerThread;
};

enum Mode { kCopy16 = 0, kAcc16 = 1, kTo32 = 2, kAcc32 = 3 };

struct FlatArgs {
    const uint16_t* src[kMaxSegs];      // element 0 of each segment (src + src_off)
    uint64_t dst_off[kMaxSegs];
    uint64_t count[kMaxSegs];
    uint32_t first_block[kMaxSegs + 1]; // prefix sum of blocks per segment
    uint32_t nsegs;
    NormPartial* partials;              // fused form: one per workgroup of this launch
};

__host__ __device__ inline uint64_t head_len(uint64_t dst_off, uint64_t count)
{
    const uint64_t h = (8 - (dst_off & 7)) & 7;
    return h < count ? h : count;
}

// The exact accumulator for what a mode stores: binary16 or binary32 values.
template <int MODE>
using AccOf = typename std::conditional<(MODE >= kTo32), exact::Acc32, exact::Acc16>::type;

// Stores one element; in the fused form also accumulates the value stored.
template <int MODE, bool NORM>
__device__ __forceinline__ void put_scalar(void* dst, uint64_t i, uint16_t s, AccOf<MODE>& acc)
{
    const _Float16 h = __builtin_bit_cast(_Float16, s);
    if constexpr (MODE == kCopy16) {
        static_cast<uint16_t*>(dst)[i] = s;
        if (NORM)
            acc.bits(s);
    } else if constexpr (MODE == kAcc16) {
        _Float16* d = static_cast<_Float16*>(dst);
        const _Float16 r = d[i] + h;                     // correctly rounded binary16 add
        d[i] = r;
        if (NORM)
            acc.bits(__builtin_bit_cast(uint16_t, r));
    } else {
        float* d = static_cast<float*>(dst);
        const float r = MODE == kAcc32 ? d[i] + float(h) : float(h);
        d[i] = r;
        if (NORM)
            acc.add(r);
    }
}

template <bool NTS, typename V>
__device__ __forceinline__ void store(V v, V* d)
{
    if (NTS)
        __builtin_nontemporal_store(v, d);
    else
        *d = v;
}

// What an accumulating mode reads back from the destination for the 8
// elements at index i (a multiple of 8): one fp16 vector or two fp32 vectors.
struct Old {
    u32x4 a, b;
};

template <int MODE>
__device__ __forceinline__ Old load_old(const void* dst, uint64_t i)
{
    Old o{};
    if constexpr (MODE == kAcc16) {
        o.a = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(dst) + i);
    } else if constexpr (MODE == kAcc32) {
        const u32x4* d = reinterpret_cast<const u32x4*>(static_cast<const float*>(dst) + i);
        o.a = d[0];
        o.b = d[1];
    }
    return o;
}

// Stores 8 elements at dst index i (a multiple of 8), nontemporally in the
// fused form, which also accumulates the values stored; the accumulating
// modes add the old destination values o (from load_old).
template <int MODE, bool NORM>
__device__ __forceinline__ void put_vector(void* dst, uint64_t i, u32x4 s, Old o, AccOf<MODE>& acc)
{
    if constexpr (MODE == kCopy16 || MODE == kAcc16) {
        u32x4* d = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(dst) + i);
        u32x4 r = s;
        if (MODE == kAcc16)
            r = __builtin_bit_cast(u32x4, __builtin_bit_cast(f16x8, o.a) + __builtin_bit_cast(f16x8, s));
        store<NORM>(r, d);
        if (NORM)
            acc.vec(r);
    } else {
        const f16x8 h = __builtin_bit_cast(f16x8, s);
        f32x4* d = reinterpret_cast<f32x4*>(static_cast<float*>(dst) + i);
        f32x4 lo = {float(h[0]), float(h[1]), float(h[2]), float(h[3])};
        f32x4 hi = {float(h[4]), float(h[5]), float(h[6]), float(h[7])};
        if (MODE == kAcc32) {
            lo = __builtin_bit_cast(f32x4, o.a) + lo;
            hi = __builtin_bit_cast(f32x4, o.b) + hi;
        }
        store<NORM>(lo, d);
        store<NORM>(hi, d + 1);
        if (NORM) {
            acc.vec(lo);
            acc.vec(hi);
        }
    }
}

// The vector body of an fp32 destination, in units of 4 elements.  Hints:
// the source is read once (nontemporal); an accumulating call rewrites the
// partition in place, so it reads the old values and stores the sums
// nontemporally (a plain load ahead of an in-place store is the slow
// pattern: the 4-micro-batch step went 1.067 -> 1.040 ms); the widening
// call keeps plain stores (11 us faster here than nontemporal ones).
// Thread t takes units u0 + t + k*kBlock, so each 8-byte fp16 load and each 16-byte
// fp32 store of a wave covers one contiguous span (8-element units would put
// a thread's two fp32 vectors 32 bytes apart across the lanes).  d points at
// element 0 of the body (32-byte aligned), s at its source (16-byte aligned).
template <int MODE, bool NORM>
__device__ __forceinline__ void body32(const uint16_t* __restrict__ s, float* __restrict__ d, uint64_t u0,
                                       uint64_t u1, AccOf<MODE>& acc)
{
    constexpr int kUnits = 2 * Geometry<NORM>::kVecsPerThread;
    const u32x2* __restrict__ S = reinterpret_cast<const u32x2*>(s);
    f32x4* __restrict__ D = reinterpret_cast<f32x4*>(d);
    auto put = [&](f32x4* at, u32x2 raw, f32x4 old) {
        const f16x4 h = __builtin_bit_cast(f16x4, raw);
        f32x4 r = {float(h[0]), float(h[1]), float(h[2]), float(h[3])};
        if (MODE == kAcc32)
            r = old + r;                                      // binary32 add
        store<NORM || MODE == kAcc32>(r, at);
        if (NORM)
            acc.vec(r);
    };
    if (u1 - u0 == uint64_t(kUnits) * kBlock) {              // a full workgroup: every load first
        u32x2 r[kUnits];
        f32x4 o[kUnits];
#pragma unroll
        for (int k = 0; k < kUnits; ++k) {
            const uint64_t u = u0 + threadIdx.x + k * kBlock;
            r[k] = __builtin_nontemporal_load(S + u);
            o[k] = MODE == kAcc32 ? __builtin_nontemporal_load(D + u) : f32x4{};
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < kUnits; ++k)
            put(D + u0 + threadIdx.x + k * kBlock, r[k], o[k]);
    } else {
#pragma unroll
        for (int k = 0; k < kUnits; ++k) {
            const uint64_t u = u0 + threadIdx.x + k * kBlock;
            if (u < u1)
                put(D + u, __builtin_nontemporal_load(S + u), MODE == kAcc32 ? D[u] : f32x4{});
        }
    }
}

template <int MODE, bool NORM>
__global__ __launch_bounds__(kBlock) void flatten_kernel(FlatArgs a, void* __restrict__ dst)
{
    constexpr int kVecsPerThread = Geometry<NORM>::kVecsPerThread;
    constexpr uint64_t kVecsPerBlock = Geometry<NORM>::kVecsPerBlock;
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

    AccOf<MODE> acc;                           // fused form: this thread's exact sum

    // body: vectors [v0, v1) of this segment
    const uint64_t v0 = local * kVecsPerBlock;
    const uint64_t v1 = v0 + kVecsPerBlock < nv ? v0 + kVecsPerBlock : nv;
    const uint16_t* __restrict__ sbody = src + head;
    const uint64_t dbody = doff + head;
    if (MODE >= kTo32 && vec_src) {
        if constexpr (MODE >= kTo32)
            body32<MODE, NORM>(sbody, static_cast<float*>(dst) + dbody, 2 * v0, 2 * v1, acc);
    } else if (vec_src && v1 - v0 == kVecsPerBlock) {
        // A full workgroup (all but a segment's last): no per-lane guards, so
        // every load is issued before the first wait.  Under per-lane guards
        // the compiler moves each load into its store's guarded block and
        // waits for it there, one load in flight per thread.
        u32x4 r[kVecsPerThread];
        Old o[kVecsPerThread];
#pragma unroll
        for (int k = 0; k < kVecsPerThread; ++k) {
            const uint64_t v = v0 + threadIdx.x + k * kBlock;
            r[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sbody) + v);
            o[k] = load_old<MODE>(dst, dbody + 8 * v);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < kVecsPerThread; ++k)
            put_vector<MODE, NORM>(dst, dbody + 8 * (v0 + threadIdx.x + k * kBlock), r[k], o[k], acc);
    } else if (vec_src) {
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
                put_vector<MODE, NORM>(dst, dbody + 8 * v, r[k], load_old<MODE>(dst, dbody + 8 * v), acc);
        }
    } else {
        for (uint64_t v = v0 + threadIdx.x; v < v1; v += kBlock) {
            const uint16_t* s = sbody + 8 * v;
            u32x4 r;
            r.x = uint32_t(s[0]) | (uint32_t(s[1]) << 16);
            r.y = uint32_t(s[2]) | (uint32_t(s[3]) << 16);
            r.z = uint32_t(s[4]) | (uint32_t(s[5]) << 16);
            r.w = uint32_t(s[6]) | (uint32_t(s[7]) << 16);
            put_vector<MODE, NORM>(dst, dbody + 8 * v, r, load_old<MODE>(dst, dbody + 8 * v), acc);
        }
    }

    // head and tail: fewer than 8 elements each, done by the segment's first block
    if (local == 0) {
        const uint64_t t0 = head + 8 * nv;
        const uint64_t t = threadIdx.x;
        if (t < head)
            put_scalar<MODE, NORM>(dst, doff + t, src[t], acc);
        if (t < cnt - t0)
            put_scalar<MODE, NORM>(dst, doff + t0 + t, src[t0 + t], acc);
    }

    if constexpr (NORM && MODE < kTo32) {       // every thread reaches this point
        // A lane has added at most 8 * kVecsPerThread + 2 binary16 squares
        // (its vectors, at most one head and one tail element), each below
        // 2^32, so the wave's h is a multiple of 2^-8 below 2^44 and its |l| a
        // multiple of 2^-48 below 2^3 while that count is at most 64: both
        // fold across the wave in binary64 without rounding, and become limbs
        // once per wave.
        static_assert(kVecsPerThread * 8 + 2 <= 64, "the binary64 wave fold needs at most 64 squares per lane");
        exact::Acc16 w = acc;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            w.h += __shfl_xor(w.h, off, 64);
            w.l += __shfl_xor(w.l, off, 64);
        }
        __shared__ exact::Limbs s_w[kBlock / 64];
        __shared__ uint32_t s_f[kBlock / 64];
        if ((threadIdx.x & 63) == 0) {
            s_w[threadIdx.x >> 6] = w.limbs();
            s_f[threadIdx.x >> 6] = w.status();
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            exact::Limbs s{0, 0, 0, 0};
            uint32_t flag = 0;
#pragma unroll
            for (int k = 0; k < kBlock / 64; ++k) {
                s.l0 += s_w[k].l0;
                s.l1 += s_w[k].l1;
                s.l2 += s_w[k].l2;
                s.l3 += s_w[k].l3;
                flag |= s_f[k];
            }
            a.partials[blockIdx.x] = exact::make_partial(s, flag);
        }
    } else if constexpr (NORM) {
        uint32_t flag = acc.status();
        exact::Limbs s = acc.limbs();
        exact::block_fold<kBlock>(s, flag);
        if (threadIdx.x == 0)
            a.partials[blockIdx.x] = exact::make_partial(s, flag);
    }
}

// One launch.  ordered = false clears the barrier bit of the dispatch packet
// (hipExtAnyOrderLaunch): the packet processor may then start this kernel's
// workgroups while earlier kernels of the stream are still running, so
// back-to-back flattens of disjoint buckets overlap their ramp and drain.
template <int MODE, bool NORM>
void launch_one(const FlatArgs& a, uint32_t blocks, void* dst, hipStream_t s, bool ordered)
{
    if (ordered)
        hipLaunchKernelGGL((flatten_kernel<MODE, NORM>), dim3(blocks), dim3(kBlock), 0, s, a, dst);
    else
        hipExtLaunchKernelGGL((flatten_kernel<MODE, NORM>), dim3(blocks), dim3(kBlock), 0, s, nullptr, nullptr,
                              uint32_t(hipExtAnyOrderLaunch), a, dst);
}

template <bool NORM>
int launch(const FlatArgs& a, uint32_t blocks, int mode, void* dst, hipStream_t s, bool ordered = true)
{
    switch (mode) {
    case kCopy16: launch_one<kCopy16, NORM>(a, blocks, dst, s, ordered); break;
    case kAcc16: launch_one<kAcc16, NORM>(a, blocks, dst, s, ordered); break;
    case kTo32: launch_one<kTo32, NORM>(a, blocks, dst, s, ordered); break;
    default: launch_one<kAcc32, NORM>(a, blocks, dst, s, ordered); break;
    }
    return launch_status();
}

// Workgroups a segment needs: one per kVecsPerBlock body vectors, at least one.
template <bool NORM>
uint64_t blocks_for(const zero_segment_t& sg)
{
    constexpr uint64_t vpb = Geometry<NORM>::kVecsPerBlock;
    const uint64_t head = head_len(sg.dst_off, sg.count);
    const uint64_t nv = (sg.count - head) / 8;
    return nv ? (nv + vpb - 1) / vpb : 1;
}

int validate(const zero_segment_t* segs, uint32_t nsegs, const void* dst, uint64_t dst_len)
{
    if (nsegs && (!segs || !dst))
        return ZERO_EINVAL;
    if (nsegs && !is_aligned(dst, 16))
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
        if (blocks_for<false>(segs[i]) > 0x7fffffffull)      // the larger of the two counts
            return ZERO_ERANGE;
    }
    return ZERO_OK;
}

// Splits the call into launches of at most kMaxSegs segments and 2^31 - 1
// workgroups; `fn(args, blocks)` is called once per launch, in order.
template <bool NORM, typename F>
int for_each_launch(const zero_segment_t* segs, uint32_t nsegs, F&& fn)
{
    FlatArgs a{};
    uint32_t k = 0;
    uint64_t blocks = 0;
    for (uint32_t i = 0; i <= nsegs; ++i) {
        const uint64_t need = (i < nsegs && segs[i].count) ? blocks_for<NORM>(segs[i]) : 0;
        if (k && (i == nsegs || k == kMaxSegs || blocks + need > 0x7fffffffull)) {
            a.first_block[k] = uint32_t(blocks);
            a.nsegs = k;
            const int rc = fn(a, uint32_t(blocks));
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

}  // namespace
}  // namespace zero

using namespace zero;

extern "C" int zero_flatten_bucket(const zero_segment_t* segs, uint32_t nsegs, void* dst, uint64_t dst_len,
                                   int dst_dtype, int accumulate, void* stream)
{
    if (dst_dtype != ZERO_F16 && dst_dtype != ZERO_F32)
        return ZERO_EINVAL;
    const int rc = validate(segs, nsegs, dst, dst_len);
    if (rc != ZERO_OK)
        return rc;
    const int mode = (dst_dtype == ZERO_F16 ? kCopy16 : kTo32) + (accumulate ? 1 : 0);
    hipStream_t s = (hipStream_t)stream;
    return for_each_launch<false>(segs, nsegs,
                                  [&](FlatArgs& a, uint32_t blocks) { return launch<false>(a, blocks, mode, dst, s); });
}

extern "C" uint64_t zero_flatten_norm_partials(const zero_segment_t* segs, uint32_t nsegs)
{
    if (!segs)
        return 0;
    uint64_t total = 0;
    for (uint32_t i = 0; i < nsegs; ++i)
        if (segs[i].count)
            total += blocks_for<true>(segs[i]);
    return total;
}

namespace zero {
namespace {

int flatten_norm(const zero_segment_t* segs, uint32_t nsegs, void* dst, uint64_t dst_len, int mode,
                 void* partials, uint64_t partials_capacity, void* stream)
{
    const int rc = validate(segs, nsegs, dst, dst_len);
    if (rc != ZERO_OK)
        return rc;
    const uint64_t need = zero_flatten_norm_partials(segs, nsegs);
    if (need && !partials)
        return ZERO_EINVAL;
    if (need && !is_aligned(partials, 16))
        return ZERO_EALIGN;
    if (need > partials_capacity)
        return ZERO_ERANGE;
    hipStream_t s = (hipStream_t)stream;
    NormPartial* next = static_cast<NormPartial*>(partials);
    return for_each_launch<true>(segs, nsegs, [&](FlatArgs& a, uint32_t blocks) {
        a.partials = next;
        next += blocks;
        return launch<true>(a, blocks, mode, dst, s);
    });
}

}  // namespace
}  // namespace zero

extern "C" int zero_flatten_norm_bucket(const zero_segment_t* segs, uint32_t nsegs, uint16_t* dst,
                                        uint64_t dst_len, int accumulate, void* partials,
                                        uint64_t partials_capacity, void* stream)
{
    return flatten_norm(segs, nsegs, dst, dst_len, accumulate ? kAcc16 : kCopy16, partials, partials_capacity,
                        stream);
}

extern "C" int zero_flatten_norm_bucket_f32(const zero_segment_t* segs, uint32_t nsegs, float* dst,
                                            uint64_t dst_len, int accumulate, void* partials,
                                            uint64_t partials_capacity, void* stream)
{
    return flatten_norm(segs, nsegs, dst, dst_len, accumulate ? kAcc32 : kTo32, partials, partials_capacity,
                        stream);
}

namespace zero {
namespace {

// ZERO_EINVAL if two nonempty segments write a common destination element
// (ZERO_ENOMEM if the host cannot hold the sorted list).
int check_disjoint(const zero_segment_t* segs, uint64_t nsegs)
{
    try {
        std::vector<std::pair<uint64_t, uint64_t>> r;
        r.reserve(nsegs);
        for (uint64_t i = 0; i < nsegs; ++i)
            if (segs[i].count)
                r.emplace_back(segs[i].dst_off, segs[i].count);
        std::sort(r.begin(), r.end());
        for (size_t i = 1; i < r.size(); ++i)
            if (r[i].first - r[i - 1].first < r[i - 1].second)     // sorted: r[i].first >= r[i-1].first
                return ZERO_EINVAL;
        return ZERO_OK;
    } catch (...) {
        return ZERO_ENOMEM;
    }
}

}  // namespace
}  // namespace zero

extern "C" int zero_flatten_buckets(const zero_segment_t* segs, const uint32_t* bucket_nsegs, uint32_t nbuckets,
                                    void* dst, uint64_t dst_len, int dst_dtype, int accumulate, void* partials,
                                    uint64_t partials_capacity, void* stream)
{
    if (dst_dtype != ZERO_F16 && dst_dtype != ZERO_F32)
        return ZERO_EINVAL;
    if (nbuckets && !bucket_nsegs)
        return ZERO_EINVAL;
    uint64_t total = 0;
    for (uint32_t b = 0; b < nbuckets; ++b)
        total += bucket_nsegs[b];
    if (total > 0xFFFFFFFFull)
        return ZERO_ERANGE;
    int rc = validate(segs, uint32_t(total), dst, dst_len);
    if (rc != ZERO_OK)
        return rc;
    rc = check_disjoint(segs, total);
    if (rc != ZERO_OK)
        return rc;
    const bool norm = partials != nullptr;
    if (norm) {
        if (!is_aligned(partials, 16))
            return ZERO_EALIGN;
        if (zero_flatten_norm_partials(segs, uint32_t(total)) > partials_capacity)
            return ZERO_ERANGE;
    }
    const int mode = (dst_dtype == ZERO_F16 ? kCopy16 : kTo32) + (accumulate ? 1 : 0);
    hipStream_t s = (hipStream_t)stream;
    NormPartial* next = static_cast<NormPartial*>(partials);
    bool ordered = true;          // the first launch waits for the stream's earlier work
    int capturing = -1;           // looked up after the first launch
    // After a launch: whether the next one keeps the dispatch barrier.  Under
    // stream capture the launches become graph nodes, ordered by the graph's
    // edges, so they are captured as ordinary launches.
    auto after_launch = [&](int rc_launch) {
        if (rc_launch != ZERO_OK)
            return rc_launch;
        if (capturing < 0) {
            hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
            const hipError_t e = hipStreamIsCapturing(s, &cap);
            if (e != hipSuccess)
                return hip_fail(e);
            capturing = cap != hipStreamCaptureStatusNone ? 1 : 0;
        }
        ordered = capturing != 0;
        return int(ZERO_OK);
    };
    // Each launch is issued once the next one is known, so that the call's
    // last launch keeps the dispatch barrier too: its completion then implies
    // that of every launch before it, for whatever waits on the stream's last
    // packet afterwards (a synchronisation, an event, a copy engine).
    FlatArgs pend{};
    uint32_t pend_blocks = 0;
    bool have = false;
    auto flush = [&](bool last) {
        if (!have)
            return int(ZERO_OK);
        have = false;
        const bool ord = ordered || last;
        return after_launch(norm ? launch<true>(pend, pend_blocks, mode, dst, s, ord)
                                 : launch<false>(pend, pend_blocks, mode, dst, s, ord));
    };
    auto defer = [&](FlatArgs& a, uint32_t blocks) {
        const int r = flush(false);
        pend = a;
        pend_blocks = blocks;
        have = true;
        return r;
    };
    const zero_segment_t* b = segs;
    for (uint32_t k = 0; k < nbuckets; ++k) {
        if (norm)
            rc = for_each_launch<true>(b, bucket_nsegs[k], [&](FlatArgs& a, uint32_t blocks) {
                a.partials = next;
                next += blocks;
                return defer(a, blocks);
            });
        else
            rc = for_each_launch<false>(b, bucket_nsegs[k], defer);
        if (rc != ZERO_OK)
            return rc;
        b += bucket_nsegs[k];
    }
    return flush(true);
}
