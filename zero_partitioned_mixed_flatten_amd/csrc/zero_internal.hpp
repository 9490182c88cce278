// zero_internal.hpp -- definitions shared by the library's translation units
// (never installed; the public interface is include/zero_mi355x.h).
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "zero_mi355x.h"

static_assert(sizeof(zero_step_state_t) == 128, "zero_step_state_t is a 128-byte ABI struct");
static_assert(offsetof(zero_step_state_t, sumsq) == 40, "state layout");
static_assert(offsetof(zero_step_state_t, gmul) == 64, "state layout");
static_assert(offsetof(zero_step_state_t, done_blocks) == 104, "state layout");
static_assert(offsetof(zero_step_state_t, sumsq_units) == 112, "state layout");
static_assert(sizeof(zero_segment_t) == 32, "segment layout");
static_assert(sizeof(zero_hparams_t) == 80, "hparams layout");
static_assert(sizeof(zero_onebit_state_t) == 72, "1-bit state layout");

namespace zero {

// 16-byte register vectors: one global_load/store_dwordx4 each.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
// 8-byte register vectors: one global_load/store_dwordx2 each.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// ---- loads ahead of the skip test (loads_first_use) ---------------------------
// The one-shot step kernels issue every load of a thread before they read the
// step's skip flag: a wave that tests the flag first starts its streams one
// scalar-load latency late (about 3% of the Adam kernel).  Used only on the
// update path, the loads would be sunk by the compiler into that path, behind
// the flag's wait; each kernel therefore also uses them on the skip path,
// inside a test that no valid call passes (n == UINT64_MAX, which no launch
// can have), so they stay ahead of the branch.  bits_of gathers a raw fp16
// group's bits into one fp32 vector for that use.
__device__ __forceinline__ f32x4 bits_of(u32x2 r)
{
    return f32x4{__builtin_bit_cast(float, r.x), __builtin_bit_cast(float, r.y), 0.0f, 0.0f};
}

__device__ __forceinline__ f32x4 bits_of(f32x4 r) { return r; }

__host__ __device__ inline bool is_aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Records a HIP error for zero_status_string and maps it to ZERO_EHIP.
int hip_fail(hipError_t e);
// Checks the launch that was just enqueued.
int launch_status();

// Bytes of dynamic LDS that, reserved by each workgroup of a kernel that
// uses none, limit the current device to blocks_per_cu resident workgroups
// per CU (0 if the device cannot be queried).
uint32_t lds_reservation(int blocks_per_cu);

// ---- norm/overflow reduction geometry (shared by the host size query and
// the launch) ----------------------------------------------------------------
constexpr int kNormBlock = 1024;                            // 16 wavefronts, one workgroup per CU
constexpr uint64_t kNormMaxBlocks = 256;                    // one per CU of an MI355X
constexpr uint64_t kNormMaxPerThread = uint64_t(1) << 12;   // keeps the binary64 partial sums exact
constexpr uint64_t kNormMaxElems = uint64_t(1) << 40;       // keeps the grid within 2^18 workgroups

// One workgroup's exact partial in 16 bytes, one vector load: the sum of
// squares in 2^-48 units, below 2^126, as w0 + 2^64 * (w1 mod 2^62), and the
// OR-ed status bits in the top two bits of w1.  No partial of a valid fast
// reduction comes near 2^126 units: a workgroup adds at most 2^22 squares,
// each below 2^96 units; a larger sum is marked for the wide pass.
struct alignas(16) NormPartial {
    uint64_t w0, w1;
};
static_assert(sizeof(NormPartial) == 16 && sizeof(NormPartial) == ZERO_NORM_PARTIAL_BYTES, "partial layout");
constexpr int kPartialStatusShift = 62;

uint64_t norm_grid(uint64_t n);

// zero_shard_adam_step that runs only while dev_state->step <= gate (the
// warm-up steps of zero_onebit_step); the same checks and errors.
int adam_step_gated(uint16_t* p16, float* p32, float* m32, float* v32, const uint16_t* grad16, uint64_t n,
                    const zero_step_state_t* dev_state, void* stream, int64_t gate);

// Partials folded by the decide-only pass (the fused flatten writes one per
// workgroup); stored partials are carried, so 2^30 of them fit in int64 sums.
constexpr uint64_t kMaxPartials = uint64_t(1) << 30;
uint64_t decide_grid(uint64_t count);

}  // namespace zero
