// Memory-safety and data-race driver for the host (ZeRO-Offload) step:
// built with host_step.cpp under AddressSanitizer + UndefinedBehaviorSanitizer,
// and separately under ThreadSanitizer, by tests/test_sanitizers.py.  It runs
// the host norm, decision and AdamW on worker pools of 1, 3 and 8 threads over
// ragged sizes and misaligned views, every buffer sized exactly.  Correctness
// is pinned by the host-step tests; this only looks for overruns, undefined
// behaviour and races in the worker pool.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

#include "zero_mi355x.h"

namespace zero {
int hip_fail(hipError_t) { return ZERO_EHIP; }   // the library's HIP error hook (the driver makes no HIP call)
}

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd()
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return uint32_t(rng_state >> 32);
}

int main()
{
    const int threads[] = {1, 3, 8};
    const uint64_t sizes[] = {0, 1, 7, 67, 4099, 100003};
    const zero_hparams_t hp = {1e-4, 0.9, 0.999, 1e-8, 0.01, 1.0, 0.5, 2.0, 1.0, 20, 0};
    for (int t : threads) {
        zero_host_ctx_t* ctx = nullptr;
        int rc = zero_host_create(t, &ctx);
        if (rc == ZERO_ENOTSUP) {
            std::puts("skip: this CPU lacks the AVX-512 the host step needs");
            return 0;
        }
        if (rc != ZERO_OK) {
            std::printf("zero_host_create(%d) = %d\n", t, rc);
            return 1;
        }
        for (uint64_t n : sizes) {
            for (uint64_t off = 0; off < 3; ++off) {            // views 0, 2 and 4 bytes past the allocation
                std::vector<uint16_t> g(off + n), p16(off + n);
                std::vector<float> p(off + n), m(off + n), v(off + n);
                for (uint64_t i = 0; i < off + n; ++i) {
                    uint16_t b = uint16_t(rnd());
                    if ((b & 0x7C00u) == 0x7C00u && (i % 5))
                        b &= 0xBFFFu;                          // mostly finite, a few inf/NaN
                    g[i] = b;
                    p[i] = float(int32_t(rnd())) * 1e-11f;
                }
                zero_step_state_t st;
                if (zero_host_state_init(&st, 65536.0) != ZERO_OK)
                    return 2;
                for (int k = 0; k < 3; ++k) {
                    rc = zero_host_norm_overflow(ctx, n ? g.data() + off : nullptr, n, &hp, &st);
                    if (rc == ZERO_OK)
                        rc = zero_host_adam_step(ctx, n ? p16.data() + off : nullptr, n ? p.data() + off : nullptr,
                                                 n ? m.data() + off : nullptr, n ? v.data() + off : nullptr,
                                                 n ? g.data() + off : nullptr, n, &st);
                    if (rc != ZERO_OK) {
                        std::printf("threads %d n %llu off %llu: rc %d\n", t, (unsigned long long)n,
                                    (unsigned long long)off, rc);
                        return 3;
                    }
                }
            }
        }
        zero_host_destroy(ctx);
    }
    std::puts("ok");
    return 0;
}
