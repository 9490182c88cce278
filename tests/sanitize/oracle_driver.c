/* Memory-safety driver for the oracle: built together with its source under
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py.
 * Every buffer is allocated at exactly the size a call may touch, so any
 * overrun reaches a redzone.  Values are seeded pseudo-random; correctness is
 * pinned elsewhere -- this only exercises every entry point on ragged sizes,
 * misaligned segments, specials and skipped steps. */
#include "../../oracle/zero_oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 32);
}

static uint16_t rnd_f16(int specials)
{
    uint16_t b = (uint16_t)(rnd() & 0xFFFFu);
    if (!specials && (b & 0x7C00u) == 0x7C00u)
        b &= 0xBFFFu;                                   /* keep it finite */
    return b;
}

int main(void)
{
    static const uint64_t sizes[] = {0, 1, 7, 8, 9, 63, 4099, 65539};
    oracle_hparams_t hp = {1e-4, 0.9, 0.999, 1e-8, 0.01, 1.0, 0.5, 2.0, 1.0, 20, 0};
    for (unsigned si = 0; si < sizeof sizes / sizeof sizes[0]; ++si) {
        const uint64_t n = sizes[si];
        const uint64_t a = n ? n : 1;
        /* segments: random pieces of n, each from its own exact-size source at a random offset */
        oracle_segment_t segs[64];
        uint16_t* srcs[64];
        uint32_t ns = 0;
        for (uint64_t d = 0; d < n && ns < 64; ++ns) {
            uint64_t c = 1 + rnd() % (n - d < 5000 ? n - d : 5000);
            if (ns == 63)
                c = n - d;
            const uint64_t off = rnd() % 17;
            srcs[ns] = (uint16_t*)malloc((off + c) * sizeof(uint16_t));
            for (uint64_t i = 0; i < off + c; ++i)
                srcs[ns][i] = rnd_f16(si & 1);
            segs[ns].src = srcs[ns];
            segs[ns].src_off = off;
            segs[ns].dst_off = d;
            segs[ns].count = c;
            d += c;
        }
        uint16_t* g16 = (uint16_t*)malloc(a * sizeof(uint16_t));
        uint16_t* p16 = (uint16_t*)malloc(a * sizeof(uint16_t));
        float* g32 = (float*)calloc(a, sizeof(float));
        float* p32 = (float*)malloc(a * sizeof(float));
        float* m32 = (float*)calloc(a, sizeof(float));
        float* v32 = (float*)calloc(a, sizeof(float));
        float* ew = (float*)calloc(a, sizeof(float));
        float* es = (float*)calloc(a, sizeof(float));
        uint8_t* bw = (uint8_t*)malloc((a + 7) / 8);
        uint8_t* bs = (uint8_t*)malloc((a + 7) / 8);
        for (uint64_t i = 0; i < a; ++i) {
            p32[i] = (float)((int32_t)rnd()) * 1e-11f;
            p16[i] = oracle_f16_from_f32(p32[i]);
        }
        oracle_state_t st;
        oracle_state_init(&st, 65536.0);
        for (int k = 0; k < 4; ++k) {
            double sumsq;
            int32_t ovf;
            oracle_flatten(segs, ns, g16, 0, 0);
            oracle_flatten(segs, ns, g32, 1, k > 0);
            oracle_norm_overflow(g16, n, &sumsq, &ovf);
            oracle_decide(&st, &hp, sumsq, ovf);
            oracle_adam_update(&st, p16, p32, m32, v32, g16, n);
            oracle_norm_overflow_f32(g32, n, &sumsq, &ovf);
            oracle_decide(&st, &hp, sumsq, ovf);
            oracle_adam_update_f32(&st, p16, p32, m32, v32, g32, n);
            float scales[2];
            if (oracle_onebit_step(&st, p16, p32, m32, v32, ew, es, g16, n, bw, bs, scales) < 0)
                return 3;
            oracle_step(&hp, &st, segs, ns, g16, p16, p32, m32, v32, n);
        }
        double scale_sum;
        (void)oracle_onebit_scale(p32, n, &scale_sum);
        oracle_onebit_pack(p32, n, bw);
        oracle_f32_from_f16_array(p16, g32, n);
        oracle_f16_from_f32_array(g32, p16, n);
        for (uint32_t s = 0; s < ns; ++s)
            free(srcs[s]);
        free(g16); free(p16); free(g32); free(p32); free(m32); free(v32); free(ew); free(es); free(bw); free(bs);
    }
    for (int stage = 0; stage <= 3; ++stage) {
        uint64_t out;
        if (oracle_state_bytes(1557611200ull, 16, 12, stage, &out) != 0)
            return 2;
    }
    for (uint32_t h = 0; h < 65536; ++h)
        (void)oracle_f16_from_f32(oracle_f32_from_f16((uint16_t)h));
    puts("ok");
    return 0;
}
