// Host driver for the 1-bit folds' integer core (window_fold.hpp): the same
// partial round trip, rounded moves and interval test the device folds use,
// run on the CPU so a test can check them against exact Python integers.
//   window_driver fold FILE     FILE: "E half count", then count lines
//                               "hi lo e": a window sum W_b = hi*2^64 + lo on
//                               the window of exponent e.  Each W_b goes
//                               through a carried partial and is moved onto
//                               the window of E (2*(E - e) bits, rounded);
//                               prints "hi lo fits decides roundtrip" for the
//                               folded sum
//   window_driver decides FILE  lines "hi lo half": prints decides per line
//   window_driver limbs FILE    lines "hi lo status repeat": each value (below
//                               2^126) becomes a carried partial with those
//                               status bits (make_partial, as a workgroup
//                               stores it) and is folded `repeat` times
//                               (fold_partial, as the decide kernels fold);
//                               prints "hi lo fits flag" for the total
#include <stdio.h>
#include <string.h>

#include "window_fold.hpp"

using namespace zero;

static exact::Limbs limbs_of(uint64_t hi, uint64_t lo)
{
    return exact::Limbs{int64_t(lo & 0xFFFFFFFFull), int64_t(lo >> 32), int64_t(hi & 0xFFFFFFFFull),
                        int64_t(hi >> 32)};
}

int main(int argc, char** argv)
{
    if (argc != 3)
        return 2;
    FILE* f = fopen(argv[2], "r");
    if (!f)
        return 2;
    unsigned long long hi, lo, half;
    if (!strcmp(argv[1], "fold")) {
        int E;
        unsigned long long count;
        if (fscanf(f, "%d %llu %llu", &E, &half, &count) != 3)
            return 3;
        exact::Limbs t{0, 0, 0, 0};
        int roundtrip = 1;
        for (unsigned long long i = 0; i < count; ++i) {
            int e;
            if (fscanf(f, "%llu %llu %d", &hi, &lo, &e) != 3)
                return 3;
            const NormPartial p = exact::make_partial(limbs_of(hi, lo), 0);
            const unsigned __int128 v = window::partial_value(p);
            roundtrip &= v == (((unsigned __int128)hi << 64) | lo);
            window::add_moved(t, v, 2 * (E - e));
        }
        uint64_t h = 0, l = 0;
        const bool fits = exact::limbs_to_u128(t, h, l);
        printf("%llu %llu %d %d %d\n", (unsigned long long)h, (unsigned long long)l, fits ? 1 : 0,
               window::decides(h, l, half) ? 1 : 0, roundtrip);
    } else if (!strcmp(argv[1], "limbs")) {
        exact::Limbs t{0, 0, 0, 0};
        uint32_t flag = 0;
        unsigned status, repeat;
        while (fscanf(f, "%llu %llu %u %u", &hi, &lo, &status, &repeat) == 4) {
            const NormPartial p = exact::make_partial(limbs_of(hi, lo), status);
            for (unsigned r = 0; r < repeat; ++r)
                exact::fold_partial(t, flag, p);
        }
        uint64_t h = 0, l = 0;
        const bool fits = exact::limbs_to_u128(t, h, l);
        printf("%llu %llu %d %u\n", (unsigned long long)h, (unsigned long long)l, fits ? 1 : 0, flag);
    } else if (!strcmp(argv[1], "decides")) {
        while (fscanf(f, "%llu %llu %llu", &hi, &lo, &half) == 3)
            printf("%d\n", window::decides(hi, lo, half) ? 1 : 0);
    } else {
        return 2;
    }
    fclose(f);
    return 0;
}
