// Host driver for the wide exact sum's integer arithmetic (wide_sum.hpp):
// the same square decomposition, carry and conversions the device pass uses,
// run on the CPU so a test can check them against exact Python integers.
//   wide_driver sum FILE    sum of squares of the binary32 values in FILE:
//                           prints the binary64 result (%a), whether it is a
//                           whole number of 2^-48 units below 2^128, and
//                           those units (high, low)
//   wide_driver digits FILE 20 uint64 digits per record: prints each
//                           record's binary64 value (%a)
#include <stdio.h>
#include <string.h>

#include <vector>

#include "wide_sum.hpp"

using namespace zero::wide;

int main(int argc, char** argv)
{
    if (argc != 3)
        return 2;
    FILE* f = fopen(argv[2], "rb");
    if (!f)
        return 2;
    if (!strcmp(argv[1], "sum")) {
        std::vector<float> v;
        float x;
        while (fread(&x, sizeof x, 1, f) == 1)
            v.push_back(x);
        fclose(f);
        uint64_t d[kDigits] = {0};
        for (float y : v) {
            const SquareDigits s = square_digits(y);
            if (s.k < 0)
                continue;
            d[s.k] += s.d0;
            d[s.k + 1] += s.d1;
            d[s.k + 2] += s.d2;
        }
        carry(d);
        uint64_t hi = 0, lo = 0;
        const bool whole = to_units48(d, hi, lo);
        printf("%a %d %llu %llu\n", to_f64(d), whole ? 1 : 0, (unsigned long long)hi, (unsigned long long)lo);
        return 0;
    }
    if (!strcmp(argv[1], "digits")) {
        uint64_t d[kDigits];
        while (fread(d, sizeof d, 1, f) == 1)
            printf("%a\n", to_f64(d));
        fclose(f);
        return 0;
    }
    return 2;
}
