/* Exhaustive checks of the two division shortcuts the HIP quantizer uses
 * (see quantize.hip): both must equal the correctly rounded IEEE result on
 * every input they can receive.  Built and run by tests/test_fastdiv.py. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(void)
{
    long bad = 0;
    /* 1. x / n for n = 2^b - 1, every non-negative finite binary32 x. */
    const int ns[4] = {3, 7, 15, 255};
    for (int k = 0; k < 4; k++) {
        const float n = (float)ns[k], c = 1.0f / n;
        long bk = 0;
#pragma omp parallel for reduction(+ : bk) schedule(static)
        for (long u = 0; u < 0x7f800000L; u++) {
            const float x = from_bits((uint32_t)u);
            const float q0 = x * c;
            const float q1 = fmaf(fmaf(-q0, n, x), c, q0);
            if (to_bits(q1) != to_bits(x / n)) bk++;
        }
        printf("divide by %d: %ld mismatches\n", ns[k], bk);
        bad += bk;
    }
    /* 2. 1/s for every positive finite binary16 s, one Newton step from any
     *    start within 2 ulp of the true reciprocal. */
    long br = 0;
    for (uint32_t h = 1; h < 0x7c00; h++) {
        const uint32_t e = (h >> 10) & 31, m = h & 1023;
        const float s = e ? ldexpf((float)(m | 1024), (int)e - 25) : ldexpf((float)m, -24);
        const float want = 1.0f / s;
        for (int d = -2; d <= 2; d++) {
            const float y0 = from_bits(to_bits(want) + (uint32_t)d);
            const float y1 = fmaf(fmaf(-s, y0, 1.0f), y0, y0);
            if (to_bits(y1) != to_bits(want)) br++;
        }
    }
    printf("reciprocal: %ld mismatches\n", br);
    bad += br;
    return bad ? 1 : 0;
}
