/* Host check of the quantiser's division: for a block scale s = RN(amax / 448) >= 2^-90 and
 * |x| <= amax, the corrected product
 *     y = RN(1 / s),  q = RN(x y),  r = RN(x - q s) (one FMA),  q' = copysign(RN(q + r y), x)
 * encodes to the same E4M3 value (round to nearest even, saturating at 448) as the IEEE
 * quotient RN(x / s).  Cases: random amax over a wide exponent range, x at amax, just below it,
 * anywhere below it, and x placed a few ulps around s times an E4M3 rounding midpoint.
 * Usage: quotient_check N  -> prints "cases C quotient_mismatches Q code_mismatches M". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t state = 0x2545F4914F6CDD1Dull;
static uint64_t next_u64(void) {
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return state;
}
static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* value of the E4M3 encoding of v: saturate to +-448, quantum 2^(e-3) for normals
 * (e >= -6), 2^-9 for subnormals, ties to even */
static double e4m3_value(float vf) {
    double v = vf;
    if (v > 448.0) v = 448.0;
    if (v < -448.0) v = -448.0;
    double a = fabs(v);
    if (a == 0.0) return v;
    int e;
    frexp(a, &e);
    e -= 1;
    if (e < -6) e = -6;
    double quantum = ldexp(1.0, e - 3);
    return copysign(nearbyint(a / quantum) * quantum, v);
}

int main(int argc, char** argv) {
    long n = argc > 1 ? atol(argv[1]) : 1000000L;
    long cases = 0, qbad = 0, cbad = 0;
    for (long i = 0; i < n; ++i) {
        uint64_t r = next_u64();
        int e = (int)(r % 208) - 80;
        uint32_t abits = ((uint32_t)(e + 127) << 23) | (uint32_t)((r >> 8) & 0x7fffffu);
        float amax = from_bits(abits);
        float s = amax / 448.0f;
        if (!isfinite(amax) || s < 0x1p-90f) continue;
        uint64_t r2 = next_u64();
        float x;
        switch (r2 & 3) {
        case 0: x = amax; break;
        case 1: x = from_bits(abits - (uint32_t)((r2 >> 8) % 0x1000000u)); break;
        default: {
            int xe = (int)(abits >> 23) - (int)((r2 >> 8) % 40);
            if (xe <= 0) continue;
            x = from_bits(((uint32_t)xe << 23) | (uint32_t)((r2 >> 16) & 0x7fffffu));
        }
        }
        if (((r2 >> 41) & 3) == 0) {
            int me = (int)((r2 >> 44) % 15) - 9;
            double mid = me <= -7 ? ldexp((double)((r2 >> 50) % 8) + 0.5, -9)
                                  : ldexp(1.0, me) * (1.0 + ((double)((r2 >> 50) % 8) + 0.5) / 8.0);
            if (mid > 448.0) mid = 440.0;
            x = from_bits(to_bits((float)(mid * (double)s)) + (uint32_t)((int)((r2 >> 54) % 9) - 4));
        }
        if (!(fabsf(x) <= amax)) continue;
        if ((r2 >> 40) & 1) x = -x;
        float y = 1.0f / s;
        float q = x * y;
        float rr = fmaf(-q, s, x);
        float qc = copysignf(fmaf(rr, y, q), x);
        float ref = x / s;
        ++cases;
        if (to_bits(qc) != to_bits(ref)) ++qbad;
        if (e4m3_value(qc) != e4m3_value(ref) || signbit(qc) != signbit(ref)) ++cbad;
    }
    printf("cases %ld quotient_mismatches %ld code_mismatches %ld\n", cases, qbad, cbad);
    return 0;
}
