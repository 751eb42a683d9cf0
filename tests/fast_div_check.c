/* The quantisers compute x / scale as RN(q0 + r * inv) with inv = RN(1/scale),
 * q0 = RN(x * inv), r = x - q0 * scale (exact, an fma) and the sign of x
 * restored (Markstein's correction), for scales >= 2^-80.  This checks, on the
 * CPU, that the INT8 code (clamp(rint(q), -127, 127)) and the OCP E4M3 code
 * (nearest even, saturating, sign kept) of that quotient equal the codes of the
 * IEEE quotient: every bf16 value up to amax, and random fp32 values, ties
 * (k + 1/2) * scale and fp32 subnormals, for `nscales` scales amax/127 and
 * amax/448 with amax from 2^-72 to the top of the fp32 range.  Exit status 1 on any difference.
 * Build: gcc -O2 -ffp-contract=off fast_div_check.c -lm. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return state;
}
static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* E4M3 code by value: the nearest of the 127 finite magnitudes (ties to the
 * even code), saturating at 448, sign bit kept. */
static double e4m3_value(uint32_t c)
{
    uint32_t e = (c >> 3) & 15, m = c & 7;
    return e == 0 ? m / 8.0 * ldexp(1.0, -6) : (1.0 + m / 8.0) * ldexp(1.0, (int)e - 7);
}
static uint32_t e4m3_code(float y)
{
    double a = fabs((double)y);
    uint32_t best = 0;
    for (uint32_t c = 1; c <= 0x7E; c++) {
        double d = fabs(e4m3_value(c) - a), db = fabs(e4m3_value(best) - a);
        if (d < db || (d == db && (c & 1) == 0)) best = c;
    }
    if (a >= 448.0) best = 0x7E;
    return (signbit(y) ? 0x80u : 0u) | best;
}
static uint32_t int8_code(float q)
{
    float r = rintf(q);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (uint32_t)(int32_t)r & 0xFFu;
}
static float div_corrected(float x, float d, float inv)
{
    float q0 = x * inv;
    float r = fmaf(-q0, d, x);
    return copysignf(fmaf(r, inv, q0), x);
}

static long total, bad;
static void check(float x, float d, int fp8)
{
    if (!isfinite(x)) return;
    float inv = 1.0f / d, exact = x / d, q = div_corrected(x, d, inv);
    uint32_t c0 = fp8 ? e4m3_code(exact) : int8_code(exact);
    uint32_t c1 = fp8 ? e4m3_code(q) : int8_code(q);
    total++;
    if (c0 != c1) {
        if (bad < 10) printf("mismatch fp8=%d x=%a scale=%a exact=%a corrected=%a\n", fp8, x, d, exact, q);
        bad++;
    }
}

int main(int argc, char **argv)
{
    long nscales = argc > 1 ? atol(argv[1]) : 200;
    for (long j = 0; j < nscales; j++) {
        int fp8 = (int)(j & 1);
        int e = (int)(next() % 210) - 72;            /* amax in [2^-72, 2^138): infinite ones skipped */
        float amax = ldexpf(1.0f + (float)(next() & 0x7FFFFF) / 8388608.0f, e);
        if (isinf(amax)) continue;
        float d = amax / (fp8 ? 448.0f : 127.0f);
        if (d < 0x1p-80f) continue;
        for (uint32_t u = 0; u < 65536; u += fp8 ? 7 : 1) {     /* bf16 values (every 7th for E4M3) */
            float x = from_bits(u << 16);
            if (isfinite(x) && fabsf(x) <= amax) check(x, d, fp8);
        }
        for (int t = 0; t < 2000; t++) {
            float x = amax * ((float)(next() & 0xFFFFFF) / 16777216.0f);
            check((t & 1) ? -x : x, d, fp8);
            float k = (float)((int)(next() % 253) - 126);    /* (k + 1/2) * scale stays below amax */
            check((k + 0.5f) * d, d, fp8);
            check(from_bits((uint32_t)(next() & 0x807FFFFFu)), d, fp8);
        }
    }
    printf("checked %ld, mismatches %ld\n", total, bad);
    return bad != 0;
}
