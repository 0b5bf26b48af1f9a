/*
 * quotient_sweep.c -- CPU check of the quantizer's element quotient (test infrastructure).
 *
 * The recipe's element code is Round(x / (B * T)) (onedev.kr MicroQonv digest, section "How it
 * differs"), read as one IEEE fp32 division q = RN(x / D), D = RN(B * T). The GPU quantizer
 * computes the 16 quotients of a square from one reciprocal:
 *     r  = RN(1 / D)
 *     q0 = RN(x * r)
 *     q  = RN(q0 + RN_exact(x - q0 * D) * r)      (two fused multiply-adds)
 *     q  = copysign(q, x)
 * and uses it only when D lies in [2^-64, 2^64] and |x / D| >= 2^-20 or x = 0 (other squares
 * divide). This program restates that arithmetic with C's fmaf and compares the bit pattern of q
 * (signed zeros included) with x / D over many (x, D) pairs: D = RN(B * T) for every positive
 * E4M3 scale B and log-uniform tensor scales T, x log-uniform in quotient and x next to every
 * rounding midpoint of the E2M1 and E2M3 grids (where a one-ulp error would change a code).
 *
 * Output: "pairs <n> mismatches <m> q0_mismatches <k> nosign_mismatches <z>", where the last two
 * count the same sweep without the correction step and without the sign step (controls: they
 * must be non-zero, so the sweep can see an error).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off quotient_sweep.c -lm (no fast-math: x / D and 1 / D
 * are IEEE divisions, fmaf is the correctly rounded fused multiply-add).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint32_t bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

static float from_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* SplitMix64: a seeded stream for the sweep (no arithmetic of the method). */
static uint64_t g_state = 0x5eedULL;
static uint64_t next64(void)
{
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ULL);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}
static double unif(void) { return (double)(next64() >> 11) * 0x1p-53; }

static long long g_pairs, g_bad, g_bad_q0, g_bad_nosign;

static void check(float x, float D)
{
    const float r = 1.0f / D;
    const float q0 = x * r;
    const float q1 = fmaf(fmaf(-q0, D, x), r, q0);
    const float q = copysignf(q1, x);
    const float want = x / D;
    g_pairs++;
    if (bits(q) != bits(want)) {
        if (g_bad < 5) fprintf(stderr, "mismatch x=%a D=%a q=%a want=%a\n", x, D, q, want);
        g_bad++;
    }
    if (bits(q0) != bits(want)) g_bad_q0++;
    if (bits(q1) != bits(want)) g_bad_nosign++;
}

/* does the GPU take the reciprocal path for this (x, D)? */
static int fast_path(float x, float D)
{
    if (!(D >= 0x1p-64f && D <= 0x1p64f)) return 0;
    return x == 0.0f || fabsf(x) >= D * 0x1p-20f;
}

int main(int argc, char **argv)
{
    const int nT = argc > 1 ? atoi(argv[1]) : 400;
    /* positive E4M3 values, decoded from s|eeee|mmm (bias 7, subnormal m * 2^-9), 0x01..0x7E */
    float e4m3[126];
    for (int c = 1; c <= 126; c++) {
        const int e = c >> 3, m = c & 7;
        e4m3[c - 1] = e == 0 ? ldexpf((float)m, -9) : ldexpf(1.0f + m / 8.0f, e - 7);
    }
    /* element-grid magnitudes: E2M1 {0,.5,...,6} and E2M3 {k/8, ..., 7.5}; midpoints between
     * neighbours are where rounding switches */
    float mids[64];
    int nm = 0;
    for (int fmt = 0; fmt < 2; fmt++) {
        const int mant = fmt == 0 ? 1 : 3, n = 1 << (2 + mant);
        float prev = 0.0f;
        for (int c = 1; c < n; c++) {
            const int e = c >> mant, m = c & ((1 << mant) - 1);
            const float v = e == 0 ? (float)m / (1 << mant) : ldexpf(1.0f + (float)m / (1 << mant), e - 1);
            mids[nm++] = 0.5f * (prev + v);
            prev = v;
        }
    }
    for (int it = 0; it < nT; it++) {
        /* T log-uniform over [2^-40, 2^24] */
        const float T = (float)exp2(-40.0 + 64.0 * unif());
        for (int b = 0; b < 126; b++) {
            const float D = e4m3[b] * T;
            if (!(D >= 0x1p-64f && D <= 0x1p64f)) continue;
            /* x next to every midpoint, +-6 ulps, both signs */
            for (int k = 0; k < nm; k++) {
                const float c = mids[k] * D;
                for (int d = -6; d <= 6; d++) {
                    const float x = from_bits(bits(c) + d);
                    if (fast_path(x, D)) { check(x, D); check(-x, D); }
                }
            }
            /* random x with |x / D| log-uniform in [2^-20, 2^4] */
            for (int j = 0; j < 64; j++) {
                const float x = (float)((unif() < 0.5 ? -1.0 : 1.0) * D * exp2(-20.0 + 24.0 * unif()));
                if (fast_path(x, D)) check(x, D);
            }
            check(0.0f, D);
            check(-0.0f, D);
        }
    }
    printf("pairs %lld mismatches %lld q0_mismatches %lld nosign_mismatches %lld\n", g_pairs, g_bad,
           g_bad_q0, g_bad_nosign);
    return g_bad != 0;
}
