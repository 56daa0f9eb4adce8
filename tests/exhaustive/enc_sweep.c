/*
 * enc_sweep.c -- every non-NaN binary32 value through the C oracle's encoders and through
 * an independent bit-manipulation encoder written here, test-only.
 *
 * The oracle encodes by searching a table of the format's values built from its bit fields
 * ("nearest finite value, ties to the even code, sign kept"; page "Towards Blackwell-native
 * 8-bit and 4-bit RL", section "Format background": E4M3 scales and elements, E2M1
 * elements; section "High-precision and dequantized backward": BF16 operands).  The
 * encoders below instead round the binary32 significand directly: the kept bits, the
 * remainder against half a step, ties to an even last bit, a carry that moves into the
 * exponent field, and saturation at the largest finite value.  Prints the number of
 * mismatches per format and the first mismatching input, and exits non-zero on any.
 *
 * Build: gcc -O2 -fopenmp enc_sweep.c -L<oracle dir> -l:liboracle.so -Wl,-rpath,<oracle dir>
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint8_t oracle_enc_e4m3(double v);
uint8_t oracle_enc_e2m1(double v);
uint16_t oracle_rne_bf16(double v);

/* Round sig * 2^-sh to an integer, nearest with ties to even (sh >= 1). */
static uint64_t rne_shift(uint64_t sig, int sh) {
    if (sh >= 64) return 0;
    uint64_t q = sig >> sh, rem = sig & ((1ull << sh) - 1), half = 1ull << (sh - 1);
    if (rem > half || (rem == half && (q & 1))) q++;
    return q;
}

/* E4M3 (OCP E4M3FN): bias 7, 3 mantissa bits, subnormal step 2^-9, largest finite 448. */
static uint8_t e4m3_bits(uint32_t u) {
    const uint8_t s = (uint8_t)((u >> 24) & 0x80);
    const uint32_t a = u & 0x7FFFFFFFu, E = a >> 23, m = a & 0x7FFFFFu;
    if (a >= 0x43E00000u) return s | 0x7E;            /* 448 or more (also inf): 448 */
    if (a < 0x3C800000u) {                             /* below 2^-6: multiples of 2^-9 */
        if (E == 0) return s;                          /* below 2^-126 */
        /* a = (2^23 + m) * 2^(E - 150); a / 2^-9 = (2^23 + m) * 2^(E - 141) */
        return s | (uint8_t)rne_shift((uint64_t)(m | 0x800000u), 141 - (int)E);
    }
    uint32_t q = m >> 20;                              /* keep 3 of 23 mantissa bits */
    const uint32_t rem = m & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) q++;
    return s | (uint8_t)(((E - 120u) << 3) + q);       /* a carry moves into the exponent */
}

/* E2M1: bias 1, 1 mantissa bit, subnormal step 0.5, largest finite 6. */
static uint8_t e2m1_bits(uint32_t u) {
    const uint8_t s = (uint8_t)((u >> 28) & 0x8);
    const uint32_t a = u & 0x7FFFFFFFu, E = a >> 23, m = a & 0x7FFFFFu;
    if (a >= 0x40C00000u) return s | 7;                /* 6 or more (also inf): 6 */
    if (a < 0x3F800000u) {                             /* below 1: multiples of 0.5 */
        if (E == 0) return s;
        return s | (uint8_t)rne_shift((uint64_t)(m | 0x800000u), 149 - (int)E);
    }
    uint32_t q = m >> 22;                              /* keep 1 of 23 mantissa bits */
    const uint32_t rem = m & 0x3FFFFFu;
    if (rem > 0x200000u || (rem == 0x200000u && (q & 1u))) q++;
    return s | (uint8_t)(((E - 126u) << 1) + q);
}

/* BF16: keep the top 16 bits, nearest with ties to even; overflow gives infinity. */
static uint16_t bf16_bits(uint32_t u) {
    const uint32_t keep = u >> 16, rem = u & 0xFFFFu;
    return (uint16_t)(keep + ((rem > 0x8000u || (rem == 0x8000u && (keep & 1u))) ? 1u : 0u));
}

int main(void) {
    long long bad[3] = {0, 0, 0};
    long long first[3] = {-1, -1, -1};
#pragma omp parallel for schedule(static, 1 << 16) reduction(+ : bad[:3])
    for (long long i = 0; i < (1ll << 32); ++i) {
        const uint32_t u = (uint32_t)i;
        if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu) != 0) continue;   /* NaN */
        float f;
        memcpy(&f, &u, sizeof f);
        const double d = (double)f;
        const int b0 = oracle_enc_e4m3(d) != e4m3_bits(u);
        const int b1 = oracle_enc_e2m1(d) != e2m1_bits(u);
        const int b2 = oracle_rne_bf16(d) != bf16_bits(u);
        if (b0 | b1 | b2) {
#pragma omp critical
            {
                if (b0 && first[0] < 0) first[0] = i;
                if (b1 && first[1] < 0) first[1] = i;
                if (b2 && first[2] < 0) first[2] = i;
            }
        }
        bad[0] += b0; bad[1] += b1; bad[2] += b2;
    }
    const char* name[3] = {"E4M3", "E2M1", "BF16"};
    for (int k = 0; k < 3; ++k) {
        if (bad[k]) printf("%s %lld mismatches, first at binary32 0x%08llx\n", name[k], bad[k], (unsigned long long)first[k]);
        else printf("%s 0 mismatches over every non-NaN binary32 value\n", name[k]);
    }
    return (bad[0] | bad[1] | bad[2]) ? 1 : 0;
}
