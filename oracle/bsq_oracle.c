/*
 * bsq_oracle.c -- plain, slow, obviously correct CPU oracle for the block-scaled
 * quantizer contract: MXFP8 (rowwise 1x32 and columnwise 32x1), per-token NVFP4,
 * and BF16 dequantization of both.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file.  Only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code, header, table or constant generator with
 * the HIP library: every format table below is built here from the bit-field
 * definition of the format.
 *
 * Sources (the pages; "Towards Blackwell-native 8-bit and 4-bit RL", Chinese
 * translation, and its Vietnamese partial translation):
 *   - MXFP8: every 32 consecutive E4M3 values share one local E8M0 scale, blocks
 *     are one-dimensional; the decoded E8M0 scale is rounded up so the block
 *     maximum is never clipped.  (section "Format background", MXFP8 paragraph)
 *   - Rowwise 1x32 and columnwise 32x1 blocks are numerically different and each
 *     copy is quantized independently from full precision.  (section "Recipe 1:
 *     end-to-end MXFP8 RL", training paragraph)
 *   - NVFP4: E2M1 values, one E4M3 scale per 16 values rounded to the nearest
 *     representable value, plus a coarse FP32 scale; the scope of the FP32 scale
 *     is a recipe choice.  (section "Format background", NVFP4 paragraph)
 *   - Per-token recipe: one FP32 activation scale per token, computed online, and
 *     one call that returns packed FP4, E4M3 block scales and FP32 token scales.
 *     (section "Per-token activation scaling")
 *   - Dequantized backward: BF16 dequantized from the exact low-precision forward
 *     operands.  (section "High-precision and dequantized backward")
 *   - Exact byte-level agreement, fast math disabled.  (section "Bit-exact
 *     quantizer contract")
 *
 * Readings of the pages where they are silent (each one is listed with its reason
 * in the design notes of the repository):
 *   - E4M3 is the OCP E4M3FN variant: bias 7, largest finite 448, codes 0x7F/0xFF
 *     are NaN, no infinity.  E2M1: bias 1, values 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 *   - Encoding to E4M3/E2M1 means: the nearest finite value of the format, ties to
 *     the even code, the sign of the input kept (a negative input that rounds to
 *     zero gives the negative-zero code).
 *   - An all-zero MXFP8 block gets E8M0 code 0.
 *   - The per-token FP32 scale is the decode scale s_t = fl(amax_t / 2688), with
 *     2688 = 6 * 448; the block scale is sb = ENC_E4M3(fl(amax_b / fl(6 * s_t)));
 *     the element multiplier is f = min(fl(1 / fl(DEC(sb) * s_t)), FLT_MAX), or 0
 *     when the decoded scale is zero; the element code is ENC_E2M1(fl(x * f)).
 *   - FP4 packing: element 2j in the low nibble, element 2j+1 in the high nibble.
 *   - Dequantization: MXFP8 y = RNE_BF16(exact DEC(q) * 2^(c-127)); NVFP4
 *     y = RNE_BF16(fl(exact(DEC(q) * DEC(sb)) * s_t)).  A NaN result is written as
 *     the BF16 pattern 0x7FC0.
 *
 * Arithmetic: everything that is exact is done in binary64 (every BF16, E4M3,
 * E2M1 and E8M0 value, and every product the contract states as exact, fits
 * binary64 exactly).  Where the contract rounds to binary32 -- the steps written
 * fl(.) above -- the oracle performs exactly that one C float operation.  The
 * build uses -fno-fast-math -ffp-contract=off and the check below rules out
 * excess precision, so each float operation is one IEEE binary32 operation,
 * rounded to nearest-even, with gradual underflow.
 *
 * Parity unpinned: the readings listed above (the all-zero block code, the sign of zero
 * codes, the nibble order, the direction of the FP32 scale and the binary32 operation
 * order of the NVFP4 scale steps), and the layouts of the grouped, per-group, 16x16-tile
 * and scatter calls, are fixed by this implementation, not by the pages, which print no
 * worked example.  They are checked against a second implementation of the same readings
 * (the exact-rational verifier), against hand-worked fixtures, and against the flat calls
 * and properties they reduce to; nothing on the pages can confirm the choices themselves.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs float operations evaluated in binary32 (FLT_EVAL_METHOD == 0)"
#endif
#if defined(__FAST_MATH__)
#error "the oracle must not be compiled with fast math"
#endif

/* ------------------------------------------------------------------------- */
/* Format tables, built from the bit-field definitions                        */
/* ------------------------------------------------------------------------- */

/* E4M3 (OCP E4M3FN): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * exponent field 0 is subnormal: m/8 * 2^(1-7); code 0x7F (all ones) is NaN. */
static double e4m3_mag[127]; /* magnitude of codes 0x00 .. 0x7E, increasing */
/* E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; field 0 subnormal. */
static double e2m1_mag[8];
static int tables_ready = 0;

static void build_tables(void) {
    if (tables_ready) return;
    for (int c = 0; c < 127; ++c) {
        int e = (c >> 3) & 0xF, m = c & 7;
        e4m3_mag[c] = (e == 0) ? ldexp((double)m / 8.0, 1 - 7)
                               : ldexp(1.0 + (double)m / 8.0, e - 7);
    }
    for (int c = 0; c < 8; ++c) {
        int e = (c >> 1) & 3, m = c & 1;
        e2m1_mag[c] = (e == 0) ? ldexp((double)m / 2.0, 1 - 1)
                               : ldexp(1.0 + (double)m / 2.0, e - 1);
    }
    tables_ready = 1;
}

/* Nearest entry of an increasing magnitude table (codes 0..n-1), ties to the
 * even code, magnitudes above the last entry go to the last entry (the nearest
 * finite value). */
static int nearest_code(const double* mag, int n, double a) {
    if (a >= mag[n - 1]) return n - 1;
    /* largest i with mag[i] <= a (mag[0] == 0 <= a) */
    int lo = 0, hi = n - 1; /* invariant: mag[lo] <= a < mag[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (mag[mid] <= a) lo = mid; else hi = mid;
    }
    double dlo = a - mag[lo], dhi = mag[hi] - a; /* both exact in binary64 here */
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo % 2 == 0) ? lo : hi;
}

double oracle_dec_e4m3(uint8_t code) {
    build_tables();
    if ((code & 0x7F) == 0x7F) return NAN;
    double v = e4m3_mag[code & 0x7F];
    return (code & 0x80) ? -v : v;
}

uint8_t oracle_enc_e4m3(double v) {
    build_tables();
    int c = nearest_code(e4m3_mag, 127, fabs(v));
    return (uint8_t)(c | (signbit(v) ? 0x80 : 0));
}

double oracle_dec_e2m1(uint8_t code) {
    build_tables();
    double v = e2m1_mag[code & 7];
    return (code & 8) ? -v : v;
}

uint8_t oracle_enc_e2m1(double v) {
    build_tables();
    int c = nearest_code(e2m1_mag, 8, fabs(v));
    return (uint8_t)(c | (signbit(v) ? 8 : 0));
}

/* E8M0: an unsigned power of two 2^(c-127); 0xFF is NaN. */
double oracle_dec_e8m0(uint8_t code) {
    if (code == 0xFF) return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* BF16: 1 sign, 8 exponent (bias 127), 7 mantissa bits. */
double oracle_bf16_to_double(uint16_t b) {
    int s = b >> 15, e = (b >> 7) & 0xFF, m = b & 0x7F;
    double v;
    if (e == 0xFF) v = (m == 0) ? INFINITY : NAN;
    else if (e == 0) v = ldexp((double)m, -126 - 7);
    else v = ldexp(128.0 + (double)m, e - 127 - 7);
    return s ? -v : v;
}

/* Round a binary64 value to the nearest BF16 (ties to even significand);
 * magnitudes at or beyond the overflow threshold give infinity; NaN gives 0x7FC0. */
uint16_t oracle_rne_bf16(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t s = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a)) return s | 0x7F80;
    if (a == 0.0) return s;
    int E;
    frexp(a, &E);                    /* a = f * 2^E, f in [0.5, 1) */
    int ex = E - 1;                  /* a in [2^ex, 2^(ex+1)) */
    if (ex < -126) ex = -126;        /* below the normal range the quantum is fixed */
    double quantum = ldexp(1.0, ex - 7);
    double n = a / quantum;          /* exact: division by a power of two */
    double r = floor(n);
    double rem = n - r;
    if (rem > 0.5 || (rem == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    double rv = r * quantum;
    if (rv >= ldexp(1.0, 128)) return s | 0x7F80;
    if (rv == 0.0) return s;
    if (rv < ldexp(1.0, -126)) {     /* subnormal: mantissa counts 2^-133 */
        return s | (uint16_t)(rv / ldexp(1.0, -133));
    }
    int E2;
    frexp(rv, &E2);
    int ex2 = E2 - 1;
    uint16_t mant = (uint16_t)(rv / ldexp(1.0, ex2 - 7) - 128.0);
    return s | (uint16_t)((ex2 + 127) << 7) | mant;
}

/* ------------------------------------------------------------------------- */
/* MXFP8                                                                      */
/* ------------------------------------------------------------------------- */

/* E8M0 code of a block whose largest magnitude is amax: the smallest integer e
 * with amax <= 448 * 2^e (so the block maximum never clips), clamped below at
 * -127, stored as e + 127.  An all-zero block gets code 0. */
uint8_t oracle_e8m0_code(double amax) {
    if (amax == 0.0) return 0;
    int E;
    frexp(amax, &E);
    int e = E - 10;                                    /* 448 * 2^e < amax here */
    while (amax > 448.0 * ldexp(1.0, e)) ++e;          /* smallest e that fits */
    if (e < -127) e = -127;
    return (uint8_t)(e + 127);
}

/* One block of n <= 32 elements (32 except for the partial last block of an expert
 * segment, see the grouped columnwise copy below): values v[0..n-1] (exact BF16
 * values), codes to q[i*qs].  The scale depends only on the largest magnitude. */
static uint8_t mx_block_n(const double* v, int n, uint8_t* q, int64_t qs) {
    double amax = 0.0;
    for (int i = 0; i < n; ++i)
        if (fabs(v[i]) > amax) amax = fabs(v[i]);
    uint8_t c = oracle_e8m0_code(amax);
    double inv_scale = ldexp(1.0, 127 - (int)c);       /* 2^-e, exact */
    for (int i = 0; i < n; ++i)
        q[i * qs] = oracle_enc_e4m3(v[i] * inv_scale);  /* exact product */
    return c;
}

static uint8_t mx_block(const double* v, uint8_t* q, int64_t qs) {
    return mx_block_n(v, 32, q, qs);
}

/* Rowwise MXFP8 of x[rows][cols] (BF16 bits): blocks of 32 along cols.
 * q[rows][cols] E4M3, s[rows][cols/32] E8M0.  cols % 32 == 0. */
void oracle_mx_quantize_rowwise(const uint16_t* x, int64_t rows, int64_t cols,
                                uint8_t* q, uint8_t* s) {
    build_tables();
    const int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double v[32];
        for (int64_t b = 0; b < nb; ++b) {
            for (int i = 0; i < 32; ++i)
                v[i] = oracle_bf16_to_double(x[r * cols + b * 32 + i]);
            s[r * nb + b] = mx_block(v, q + r * cols + b * 32, 1);
        }
    }
}

/* Columnwise MXFP8 of x[M][K]: blocks of 32 consecutive rows of one column,
 * stored transposed: q_col[K][M] E4M3, s_col[K][M/32] E8M0.  M % 32 == 0. */
void oracle_mx_quantize_colwise(const uint16_t* x, int64_t M, int64_t K,
                                uint8_t* q_col, uint8_t* s_col) {
    build_tables();
    const int64_t nb = M / 32;
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k) {
        double v[32];
        for (int64_t b = 0; b < nb; ++b) {
            for (int i = 0; i < 32; ++i)
                v[i] = oracle_bf16_to_double(x[(b * 32 + i) * K + k]);
            s_col[k * nb + b] = mx_block(v, q_col + k * M + b * 32, 1);
        }
    }
}

/* Grouped columnwise MXFP8 for the weight-gradient operand of MoE experts (MXFP8
 * recipe: experts are MXFP8 and the weight-gradient GEMM runs in MXFP8 on the
 * columnwise copy; section "Recipe 1: end-to-end MXFP8 RL").  The rows of x[M][K]
 * are E consecutive expert segments [off[e], off[e+1]); an expert's GEMM reduces
 * over its own rows only, so a 32x1 block never crosses a segment.  Expert e's rows
 * form nb_e = ceil(m_e / 32) blocks of 32 consecutive rows from off[e]; the last one
 * holds the remaining m_e mod 32 rows when m_e is not a multiple of 32, and its scale
 * is taken over the rows present.  Layout: q_col[K][M] as in the flat copy (expert
 * e's copy is entries off[e] .. off[e+1]-1 of every row); s_col[K][s_ld], expert e's
 * blocks at entries blk_e .. blk_e + nb_e - 1 of every row, blk_e = nb_0 + ... +
 * nb_(e-1).  With every m_e a multiple of 32 this is exactly the flat copy.  The
 * offsets must be valid (off[0] = 0, non-decreasing, off[E] = M) and s_ld at least
 * the total block count; the caller checks both. */
void oracle_mx_quantize_colwise_grouped(const uint16_t* x, int64_t M, int64_t K,
                                        const int64_t* off, int64_t E,
                                        uint8_t* q_col, uint8_t* s_col, int64_t s_ld) {
    build_tables();
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k) {
        double v[32];
        int64_t blk = 0;
        for (int64_t e = 0; e < E; ++e) {
            for (int64_t r0 = off[e]; r0 < off[e + 1]; r0 += 32) {
                const int n = (off[e + 1] - r0 < 32) ? (int)(off[e + 1] - r0) : 32;
                for (int i = 0; i < n; ++i)
                    v[i] = oracle_bf16_to_double(x[(r0 + i) * K + k]);
                s_col[k * s_ld + blk] = mx_block_n(v, n, q_col + k * M + r0, 1);
                ++blk;
            }
        }
    }
}

/* MXFP8 dequantization in the stored layout: q[rows][cols], s[rows][cols/32].
 * y = RNE_BF16(DEC_E4M3(q) * 2^(c-127)); the product is exact in binary64. */
void oracle_mx_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols,
                          uint16_t* y) {
    build_tables();
    const int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k) {
            double v = oracle_dec_e4m3(q[r * cols + k]) * oracle_dec_e8m0(s[r * nb + k / 32]);
            y[r * cols + k] = oracle_rne_bf16(v);
        }
}

/* ------------------------------------------------------------------------- */
/* Per-token NVFP4                                                            */
/* ------------------------------------------------------------------------- */

/* The per-token FP32 decode scale of a row whose largest magnitude is amax. */
float oracle_nv_token_scale(float amax) {
    return amax / 2688.0f;                              /* fl(amax / (6 * 448)) */
}

/* The E4M3 block scale of a 16-element block with largest magnitude amax_b. */
uint8_t oracle_nv_block_scale(float amax_b, float s_t) {
    if (s_t == 0.0f) return 0x00;
    float p = 6.0f * s_t;                               /* fl(6 * s_t) */
    float t = amax_b / p;                               /* fl(amax_b / p) */
    return oracle_enc_e4m3((double)t);
}

/* The multiplier applied to each element of a block with scale code sb. */
float oracle_nv_block_multiplier(uint8_t sb, float s_t) {
    float d = (float)oracle_dec_e4m3(sb) * s_t;         /* fl(DEC(sb) * s_t) */
    if (d == 0.0f) return 0.0f;
    float f = 1.0f / d;                                 /* fl(1 / D) */
    return (f > FLT_MAX) ? FLT_MAX : f;
}

/* Largest magnitude of n BF16 values (exact). */
static double bf16_amax(const uint16_t* v, int64_t n) {
    double amax = 0.0;
    for (int64_t k = 0; k < n; ++k) {
        double a = fabs(oracle_bf16_to_double(v[k]));
        if (a > amax) amax = a;
    }
    return amax;
}

/* One row of K elements under the FP32 decode scale s: its K/16 block scales and K/2
 * packed bytes. */
static void nv_row(const uint16_t* xr, int64_t K, float s, uint8_t* qr, uint8_t* sbr) {
    const int64_t nb = K / 16;
    for (int64_t b = 0; b < nb; ++b) {
        double amax_b = bf16_amax(xr + b * 16, 16);
        uint8_t code_b = oracle_nv_block_scale((float)amax_b, s);
        sbr[b] = code_b;
        float f = oracle_nv_block_multiplier(code_b, s);
        for (int i = 0; i < 16; i += 2) {
            float x0 = (float)oracle_bf16_to_double(xr[b * 16 + i]);
            float x1 = (float)oracle_bf16_to_double(xr[b * 16 + i + 1]);
            uint8_t c0 = oracle_enc_e2m1((double)(x0 * f));  /* fl(x * f) */
            uint8_t c1 = oracle_enc_e2m1((double)(x1 * f));
            qr[(b * 16 + i) / 2] = (uint8_t)(c0 | (c1 << 4));
        }
    }
}

/* Per-token NVFP4 of x[R][K] (BF16 bits), K % 16 == 0.
 * q[R][K/2] packed E2M1 (element 2j low nibble), sb[R][K/16] E4M3, st[R] FP32. */
void oracle_nv_quantize_per_token(const uint16_t* x, int64_t R, int64_t K,
                                  uint8_t* q, uint8_t* sb, float* st) {
    build_tables();
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        const uint16_t* xr = x + r * K;
        float s_t = oracle_nv_token_scale((float)bf16_amax(xr, K));   /* BF16 -> float exact */
        st[r] = s_t;
        nv_row(xr, K, s_t, q + r * (K / 2), sb + r * (K / 16));
    }
}

/* Standard NVFP4 with one FP32 scale per group of rows: the two-level hierarchy with the
 * coarse FP32 scale taken over a tensor instead of a token ("Format background": the
 * scope of the FP32 scale is a recipe choice).  Groups are row ranges [off[g], off[g+1])
 * -- a whole tensor, or an expert's tensor; an expert's gate and up projections go in one
 * group so that both get the same scale ("Per-token activation scaling": gate and up
 * share one FP32 scale in conversion and weight export).  The scale of group g is
 * s_g = fl(amax_g / 2688) over all its elements (0 for an empty or all-zero group), and
 * each of its rows is then encoded exactly as a per-token row with s_t = s_g.
 * Offsets must be valid (off[0] = 0, non-decreasing, off[G] = R); the caller checks. */
void oracle_nv_quantize_per_group(const uint16_t* x, int64_t R, int64_t K,
                                  const int64_t* off, int64_t G,
                                  uint8_t* q, uint8_t* sb, float* s_group) {
    build_tables();
    (void)R;
    for (int64_t g = 0; g < G; ++g) {
        double amax = 0.0;
        for (int64_t r = off[g]; r < off[g + 1]; ++r) {
            double a = bf16_amax(x + r * K, K);
            if (a > amax) amax = a;
        }
        s_group[g] = oracle_nv_token_scale((float)amax);
    }
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t r = 0; r < off[G]; ++r) {
        int64_t g = 0;
        while (off[g + 1] <= r) ++g;                   /* the group of row r */
        nv_row(x + r * K, K, s_group[g], q + r * (K / 2), sb + r * (K / 16));
    }
}

/* NVFP4 with 16x16 weight blocks (two-dimensional block scaling of the weights, one of the
 * four parts of NVIDIA's NVFP4 pretraining recipe: page "NVIDIA verified the 4-bit NVFP4
 * format on a Mamba-Transformer (12B) at 10 trillion tokens"; Miles turns it off, "Towards
 * Blackwell-native 8-bit and 4-bit RL", section "Try the NVFP4 recipe in Miles"): every 16x16 tile of a
 * weight shares one E4M3 scale, under the FP32 scale of its row group (as in
 * oracle_nv_quantize_per_group), so the same codes and scales serve the weight and its
 * transpose.  Reading: the per-token steps with the tile in place of the 1x16 block:
 *   s_g = fl(amax_g / 2688);  sb = ENC_E4M3(fl(amax_tile / fl(6 s_g)));
 *   f = min(fl(1 / fl(DEC(sb) s_g)), FLT_MAX) (0 if that product is 0);  q = ENC_E2M1(fl(x f)).
 * x[R][K], R % 16 == 0, K % 16 == 0, every group a whole number of 16-row tiles (the
 * caller checks).  q[R][K/2] packed as usual, sb[R/16][K/16], s_group[G]. */
void oracle_nv_quantize_2d(const uint16_t* x, int64_t R, int64_t K, const int64_t* off, int64_t G,
                           uint8_t* q, uint8_t* sb, float* s_group) {
    build_tables();
    (void)R;
    for (int64_t g = 0; g < G; ++g) {
        double amax = 0.0;
        for (int64_t r = off[g]; r < off[g + 1]; ++r) {
            double a = bf16_amax(x + r * K, K);
            if (a > amax) amax = a;
        }
        s_group[g] = oracle_nv_token_scale((float)amax);
    }
    const int64_t tiles_r = off[G] / 16, tiles_c = K / 16;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t tr = 0; tr < tiles_r; ++tr) {
        int64_t g = 0;
        while (off[g + 1] <= tr * 16) ++g;                /* the group of the tile's rows */
        const float s = s_group[g];
        for (int64_t tc = 0; tc < tiles_c; ++tc) {
            double amax_t = 0.0;
            for (int i = 0; i < 16; ++i) {
                double a = bf16_amax(x + (tr * 16 + i) * K + tc * 16, 16);
                if (a > amax_t) amax_t = a;
            }
            uint8_t code = oracle_nv_block_scale((float)amax_t, s);
            sb[tr * tiles_c + tc] = code;
            float f = oracle_nv_block_multiplier(code, s);
            for (int i = 0; i < 16; ++i) {
                const uint16_t* xr = x + (tr * 16 + i) * K + tc * 16;
                for (int j = 0; j < 16; j += 2) {
                    float x0 = (float)oracle_bf16_to_double(xr[j]);
                    float x1 = (float)oracle_bf16_to_double(xr[j + 1]);
                    uint8_t c0 = oracle_enc_e2m1((double)(x0 * f));
                    uint8_t c1 = oracle_enc_e2m1((double)(x1 * f));
                    q[(tr * 16 + i) * (K / 2) + (tc * 16 + j) / 2] = (uint8_t)(c0 | (c1 << 4));
                }
            }
        }
    }
}

/* Dequantization of the 16x16-tile layout: y = RNE_BF16(fl(exact(DEC_E2M1(q) *
 * DEC_E4M3(sb[r/16][c/16])) * s_g)) with s_g the scale of row r's group. */
void oracle_nv_dequantize_2d(const uint8_t* q, const uint8_t* sb, const float* s_group,
                             const int64_t* off, int64_t G, int64_t R, int64_t K, uint16_t* y) {
    build_tables();
    (void)G;
    const int64_t tiles_c = K / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        int64_t g = 0;
        while (off[g + 1] <= r) ++g;
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = q[r * (K / 2) + k / 2];
            uint8_t code = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
            uint8_t bs = sb[(r / 16) * tiles_c + k / 16];
            double e = oracle_dec_e2m1(code) * oracle_dec_e4m3(bs);   /* exact */
            y[r * K + k] = oracle_rne_bf16((double)((float)e * s_group[g]));
        }
    }
}

/* NVFP4 dequantization: y = RNE_BF16(fl(exact(DEC_E2M1(q) * DEC_E4M3(sb)) * s_t)). */
void oracle_nv_dequantize(const uint8_t* q, const uint8_t* sb, const float* st,
                          int64_t R, int64_t K, uint16_t* y) {
    build_tables();
    const int64_t nb = K / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = q[r * (K / 2) + k / 2];
            uint8_t code = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
            double inner = oracle_dec_e2m1(code) * oracle_dec_e4m3(sb[r * nb + k / 16]);
            float prod = (float)inner * st[r];          /* inner is exact in float */
            y[r * K + k] = oracle_rne_bf16((double)prod);
        }
}

/* ------------------------------------------------------------------------- */
/* Vector helpers for the tests (element-wise maps over arrays).              */
/* ------------------------------------------------------------------------- */

void oracle_enc_e4m3_array(const double* v, int64_t n, uint8_t* out) {
    build_tables();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_enc_e4m3(v[i]);
}

void oracle_enc_e2m1_array(const double* v, int64_t n, uint8_t* out) {
    build_tables();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_enc_e2m1(v[i]);
}

void oracle_rne_bf16_array(const double* v, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_rne_bf16(v[i]);
}

/* The encoders applied to every binary32 bit pattern start, start+1, ..., start+n-1 (for
 * exhaustive sweeps of a conversion over all 2^32 inputs, in chunks).  Inputs that are
 * NaN get the output 0 (E2M1) / 0x7FC0 (BF16) and are skipped by the sweeps. */
static double f32_from_bits(uint32_t b) {
    float f;
    memcpy(&f, &b, sizeof f);
    return (double)f;
}

void oracle_enc_e2m1_f32_range(uint32_t start, int64_t n, uint8_t* out) {
    build_tables();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double v = f32_from_bits(start + (uint32_t)i);
        out[i] = isnan(v) ? 0 : oracle_enc_e2m1(v);
    }
}

void oracle_rne_bf16_f32_range(uint32_t start, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_rne_bf16(f32_from_bits(start + (uint32_t)i));
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the parallel loops above (timing only; the results do not depend on it). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
