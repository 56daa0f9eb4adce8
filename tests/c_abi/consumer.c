/*
 * consumer.c -- a plain C program that uses libbsq.so through include/bsq.h and the HIP
 * runtime's C API only (no Python, no C++): it quantizes a seeded BF16 tensor to MXFP8
 * (both copies) and per-token NVFP4, dequantizes all of it, and compares every byte with
 * the CPU oracle (liboracle.so, test infrastructure).  It also checks that argument errors
 * come back synchronously and leave the outputs untouched.  Exit status 0 when all agree.
 *
 * Usage: consumer [M K]   (M % 32 == 0, K % 32 == 0)
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bsq.h"

/* the oracle's entry points */
void oracle_mx_quantize_rowwise(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s);
void oracle_mx_quantize_colwise(const uint16_t* x, int64_t M, int64_t K, uint8_t* q_col, uint8_t* s_col);
void oracle_mx_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols, uint16_t* y);
void oracle_nv_quantize_per_token(const uint16_t* x, int64_t R, int64_t K, uint8_t* q, uint8_t* sb, float* st);
void oracle_nv_dequantize(const uint8_t* q, const uint8_t* sb, const float* st, int64_t R, int64_t K, uint16_t* y);

#define HIP_OK(call)                                                                      \
    do {                                                                                  \
        hipError_t e_ = (call);                                                           \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                   \
            exit(2);                                                                      \
        }                                                                                 \
    } while (0)

static int failures = 0;

static void expect_status(const char* what, int got, int want) {
    if (got != want) {
        fprintf(stderr, "%s: status %d (%s), expected %d (%s)\n", what, got, bsq_status_string(got), want,
                bsq_status_string(want));
        ++failures;
    }
}

static void compare(const char* what, const void* gpu_dev, const void* cpu, size_t n) {
    unsigned char* h = (unsigned char*)malloc(n);
    HIP_OK(hipMemcpy(h, gpu_dev, n, hipMemcpyDeviceToHost));
    size_t bad = 0, first = 0;
    for (size_t i = 0; i < n; ++i)
        if (h[i] != ((const unsigned char*)cpu)[i] && bad++ == 0) first = i;
    if (bad) {
        fprintf(stderr, "%s: %zu of %zu bytes differ (first at byte %zu)\n", what, bad, n, first);
        ++failures;
    } else {
        printf("%-24s %10zu bytes equal\n", what, n);
    }
    free(h);
}

/* A finite BF16 value: N(0,1)-ish magnitudes spread over 2^-20 .. 2^12 from a fixed LCG. */
static uint16_t next_bf16(uint64_t* st) {
    *st = *st * 6364136223846793005ull + 1442695040888963407ull;
    const uint32_t r = (uint32_t)(*st >> 33);
    const uint32_t sign = (r & 1u) << 15, exp = 107u + (r >> 1) % 33u, man = (r >> 7) & 0x7Fu;
    return (uint16_t)(sign | (exp << 7) | man);
}

int main(int argc, char** argv) {
    const int64_t M = argc > 2 ? atoll(argv[1]) : 256, K = argc > 2 ? atoll(argv[2]) : 2048;
    const int64_t n = M * K;
    printf("libbsq ABI version %d, tensor %lld x %lld\n", bsq_abi_version(), (long long)M, (long long)K);
    if (bsq_abi_version() != BSQ_ABI_VERSION) { fprintf(stderr, "ABI version mismatch\n"); return 1; }

    uint16_t* x = (uint16_t*)malloc(2 * n);
    uint64_t seed = 20240611ull;
    for (int64_t i = 0; i < n; ++i) x[i] = next_bf16(&seed);
    for (int64_t j = 0; j < 32; ++j) x[5 * K + 64 + j] = 0;          /* one all-zero block */

    /* device buffers */
    void *dx, *dqr, *dsr, *dqc, *dsc, *dq4, *dsb, *dst, *dyr, *dyc, *dy4;
    HIP_OK(hipMalloc(&dx, 2 * n));
    HIP_OK(hipMalloc(&dqr, n));
    HIP_OK(hipMalloc(&dsr, n / 32));
    HIP_OK(hipMalloc(&dqc, n));
    HIP_OK(hipMalloc(&dsc, n / 32));
    HIP_OK(hipMalloc(&dq4, n / 2));
    HIP_OK(hipMalloc(&dsb, n / 16));
    HIP_OK(hipMalloc(&dst, 4 * M));
    HIP_OK(hipMalloc(&dyr, 2 * n));
    HIP_OK(hipMalloc(&dyc, 2 * n));
    HIP_OK(hipMalloc(&dy4, 2 * n));
    HIP_OK(hipMemcpy(dx, x, 2 * n, hipMemcpyHostToDevice));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    /* the path */
    expect_status("mx_quantize_mxfp8", mx_quantize_mxfp8(dx, M, K, MX_BOTH, dqr, dsr, dqc, dsc, stream), BSQ_OK);
    expect_status("nv_quantize_nvfp4_per_token",
                  nv_quantize_nvfp4_per_token(dx, M, K, dq4, dsb, (float*)dst, stream), BSQ_OK);
    expect_status("mx_dequantize rowwise", mx_dequantize(dqr, dsr, M, K, dyr, stream), BSQ_OK);
    expect_status("mx_dequantize colwise", mx_dequantize(dqc, dsc, K, M, dyc, stream), BSQ_OK);
    expect_status("nv_dequantize", nv_dequantize(dq4, dsb, (const float*)dst, M, K, dy4, stream), BSQ_OK);
    HIP_OK(hipStreamSynchronize(stream));

    /* the oracle */
    uint8_t *qr = malloc(n), *sr = malloc(n / 32), *qc = malloc(n), *sc = malloc(n / 32);
    uint8_t *q4 = malloc(n / 2), *sb = malloc(n / 16);
    float* st = malloc(4 * M);
    uint16_t *yr = malloc(2 * n), *yc = malloc(2 * n), *y4 = malloc(2 * n);
    oracle_mx_quantize_rowwise(x, M, K, qr, sr);
    oracle_mx_quantize_colwise(x, M, K, qc, sc);
    oracle_mx_dequantize(qr, sr, M, K, yr);
    oracle_mx_dequantize(qc, sc, K, M, yc);
    oracle_nv_quantize_per_token(x, M, K, q4, sb, st);
    oracle_nv_dequantize(q4, sb, st, M, K, y4);
    compare("MXFP8 q_row", dqr, qr, n);
    compare("MXFP8 s_row", dsr, sr, n / 32);
    compare("MXFP8 q_col", dqc, qc, n);
    compare("MXFP8 s_col", dsc, sc, n / 32);
    compare("MXFP8 dequant rowwise", dyr, yr, 2 * n);
    compare("MXFP8 dequant colwise", dyc, yc, 2 * n);
    compare("NVFP4 q", dq4, q4, n / 2);
    compare("NVFP4 sb", dsb, sb, n / 16);
    compare("NVFP4 st", dst, st, 4 * M);
    compare("NVFP4 dequant", dy4, y4, 2 * n);

    /* argument errors: returned at once, outputs untouched */
    HIP_OK(hipMemset(dqr, 0x5A, n));
    HIP_OK(hipDeviceSynchronize());
    expect_status("misaligned input", mx_quantize_mxfp8((char*)dx + 2, M, K, MX_ROWWISE, dqr, dsr, NULL, NULL, stream),
                  BSQ_ERR_ALIGN);
    expect_status("missing output", mx_quantize_mxfp8(dx, M, K, MX_BOTH, dqr, dsr, NULL, dsc, stream), BSQ_ERR_NULL);
    expect_status("K not a multiple of 32", mx_quantize_mxfp8(dx, M, K - 16, MX_ROWWISE, dqr, dsr, NULL, NULL, stream),
                  BSQ_ERR_SHAPE);
    expect_status("unknown mode", mx_quantize_mxfp8(dx, M, K, 7, dqr, dsr, dqc, dsc, stream), BSQ_ERR_MODE);
    expect_status("output overlaps input", mx_quantize_mxfp8(dx, M, K, MX_ROWWISE, dx, dsr, NULL, NULL, stream),
                  BSQ_ERR_ALIAS);
    expect_status("zero rows", nv_quantize_nvfp4_per_token(dx, 0, K, dq4, dsb, (float*)dst, stream), BSQ_OK);
    HIP_OK(hipStreamSynchronize(stream));
    memset(qr, 0x5A, n);
    compare("untouched after errors", dqr, qr, n);

    HIP_OK(hipStreamDestroy(stream));
    void* bufs[] = {dx, dqr, dsr, dqc, dsc, dq4, dsb, dst, dyr, dyc, dy4};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIP_OK(hipFree(bufs[i]));
    free(x); free(qr); free(sr); free(qc); free(sc); free(q4); free(sb); free(st); free(yr); free(yc); free(y4);
    printf(failures ? "FAILED (%d)\n" : "all equal\n", failures);
    return failures ? 1 : 0;
}
