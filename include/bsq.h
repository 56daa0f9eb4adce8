/*
 * bsq.h -- C ABI of the block-scaled quantizer library (libbsq.so) for AMD MI355X (gfx950).
 *
 * One definition of the MXFP8 and per-token NVFP4 bytes, with their BF16 dequantization,
 * so that every producer and consumer of these tensors (training, rollout, checkpoint
 * conversion, live weight export) can share it byte for byte.
 *
 * The passages cited below are sections of the page "Towards Blackwell-native 8-bit and
 * 4-bit RL" (end-to-end MXFP8 and per-token NVFP4 RL in Miles).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers (HIP device memory of the current device),
 *    owned by the caller.  The library never allocates, frees or synchronises, keeps no
 *    global state, and is safe to call from several host threads at once.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work is
 *    enqueued on it and the call returns at once.
 *  - BF16 tensors are contiguous row-major arrays of 16-bit patterns.  Inputs are finite;
 *    NaN or infinite inputs are outside the contract (no crash, output unspecified).
 *  - Element formats: E4M3 is OCP E4M3FN (bias 7, largest finite 448, 0x7F/0xFF NaN);
 *    E8M0 code c is 2^(c-127) (0xFF NaN); E2M1 codes are 0, 0.5, 1, 1.5, 2, 3, 4, 6 with
 *    a sign bit, packed two per byte, element 2j in the low nibble of byte j.
 *  - Rounding to E4M3/E2M1 is "nearest finite value, ties to the even code, sign kept";
 *    FP32 steps are single IEEE binary32 operations rounded to nearest-even, with
 *    denormals, no fused multiply-add and no approximate division.
 *  - Argument errors are detected on the host before anything is launched and are
 *    returned synchronously; outputs are then untouched:
 *      BSQ_ERR_NULL    a required pointer is NULL (or a pointer the mode needs is missing)
 *      BSQ_ERR_SHAPE   a size is negative, violates the divisibility rule of the call, or
 *                      is too large for one kernel launch (a launch holds fewer than 2^32
 *                      threads: e.g. per-token NVFP4 takes 32 threads per row up to K = 768
 *                      and 64 above, MXFP8 dequant one per 16 elements; the dequantizers
 *                      need K <= 2^34, the 16x16-tile one K <= 2^30)
 *      BSQ_ERR_ALIGN   a tensor pointer is not 16-byte aligned
 *      BSQ_ERR_MODE    unknown mode
 *      BSQ_ERR_ALIAS   two of the call's buffers overlap
 *    Sizes of zero are valid and launch nothing.  A failed launch returns BSQ_ERR_HIP.
 */
#ifndef BSQ_H
#define BSQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSQ_ABI_VERSION 1

enum bsq_status {
    BSQ_OK = 0,
    BSQ_ERR_NULL = 1,
    BSQ_ERR_SHAPE = 2,
    BSQ_ERR_ALIGN = 3,
    BSQ_ERR_MODE = 4,
    BSQ_ERR_ALIAS = 5,
    BSQ_ERR_OFFSETS = 6,
    BSQ_ERR_HIP = 7
};

enum bsq_mx_mode { MX_ROWWISE = 1, MX_COLWISE = 2, MX_BOTH = 3 };

/*
 * MXFP8 quantization of x[M][K] (BF16).
 * Passages: "Format background" (32 consecutive E4M3 values share one E8M0 scale, blocks
 * are one-dimensional, the decoded scale is rounded up so the block maximum never clips)
 * and "Recipe 1: end-to-end MXFP8 RL" (rowwise 1x32 and columnwise 32x1 blocks are
 * numerically different; both copies are quantized independently from full precision).
 *
 * For each block: amax = max |x_i|; the E8M0 code c is e + 127 for the smallest integer
 * e >= -127 with amax <= 448 * 2^e (c = 0 for an all-zero block); q_i = ENC_E4M3(x_i*2^-e)
 * (the product is exact and never exceeds 448).
 *
 * mode MX_ROWWISE: blocks of 32 along K.  Needs K % 32 == 0.
 *   q_row u8 [M][K] E4M3,   s_row u8 [M][K/32] E8M0.
 * mode MX_COLWISE: blocks of 32 consecutive rows of one column, stored transposed so each
 *   block is contiguous.  Needs M % 32 == 0, and K % 8 == 0 (rows of x are whole 16-byte
 *   pieces; the blocks themselves put no condition on K).
 *   q_col u8 [K][M] E4M3,   s_col u8 [K][M/32] E8M0.
 * mode MX_BOTH: both copies from one read of x (M % 32 == 0 and K % 32 == 0).
 * Pointers of the copy a mode does not produce are ignored and may be NULL.
 */
int mx_quantize_mxfp8(const void* x_bf16, int64_t M, int64_t K, int mode,
                      void* q_row, void* s_row, void* q_col, void* s_col, void* stream);

/*
 * Per-token NVFP4 quantization of x[R][K] (BF16), one call producing all three outputs.
 * Passages: "Format background" (E2M1 values, one E4M3 scale per 16 values rounded to the
 * nearest representable value, a coarse FP32 scale on top whose scope is a recipe choice)
 * and "Per-token activation scaling" (one FP32 scale per token computed online; the call
 * that emits packed FP4 and E4M3 block scales also returns the per-token FP32 scales).
 *
 * Per row: s_t = fl(amax_row / 2688)  (2688 = 6 * 448).
 * Per 16-element block: sb = ENC_E4M3(fl(amax_b / fl(6 * s_t))), or 0 when s_t == 0;
 *   D = fl(DEC_E4M3(sb) * s_t); f = 0 if D == 0 else min(fl(1 / D), FLT_MAX);
 *   q_i = ENC_E2M1(fl(x_i * f)).
 * Needs K % 16 == 0.
 *   q  u8 [R][K/2] packed E2M1,  sb u8 [R][K/16] E4M3,  st f32 [R] (the s_t values).
 * A row's bytes depend on that row only.
 */
int nv_quantize_nvfp4_per_token(const void* x_bf16, int64_t R, int64_t K,
                                void* q, void* sb, float* st, void* stream);

/*
 * Per-token NVFP4 of rows grouped by expert: rows [offsets[e], offsets[e+1]) belong to
 * expert e.  Since per-token scaling is row-local the bytes are exactly those of
 * nv_quantize_nvfp4_per_token on the same R rows (empty experts allowed).
 * expert_offsets: DEVICE int64 [E+1], E >= 1.  They are checked on the device
 * (offsets[0] == 0, non-decreasing, offsets[E] == R) without any host synchronisation:
 * if status_dev is not NULL the kernel writes BSQ_OK or BSQ_ERR_OFFSETS to *status_dev
 * (a device int32).  All R rows are quantized either way.
 */
int nv_quantize_nvfp4_per_token_grouped(const void* x_bf16, int64_t R, int64_t K,
                                        const int64_t* expert_offsets, int64_t E,
                                        void* q, void* sb, float* st,
                                        int32_t* status_dev, void* stream);

/*
 * MXFP8 quantization of x[M][K] (BF16) whose rows are grouped by expert, for the MoE
 * weight-gradient operand: rows [offsets[e], offsets[e+1]) belong to expert e.
 * Passages: "Recipe 1: end-to-end MXFP8 RL" (MoE experts run in MXFP8, the weight-gradient
 * GEMM included, on the columnwise copy quantized from full precision) and "Format
 * background" (32-value blocks, E8M0 scale rounded up).  An expert's GEMM reduces over
 * its own rows only, so a 32x1 block never crosses an expert boundary: expert e's
 * m_e = offsets[e+1] - offsets[e] rows form ceil(m_e / 32) blocks of 32 consecutive rows
 * starting at offsets[e]; when m_e % 32 != 0 the last one is partial and its scale is
 * taken over the rows present.  Scale and code rules are those of mx_quantize_mxfp8.
 * Blocks are numbered n = 0, 1, ... in row order over all experts.
 *
 * mode MX_COLWISE or MX_BOTH (MX_ROWWISE is plain mx_quantize_mxfp8: rowwise blocks never
 * cross rows, so grouping does not change them).  Needs K % 32 == 0; M may be any size.
 *   q_col u8 [K][M] E4M3, the flat columnwise layout (expert e's copy is entries
 *         offsets[e] .. offsets[e+1]-1 of every row);
 *   s_col u8 [K][s_ld] E8M0, block n at entry n of every row (expert e's blocks follow
 *         those of experts 0 .. e-1); entries past the last block are not written;
 *   q_row, s_row (MX_BOTH only): exactly as mx_quantize_mxfp8's rowwise copy.
 * With every m_e a multiple of 32 and s_ld = M/32 the bytes equal mx_quantize_mxfp8's.
 * s_ld >= ceil(M/32) (the fewest blocks any offsets give); (M + 31 E) / 32 is enough for
 * any offsets; ceil(M/32) + E < 2^31.
 * expert_offsets: DEVICE int64 [E+1], E >= 1, checked on the device without any host
 * synchronisation: if status_dev is not NULL the kernel writes BSQ_ERR_OFFSETS to
 * *status_dev when offsets[0] != 0, offsets[E] != M, the offsets decrease, or the blocks
 * need more than s_ld scale entries, and BSQ_OK otherwise.  With invalid offsets the
 * output bytes are unspecified, but nothing outside the given buffers is written.
 */
int mx_quantize_mxfp8_grouped(const void* x_bf16, int64_t M, int64_t K, int mode,
                              const int64_t* expert_offsets, int64_t E,
                              void* q_row, void* s_row, void* q_col, void* s_col, int64_t s_ld,
                              int32_t* status_dev, void* stream);

/*
 * Per-token NVFP4 of routed rows without gathering them: quantize-then-scatter.
 * Passage: "Per-token activation scaling" (a token's bytes depend on that token only).
 * The routed rows are X[dst[t][j]] = H[t] for every token t < T and choice j < top_k (a
 * token is routed to top_k experts); this call quantizes each token row of H[T][K] once and
 * writes its q / sb / st to each of its routed rows, so the outputs are exactly those of
 * nv_quantize_nvfp4_per_token on X (N rows) while H is read once instead of X.
 * dst_rows: DEVICE int64 [T][top_k], the routed row of each (token, choice); a negative
 * entry is a dropped choice; entries must be distinct.  Rows of X that no entry names are
 * not written.  Needs K % 16 == 0.  Outputs as nv_quantize_nvfp4_per_token on N rows:
 *   q u8 [N][K/2],  sb u8 [N][K/16],  st f32 [N].
 * If status_dev is not NULL the kernel writes BSQ_ERR_OFFSETS to *status_dev when an entry
 * is >= N (it is skipped) and BSQ_OK otherwise.
 */
int nv_quantize_nvfp4_per_token_scatter(const void* h_bf16, int64_t T, int64_t K,
                                        const int64_t* dst_rows, int64_t top_k, int64_t N,
                                        void* q, void* sb, float* st,
                                        int32_t* status_dev, void* stream);

/*
 * Standard NVFP4 of x[R][K] (BF16) with one FP32 scale per group of rows: rows
 * [offsets[g], offsets[g+1]) form group g (a whole tensor, or one expert's tensor; an
 * expert's gate and up projections belong in one group).
 * Passages: "Format background" (the coarse FP32 scale maps a tensor or a token into the
 * NVFP4 range; its scope is a recipe choice) and "Per-token activation scaling" (gate and
 * up share one FP32 scale in conversion and live weight export).
 * Per group: s_g = fl(amax_g / 2688) over all its elements (0 for an empty group); every
 * row of the group is then encoded with the per-token steps under s_t = s_g.
 * Needs K % 16 == 0.  Outputs:  q u8 [R][K/2],  sb u8 [R][K/16] (as per-token), and
 * s_group f32 [G] (DEVICE).  The group maximum needs the whole group before any element
 * can be encoded, so x is read twice (two passes); s_group also holds the group maxima
 * between the passes (four launches on `stream`).
 * group_offsets: DEVICE int64 [G+1], G >= 1, checked on the device: if status_dev is not
 * NULL the kernel writes BSQ_ERR_OFFSETS when offsets[0] != 0, offsets[G] != R or the
 * offsets decrease, BSQ_OK otherwise.  With invalid offsets the output bytes are
 * unspecified, but nothing outside the given buffers is written.
 */
int nv_quantize_nvfp4_per_group(const void* x_bf16, int64_t R, int64_t K,
                                const int64_t* group_offsets, int64_t G,
                                void* q, void* sb, float* s_group,
                                int32_t* status_dev, void* stream);

/*
 * BF16 [R][K] from NVFP4 with one FP32 scale per group of rows (the output of
 * nv_quantize_nvfp4_per_group): y = RNE_BF16(fl(exact(DEC_E2M1(q) * DEC_E4M3(sb)) * s_g))
 * for the group g of the row; a NaN result is 0x7FC0.  Passage: "High-precision and
 * dequantized backward".  Needs K % 16 == 0; s_group and group_offsets are DEVICE arrays
 * [G] and [G+1] (valid offsets assumed).
 */
int nv_dequantize_per_group(const void* q, const void* sb, const float* s_group,
                            const int64_t* group_offsets, int64_t G, int64_t R, int64_t K,
                            void* y_bf16, void* stream);

/*
 * NVFP4 with 16x16 weight tiles (two-dimensional block scaling) under one FP32 scale per
 * group of rows.  Passages: page "NVIDIA verified the 4-bit NVFP4 format on a
 * Mamba-Transformer (12B) at 10 trillion tokens" (two-dimensional block scaling of the
 * weights is one of the four parts of NVIDIA's pretraining recipe) and "Towards
 * Blackwell-native 8-bit and 4-bit RL", section "Try the NVFP4 recipe in Miles" (Miles
 * turns it off).  Square tiles make the codes and scales of the transposed weight the
 * transposes of these, so one copy serves both GEMM orientations.
 * Per group (as nv_quantize_nvfp4_per_group): s_g = fl(amax_g / 2688).  Per 16x16 tile:
 *   sb = ENC_E4M3(fl(amax_tile / fl(6 s_g))); D = fl(DEC(sb) s_g);
 *   f = 0 if D == 0 else min(fl(1/D), FLT_MAX);  q = ENC_E2M1(fl(x f)).
 * Needs R % 16 == 0 and K % 16 == 0.  Outputs: q u8 [R][K/2] (packed as usual),
 * sb u8 [R/16][K/16] (one byte per tile), s_group f32 [G] (DEVICE; it also holds the group
 * maxima between the two passes).  group_offsets: DEVICE int64 [G+1], every one a multiple
 * of 16, checked on the device into *status_dev (BSQ_ERR_OFFSETS / BSQ_OK) when it is not
 * NULL; with invalid offsets the bytes are unspecified but stay inside the buffers.
 */
int nv_quantize_nvfp4_2d(const void* x_bf16, int64_t R, int64_t K,
                         const int64_t* group_offsets, int64_t G,
                         void* q, void* sb, float* s_group,
                         int32_t* status_dev, void* stream);

/*
 * BF16 [R][K] from the 16x16-tile layout of nv_quantize_nvfp4_2d:
 * y = RNE_BF16(fl(exact(DEC_E2M1(q) * DEC_E4M3(sb[r/16][c/16])) * s_g)); NaN -> 0x7FC0.
 * Passage: "High-precision and dequantized backward".  Needs R % 16 == 0, K % 16 == 0.
 */
int nv_dequantize_2d(const void* q, const void* sb, const float* s_group,
                     const int64_t* group_offsets, int64_t G, int64_t R, int64_t K,
                     void* y_bf16, void* stream);

/*
 * MXFP8 dequantization to BF16, in the stored layout: q u8 [rows][cols] E4M3 and
 * s u8 [rows][cols/32] E8M0 (blocks of 32 along the stored last dimension).
 * Passage: "High-precision and dequantized backward" (backward GEMMs consume BF16
 * dequantized from the exact low-precision forward operands).
 * y = RNE_BF16(DEC_E4M3(q) * 2^(c-127)) (the product is exact; overflow gives +-inf).
 * A NaN result (q in {0x7F, 0xFF} or c == 0xFF) is written as 0x7FC0.
 * The columnwise copy is passed as (q_col, s_col, rows = K, cols = M) and gives [K][M].
 * Needs cols % 32 == 0.
 */
int mx_dequantize(const void* q, const void* s, int64_t rows, int64_t cols,
                  void* y_bf16, void* stream);

/*
 * Per-token NVFP4 dequantization to BF16 [R][K].
 * Passage: "High-precision and dequantized backward".
 * y = RNE_BF16(fl(exact(DEC_E2M1(q) * DEC_E4M3(sb)) * s_t)); a NaN result is 0x7FC0.
 * Needs K % 16 == 0.  st is a DEVICE float array [R].
 */
int nv_dequantize(const void* q, const void* sb, const float* st, int64_t R, int64_t K,
                  void* y_bf16, void* stream);

/* Static description of a status code (never NULL). */
const char* bsq_status_string(int status);

/* BSQ_ABI_VERSION of the library that was loaded. */
int bsq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSQ_H */
