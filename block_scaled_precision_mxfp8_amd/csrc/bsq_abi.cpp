// bsq_abi.cpp -- the extern "C" entry points of libbsq.so (declared in include/bsq.h).
//
// Every argument is validated on the host, before any HIP call, so that argument errors
// come back synchronously with the outputs untouched and the library can be loaded and
// exercised on a machine without a GPU.  Valid calls enqueue one kernel on the caller's
// stream and return; nothing is allocated or synchronised here.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsq.h"

namespace bsq {
hipError_t launch_mx_quant(const void* x, int64_t M, int64_t K, int mode, void* q_row,
                           void* s_row, void* q_col, void* s_col, hipStream_t stream);
hipError_t launch_mx_quant_grouped(const void* x, int64_t M, int64_t K, int mode, const int64_t* off,
                                   int64_t E, void* q_row, void* s_row, void* q_col, void* s_col,
                                   int64_t s_ld, int32_t* status, hipStream_t stream);
hipError_t launch_mx_dequant(const void* q, const void* s, int64_t rows, int64_t cols, void* y,
                             hipStream_t stream);
hipError_t launch_nv_quant(const void* x, int64_t R, int64_t K, void* q, void* sb, float* st,
                           const int64_t* offsets, int64_t E, int32_t* status,
                           hipStream_t stream);
hipError_t launch_nv_dequant(const void* q, const void* sb, const float* st, int64_t R,
                             int64_t K, void* y, hipStream_t stream);
hipError_t launch_nv_quant_group(const void* x, int64_t R, int64_t K, const int64_t* off, int64_t G,
                                 void* q, void* sb, float* s_group, int32_t* status, hipStream_t stream);
hipError_t launch_nv_dequant_group(const void* q, const void* sb, const float* s_group, const int64_t* off,
                                   int64_t G, int64_t R, int64_t K, void* y, hipStream_t stream);
hipError_t launch_nv_quant_scatter(const void* h, int64_t T, int64_t K, const int64_t* dst, int64_t top_k,
                                   int64_t N, void* q, void* sb, float* st, int32_t* status,
                                   hipStream_t stream);
hipError_t launch_nv_quant_2d(const void* x, int64_t R, int64_t K, const int64_t* off, int64_t G,
                              void* q, void* sb, float* s_group, int32_t* status, hipStream_t stream);
hipError_t launch_nv_dequant_2d(const void* q, const void* sb, const float* s_group, const int64_t* off,
                                int64_t G, int64_t R, int64_t K, void* y, hipStream_t stream);
// Whether each launcher's grid fits one dispatch (next to the launchers' grid formulas).
bool mx_quant_launch_fits(int64_t M, int64_t K, int mode);
bool mx_quant_grouped_launch_fits(int64_t M, int64_t K);
bool mx_dequant_launch_fits(int64_t rows, int64_t cols);
bool nv_quant_launch_fits(int64_t R, int64_t K);
bool nv_group_launch_fits(int64_t R, int64_t K, int64_t G);
bool nv_2d_launch_fits(int64_t R, int64_t K, int64_t G);
bool nv_dequant_launch_fits(int64_t R, int64_t K);
bool nv_dequant_2d_launch_fits(int64_t R, int64_t K);
}  // namespace bsq

namespace {

struct Buf {
    const void* p;
    int64_t bytes;
};

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; }

// Any two non-empty byte ranges of the list overlap?
bool overlap(const Buf* b, int n) {
    for (int i = 0; i < n; ++i)
        for (int j = i + 1; j < n; ++j) {
            if (b[i].bytes <= 0 || b[j].bytes <= 0) continue;
            const uintptr_t a0 = reinterpret_cast<uintptr_t>(b[i].p), a1 = a0 + (uintptr_t)b[i].bytes;
            const uintptr_t c0 = reinterpret_cast<uintptr_t>(b[j].p), c1 = c0 + (uintptr_t)b[j].bytes;
            if (a0 < c1 && c0 < a1) return true;
        }
    return false;
}

// rows * cols * elem_bytes representable (and every derived size with it)?
bool size_ok(int64_t rows, int64_t cols, int64_t elem_bytes) {
    if (rows < 0 || cols < 0) return false;
    if (rows == 0 || cols == 0) return true;
    return rows <= INT64_MAX / cols / elem_bytes;
}

int hip_status(hipError_t e) { return e == hipSuccess ? BSQ_OK : BSQ_ERR_HIP; }

}  // namespace

extern "C" {

int bsq_abi_version(void) { return BSQ_ABI_VERSION; }

const char* bsq_status_string(int status) {
    switch (status) {
        case BSQ_OK: return "ok";
        case BSQ_ERR_NULL: return "a required pointer is NULL";
        case BSQ_ERR_SHAPE: return "invalid shape (negative, too large, or breaking the block divisibility rule)";
        case BSQ_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case BSQ_ERR_MODE: return "unknown MXFP8 mode (expected MX_ROWWISE, MX_COLWISE or MX_BOTH)";
        case BSQ_ERR_ALIAS: return "two buffers of the call overlap";
        case BSQ_ERR_OFFSETS: return "expert offsets are not 0 = o[0] <= ... <= o[E] = R";
        case BSQ_ERR_HIP: return "HIP kernel launch failed";
        default: return "unknown status";
    }
}

int mx_quantize_mxfp8(const void* x, int64_t M, int64_t K, int mode, void* q_row, void* s_row,
                      void* q_col, void* s_col, void* stream) {
    if (mode != MX_ROWWISE && mode != MX_COLWISE && mode != MX_BOTH) return BSQ_ERR_MODE;
    const bool row = (mode & MX_ROWWISE) != 0, col = (mode & MX_COLWISE) != 0;
    if (!size_ok(M, K, 2)) return BSQ_ERR_SHAPE;
    if (row && K % 32 != 0) return BSQ_ERR_SHAPE;       // rowwise blocks along K
    if (K % 8 != 0) return BSQ_ERR_SHAPE;               // 16-byte rows (columnwise only)
    if (col && M % 32 != 0) return BSQ_ERR_SHAPE;       // columnwise blocks along M
    if (!bsq::mx_quant_launch_fits(M, K, mode)) return BSQ_ERR_SHAPE;
    if (M == 0 || K == 0) return BSQ_OK;
    if (x == nullptr) return BSQ_ERR_NULL;
    if (row && (q_row == nullptr || s_row == nullptr)) return BSQ_ERR_NULL;
    if (col && (q_col == nullptr || s_col == nullptr)) return BSQ_ERR_NULL;
    if (misaligned(x, 16)) return BSQ_ERR_ALIGN;
    if (row && (misaligned(q_row, 16) || misaligned(s_row, 16))) return BSQ_ERR_ALIGN;
    if (col && (misaligned(q_col, 16) || misaligned(s_col, 16))) return BSQ_ERR_ALIGN;
    const int64_t n = M * K;
    const Buf bufs[5] = {{x, 2 * n},
                         {q_row, row ? n : 0}, {s_row, row ? n / 32 : 0},
                         {q_col, col ? n : 0}, {s_col, col ? n / 32 : 0}};
    if (overlap(bufs, 5)) return BSQ_ERR_ALIAS;
    return hip_status(bsq::launch_mx_quant(x, M, K, mode, q_row, s_row, q_col, s_col,
                                           static_cast<hipStream_t>(stream)));
}

int mx_quantize_mxfp8_grouped(const void* x, int64_t M, int64_t K, int mode,
                              const int64_t* expert_offsets, int64_t E, void* q_row, void* s_row,
                              void* q_col, void* s_col, int64_t s_ld, int32_t* status_dev,
                              void* stream) {
    if (mode != MX_COLWISE && mode != MX_BOTH) return BSQ_ERR_MODE;
    const bool row = mode == MX_BOTH;
    if (!size_ok(M, K, 2)) return BSQ_ERR_SHAPE;
    if (K % 32 != 0) return BSQ_ERR_SHAPE;
    if (E < 1 || E >= (int64_t(1) << 31)) return BSQ_ERR_SHAPE;
    const int64_t min_blocks = (M + 31) / 32;
    if (min_blocks + E >= (int64_t(1) << 31)) return BSQ_ERR_SHAPE;
    if (s_ld < min_blocks || !size_ok(K, s_ld, 1)) return BSQ_ERR_SHAPE;
    if (!bsq::mx_quant_grouped_launch_fits(M, K)) return BSQ_ERR_SHAPE;
    if (expert_offsets == nullptr) return BSQ_ERR_NULL;
    if (misaligned(expert_offsets, 8)) return BSQ_ERR_ALIGN;
    if (status_dev != nullptr && misaligned(status_dev, 4)) return BSQ_ERR_ALIGN;
    const bool empty = (M == 0 || K == 0);
    if (empty && status_dev == nullptr) return BSQ_OK;
    if (!empty) {
        if (x == nullptr || q_col == nullptr || s_col == nullptr) return BSQ_ERR_NULL;
        if (row && (q_row == nullptr || s_row == nullptr)) return BSQ_ERR_NULL;
        if (misaligned(x, 16) || misaligned(q_col, 16) || misaligned(s_col, 16)) return BSQ_ERR_ALIGN;
        if (row && (misaligned(q_row, 16) || misaligned(s_row, 16))) return BSQ_ERR_ALIGN;
    }
    const int64_t n = empty ? 0 : M * K;
    const Buf bufs[7] = {{x, 2 * n},
                         {q_row, row ? n : 0}, {s_row, row ? n / 32 : 0},
                         {q_col, n}, {s_col, empty ? 0 : K * s_ld},
                         {expert_offsets, 8 * (E + 1)},
                         {status_dev, status_dev != nullptr ? 4 : 0}};
    if (overlap(bufs, 7)) return BSQ_ERR_ALIAS;
    return hip_status(bsq::launch_mx_quant_grouped(x, M, K, mode, expert_offsets, E, q_row, s_row,
                                                   q_col, s_col, s_ld, status_dev,
                                                   static_cast<hipStream_t>(stream)));
}

static int nv_quant_common(const void* x, int64_t R, int64_t K, const int64_t* offsets, int64_t E,
                           bool grouped, void* q, void* sb, float* st, int32_t* status,
                           void* stream) {
    if (!size_ok(R, K, 2)) return BSQ_ERR_SHAPE;
    if (K % 16 != 0) return BSQ_ERR_SHAPE;
    if (grouped && (E < 1 || E > INT64_MAX / 8 - 1)) return BSQ_ERR_SHAPE;
    if (!bsq::nv_quant_launch_fits(R, K)) return BSQ_ERR_SHAPE;
    if (grouped && offsets == nullptr) return BSQ_ERR_NULL;
    if (grouped && misaligned(offsets, 8)) return BSQ_ERR_ALIGN;
    if (grouped && status != nullptr && misaligned(status, 4)) return BSQ_ERR_ALIGN;
    const bool empty = (R == 0 || K == 0);
    if (empty && !(grouped && status != nullptr)) return BSQ_OK;
    if (!empty) {
        if (x == nullptr || q == nullptr || sb == nullptr || st == nullptr) return BSQ_ERR_NULL;
        if (misaligned(x, 16) || misaligned(q, 16) || misaligned(sb, 16) || misaligned(st, 16))
            return BSQ_ERR_ALIGN;
    }
    const int64_t n = empty ? 0 : R * K;
    const Buf bufs[6] = {{x, 2 * n}, {q, n / 2}, {sb, n / 16}, {st, empty ? 0 : 4 * R},
                         {offsets, grouped ? 8 * (E + 1) : 0},
                         {status, (grouped && status != nullptr) ? 4 : 0}};
    if (overlap(bufs, 6)) return BSQ_ERR_ALIAS;
    return hip_status(bsq::launch_nv_quant(x, R, K, q, sb, st, grouped ? offsets : nullptr, E,
                                           grouped ? status : nullptr,
                                           static_cast<hipStream_t>(stream)));
}

int nv_quantize_nvfp4_per_token(const void* x, int64_t R, int64_t K, void* q, void* sb,
                                float* st, void* stream) {
    return nv_quant_common(x, R, K, nullptr, 0, false, q, sb, st, nullptr, stream);
}

int nv_quantize_nvfp4_per_token_grouped(const void* x, int64_t R, int64_t K,
                                        const int64_t* expert_offsets, int64_t E, void* q,
                                        void* sb, float* st, int32_t* status_dev,
                                        void* stream) {
    return nv_quant_common(x, R, K, expert_offsets, E, true, q, sb, st, status_dev, stream);
}

int nv_quantize_nvfp4_per_token_scatter(const void* h, int64_t T, int64_t K, const int64_t* dst_rows,
                                        int64_t top_k, int64_t N, void* q, void* sb, float* st,
                                        int32_t* status_dev, void* stream) {
    if (!size_ok(T, K, 2) || !size_ok(N, K, 2)) return BSQ_ERR_SHAPE;
    if (K % 16 != 0) return BSQ_ERR_SHAPE;
    if (top_k < 1 || !size_ok(T, top_k, 8)) return BSQ_ERR_SHAPE;
    if (!bsq::nv_quant_launch_fits(T, K)) return BSQ_ERR_SHAPE;
    if (status_dev != nullptr && misaligned(status_dev, 4)) return BSQ_ERR_ALIGN;
    const bool no_rows = (T == 0 || K == 0);
    if (no_rows && status_dev == nullptr) return BSQ_OK;
    if (!no_rows) {
        if (h == nullptr || dst_rows == nullptr) return BSQ_ERR_NULL;
        if (misaligned(h, 16) || misaligned(dst_rows, 8)) return BSQ_ERR_ALIGN;
    }
    const bool out = !no_rows && N > 0;
    if (out) {
        if (q == nullptr || sb == nullptr || st == nullptr) return BSQ_ERR_NULL;
        if (misaligned(q, 16) || misaligned(sb, 16) || misaligned(st, 16)) return BSQ_ERR_ALIGN;
    }
    const int64_t nh = no_rows ? 0 : T * K, nx = out ? N * K : 0;
    const Buf bufs[6] = {{h, 2 * nh}, {dst_rows, no_rows ? 0 : 8 * T * top_k},
                         {q, nx / 2}, {sb, nx / 16}, {st, out ? 4 * N : 0},
                         {status_dev, status_dev != nullptr ? 4 : 0}};
    if (overlap(bufs, 6)) return BSQ_ERR_ALIAS;
    return hip_status(bsq::launch_nv_quant_scatter(h, no_rows ? 0 : T, K, dst_rows, top_k, N, q, sb, st,
                                                   status_dev, static_cast<hipStream_t>(stream)));
}

int nv_quantize_nvfp4_per_group(const void* x, int64_t R, int64_t K, const int64_t* group_offsets,
                                int64_t G, void* q, void* sb, float* s_group, int32_t* status_dev,
                                void* stream) {
    if (!size_ok(R, K, 2)) return BSQ_ERR_SHAPE;
    if (K % 16 != 0) return BSQ_ERR_SHAPE;
    if (G < 1 || G > INT64_MAX / 8 - 1) return BSQ_ERR_SHAPE;
    if (!bsq::nv_group_launch_fits(R, K, G)) return BSQ_ERR_SHAPE;
    if (group_offsets == nullptr || s_group == nullptr) return BSQ_ERR_NULL;
    if (misaligned(group_offsets, 8) || misaligned(s_group, 16)) return BSQ_ERR_ALIGN;
    if (status_dev != nullptr && misaligned(status_dev, 4)) return BSQ_ERR_ALIGN;
    const bool empty = (R == 0 || K == 0);
    if (!empty) {
        if (x == nullptr || q == nullptr || sb == nullptr) return BSQ_ERR_NULL;
        if (misaligned(x, 16) || misaligned(q, 16) || misaligned(sb, 16)) return BSQ_ERR_ALIGN;
    }
    const int64_t n = empty ? 0 : R * K;
    const Buf bufs[6] = {{x, 2 * n}, {q, n / 2}, {sb, n / 16}, {s_group, 4 * G},
                         {group_offsets, 8 * (G + 1)}, {status_dev, status_dev != nullptr ? 4 : 0}};
    if (overlap(bufs, 6)) return BSQ_ERR_ALIAS;
    return hip_status(bsq::launch_nv_quant_group(x, R, K, group_offsets, G, q, sb, s_group, status_dev,
                                                 static_cast<hipStream_t>(stream)));
}

int nv_dequantize_per_group(const void* q, const void* sb, const float* s_group,
                            const int64_t* group_offsets, int64_t G, int64_t R, int64_t K, void* y,
                            void* stream) {
    if (!size_ok(R, K, 2)) return BSQ_ERR_SHAPE;
    if (K % 16 != 0) return BSQ_ERR_SHAPE;
    if (G < 1 || G > INT64_MAX / 8 - 1) return BSQ_ERR_SHAPE;
    if (!bsq::nv_dequant_launch_fits(R, K)) return BSQ_ERR_SHAPE;
    if (R == 0 || K == 0) return BSQ_OK;
    if (q == nullptr || sb == nullptr || s_group == nullptr || group_offsets == nullptr || y == nullptr)
        return BSQ_ERR_NULL;
    if (misaligned(q, 16) || misaligned(sb, 16) || misaligned(s_group, 16) || misaligned(y, 16) ||
        misaligned(group_offsets, 8))
        return BSQ_ERR_ALIGN;
    const int64_t n = R * K;
    const Buf bufs[5] = {{q, n / 2}, {sb, n / 16}, {s_group, 4 * G}, {group_offsets, 8 * (G + 1)},
                         {y, 2 * n}};
    if (overlap(bufs, 5)) return BSQ_ERR_ALIAS;
    return hip_status(bsq::launch_nv_dequant_group(q, sb, s_group, group_offsets, G, R, K, y,
                                                   static_cast<hipStream_t>(stream)));
}

int nv_quantize_nvfp4_2d(const void* x, int64_t R, int64_t K, const int64_t* group_offsets, int64_t G,
                         void* q, void* sb, float* s_group, int32_t* status_dev, void* stream) {
    if (!size_ok(R, K, 2)) return BSQ_ERR_SHAPE;
    if (R % 16 != 0 || K % 16 != 0) return BSQ_ERR_SHAPE;
    if (G < 1 || G > INT64_MAX / 8 - 1) return BSQ_ERR_SHAPE;
    if (!bsq::nv_2d_launch_fits(R, K, G)) return BSQ_ERR_SHAPE;
    if (group_offsets == nullptr || s_group == nullptr) return BSQ_ERR_NULL;
    if (misaligned(group_offsets, 8) || misaligned(s_group, 16)) return BSQ_ERR_ALIGN;
    if (status_dev != nullptr && misaligned(status_dev, 4)) return BSQ_ERR_ALIGN;
    const bool empty = (R == 0 || K == 0);
    if (!empty) {
        if (x == nullptr || q == nullptr || sb == nullptr) return BSQ_ERR_NULL;
        if (misaligned(x, 16) || misaligned(q, 16) || misaligned(sb, 16)) return BSQ_ERR_ALIGN;
    }
    const int64_t n = empty ? 0 : R * K;
    const Buf bufs[6] = {{x, 2 * n}, {q, n / 2}, {sb, n / 256}, {s_group, 4 * G},
                         {group_offsets, 8 * (G + 1)}, {status_dev, status_dev != nullptr ? 4 : 0}};
    if (overlap(bufs, 6)) return BSQ_ERR_ALIAS;
    return hip_status(bsq::launch_nv_quant_2d(x, R, K, group_offsets, G, q, sb, s_group, status_dev,
                                              static_cast<hipStream_t>(stream)));
}

int nv_dequantize_2d(const void* q, const void* sb, const float* s_group, const int64_t* group_offsets,
                     int64_t G, int64_t R, int64_t K, void* y, void* stream) {
    if (!size_ok(R, K, 2)) return BSQ_ERR_SHAPE;
    if (R % 16 != 0 || K % 16 != 0) return BSQ_ERR_SHAPE;
    if (G < 1 || G > INT64_MAX / 8 - 1) return BSQ_ERR_SHAPE;
    if (!bsq::nv_dequant_2d_launch_fits(R, K)) return BSQ_ERR_SHAPE;
    if (R == 0 || K == 0) return BSQ_OK;
    if (q == nullptr || sb == nullptr || s_group == nullptr || group_offsets == nullptr || y == nullptr)
        return BSQ_ERR_NULL;
    if (misaligned(q, 16) || misaligned(sb, 16) || misaligned(s_group, 16) || misaligned(y, 16) ||
        misaligned(group_offsets, 8))
        return BSQ_ERR_ALIGN;
    const int64_t n = R * K;
    const Buf bufs[5] = {{q, n / 2}, {sb, n / 256}, {s_group, 4 * G}, {group_offsets, 8 * (G + 1)},
                         {y, 2 * n}};
    if (overlap(bufs, 5)) return BSQ_ERR_ALIAS;
    return hip_status(bsq::launch_nv_dequant_2d(q, sb, s_group, group_offsets, G, R, K, y,
                                                static_cast<hipStream_t>(stream)));
}

int mx_dequantize(const void* q, const void* s, int64_t rows, int64_t cols, void* y,
                  void* stream) {
    if (!size_ok(rows, cols, 2)) return BSQ_ERR_SHAPE;
    if (cols % 32 != 0) return BSQ_ERR_SHAPE;
    if (!bsq::mx_dequant_launch_fits(rows, cols)) return BSQ_ERR_SHAPE;
    if (rows == 0 || cols == 0) return BSQ_OK;
    if (q == nullptr || s == nullptr || y == nullptr) return BSQ_ERR_NULL;
    if (misaligned(q, 16) || misaligned(s, 16) || misaligned(y, 16)) return BSQ_ERR_ALIGN;
    const int64_t n = rows * cols;
    const Buf bufs[3] = {{q, n}, {s, n / 32}, {y, 2 * n}};
    if (overlap(bufs, 3)) return BSQ_ERR_ALIAS;
    return hip_status(bsq::launch_mx_dequant(q, s, rows, cols, y, static_cast<hipStream_t>(stream)));
}

int nv_dequantize(const void* q, const void* sb, const float* st, int64_t R, int64_t K, void* y,
                  void* stream) {
    if (!size_ok(R, K, 2)) return BSQ_ERR_SHAPE;
    if (K % 16 != 0) return BSQ_ERR_SHAPE;
    if (!bsq::nv_dequant_launch_fits(R, K)) return BSQ_ERR_SHAPE;
    if (R == 0 || K == 0) return BSQ_OK;
    if (q == nullptr || sb == nullptr || st == nullptr || y == nullptr) return BSQ_ERR_NULL;
    if (misaligned(q, 16) || misaligned(sb, 16) || misaligned(st, 16) || misaligned(y, 16))
        return BSQ_ERR_ALIGN;
    const int64_t n = R * K;
    const Buf bufs[4] = {{q, n / 2}, {sb, n / 16}, {st, 4 * R}, {y, 2 * n}};
    if (overlap(bufs, 4)) return BSQ_ERR_ALIAS;
    return hip_status(bsq::launch_nv_dequant(q, sb, st, R, K, y, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
