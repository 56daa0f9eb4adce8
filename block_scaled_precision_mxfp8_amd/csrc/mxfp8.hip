// mxfp8.hip -- MXFP8 quantization (rowwise 1x32, columnwise 32x1, both) and MXFP8
// dequantization to BF16 for gfx950.
//
// Page "Towards Blackwell-native 8-bit and 4-bit RL":
//  * section "Format background": 32 consecutive E4M3 values share one E8M0 scale; the
//    blocks are one-dimensional; the decoded scale is rounded up so the block maximum is
//    never clipped.
//  * section "Recipe 1: end-to-end MXFP8 RL": rowwise (1x32) and columnwise (32x1) blocks
//    are numerically different, so both copies are quantized from the full-precision
//    input, not one from the other.
//  * section "High-precision and dequantized backward": BF16 dequantized operands.
//
// The work is pure streaming (about 3-4 bytes of HBM traffic per element and a few
// integer/FP32 operations), so the kernels are written for HBM bandwidth: 16-byte loads
// and stores that cover whole cache lines per instruction, block maxima reduced inside a
// quad of lanes with DPP, and no LDS traffic on the element data.
#include "bsq_device.h"

namespace bsq {

// Cache policy of each kernel family's one-touch accesses: bit 0 = non-temporal loads,
// bit 1 = non-temporal stores.  Measured on the layer-step stream (MX dual, NV quant,
// dequants back to back): non-temporal loads speed up the read-heavy kernels in isolation
// (rowwise 206 -> 184 us on 196608 x 2048) but slow the dual kernel; non-temporal stores
// leave no dirty Infinity-Cache lines for the next kernel to write back, which speeds up
// the stream (5623 -> 6001 GB/s per step) at some cost to a write-heavy kernel timed alone.
#ifndef BSQ_POLICY_MXROW
#define BSQ_POLICY_MXROW 3
#endif
#ifndef BSQ_POLICY_MXTILE
#define BSQ_POLICY_MXTILE 2
#endif
#ifndef BSQ_POLICY_MXDQ
#define BSQ_POLICY_MXDQ 2
#endif
constexpr bool MXROW_NT_LOAD = (BSQ_POLICY_MXROW & 1) != 0, MXROW_NT_STORE = (BSQ_POLICY_MXROW & 2) != 0;
constexpr bool MXTILE_NT_LOAD = (BSQ_POLICY_MXTILE & 1) != 0, MXTILE_NT_STORE = (BSQ_POLICY_MXTILE & 2) != 0;
constexpr bool MXDQ_NT_LOAD = (BSQ_POLICY_MXDQ & 1) != 0, MXDQ_NT_STORE = (BSQ_POLICY_MXDQ & 2) != 0;

// ----------------------------------------------------------------------------- encode

// Eight E4M3 codes of a 16-byte chunk of BF16 divided by the block scale 2^(c-127): the
// quotient is exact and at most 448 (the scale never clips), where the gfx950 scaled
// convert is exactly round-to-nearest-even of the quotient.
__device__ __forceinline__ uint2 mx_enc8(const uint4& v, float scale) {
    return make_uint2(cvt_e4m3x4_bf16(v.x, v.y, scale), cvt_e4m3x4_bf16(v.z, v.w, scale));
}

// Dword d (0..3) of a 16-byte chunk; d is a compile-time constant after unrolling.
__device__ __forceinline__ uint32_t dword_of(const uint4& v, int d) {
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

// Magnitude maximum (BF16 bits) of the 8 BF16 values of a 16-byte chunk.
__device__ __forceinline__ uint32_t chunk_absmax(const uint4& v) {
    uint32_t m = absmax2(absmax2(absmax2(absmax2(0u, v.x), v.y), v.z), v.w);
    return fold2(m);
}

// ----------------------------------------------------------------------------- rowwise

// Rowwise blocks of 32 never straddle a row (K % 32 == 0), and the row-major E4M3 and
// E8M0 arrays are exactly the element and block orders of the flattened tensor, so the
// rowwise copy is a 1-D stream over M*K elements.  One wave handles a tile of
// ROW_SLOTS x 512 elements: in slot j lane l owns the 16-byte chunk (8 BF16) number
// tile*64*ROW_SLOTS + 64*j + l, so each load instruction covers 1 KiB contiguous and each
// quad of lanes holds one block.  The 16*ROW_SLOTS scale bytes of the tile are gathered
// in LDS and written as 16-byte stores (one full 128-byte line for ROW_SLOTS = 8).
constexpr int ROW_SLOTS = 8;
constexpr int ROW_WAVES = 4;

__global__ __launch_bounds__(64 * ROW_WAVES)
void mx_quant_rowwise_kernel(const uint4* __restrict__ x, uint2* __restrict__ q,
                             uint8_t* __restrict__ s, int64_t n_chunks) {
    __shared__ __align__(16) uint8_t lds_s[ROW_WAVES][16 * ROW_SLOTS];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t base = ((int64_t)blockIdx.x * ROW_WAVES + wave) * (64 * ROW_SLOTS);
    if (base >= n_chunks) return;

    uint4 v[ROW_SLOTS];
#pragma unroll
    for (int j = 0; j < ROW_SLOTS; ++j) {
        const int64_t c = base + 64 * j + lane;
        v[j] = (c < n_chunks) ? ld_stream<MXROW_NT_LOAD>(x + c) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < ROW_SLOTS; ++j) {
        const uint32_t amax = quad_max(chunk_absmax(v[j]));
        const uint32_t code = e8m0_code_from_bf16_mag(amax);
        const uint2 out = mx_enc8(v[j], e8m0_decode(code));
        const int64_t c = base + 64 * j + lane;
        if (c < n_chunks) st_stream<MXROW_NT_STORE>(q + c, out);
        if ((lane & 3) == 0) lds_s[wave][16 * j + (lane >> 2)] = (uint8_t)code;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const int64_t nblk = n_chunks >> 2;
    const int64_t b0 = base >> 2;
    if (b0 + 16 * ROW_SLOTS <= nblk) {
        if (lane < ROW_SLOTS)
            st_stream<MXROW_NT_STORE>(reinterpret_cast<uint4*>(s + b0) + lane, reinterpret_cast<const uint4*>(lds_s[wave])[lane]);
    } else {
        for (int i = lane; i < 16 * ROW_SLOTS; i += 64)
            if (b0 + i < nblk) s[b0 + i] = lds_s[wave][i];
    }
}

// ----------------------------------------------------------------------------- col / both

// Columnwise (and dual) quantization of x[M][K].  One wave owns a 128-row x 64-column
// tile.  Lane l = 8*g + c holds rows 16*g .. 16*g+15 of the tile and columns 8*c .. 8*c+7
// (one 16-byte chunk per row, 16 chunks = 64 VGPRs):
//  * a 32x1 column block is held by the lane pair (g, g^1) -- 16 rows each -- so its
//    maximum is a lane-local packed max plus one lane exchange;
//  * a 1x32 row block is the quad of lanes c = 4k .. 4k+3 of one row (DPP);
//  * every load instruction reads 8 rows x 128 bytes (full lines);
//  * the columnwise copy q_col[K][M] is written as one 16-byte store per lane and
//    column (16 rows of E4M3), so 8 lanes g = 0..7 fill 128 contiguous bytes of one
//    q_col row: the transpose happens in registers and the writes stay coalesced.
// A workgroup is WR x WC waves: WR wave tiles stacked down the rows and WC side by side
// along the columns, so one workgroup covers (128 WR) x (64 WC) and its q_row lines are
// 64 WC bytes and its q_col lines 128 WR bytes long.  Scale codes are gathered in LDS and
// leave as one store per row / column of the workgroup tile.  Workgroups are renumbered
// so that each XCD (workgroups are dealt round-robin over the 8 XCDs) gets a contiguous
// range of row stripes.
constexpr int TILE_ROWS = 128;
constexpr int TILE_COLS = 64;

template <int N>
__device__ __forceinline__ void store_bytes(uint8_t* dst, const uint8_t* src, int n, bool aligned) {
    if (n == N && aligned) {
        if constexpr (N == 16) *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        else if constexpr (N == 8) *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
        else if constexpr (N == 4) *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(src);
        else if constexpr (N == 2) *reinterpret_cast<uint16_t*>(dst) = *reinterpret_cast<const uint16_t*>(src);
        else dst[0] = src[0];
    } else {
        for (int i = 0; i < n; ++i) dst[i] = src[i];
    }
}

// Tile geometry of workgroup tile w (w in [0, n_wg)): first row and first column.
//   ORDER 0: each XCD (workgroups are dealt round-robin over the 8 XCDs) a contiguous
//            range of tile ids, row stripe major (columns fastest)
//   ORDER 1: plain ids, row stripe major
template <int ORDER>
__device__ __forceinline__ void tile_origin(int64_t w, int64_t n_wg, int64_t col_groups,
                                            int wg_rows, int wg_cols, int64_t& rw, int64_t& kw) {
    if (ORDER == 0 && (n_wg & 7) == 0) w = (w & 7) * (n_wg >> 3) + (w >> 3);
    rw = (w / col_groups) * wg_rows;
    kw = (w % col_groups) * wg_cols;
}

// Load the lane's 16 rows x 8 columns of the wave tile (zeros outside the tensor).
__device__ __forceinline__ void load_tile(uint4 (&v)[16], const uint16_t* __restrict__ x,
                                          int64_t K, int64_t row0, int64_t col0, bool ok) {
    const uint16_t* src = x + row0 * K + col0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        v[i] = ok ? ld_stream<MXTILE_NT_LOAD>(reinterpret_cast<const uint4*>(src + (int64_t)i * K)) : make_uint4(0u, 0u, 0u, 0u);
}

// Everything after the load for one workgroup tile: both copies' codes and stores, the
// scale gather in LDS and the scale stores.  Called by every thread of the workgroup.
template <bool ROW, int WR, int WC>
__device__ __forceinline__ void process_tile(uint4 (&v)[16], int64_t M, int64_t K, int64_t rw, int64_t kw,
                                             uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                                             uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col,
                                             uint8_t (*lds_srow)[TILE_COLS * WC / 32],
                                             uint8_t (*lds_scol)[TILE_ROWS * WR / 32]) {
    constexpr int WG_ROWS = TILE_ROWS * WR, WG_COLS = TILE_COLS * WC;
    constexpr int SROW_B = WG_COLS / 32, SCOL_B = WG_ROWS / 32;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wr = wave / WC, wc = wave % WC;
    const int g = lane >> 3;
    const int c = lane & 7;
    const int64_t row0 = rw + wr * TILE_ROWS + 16 * g;
    const int64_t col0 = kw + wc * TILE_COLS + 8 * c;
    const bool ok = row0 < M && col0 < K;      // M, K % 32 == 0: lane pairs / quads agree
    const int lrow = wr * TILE_ROWS + 16 * g;  // lane's first row inside the workgroup tile
    const int lcol = wc * TILE_COLS + 8 * c;   // lane's first column inside the workgroup tile

    // ---- rowwise copy: each row of the lane, block = quad of lanes
    if (ROW) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t amax = quad_max(chunk_absmax(v[i]));
            const uint32_t code = e8m0_code_from_bf16_mag(amax);
            const uint2 out = mx_enc8(v[i], e8m0_decode(code));
            if (ok) st_stream<MXTILE_NT_STORE>(reinterpret_cast<uint2*>(q_row + (row0 + i) * K + col0), out);
            if ((c & 3) == 0) lds_srow[lrow + i][lcol >> 5] = (uint8_t)code;
        }
        // The column pass below re-derives its FP32 operands from the packed tile; this
        // empty register barrier stops the compiler from instead keeping the row pass's
        // unpacked values alive (which would double the live tile and spill).
#pragma unroll
        for (int i = 0; i < 16; ++i)
            asm volatile("" : "+v"(v[i].x), "+v"(v[i].y), "+v"(v[i].z), "+v"(v[i].w));
    }

    // ---- columnwise copy: packed column maxima over 16 rows, then over the lane pair
    uint32_t cm[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        cm[0] = absmax2(cm[0], v[i].x);
        cm[1] = absmax2(cm[1], v[i].y);
        cm[2] = absmax2(cm[2], v[i].z);
        cm[3] = absmax2(cm[3], v[i].w);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t other = (uint32_t)__shfl_xor((int)cm[d], 8, 64);
        u16x2 a = __builtin_bit_cast(u16x2, cm[d]);
        u16x2 b = __builtin_bit_cast(u16x2, other);
        cm[d] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t code0 = e8m0_code_from_bf16_mag(cm[d] & 0xFFFFu);   // column 2d
        const uint32_t code1 = e8m0_code_from_bf16_mag(cm[d] >> 16);       // column 2d+1
        const float sc0 = e8m0_decode(code0);
        const float sc1 = e8m0_decode(code1);
        // Column-major pairs (row i, row i+1) of one column, built with one byte permute
        // each, so one scaled convert (one scale = the column's) encodes two rows.
        uint32_t a[4], b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t r0w = dword_of(v[4 * t + 0], d), r1w = dword_of(v[4 * t + 1], d);
            const uint32_t r2w = dword_of(v[4 * t + 2], d), r3w = dword_of(v[4 * t + 3], d);
            a[t] = cvt_e4m3x4_bf16(__builtin_amdgcn_perm(r1w, r0w, 0x05040100u),
                                   __builtin_amdgcn_perm(r3w, r2w, 0x05040100u), sc0);
            b[t] = cvt_e4m3x4_bf16(__builtin_amdgcn_perm(r1w, r0w, 0x07060302u),
                                   __builtin_amdgcn_perm(r3w, r2w, 0x07060302u), sc1);
        }
        if (ok) {
            const int64_t ka = col0 + 2 * d;
            st_stream<MXTILE_NT_STORE>(reinterpret_cast<uint4*>(q_col + ka * M + row0), make_uint4(a[0], a[1], a[2], a[3]));
            st_stream<MXTILE_NT_STORE>(reinterpret_cast<uint4*>(q_col + (ka + 1) * M + row0), make_uint4(b[0], b[1], b[2], b[3]));
        }
        if ((g & 1) == 0) {
            lds_scol[lcol + 2 * d][lrow >> 5] = (uint8_t)code0;
            lds_scol[lcol + 2 * d + 1][lrow >> 5] = (uint8_t)code1;
        }
    }

    __syncthreads();
    // rowwise scales: one store of SROW_B bytes per row of the workgroup tile
    if (ROW) {
        const int64_t nb_row = K >> 5;
        const int64_t b0 = kw >> 5;
        const int nb = (int)min((int64_t)SROW_B, nb_row - b0);
        for (int t = threadIdx.x; t < WG_ROWS; t += 64 * WR * WC) {
            if (rw + t < M)
                store_bytes<SROW_B>(s_row + (rw + t) * nb_row + b0, lds_srow[t], nb,
                                    (nb_row % SROW_B) == 0);
        }
    }
    // columnwise scales: one store of SCOL_B bytes per column of the workgroup tile
    {
        const int64_t nb_col = M >> 5;
        const int64_t b0 = rw >> 5;
        const int nb = (int)min((int64_t)SCOL_B, nb_col - b0);
        for (int t = threadIdx.x; t < WG_COLS; t += 64 * WR * WC) {
            if (kw + t < K)
                store_bytes<SCOL_B>(s_col + (kw + t) * nb_col + b0, lds_scol[t], nb,
                                    (nb_col % SCOL_B) == 0);
        }
    }
    __syncthreads();                           // LDS is reused by the next tile
}

// One workgroup tile per workgroup.
template <bool ROW, int WR, int WC, int ORDER>
__global__ __launch_bounds__(64 * WR * WC) __attribute__((amdgpu_waves_per_eu(4)))
void mx_quant_tile_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                          uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                          uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col,
                          int64_t col_groups, int64_t n_wg) {
    __shared__ __align__(16) uint8_t lds_srow[TILE_ROWS * WR][TILE_COLS * WC / 32];
    __shared__ __align__(16) uint8_t lds_scol[TILE_COLS * WC][TILE_ROWS * WR / 32];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int64_t rw, kw;
    tile_origin<ORDER>(blockIdx.x, n_wg, col_groups, TILE_ROWS * WR, TILE_COLS * WC, rw, kw);
    const int64_t row0 = rw + (wave / WC) * TILE_ROWS + 16 * (lane >> 3);
    const int64_t col0 = kw + (wave % WC) * TILE_COLS + 8 * (lane & 7);
    uint4 v[16];
    load_tile(v, x, K, row0, col0, row0 < M && col0 < K);
    process_tile<ROW, WR, WC>(v, M, K, rw, kw, q_row, s_row, q_col, s_col, lds_srow, lds_scol);
}

// Persistent variant: each workgroup walks tiles blockIdx.x, blockIdx.x + gridDim.x, ...
// and issues the loads of its next tile before encoding the current one, so HBM reads
// stay in flight while the codes are computed and stored.
template <bool ROW, int WR, int WC, int ORDER>
__global__ __launch_bounds__(64 * WR * WC) __attribute__((amdgpu_waves_per_eu(3)))
void mx_quant_tile_persistent_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                     uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                                     uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col,
                                     int64_t col_groups, int64_t n_wg) {
    __shared__ __align__(16) uint8_t lds_srow[TILE_ROWS * WR][TILE_COLS * WC / 32];
    __shared__ __align__(16) uint8_t lds_scol[TILE_COLS * WC][TILE_ROWS * WR / 32];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t lr = (wave / WC) * TILE_ROWS + 16 * (lane >> 3);
    const int64_t lc = (wave % WC) * TILE_COLS + 8 * (lane & 7);
    int64_t w = blockIdx.x;
    if (w >= n_wg) return;                     // uniform over the workgroup
    int64_t rw, kw;
    tile_origin<ORDER>(w, n_wg, col_groups, TILE_ROWS * WR, TILE_COLS * WC, rw, kw);
    uint4 v[16];
    load_tile(v, x, K, rw + lr, kw + lc, rw + lr < M && kw + lc < K);
    for (;;) {
        const int64_t wn = w + gridDim.x;
        int64_t rn = 0, kn = 0;
        uint4 vn[16];
        if (wn < n_wg) {
            tile_origin<ORDER>(wn, n_wg, col_groups, TILE_ROWS * WR, TILE_COLS * WC, rn, kn);
            load_tile(vn, x, K, rn + lr, kn + lc, rn + lr < M && kn + lc < K);
        }
        process_tile<ROW, WR, WC>(v, M, K, rw, kw, q_row, s_row, q_col, s_col, lds_srow, lds_scol);
        if (wn >= n_wg) break;
        w = wn;
        rw = rn;
        kw = kn;
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = vn[i];
    }
}

template <bool ROW, int WR, int WC, int ORDER = 0>
static void launch_tile(const void* x, int64_t M, int64_t K, void* q_row, void* s_row,
                        void* q_col, void* s_col, hipStream_t stream, int64_t persistent_wgs = 0) {
    const int64_t row_stripes = (M + TILE_ROWS * WR - 1) / (TILE_ROWS * WR);
    const int64_t col_groups = (K + TILE_COLS * WC - 1) / (TILE_COLS * WC);
    const int64_t n_wg = row_stripes * col_groups;
    if (persistent_wgs > 0 && persistent_wgs < n_wg) {
        hipLaunchKernelGGL((mx_quant_tile_persistent_kernel<ROW, WR, WC, ORDER>), dim3((unsigned)persistent_wgs),
                           dim3(64 * WR * WC), 0, stream, (const uint16_t*)x, M, K, (uint8_t*)q_row,
                           (uint8_t*)s_row, (uint8_t*)q_col, (uint8_t*)s_col, col_groups, n_wg);
    } else {
        hipLaunchKernelGGL((mx_quant_tile_kernel<ROW, WR, WC, ORDER>), dim3((unsigned)n_wg), dim3(64 * WR * WC),
                           0, stream, (const uint16_t*)x, M, K, (uint8_t*)q_row, (uint8_t*)s_row,
                           (uint8_t*)q_col, (uint8_t*)s_col, col_groups, n_wg);
    }
}

// Workgroup arrangement used by the library (wave tiles down x across), and the number of
// persistent workgroups (one per compute unit of an MI355X) used once a tensor has more
// tiles than that many workgroups can hold twice over.  Measured on the 65536 x 2048
// activations: 130 us with one tile per workgroup, 114 us persistent with 256 workgroups
// walking the tiles in row-stripe order (the tiles in flight then form one contiguous
// band, so concurrent reads and the concurrent q_col writes of each k-row are contiguous).
constexpr int TILE_WR = 1;
constexpr int TILE_WC = 4;
constexpr int TILE_PERSISTENT_WGS = 256;

// ----------------------------------------------------------------------------- dequant

// MXFP8 -> BF16 in the stored layout, a 1-D stream: element i uses scale i/32.  Thread t of
// a workgroup owns, in slot j, the 8 codes of chunk blockIdx*256*DQ_SLOTS + 256 j + t and
// writes their 16 bytes of BF16, so every load instruction reads 512 contiguous bytes
// and every store instruction writes 1 KiB contiguous; 4 neighbouring lanes share a scale.
constexpr int MX_DQ_SLOTS = 2;

__device__ __forceinline__ uint32_t fix_nan_pair(uint32_t y, uint32_t codes2) {
    const uint32_t lo = ((codes2 & 0x7Fu) == 0x7Fu) ? 0x7FC0u : (y & 0xFFFFu);
    const uint32_t hi = (((codes2 >> 8) & 0x7Fu) == 0x7Fu) ? 0x7FC00000u : (y & 0xFFFF0000u);
    return lo | hi;
}

// Eight BF16 (16 bytes) of the eight E4M3 codes in (w0, w1) times the block scale.  The
// product is exact in binary32 for every finite code and scale, and the convert rounds it
// to BF16 to nearest-even (overflow to infinity).  NaN codes (0x7F, 0xFF) and the NaN
// scale 0xFF give 0x7FC0; the hardware writes 0xFFC0 for a NaN code, so those rare
// chunks are patched.
__device__ __forceinline__ uint4 mx_dec8(uint32_t w0, uint32_t w1, uint32_t c) {
    const float scale = e8m0_decode(c);
    uint4 o = make_uint4(cvt_bf16x2_e4m3<false>(w0, scale), cvt_bf16x2_e4m3<true>(w0, scale),
                         cvt_bf16x2_e4m3<false>(w1, scale), cvt_bf16x2_e4m3<true>(w1, scale));
    const uint32_t nan0 = ((w0 & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
    const uint32_t nan1 = ((w1 & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
    if (c == 255u) {
        o = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
    } else if ((nan0 | nan1) != 0u) {
        o.x = fix_nan_pair(o.x, w0);
        o.y = fix_nan_pair(o.y, w0 >> 16);
        o.z = fix_nan_pair(o.z, w1);
        o.w = fix_nan_pair(o.w, w1 >> 16);
    }
    return o;
}

template <int DQ_SLOTS>
__global__ __launch_bounds__(256)
void mx_dequant_kernel(const uint2* __restrict__ q, const uint8_t* __restrict__ s,
                       uint4* __restrict__ y, int64_t n_chunks) {
    const int64_t base = (int64_t)blockIdx.x * (256 * DQ_SLOTS) + threadIdx.x;
    uint2 w[DQ_SLOTS];
    uint32_t sc[DQ_SLOTS];
#pragma unroll
    for (int j = 0; j < DQ_SLOTS; ++j) {
        const int64_t c = base + 256 * j;
        const bool ok = c < n_chunks;
        w[j] = ok ? ld_stream<MXDQ_NT_LOAD>(q + c) : make_uint2(0u, 0u);
        sc[j] = ok ? s[c >> 2] : 0u;
    }
#pragma unroll
    for (int j = 0; j < DQ_SLOTS; ++j) {
        const int64_t c = base + 256 * j;
        const uint4 o = mx_dec8(w[j].x, w[j].y, sc[j]);
        if (c < n_chunks) st_stream<MXDQ_NT_STORE>(y + c, o);
    }
}

// ----------------------------------------------------------------------------- launch

hipError_t launch_mx_quant(const void* x, int64_t M, int64_t K, int mode,
                           void* q_row, void* s_row, void* q_col, void* s_col,
                           hipStream_t stream) {
    if (mode == 1) {
        const int64_t n_chunks = M * K / 8;
        const int64_t tiles = (n_chunks + 64 * ROW_SLOTS - 1) / (64 * ROW_SLOTS);
        const int64_t grid = (tiles + ROW_WAVES - 1) / ROW_WAVES;
        hipLaunchKernelGGL(mx_quant_rowwise_kernel, dim3((unsigned)grid), dim3(64 * ROW_WAVES), 0,
                           stream, (const uint4*)x, (uint2*)q_row, (uint8_t*)s_row, n_chunks);
        return hipGetLastError();
    }
    const int64_t n_wg = ((M + TILE_ROWS * TILE_WR - 1) / (TILE_ROWS * TILE_WR)) *
                         ((K + TILE_COLS * TILE_WC - 1) / (TILE_COLS * TILE_WC));
    const int64_t pw = (n_wg > 2 * TILE_PERSISTENT_WGS) ? TILE_PERSISTENT_WGS : 0;
    if (mode == 3)
        launch_tile<true, TILE_WR, TILE_WC, 1>(x, M, K, q_row, s_row, q_col, s_col, stream, pw);
    else
        launch_tile<false, TILE_WR, TILE_WC, 1>(x, M, K, nullptr, nullptr, q_col, s_col, stream, pw);
    return hipGetLastError();
}

template <int SLOTS>
static void launch_mx_dequant_slots(const void* q, const void* s, int64_t rows, int64_t cols,
                                    void* y, hipStream_t stream) {
    const int64_t n_chunks = rows * cols / 8;
    const int64_t grid = (n_chunks + 256 * SLOTS - 1) / (256 * SLOTS);
    hipLaunchKernelGGL(mx_dequant_kernel<SLOTS>, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint2*)q, (const uint8_t*)s, (uint4*)y, n_chunks);
}

hipError_t launch_mx_dequant(const void* q, const void* s, int64_t rows, int64_t cols,
                             void* y, hipStream_t stream) {
    launch_mx_dequant_slots<MX_DQ_SLOTS>(q, s, rows, cols, y, stream);
    return hipGetLastError();
}

}  // namespace bsq
