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
// and stores that cover whole cache lines per instruction, and block maxima reduced inside
// a quad or pair of lanes with DPP.  LDS carries no element data in, only codes and scale
// bytes on their way out, where staging lets whole lines leave in one store.
#include "bsq_device.h"

namespace bsq {

// Cache policy of each kernel family's one-touch accesses: bit 0 = non-temporal loads,
// bit 1 = non-temporal stores.  Measured on the layer-step stream (MX dual, NV quant,
// dequants back to back): non-temporal loads speed up the read-heavy kernels in isolation
// (rowwise 206 -> 184 us on 196608 x 2048); non-temporal stores leave no dirty
// Infinity-Cache lines for the next kernel to write back, which speeds up the stream (5623
// -> 6001 GB/s per step) at some cost to a write-heavy kernel timed alone.  The tile
// kernels take non-temporal loads too: the dual kernel alone is unchanged (101.5 against
// 100.5 us on 65536 x 2048, 14.3 against 14.5 on 8192 x 2048), the columnwise mode 1%
// faster (627 against 634 us on 524288 x 2048), the read that follows either kernel 7 us
// faster, and the step 6141-6147 against 6131-6139 GB/s.  Non-temporal stores carry only
// whole lines: the scale bytes (8 or 4 per row or column of a workgroup tile) use ordinary
// stores, so that pieces of one line written by different workgroups meet in the caches;
// stored non-temporally they made the dual kernel 40% slower (141 against 101 us).
#ifndef BSQ_POLICY_MXROW
#define BSQ_POLICY_MXROW 3
#endif
#ifndef BSQ_POLICY_MXTILE
#define BSQ_POLICY_MXTILE 3
#endif
#ifndef BSQ_POLICY_MXDQ
#define BSQ_POLICY_MXDQ 2
#endif
// The grouped kernel reads the rows of a block that reaches past its window a second time,
// mostly from the caches, so its loads keep the ordinary policy.
#ifndef BSQ_POLICY_MXGRP
#define BSQ_POLICY_MXGRP 2
#endif
constexpr bool MXROW_NT_LOAD = (BSQ_POLICY_MXROW & 1) != 0, MXROW_NT_STORE = (BSQ_POLICY_MXROW & 2) != 0;
constexpr bool MXTILE_NT_LOAD = (BSQ_POLICY_MXTILE & 1) != 0, MXTILE_NT_STORE = (BSQ_POLICY_MXTILE & 2) != 0;
constexpr bool MXGRP_NT_LOAD = (BSQ_POLICY_MXGRP & 1) != 0, MXGRP_NT_STORE = (BSQ_POLICY_MXGRP & 2) != 0;
constexpr bool MXDQ_NT_LOAD = (BSQ_POLICY_MXDQ & 1) != 0, MXDQ_NT_STORE = (BSQ_POLICY_MXDQ & 2) != 0;

// A workgroup writes the rows of the columnwise copy q_col [K][M] it covers as one run of
// bytes per column.  When M is a multiple of 128 the runs cover whole lines; when it is not,
// the first and last line of a run are shared with the run of the workgroup holding the
// neighbouring rows, and pieces of one line stored non-temporally reach HBM as separate
// partial writes.  So a 16-byte piece goes non-temporal only if its whole 128-byte line lies
// inside the run [run0, run1); the pieces of shared lines use ordinary stores and meet in the
// caches first (the neighbouring row window is col_groups workgroups later, on the same XCD
// when col_groups is a multiple of 8).  Measured with M % 128 = 32, each kernel timed
// together with the 512 MiB read that follows it (the read's own time subtracted): dual
// 65568 x 2048 137.5 -> 112.4 us, columnwise 1012 -> 749 us on 524320 x 2048, grouped dual /
// columnwise on 524192 Zipf-routed rows 1182 / 940 -> 919 / 716 us; aligned shapes
// unchanged.  The rowwise copy keeps non-temporal stores throughout: with K % 128 = 32 the
// same rule made the dual kernel slower (129.8 -> 135.3 us on 65536 x 2080), the pieces of
// a shared q_row line coming from workgroups on different XCDs.
template <bool NT>
__device__ __forceinline__ void st_run(uint4* p, const uint4& v, const uint8_t* run0, const uint8_t* run1) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p) & ~(uintptr_t)127;
    if (NT && a >= reinterpret_cast<uintptr_t>(run0) && a + 128 <= reinterpret_cast<uintptr_t>(run1))
        st_stream<true>(p, v);
    else
        st_stream<false>(p, v);
}

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

// Columnwise (and dual) quantization of x[M][K] (M % 32 == 0, K % 32 == 0).  One wave
// owns a 128-row x 64-column tile.  Lane l = 8*g + c holds rows 16*g .. 16*g+15 of the
// tile and columns 8*c .. 8*c+7 (one 16-byte chunk per row, 16 chunks = 64 VGPRs):
//  * a 32x1 column block is held by the lane pair (g, g^1) -- 16 rows each -- so its
//    maximum is a lane-local packed max plus one DPP exchange between lanes 8 apart;
//  * a 1x32 row block is the quad of lanes c = 4k .. 4k+3 of one row (DPP);
//  * every load instruction reads 8 rows x 128 bytes (full lines);
//  * the columnwise copy q_col[K][M] is encoded as 16 bytes per lane and column (16 rows
//    of E4M3), so the 8 lanes g = 0..7 hold 128 contiguous bytes of one q_col row: the
//    transpose happens in registers.  The columnwise-only mode stores them directly; the
//    dual mode passes them through LDS first (see TILE_QCOL_LDS);
//  * the rowwise codes of the whole workgroup tile are staged in LDS and leave as
//    16-byte stores covering whole rows of the tile, so no store writes part of a line.
// A workgroup is WR x WC wave tiles (TileGeom).  Scale codes are gathered in LDS and
// leave as one store per row / column of the workgroup tile.
//
// Addressing: every pointer is a uniform (scalar) tile base plus a per-lane byte offset
// that does not change from tile to tile.  When all offsets inside a workgroup tile fit
// in 31 bits (OffT = uint32_t) the loads and stores take the scalar-base + 32-bit-offset
// form and no per-access vector address arithmetic is left; larger tensors use 64-bit
// offsets.  FULL (M and K multiples of the workgroup tile) drops every bounds mask.  In
// ragged tiles lanes outside the tensor load the tile origin instead (always inside the
// tensor, since M - row0 >= 32 for a tile that starts inside it) and skip their stores;
// because M and K are multiples of 32, a row quad or column pair never mixes lanes inside
// and outside the tensor.
constexpr int TILE_ROWS = 128;
constexpr int TILE_COLS = 64;
// Dual mode: the columnwise codes also go through LDS (CPITCH bytes per column), so that
// eight neighbouring lanes write each 128-byte line of q_col instead of eight lanes eight
// apart.  Measured: 2048 x 6144 dual 14.8 -> 12.4 us, 524288 x 2048 dual 891 -> 883 us,
// 65536 x 2048 unchanged; the columnwise-only mode is 1-3% slower that way on large
// tensors, so it keeps the direct stores.
#ifndef BSQ_TILE_QCOL_LDS
#define BSQ_TILE_QCOL_LDS 1
#endif
constexpr bool TILE_QCOL_LDS = BSQ_TILE_QCOL_LDS != 0;


// N scale bytes (N = 2, 4, 8 or 16) from LDS to an N-aligned global address.
template <int N>
__device__ __forceinline__ void store_scales(uint8_t* dst, const uint8_t* src) {
    if constexpr (N == 16) *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    else if constexpr (N == 8) *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
    else if constexpr (N == 4) *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(src);
    else *reinterpret_cast<uint16_t*>(dst) = *reinterpret_cast<const uint16_t*>(src);
}

// Workgroup geometry: WR x WC wave tiles (WR down the rows, WC along the columns).
template <int WR_, int WC_>
struct TileGeom {
    static constexpr int WR = WR_, WC = WC_;
    static constexpr int ROWS = TILE_ROWS * WR;     // workgroup tile rows
    static constexpr int COLS = TILE_COLS * WC;     // workgroup tile columns
    static constexpr int SROW_B = COLS / 32;        // row-scale bytes per row of the tile
    static constexpr int SCOL_B = ROWS / 32;        // column-scale bytes per column
    static constexpr int CPITCH = ROWS + 16;        // LDS row of one column's codes
    static constexpr int THREADS = 64 * WR * WC;
    static constexpr int QPITCH = COLS + 16;        // LDS row pitch of the staged q_row tile
};

// E8M0 code of a block from its maximum magnitude (BF16 bits, finite): E - 8 + [m > 0x60]
// clamped at 0, computed as (max(a - 0x3E1, 0)) >> 7 -- adding 0x1F carries into the
// exponent field exactly when the mantissa exceeds 0x60, and 0x400 = 8 << 7.
__device__ __forceinline__ uint32_t mx_code(uint32_t amax) {
    return __builtin_elementwise_sub_sat(amax, 0x3E1u) >> 7;
}
// Same for the high half of a packed pair (the low half only affects bits below 16).
__device__ __forceinline__ uint32_t mx_code_hi(uint32_t pair) {
    return __builtin_elementwise_sub_sat(pair, 0x3E1u << 16) >> 23;
}
// The scale operand of the scaled convert: the binary32 value 2^(c-127) (2^-127 is the
// subnormal 0x00400000, which the convert reads as exponent -127).
__device__ __forceinline__ float mx_scale(uint32_t c) {
    return __builtin_amdgcn_ldexpf(__uint_as_float(0x00400000u), (int)c);
}

__device__ __forceinline__ uint32_t pk_absmax(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}
// Both halves of a packed magnitude pair replaced by the larger one (one packed max with
// swapped halves); the result orders like the maximum itself under unsigned compares.
__device__ __forceinline__ uint32_t pk_fold(uint32_t m) {
    const u16x2 a = __builtin_bit_cast(u16x2, m);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, a.yx));
}

// Four E4M3 codes of the BF16 pairs w0 (bytes 0-1) and w1 (bytes 2-3) at one block scale.
// The convert writes half of its destination; `spare` is any value that is dead after
// the call, handed over as that destination so that no register has to be cleared.
__device__ __forceinline__ uint32_t cvt_e4m3x4_into(uint32_t spare, uint32_t w0, uint32_t w1, float scale) {
    short2_t r = __builtin_bit_cast(short2_t, spare);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, w0), scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, w1), scale, true);
    return __builtin_bit_cast(uint32_t, r);
}

// One 16-byte chunk (8 BF16 of one row) of a tile: folds its magnitudes into the lane's
// packed column maxima cm (two columns per dword) and, for the rowwise copy, returns its
// 8 E4M3 codes and the E8M0 code of its 1x32 block (the quad of lanes of the row).
template <bool ROW>
__device__ __forceinline__ uint2 tile_row_chunk(const uint4& v, uint32_t (&cm)[4], uint32_t& code) {
    const uint32_t a0 = v.x & 0x7FFF7FFFu, a1 = v.y & 0x7FFF7FFFu;
    const uint32_t a2 = v.z & 0x7FFF7FFFu, a3 = v.w & 0x7FFF7FFFu;
    cm[0] = pk_absmax(cm[0], a0);
    cm[1] = pk_absmax(cm[1], a1);
    cm[2] = pk_absmax(cm[2], a2);
    cm[3] = pk_absmax(cm[3], a3);
    if (!ROW) return make_uint2(0u, 0u);
    const uint32_t m = pk_absmax(pk_absmax(a0, a1), pk_absmax(a2, a3));
    code = mx_code_hi(quad_max(pk_fold(m)));
    const float sc = mx_scale(code);
    return make_uint2(cvt_e4m3x4_into(a0, v.x, v.y, sc), cvt_e4m3x4_into(a2, v.z, v.w, sc));
}

// The lane's packed column maxima over its 16 rows joined with the partner lane 8 apart
// (the other 16 rows of the 32-row block; DPP row_ror:8 within each 16-lane row).
__device__ __forceinline__ void tile_join_pairs(uint32_t (&cm)[4]) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
        cm[d] = pk_absmax(cm[d], (uint32_t)__builtin_amdgcn_mov_dpp((int)cm[d], 0x128, 0xF, 0xF, false));
}

// Columnwise codes of dword d of the lane's 16 rows: columns 2d (a, code0) and 2d+1 (b,
// code1), 16 rows each in row order.  Column-major pairs (row i, row i+1) of one column
// are built with one byte permute each, so one scaled convert (one scale = the column's)
// encodes two rows.
__device__ __forceinline__ void tile_col_codes(const uint4 (&v)[16], uint32_t cmd, int d, uint4& a, uint4& b,
                                               uint32_t& code0, uint32_t& code1) {
    code0 = mx_code(cmd & 0xFFFFu);
    code1 = mx_code_hi(cmd);
    const float sc0 = mx_scale(code0);
    const float sc1 = mx_scale(code1);
    uint32_t ra[4], rb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const uint32_t r0w = dword_of(v[4 * u + 0], d), r1w = dword_of(v[4 * u + 1], d);
        const uint32_t r2w = dword_of(v[4 * u + 2], d), r3w = dword_of(v[4 * u + 3], d);
        const uint32_t pa0 = __builtin_amdgcn_perm(r1w, r0w, 0x05040100u);
        const uint32_t pa1 = __builtin_amdgcn_perm(r3w, r2w, 0x05040100u);
        const uint32_t pb0 = __builtin_amdgcn_perm(r1w, r0w, 0x07060302u);
        const uint32_t pb1 = __builtin_amdgcn_perm(r3w, r2w, 0x07060302u);
        ra[u] = cvt_e4m3x4_into(pa0, pa0, pa1, sc0);
        rb[u] = cvt_e4m3x4_into(pb0, pb0, pb1, sc1);
    }
    a = make_uint4(ra[0], ra[1], ra[2], ra[3]);
    b = make_uint4(rb[0], rb[1], rb[2], rb[3]);
}

// The compiler would otherwise keep row-pass temporaries of the packed tile alive into
// the column pass (doubling the live tile); this empty register barrier pins the tile.
__device__ __forceinline__ void tile_pin(uint4 (&v)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
        asm volatile("" : "+v"(v[i].x), "+v"(v[i].y), "+v"(v[i].z), "+v"(v[i].w));
}

// Workgroup tile w -> first row and first column.
//   ORDER 0: row stripes in order, column groups fastest (the tiles in flight form one
//            band of full rows: contiguous reads and q_row writes)
//   ORDER 1: column groups in order, row stripes fastest (the tiles in flight form one
//            band of full columns: contiguous q_col writes)
template <class G, int ORDER>
__device__ __forceinline__ void tile_origin(int64_t w, int64_t row_stripes, int64_t col_groups,
                                            int64_t& rw, int64_t& kw) {
    if (ORDER == 0) {
        const int64_t s = w / col_groups;
        rw = s * G::ROWS;
        kw = (w - s * col_groups) * G::COLS;
    } else {
        const int64_t g = w / row_stripes;
        kw = g * G::COLS;
        rw = (w - g * row_stripes) * G::ROWS;
    }
}

// Per-lane constants of the tile layout.
template <typename OffT>
struct TileLane {
    int lrow, lcol;          // lane's first row / column inside the workgroup tile
    OffT xo, co;             // byte offsets from the tile origin in x and q_col
};

template <class G, typename OffT>
__device__ __forceinline__ TileLane<OffT> tile_lane(int64_t M, int64_t K) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    TileLane<OffT> t;
    t.lrow = (wave / G::WC) * TILE_ROWS + 16 * (lane >> 3);
    t.lcol = (wave % G::WC) * TILE_COLS + 8 * (lane & 7);
    t.xo = (OffT)(2 * ((int64_t)t.lrow * K + t.lcol));
    t.co = (OffT)((int64_t)t.lcol * M + t.lrow);
    return t;
}

template <bool FULL, typename OffT>
__device__ __forceinline__ void load_tile(uint4 (&v)[16], const uint16_t* __restrict__ x, int64_t M,
                                          int64_t K, int64_t rw, int64_t kw, const TileLane<OffT>& t) {
    const uint8_t* base = reinterpret_cast<const uint8_t*>(x + rw * K + kw);
    OffT o = t.xo;
    if (!FULL && !(rw + t.lrow < M && kw + t.lcol < K)) o = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        v[i] = ld_stream<MXTILE_NT_LOAD>(reinterpret_cast<const uint4*>(base + 2 * i * K + o));
}

// Everything after the load for one workgroup tile: both copies' codes and stores, the
// scale gather in LDS and the scale stores.  Called by every thread of the workgroup.
// The rowwise codes and scales of the workgroup tile, from LDS to global memory (after a
// barrier): 16-byte stores covering whole rows of the tile (COLS bytes each), instead of
// each wave writing 64-byte halves of the lines of its own columns.
template <class G, bool FULL>
__device__ __forceinline__ void store_rowwise_tile(int64_t M, int64_t K, int64_t rw, int64_t kw,
                                                   uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                                                   uint8_t (*lds_srow)[G::SROW_B], uint8_t (*lds_q)[G::QPITCH]) {
    constexpr int CHUNKS = G::COLS / 16;                      // 16-byte chunks per row
    uint8_t* qr = q_row + rw * K + kw;
#pragma unroll
    for (int j = 0; j < G::ROWS * CHUNKS / G::THREADS; ++j) {
        const int idx = j * G::THREADS + (int)threadIdx.x;
        const int r = idx / CHUNKS, c16 = idx % CHUNKS;
        const uint4 val = *reinterpret_cast<const uint4*>(&lds_q[r][16 * c16]);
        if (FULL || (rw + r < M && kw + 16 * c16 < K))
            st_stream<MXTILE_NT_STORE>(reinterpret_cast<uint4*>(qr + (int64_t)r * K + 16 * c16), val);
    }
    // SROW_B scale bytes per row of the workgroup tile
    const int64_t nb_row = K >> 5;
    const int64_t b0 = kw >> 5;
    const int nb = FULL ? G::SROW_B : (int)min((int64_t)G::SROW_B, nb_row - b0);
    const bool al = FULL || ((nb == G::SROW_B) && (nb_row % G::SROW_B) == 0);
#pragma unroll
    for (int r = threadIdx.x; r < G::ROWS; r += G::THREADS) {
        if (FULL || rw + r < M) {
            uint8_t* dst = s_row + (rw + r) * nb_row + b0;
            if (al) store_scales<G::SROW_B>(dst, lds_srow[r]);
            else for (int j = 0; j < nb; ++j) dst[j] = lds_srow[r][j];
        }
    }
}

// Everything after the load for one workgroup tile: both copies' codes and stores, the
// scale gather in LDS and the scale stores.  Called by every thread of the workgroup.
// (Sharing one LDS buffer between the staged rowwise and columnwise codes, with the
// rowwise codes stored before the column pass, was measured slower in spite of the higher
// occupancy: 65536 x 2048 dual 100.9 -> 103.2 us, 2048 x 6144 12.6 -> 14.1 us.)
template <class G, bool ROW, bool FULL, typename OffT>
__device__ __forceinline__ void process_tile(uint4 (&v)[16], int64_t M, int64_t K, int64_t rw, int64_t kw,
                                             const TileLane<OffT>& t,
                                             uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                                             uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col,
                                             uint8_t (*lds_srow)[G::SROW_B], uint8_t (*lds_scol)[G::SCOL_B],
                                             uint8_t (*lds_q)[G::QPITCH], uint8_t (*lds_c)[G::CPITCH]) {
    constexpr bool QSTAGE = TILE_QCOL_LDS && ROW;             // columnwise codes through LDS
    const bool ok = FULL || (rw + t.lrow < M && kw + t.lcol < K);
    uint8_t* qc = q_col + kw * M + rw;

    // ---- rowwise copy (each row of the lane; block = quad of lanes) and the packed
    //      column maxima over the lane's 16 rows, from one set of magnitudes
    uint32_t cm[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        uint32_t code = 0u;
        const uint2 out = tile_row_chunk<ROW>(v[i], cm, code);
        if (ROW) {
            *reinterpret_cast<uint2*>(&lds_q[t.lrow + i][t.lcol]) = out;
            lds_srow[t.lrow + i][t.lcol >> 5] = (uint8_t)code;   // the quad writes one value
        }
    }
    if (ROW) tile_pin(v);

    // ---- columnwise copy
    tile_join_pairs(cm);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint4 a, b;
        uint32_t code0, code1;
        tile_col_codes(v, cm[d], d, a, b, code0, code1);
        if (QSTAGE) {
            *reinterpret_cast<uint4*>(&lds_c[t.lcol + 2 * d][t.lrow]) = a;
            *reinterpret_cast<uint4*>(&lds_c[t.lcol + 2 * d + 1][t.lrow]) = b;
        } else if (ok) {
            uint8_t* ra = qc + (int64_t)(t.lcol + 2 * d) * M;     // this column's run: the tile's rows
            uint8_t* rb = ra + M;
            const int64_t rn = min((int64_t)G::ROWS, M - rw);
            if (FULL) {
                st_stream<MXTILE_NT_STORE>(reinterpret_cast<uint4*>(qc + (2 * d) * M + t.co), a);
                st_stream<MXTILE_NT_STORE>(reinterpret_cast<uint4*>(qc + (2 * d + 1) * M + t.co), b);
            } else {
                st_run<MXTILE_NT_STORE>(reinterpret_cast<uint4*>(qc + (2 * d) * M + t.co), a, ra, ra + rn);
                st_run<MXTILE_NT_STORE>(reinterpret_cast<uint4*>(qc + (2 * d + 1) * M + t.co), b, rb, rb + rn);
            }
        }
        lds_scol[t.lcol + 2 * d][t.lrow >> 5] = (uint8_t)code0;      // the lane pair writes
        lds_scol[t.lcol + 2 * d + 1][t.lrow >> 5] = (uint8_t)code1;  // one value each
    }

    __syncthreads();
    // the rowwise copy leaves first (65536 x 2048 dual 101.2 -> 99.8 us, 196608 x 2048 303.8
    // -> 298.6 us, measured against storing it after the columnwise copy)
    if (ROW) store_rowwise_tile<G, FULL>(M, K, rw, kw, q_row, s_row, lds_srow, lds_q);
    if (QSTAGE) {
        // columnwise codes, staged in LDS: eight neighbouring lanes write one 128-byte line
        constexpr int PARTS = G::ROWS / 16;                   // 16-byte chunks per column
#pragma unroll
        for (int j = 0; j < G::COLS * PARTS / G::THREADS; ++j) {
            const int idx = j * G::THREADS + (int)threadIdx.x;
            const int c = idx / PARTS, part = idx % PARTS;
            const uint4 val = *reinterpret_cast<const uint4*>(&lds_c[c][16 * part]);
            if (FULL || (kw + c < K && rw + 16 * part < M))
            {
                uint8_t* run = qc + (int64_t)c * M;
                if (FULL) st_stream<MXTILE_NT_STORE>(reinterpret_cast<uint4*>(run + 16 * part), val);
                else st_run<MXTILE_NT_STORE>(reinterpret_cast<uint4*>(run + 16 * part), val, run, run + min((int64_t)G::ROWS, M - rw));
            }
        }
    }
    // columnwise scales: SCOL_B bytes per column of the workgroup tile
    {
        const int64_t nb_col = M >> 5;
        const int64_t b0 = rw >> 5;
        const int nb = FULL ? G::SCOL_B : (int)min((int64_t)G::SCOL_B, nb_col - b0);
        const bool al = FULL || ((nb == G::SCOL_B) && (nb_col % G::SCOL_B) == 0);
#pragma unroll
        for (int c = threadIdx.x; c < G::COLS; c += G::THREADS) {
            if (FULL || kw + c < K) {
                uint8_t* dst = s_col + (kw + c) * nb_col + b0;
                if (al) store_scales<G::SCOL_B>(dst, lds_scol[c]);
                else for (int j = 0; j < nb; ++j) dst[j] = lds_scol[c][j];
            }
        }
    }
}

// One workgroup tile per workgroup.
template <class G, bool ROW, bool FULL, typename OffT, int ORDER>
__global__ __launch_bounds__(G::THREADS)
void mx_quant_tile_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                          uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                          uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col,
                          int64_t row_stripes, int64_t col_groups) {
    __shared__ __align__(16) uint8_t lds_srow[G::ROWS][G::SROW_B];
    __shared__ __align__(16) uint8_t lds_scol[G::COLS][G::SCOL_B];
    __shared__ __align__(16) uint8_t lds_q[ROW ? G::ROWS : 1][G::QPITCH];
    __shared__ __align__(16) uint8_t lds_c[TILE_QCOL_LDS && ROW ? G::COLS : 1][G::CPITCH];
    int64_t rw, kw;
    tile_origin<G, ORDER>(blockIdx.x, row_stripes, col_groups, rw, kw);
    const TileLane<OffT> t = tile_lane<G, OffT>(M, K);
    uint4 v[16];
    // The wave issues its tile's loads at raised priority, so that the waves of newly started
    // tiles get their reads out ahead of the arithmetic and stores of the others: dual
    // 65536 x 2048 99.8 -> 98.2 us (with the rowwise copy stored first; 101.2 before either),
    // the step 6135 -> 6147 GB/s (means of three interleaved runs).
    __builtin_amdgcn_s_setprio(3);
    load_tile<FULL>(v, x, M, K, rw, kw, t);
    __builtin_amdgcn_s_setprio(0);
    process_tile<G, ROW, FULL>(v, M, K, rw, kw, t, q_row, s_row, q_col, s_col, lds_srow, lds_scol, lds_q, lds_c);
}

// Persistent variant: each workgroup walks tiles blockIdx.x, blockIdx.x + gridDim.x, ...
// and issues the loads of its next tile before encoding the current one, so HBM reads
// stay in flight while the codes are computed and stored.
template <class G, bool ROW, bool FULL, typename OffT, int ORDER>
__global__ __launch_bounds__(G::THREADS)
void mx_quant_tile_persistent_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                     uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                                     uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col,
                                     int64_t row_stripes, int64_t col_groups) {
    __shared__ __align__(16) uint8_t lds_srow[G::ROWS][G::SROW_B];
    __shared__ __align__(16) uint8_t lds_scol[G::COLS][G::SCOL_B];
    __shared__ __align__(16) uint8_t lds_q[ROW ? G::ROWS : 1][G::QPITCH];
    __shared__ __align__(16) uint8_t lds_c[TILE_QCOL_LDS && ROW ? G::COLS : 1][G::CPITCH];
    const int64_t n_wg = row_stripes * col_groups;
    const TileLane<OffT> t = tile_lane<G, OffT>(M, K);
    int64_t w = blockIdx.x;
    if (w >= n_wg) return;                     // uniform over the workgroup
    int64_t rw, kw;
    tile_origin<G, ORDER>(w, row_stripes, col_groups, rw, kw);
    uint4 v[16];
    load_tile<FULL>(v, x, M, K, rw, kw, t);
    for (;;) {
        const int64_t wn = w + gridDim.x;
        int64_t rn = 0, kn = 0;
        uint4 vn[16];
        if (wn < n_wg) {
            tile_origin<G, ORDER>(wn, row_stripes, col_groups, rn, kn);
            load_tile<FULL>(vn, x, M, K, rn, kn, t);

        }
        process_tile<G, ROW, FULL>(v, M, K, rw, kw, t, q_row, s_row, q_col, s_col, lds_srow, lds_scol, lds_q, lds_c);
        if (wn >= n_wg) break;
        __syncthreads();                       // LDS is reused by the next tile
        w = wn;
        rw = rn;
        kw = kn;
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = vn[i];
    }
}

template <class G, bool ROW, bool FULL, typename OffT, int ORDER>
static void launch_tile_geom(const void* x, int64_t M, int64_t K, void* q_row, void* s_row, void* q_col,
                             void* s_col, hipStream_t stream, int64_t persistent_wgs) {
    const int64_t row_stripes = (M + G::ROWS - 1) / G::ROWS;
    const int64_t col_groups = (K + G::COLS - 1) / G::COLS;
    const int64_t n_wg = row_stripes * col_groups;
    if (persistent_wgs > 0 && persistent_wgs < n_wg) {
        hipLaunchKernelGGL((mx_quant_tile_persistent_kernel<G, ROW, FULL, OffT, ORDER>), dim3((unsigned)persistent_wgs),
                           dim3(G::THREADS), 0, stream, (const uint16_t*)x, M, K, (uint8_t*)q_row,
                           (uint8_t*)s_row, (uint8_t*)q_col, (uint8_t*)s_col, row_stripes, col_groups);
    } else {
        hipLaunchKernelGGL((mx_quant_tile_kernel<G, ROW, FULL, OffT, ORDER>), dim3((unsigned)n_wg), dim3(G::THREADS),
                           0, stream, (const uint16_t*)x, M, K, (uint8_t*)q_row, (uint8_t*)s_row,
                           (uint8_t*)q_col, (uint8_t*)s_col, row_stripes, col_groups);
    }
}

// Offsets inside one workgroup tile: x up to 2*ROWS*K bytes, q_col up to COLS*M bytes.
template <class G>
static bool tile_offsets_fit_32(int64_t M, int64_t K) {
    return 2 * (int64_t)G::ROWS * K < (int64_t(1) << 31) && (int64_t)G::COLS * M < (int64_t(1) << 31);
}

template <class G, bool ROW, int ORDER>
static void launch_tile(const void* x, int64_t M, int64_t K, void* q_row, void* s_row, void* q_col,
                        void* s_col, hipStream_t stream, int64_t persistent_wgs) {
    const bool full = (M % G::ROWS) == 0 && (K % G::COLS) == 0;
    if (tile_offsets_fit_32<G>(M, K)) {
        if (full) launch_tile_geom<G, ROW, true, uint32_t, ORDER>(x, M, K, q_row, s_row, q_col, s_col, stream, persistent_wgs);
        else launch_tile_geom<G, ROW, false, uint32_t, ORDER>(x, M, K, q_row, s_row, q_col, s_col, stream, persistent_wgs);
    } else {
        if (full) launch_tile_geom<G, ROW, true, int64_t, ORDER>(x, M, K, q_row, s_row, q_col, s_col, stream, persistent_wgs);
        else launch_tile_geom<G, ROW, false, int64_t, ORDER>(x, M, K, q_row, s_row, q_col, s_col, stream, persistent_wgs);
    }
}

// Geometry, tile order and persistent workgroup count used by the library for the
// columnwise-only mode (0 = one tile per workgroup always; otherwise used once a tensor
// has more than twice as many tiles); the dual mode always runs one tile per workgroup.
// Measured on the 65536 x 2048 activations (dual, one launch after a 512 MiB read, before
// the dual mode staged its columnwise codes in LDS): 1x4 row-band 105.6 us with 256
// persistent workgroups, 106.2 us with one tile per workgroup; 2x2 106.5, 1x8 108.2, 2x4
// 115.5; column-band order 138-170.  With the LDS staging the persistent form needs 208
// VGPRs for its two tiles and one tile per workgroup is faster in the dual mode: 106.3 ->
// 101.0 us (65536 x 2048), 325 -> 305 us (196608 x 2048), 882 -> 802 us (524288 x 2048),
// and the layer step 6115 -> 6145 GB/s; the columnwise-only mode stays faster persistent
// (78.6 against 81.3 us, 240 against 250 us).
#ifndef BSQ_TILE_WR
#define BSQ_TILE_WR 1
#endif
#ifndef BSQ_TILE_WC
#define BSQ_TILE_WC 4
#endif
#ifndef BSQ_TILE_ORDER
#define BSQ_TILE_ORDER 0
#endif
#ifndef BSQ_TILE_PERSISTENT_WGS
#define BSQ_TILE_PERSISTENT_WGS 256
#endif
using LibTile = TileGeom<BSQ_TILE_WR, BSQ_TILE_WC>;
constexpr int TILE_ORDER = BSQ_TILE_ORDER;
constexpr int TILE_PERSISTENT_WGS = BSQ_TILE_PERSISTENT_WGS;

// ----------------------------------------------------------------------------- grouped col / both

// Columnwise (and dual) MXFP8 over expert segments of the rows, for the weight-gradient
// operand of MoE experts.  Page "Towards Blackwell-native 8-bit and 4-bit RL", section
// "Recipe 1: end-to-end MXFP8 RL": the experts run in MXFP8 including the weight-gradient
// GEMM, whose operand is the columnwise copy, and each expert's GEMM reduces over its own
// rows only.  So a 32x1 block never crosses an expert boundary: expert e's m_e rows form
// ceil(m_e / 32) blocks from its first row, the last one partial when m_e % 32 != 0 (its
// scale comes from the rows present).  Blocks are numbered in row order over all experts;
// q_col keeps the flat [K][M] layout and s_col[K][s_ld] holds block n at entry n of every
// row.  The rowwise copy is row-local, identical to the flat one.
//
// One kernel serves both modes; its workgroups own 128-row windows of the rows (one 128-byte
// line of every q_col row they touch).  Lines of q_col that two workgroups each fill in
// part cost far more than their bytes: an earlier kernel that gave each workgroup four
// consecutive blocks (and so split lines wherever segments start off a 32-row boundary)
// took 980 us for the dual mode on 524288 x 2048 Zipf-routed rows, timed with the
// write-back of the lines it left dirty, against 858 us for the window kernel.  Block
// indices are 32-bit (ceil(M/32) + E < 2^31, checked by the caller).

__device__ __forceinline__ int64_t clamp_row(int64_t r, int64_t M) { return r < 0 ? 0 : (r > M ? M : r); }

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int32_t wave_incl_scan(int32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    return v;
}

// Wave 0 of workgroup 0: offsets valid (o[0] = 0, non-decreasing, o[E] = M) and the
// total block count within s_ld?
__device__ void group_check(const int64_t* __restrict__ off, int64_t E, int64_t M, int64_t s_ld,
                            int32_t* __restrict__ status) {
    const int lane = threadIdx.x & 63;
    bool bad = false;
    int64_t blocks = 0;
    for (int64_t e = lane; e < E; e += 64) {
        const int64_t lo = off[e], hi = off[e + 1];
        bad |= hi < lo;
        if (hi > lo) blocks += (hi - lo + 31) >> 5;
    }
    if (lane == 0) bad |= (off[0] != 0) || (off[E] != M);
    for (int o = 32; o > 0; o >>= 1) blocks += __shfl_xor(blocks, o, 64);
    bad |= blocks > s_ld;
    const bool any_bad = __any(bad);
    if (lane == 0) *status = any_bad ? 6 /* BSQ_ERR_OFFSETS */ : 0;
}

// A workgroup owns a window of 128 rows (one 128-byte line of every q_col row it touches)
// and 256 columns.  Its table lists the blocks that overlap the window, in row order: with
// segments of 32 rows or more, four or five, the first and last possibly reaching outside.
constexpr int WIN_ROWS = 128;
constexpr int WIN_SLOTS = 8;                          // blocks per pass of the block-slot path
constexpr int WIN_TAB = WIN_ROWS;                     // each overlapping block holds a window row

struct WindowTable {
    int64_t start[WIN_TAB];        // first row of each overlapping block, in row order
    int64_t n[WIN_TAB];            // its global block index
    int32_t len[WIN_TAB];          // its row count (1..32); 0 for an unused entry
    int32_t count;
};

// Wave 0: the blocks that overlap rows [w0, w0 + WIN_ROWS).  Offsets are clamped into
// [0, M]; with invalid offsets entries may be missing (len 0), never out of bounds.
__device__ void window_find_blocks(const int64_t* __restrict__ off, int64_t E, int64_t M, int64_t w0,
                                   int64_t n_limit, WindowTable& tab) {
    const int lane = threadIdx.x & 63;
    const int64_t w1 = w0 + WIN_ROWS;
    for (int i = lane; i < WIN_TAB; i += 64) { tab.start[i] = w0; tab.n[i] = 0; tab.len[i] = 0; }
    int64_t base = 0;                                  // blocks of the experts before e0
    int32_t slots = 0;                                 // table entries so far
    for (int64_t e0 = 0; e0 < E; e0 += 64) {
        if (clamp_row(off[e0], M) >= w1) break;        // uniform; later segments start past the window
        const int64_t e = e0 + lane;
        const int64_t lo = e < E ? clamp_row(off[e], M) : M;
        const int64_t hi = e < E ? clamp_row(off[e + 1], M) : M;
        const int32_t c = hi > lo ? (int32_t)((hi - lo + 31) >> 5) : 0;
        const int32_t incl = wave_incl_scan(c);
        const int64_t excl = base + (incl - c);
        int32_t jf = 0, cnt = 0;
        if (c > 0 && hi > w0 && lo < w1) {
            jf = w0 > lo ? (int32_t)((w0 - lo) >> 5) : 0;
            const int32_t jl = min(c - 1, (int32_t)((w1 - 1 - lo) >> 5));
            cnt = max(jl - jf + 1, 0);
        }
        const int32_t sincl = wave_incl_scan(cnt);
        const int32_t s0 = slots + (sincl - cnt);
        for (int32_t k = 0; k < cnt; ++k) {
            const int32_t sl = s0 + k;
            const int64_t n = excl + jf + k;
            if (sl < WIN_TAB && n < n_limit) {
                const int64_t r = lo + 32 * (int64_t)(jf + k);   // < hi <= M
                tab.start[sl] = r;
                tab.n[sl] = n;
                tab.len[sl] = (int32_t)(hi - r < 32 ? hi - r : 32);
            }
        }
        base += __shfl(incl, 63, 64);
        slots += __shfl(sincl, 63, 64);
    }
    if (lane == 0) tab.count = slots < WIN_TAB ? slots : WIN_TAB;
}

// Packed column maxima joined with the partner lane 4 apart (the other half of the block).
__device__ __forceinline__ void win_join_pairs(uint32_t (&cm)[4]) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
        cm[d] = pk_absmax(cm[d], (uint32_t)__builtin_amdgcn_ds_swizzle((int)cm[d], 0x101F));  // lane ^ 4
}

// The window kernel.  Each wave holds the window's rows in the flat tile's layout (lane
// 8g + c holds window rows 16g .. 16g+15, columns 8c .. 8c+7 of its wave's 64), so every
// lane works on rows of the window and the rowwise copy (ROWWISE) costs what it costs in
// the flat kernel.  The 32x1 block maxima are segmented: each lane folds its rows into at
// most two partial maxima (the fast path requires that no lane's rows meet three blocks,
// which holds whenever every block has 16 rows or more), the rows of the blocks that reach
// outside the window are folded too (one list of four rows a lane when both edge blocks
// lie in one segment), and the partial maxima meet in an LDS table of the window's blocks
// (ds_max per column; each wave has its own table for its 64 columns, so only a wave
// barrier waits for it).  Each row is then encoded with its own block's scale: the codes
// of a lane's rows before and after its block boundary come from two converts and a byte
// select (one convert when no lane of the wave has a boundary inside its rows).  The
// columnwise codes leave as one 16-byte store per lane and column, eight lanes filling a
// q_col line.  Other windows (more than DW_BLOCKS blocks, or a lane meeting three) take a
// block-slot path: lane 4 rg + c holds rows 16 (rg & 1) .. + 15 of block slot rg >> 1, 32
// columns at a time, a block whose rows reach outside the window is loaded whole and only
// the window's rows are stored.  A FULL variant (M % 128 == 0, K % 256 == 0) drops the
// bounds masks.
// Launched for three workgroups per compute unit (168 VGPRs for the dual mode, where the
// compiler spills a few 64-bit values, 28 bytes a lane, outside the per-row work; 152 for
// the columnwise mode).  On the 524288 x 2048 Zipf-routed rows, on one box: dual mode 858
// us (892 before the FULL variant and the shared edge list, 1010 at two workgroups per
// compute unit); issuing the window loads before the block table is built, so that the
// table's lookups overlap them, measured 10 us slower.  Columnwise mode 651 us against 682
// for a block-slot kernel of eight waves (half its lanes idle on aligned windows; it wins
// only there, 603 against 620 us).
constexpr int DW_BLOCKS = 8;


// Bytes k of a 4-row group whose row 4u + k lies before the boundary b (t = b - 4u).
__device__ __forceinline__ uint32_t split_mask(int t) {
    return t <= 0 ? 0u : t >= 4 ? 0xFFFFFFFFu : (1u << (8 * t)) - 1u;
}

// Columnwise codes of dword d of the lane's 16 rows, rows [0, b) at the scales (sA0, sA1)
// of columns 2d and 2d+1, rows [b, 16) at (sB0, sB1).
__device__ __forceinline__ void tile_col_codes_split(const uint4 (&v)[16], int d, int b, float sA0, float sA1,
                                                     float sB0, float sB1, uint4& a, uint4& bo) {
    uint32_t ra[4], rb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const uint32_t r0w = dword_of(v[4 * u + 0], d), r1w = dword_of(v[4 * u + 1], d);
        const uint32_t r2w = dword_of(v[4 * u + 2], d), r3w = dword_of(v[4 * u + 3], d);
        const uint32_t pa0 = __builtin_amdgcn_perm(r1w, r0w, 0x05040100u);
        const uint32_t pa1 = __builtin_amdgcn_perm(r3w, r2w, 0x05040100u);
        const uint32_t pb0 = __builtin_amdgcn_perm(r1w, r0w, 0x07060302u);
        const uint32_t pb1 = __builtin_amdgcn_perm(r3w, r2w, 0x07060302u);
        const uint32_t aA = cvt_e4m3x4_into(pa0, pa0, pa1, sA0);
        const uint32_t bA = cvt_e4m3x4_into(pb0, pb0, pb1, sA1);
        if (b >= 16) { ra[u] = aA; rb[u] = bA; continue; }
        const uint32_t m = split_mask(b - 4 * u);
        const uint32_t aB = cvt_e4m3x4_into(pa1, pa0, pa1, sB0);
        const uint32_t bB = cvt_e4m3x4_into(pb1, pb0, pb1, sB1);
        ra[u] = (aA & m) | (aB & ~m);
        rb[u] = (bA & m) | (bB & ~m);
    }
    a = make_uint4(ra[0], ra[1], ra[2], ra[3]);
    bo = make_uint4(rb[0], rb[1], rb[2], rb[3]);
}

// The 8 column maxima of a lane (packed pairs) into row j of the block table.
__device__ __forceinline__ void dw_put(uint32_t (*bmax)[TILE_COLS], int j, int lcol, const uint32_t (&cm)[4]) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
        atomicMax(&bmax[j][lcol + e], (e & 1) ? (cm[e >> 1] >> 16) : (cm[e >> 1] & 0xFFFFu));
}

typedef uint32_t u32x4u_t __attribute__((ext_vector_type(4), aligned(1)));

#ifndef BSQ_GRP_WGS_PER_CU
#define BSQ_GRP_WGS_PER_CU 3
#endif
template <bool FULL, bool ROWWISE>
__global__ __launch_bounds__(256, BSQ_GRP_WGS_PER_CU)
void mx_quant_grouped_window_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                         const int64_t* __restrict__ off, int64_t E,
                                         uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                                         uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col, int64_t s_ld,
                                         int64_t n_limit, int64_t col_groups, int32_t* __restrict__ status) {
    using G = TileGeom<1, 4>;                          // 128 rows x 256 columns, 4 waves
    __shared__ WindowTable tab;
    __shared__ __align__(16) uint8_t lds_srow[ROWWISE ? G::ROWS : 1][G::SROW_B];
    __shared__ __align__(16) uint8_t lds_q[ROWWISE ? G::ROWS : 1][G::QPITCH];
    __shared__ uint32_t bmax_w[4][DW_BLOCKS][TILE_COLS];       // per wave: its 64 columns
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t win = blockIdx.x / col_groups;
    const int64_t kw = (blockIdx.x - win * col_groups) * G::COLS;
    const int64_t w0 = win * WIN_ROWS, w1 = w0 + WIN_ROWS;
    if (wave == 0) window_find_blocks(off, E, M, w0, n_limit, tab);
    if (wave == 1 && status != nullptr && blockIdx.x == 0) group_check(off, E, M, s_ld, status);
    __syncthreads();
    const int count = tab.count;
    // fast path: every lane's 16 rows meet at most two blocks, i.e. no block that starts off a
    // lane's first row is followed by another start among the same lane's rows (uniform)
    bool fast = count >= 1 && count <= DW_BLOCKS;
    for (int j = 1; j + 1 < count && fast; ++j) {
        const int64_t a = tab.start[j] - w0, b = tab.start[j + 1] - w0;   // 0 < a < b < WIN_ROWS
        fast = (a & 15) == 0 || (a >> 4) != (b >> 4);
    }

    if (fast) {
        const int g = lane >> 3, c = lane & 7;
        const int lcol = wave * TILE_COLS + 8 * c;
        const int64_t col = kw + lcol;
        const bool colok = FULL || col < K;
        const uint16_t* xc = x + (colok ? col : kw);
        uint32_t (*bmax)[TILE_COLS] = bmax_w[wave];
        const int wcol = 8 * c;                        // the lane's first column in the wave
#pragma unroll
        for (int i = 0; i < DW_BLOCKS; ++i) bmax[i][lane] = 0u;
        const int64_t r0 = w0 + 16 * g;                // the lane's first row
        const int hi = FULL ? 16 : (int)max<int64_t>(min<int64_t>(M - r0, 16), 0);   // its rows in the tensor
        // rows of the blocks that reach outside the window, folded before the window rows are
        // loaded (fewer registers live at once): nh rows before it and nt after it, 1..31 each.
        // Inside one segment nh + nt = 32, and the two lists share one set of four loads a lane;
        // otherwise each list takes four.
        const int64_t hs = tab.start[0];               // head block, if it starts before w0
        const int64_t te = tab.start[count - 1] + tab.len[count - 1];   // tail block's end
        const bool head = hs < w0, tail = te > w1;     // uniform
        const int nh = head ? (int)(w0 - hs) : 0, nt = tail ? (int)(te - w1) : 0;
        uint32_t ch[4] = {0u, 0u, 0u, 0u}, ct[4] = {0u, 0u, 0u, 0u};
        // loads at raised priority, as in the flat kernel (dual 849 -> 833 us, columnwise 652 ->
        // 638 us on the Zipf-routed rows)
        __builtin_amdgcn_s_setprio(3);
        if ((head || tail) && nh + nt <= 32) {
            uint4 e[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int idx = 4 * g + t;             // entry of the list [hs, w0) ++ [w1, te)
                const int64_t r = idx < nh ? hs + idx : idx < nh + nt ? w1 + (idx - nh) : w0;
                e[t] = ld_stream<MXGRP_NT_LOAD>(reinterpret_cast<const uint4*>(xc + r * K));
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int idx = 4 * g + t;
                const bool vh = idx < nh, vt = idx >= nh && idx < nh + nt;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t m = dword_of(e[t], d) & 0x7FFF7FFFu;
                    ch[d] = pk_absmax(ch[d], vh ? m : 0u);
                    ct[d] = pk_absmax(ct[d], vt ? m : 0u);
                }
            }
        } else if (head || tail) {
            uint4 eh[4], et[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int64_t rh = w0 - 32 + 4 * g + t, rt = w1 + 4 * g + t;
                eh[t] = ld_stream<MXGRP_NT_LOAD>(reinterpret_cast<const uint4*>(xc + (head && rh >= hs ? rh : w0) * K));
                et[t] = ld_stream<MXGRP_NT_LOAD>(reinterpret_cast<const uint4*>(xc + (tail && rt < te ? rt : w0) * K));
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bool vh = head && w0 - 32 + 4 * g + t >= hs, vt = tail && w1 + 4 * g + t < te;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    ch[d] = vh ? pk_absmax(ch[d], dword_of(eh[t], d) & 0x7FFF7FFFu) : ch[d];
                    ct[d] = vt ? pk_absmax(ct[d], dword_of(et[t], d) & 0x7FFF7FFFu) : ct[d];
                }
            }
        }
        uint4 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            v[i] = ld_stream<MXGRP_NT_LOAD>(reinterpret_cast<const uint4*>(xc + (i < hi ? r0 + i : w0) * K));
        __builtin_amdgcn_s_setprio(0);
        // rowwise codes, staged in LDS
#pragma unroll
        for (int i = 0; i < 16 && ROWWISE; ++i) {
            uint32_t code = 0u, unused[4] = {0u, 0u, 0u, 0u};
            const uint2 out = tile_row_chunk<true>(v[i], unused, code);
            if (i < hi) {
                *reinterpret_cast<uint2*>(&lds_q[16 * g + i][lcol]) = out;
                lds_srow[16 * g + i][lcol >> 5] = (uint8_t)code;
            }
        }
        tile_pin(v);
        // the lane's blocks: ja holds rows [0, b), ja + 1 rows [b, hi)
        int ja = 0;
        for (int j = 1; j < count; ++j) ja = tab.start[j] <= r0 ? j : ja;
        const int jb = ja + 1 < count ? ja + 1 : ja;
        const int b = ja + 1 < count ? (int)max<int64_t>(min<int64_t>(tab.start[ja + 1] - r0, 16), 0) : 16;
        uint32_t ca[4] = {0u, 0u, 0u, 0u}, cb[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const bool in_a = i < b && i < hi, in_b = i >= b && i < hi;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t m = dword_of(v[i], d) & 0x7FFF7FFFu;
                ca[d] = in_a ? pk_absmax(ca[d], m) : ca[d];
                cb[d] = in_b ? pk_absmax(cb[d], m) : cb[d];
            }
        }
        if (hi > 0) dw_put(bmax, ja, wcol, ca);
        if (b < hi) dw_put(bmax, jb, wcol, cb);
        if (head) dw_put(bmax, 0, wcol, ch);
        if (tail) dw_put(bmax, count - 1, wcol, ct);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // the wave's own table
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // scales of the lane's two blocks, column codes, stores
        uint32_t codeA[8], codeB[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            codeA[e] = mx_code(bmax[ja][wcol + e]);
            codeB[e] = mx_code(bmax[jb][wcol + e]);
        }
        const bool own_a = hi > 0 && tab.start[ja] == r0 && colok;   // block ja starts at row r0
        const bool own_b = b < hi && colok;                           // block jb starts inside
        const int64_t na = tab.n[ja], nb = tab.n[jb];
        const bool one_block = __builtin_amdgcn_ballot_w64(b < hi) == 0;   // no lane of the wave splits
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint4 a, bo;
            if (one_block)
                tile_col_codes_split(v, d, 16, mx_scale(codeA[2 * d]), mx_scale(codeA[2 * d + 1]),
                                     mx_scale(codeA[2 * d]), mx_scale(codeA[2 * d + 1]), a, bo);
            else
                tile_col_codes_split(v, d, b, mx_scale(codeA[2 * d]), mx_scale(codeA[2 * d + 1]),
                                     mx_scale(codeB[2 * d]), mx_scale(codeB[2 * d + 1]), a, bo);
            if (colok && hi > 0) {
                uint8_t* pa = q_col + (col + 2 * d) * M + r0;
                uint8_t* pb = pa + M;
                // the window's run of this column: rows w0 .. min(w1, M) - 1; a 16-byte piece
                // goes non-temporal only inside a line the run covers whole (see st_run)
                const uintptr_t la = reinterpret_cast<uintptr_t>(pa) & ~(uintptr_t)127;
                const uintptr_t lb = reinterpret_cast<uintptr_t>(pb) & ~(uintptr_t)127;
                const uintptr_t ra0 = reinterpret_cast<uintptr_t>(pa) - (uintptr_t)(r0 - w0);
                const uintptr_t rlen = (uintptr_t)(FULL ? WIN_ROWS : min<int64_t>(WIN_ROWS, M - w0));
                const bool nta = FULL || (la >= ra0 && la + 128 <= ra0 + rlen);
                const bool ntb = FULL || (lb >= ra0 + M && lb + 128 <= ra0 + M + rlen);
                if (hi == 16) {
                    if (nta) __builtin_nontemporal_store(u32x4_t{a.x, a.y, a.z, a.w}, reinterpret_cast<u32x4u_t*>(pa));
                    else __builtin_memcpy(pa, &a, 16);
                    if (ntb) __builtin_nontemporal_store(u32x4_t{bo.x, bo.y, bo.z, bo.w}, reinterpret_cast<u32x4u_t*>(pb));
                    else __builtin_memcpy(pb, &bo, 16);
                } else {
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        if (j < hi) {
                            pa[j] = (uint8_t)(dword_of(a, j >> 2) >> (8 * (j & 3)));
                            pb[j] = (uint8_t)(dword_of(bo, j >> 2) >> (8 * (j & 3)));
                        }
                    }
                }
            }
            if (own_a) {
                s_col[(col + 2 * d) * s_ld + na] = (uint8_t)codeA[2 * d];
                s_col[(col + 2 * d + 1) * s_ld + na] = (uint8_t)codeA[2 * d + 1];
            }
            if (own_b) {
                s_col[(col + 2 * d) * s_ld + nb] = (uint8_t)codeB[2 * d];
                s_col[(col + 2 * d + 1) * s_ld + nb] = (uint8_t)codeB[2 * d + 1];
            }
        }
    } else {
        // block-slot path: lane 4 rg + c, 32 columns at a time (two halves of the wave's 64)
        const int rg = lane >> 2, c = lane & 3;
        const int slot = rg >> 1, half = rg & 1;
        for (int h2 = 0; h2 < 2; ++h2) {
            const int lcol = wave * TILE_COLS + 32 * h2 + 8 * c;
            const int64_t col = kw + lcol;
            const bool colok = col < K;
            const uint16_t* xc = x + (colok ? col : kw);
            for (int p = 0; p * WIN_SLOTS < count; ++p) {
                const int sl = WIN_SLOTS * p + slot;
                const int blen = sl < count ? tab.len[sl] : 0;
                const int64_t bstart = blen > 0 ? tab.start[sl] : tab.start[WIN_SLOTS * p];
                const int last = (blen > 0 ? blen : 1) - 1;
                const int64_t r0 = bstart + 16 * half;
                uint4 v[16];
                __builtin_amdgcn_s_setprio(3);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int ri = min(16 * half + i, last);
                    v[i] = ld_stream<MXGRP_NT_LOAD>(reinterpret_cast<const uint4*>(xc + (bstart + ri) * K));
                }
                __builtin_amdgcn_s_setprio(0);
                const int vc = min(max(blen - 16 * half, 0), 16);
                const int ilo = (int)max<int64_t>(w0 - r0, 0);
                const int ihi = (int)min<int64_t>(w1 - r0, (int64_t)vc);
                uint32_t cm[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    uint32_t code = 0u;
                    const uint2 out = tile_row_chunk<ROWWISE>(v[i], cm, code);
                    if (ROWWISE && i >= ilo && i < ihi) {
                        const int wr = (int)(r0 - w0) + i;             // 0 <= wr < WIN_ROWS
                        *reinterpret_cast<uint2*>(&lds_q[wr][lcol]) = out;
                        lds_srow[wr][lcol >> 5] = (uint8_t)code;
                    }
                }
                tile_pin(v);
                win_join_pairs(cm);
                const bool own_scale = blen > 0 && half == 0 && bstart >= w0 && colok;
                const int64_t n = tab.n[sl < WIN_TAB ? sl : 0];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    uint4 a, bo;
                    uint32_t code0, code1;
                    tile_col_codes(v, cm[d], d, a, bo, code0, code1);
                    if (colok && ihi > ilo) {
                        uint8_t* pa = q_col + (col + 2 * d) * M + r0;
                        uint8_t* pb = pa + M;
                        if (ilo == 0 && ihi == 16) {
                            __builtin_memcpy(pa, &a, 16);
                            __builtin_memcpy(pb, &bo, 16);
                        } else {
#pragma unroll
                            for (int j = 0; j < 16; ++j) {
                                if (j >= ilo && j < ihi) {
                                    pa[j] = (uint8_t)(dword_of(a, j >> 2) >> (8 * (j & 3)));
                                    pb[j] = (uint8_t)(dword_of(bo, j >> 2) >> (8 * (j & 3)));
                                }
                            }
                        }
                    }
                    if (own_scale) {
                        s_col[(col + 2 * d) * s_ld + n] = (uint8_t)code0;
                        s_col[(col + 2 * d + 1) * s_ld + n] = (uint8_t)code1;
                    }
                }
            }
        }
    }
    if (!ROWWISE) return;
    __syncthreads();
    // rowwise codes and scales of the window's rows
    const int L = FULL ? WIN_ROWS : (int)min<int64_t>(WIN_ROWS, M - w0);
    constexpr int CHUNKS = G::COLS / 16;
    for (int idx = threadIdx.x; idx < L * CHUNKS; idx += G::THREADS) {
        const int r = idx / CHUNKS, c16 = idx % CHUNKS;
        if (FULL || kw + 16 * c16 < K) {
            const uint4 val = *reinterpret_cast<const uint4*>(&lds_q[r][16 * c16]);
            st_stream<MXGRP_NT_STORE>(reinterpret_cast<uint4*>(q_row + (w0 + r) * K + kw + 16 * c16), val);
        }
    }
    const int64_t nb_row = K >> 5;
    const int nbr = (int)min((int64_t)G::SROW_B, nb_row - (kw >> 5));
    for (int r = threadIdx.x; r < L; r += G::THREADS) {
        uint8_t* dst = s_row + (w0 + r) * nb_row + (kw >> 5);
        if (nbr == G::SROW_B && (nb_row % G::SROW_B) == 0) store_scales<G::SROW_B>(dst, lds_srow[r]);
        else for (int j = 0; j < nbr; ++j) dst[j] = lds_srow[r][j];
    }
}

__global__ __launch_bounds__(64)
void mx_group_check_kernel(const int64_t* __restrict__ off, int64_t E, int64_t M, int64_t s_ld,
                           int32_t* __restrict__ status) {
    group_check(off, E, M, s_ld, status);
}

hipError_t launch_mx_quant_grouped(const void* x, int64_t M, int64_t K, int mode, const int64_t* off,
                                   int64_t E, void* q_row, void* s_row, void* q_col, void* s_col,
                                   int64_t s_ld, int32_t* status, hipStream_t stream) {
    // blocks that can exist: at most one per row, at most ceil(m_e/32) per expert, at most s_ld
    int64_t n_limit = (M + 31 * E) / 32;
    if (n_limit > M) n_limit = M;
    if (n_limit > s_ld) n_limit = s_ld;
    if (n_limit == 0 || K == 0) {
        if (status != nullptr)
            hipLaunchKernelGGL(mx_group_check_kernel, dim3(1), dim3(64), 0, stream, off, E, M, s_ld, status);
        return hipGetLastError();
    }
    const int64_t col_groups = (K + 255) / 256;
    const int64_t grid = (M + WIN_ROWS - 1) / WIN_ROWS * col_groups;
    const bool full = M % WIN_ROWS == 0 && K % 256 == 0;   // no ragged window or column group
    const auto kernel = mode == 3 ? (full ? mx_quant_grouped_window_kernel<true, true> : mx_quant_grouped_window_kernel<false, true>)
                                  : (full ? mx_quant_grouped_window_kernel<true, false> : mx_quant_grouped_window_kernel<false, false>);
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint16_t*)x, M, K, off, E, (uint8_t*)q_row, (uint8_t*)s_row,
                       (uint8_t*)q_col, (uint8_t*)s_col, s_ld, n_limit, col_groups, status);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------- dequant

// MXFP8 -> BF16 in the stored layout, a 1-D stream: element i uses scale i/32.  Thread t of
// a workgroup owns, in slot j, the 8 codes of chunk blockIdx*256*DQ_SLOTS + 256 j + t and
// writes their 16 bytes of BF16, so every load instruction reads 512 contiguous bytes
// and every store instruction writes 1 KiB contiguous; 4 neighbouring lanes share a scale.
#ifndef BSQ_MX_DQ_SLOTS
#define BSQ_MX_DQ_SLOTS 2
#endif
constexpr int MX_DQ_SLOTS = BSQ_MX_DQ_SLOTS;

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
    __builtin_amdgcn_s_setprio(3);                   // loads at raised priority (see the tile kernel)
#pragma unroll
    for (int j = 0; j < DQ_SLOTS; ++j) {
        const int64_t c = base + 256 * j;
        const bool ok = c < n_chunks;
        w[j] = ok ? ld_stream<MXDQ_NT_LOAD>(q + c) : make_uint2(0u, 0u);
        sc[j] = ok ? s[c >> 2] : 0u;
    }
    __builtin_amdgcn_s_setprio(0);
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
    const int64_t n_wg = ((M + LibTile::ROWS - 1) / LibTile::ROWS) * ((K + LibTile::COLS - 1) / LibTile::COLS);
    const int64_t pw = (mode == 2 && n_wg > 2 * TILE_PERSISTENT_WGS) ? TILE_PERSISTENT_WGS : 0;
    if (mode == 3)
        launch_tile<LibTile, true, TILE_ORDER>(x, M, K, q_row, s_row, q_col, s_col, stream, pw);
    else
        launch_tile<LibTile, false, TILE_ORDER>(x, M, K, nullptr, nullptr, q_col, s_col, stream, pw);
    return hipGetLastError();
}

// The grids of launch_mx_quant / launch_mx_quant_grouped / launch_mx_dequant fit one dispatch?
bool mx_quant_launch_fits(int64_t M, int64_t K, int mode) {
    if (mode == 1) {
        const int64_t tiles = (M * K / 8 + 64 * ROW_SLOTS - 1) / (64 * ROW_SLOTS);
        return dispatch_fits((tiles + ROW_WAVES - 1) / ROW_WAVES, 64 * ROW_WAVES);
    }
    const int64_t n_wg = ((M + LibTile::ROWS - 1) / LibTile::ROWS) * ((K + LibTile::COLS - 1) / LibTile::COLS);
    if (mode == 2 && n_wg > 2 * TILE_PERSISTENT_WGS) return true;   // persistent grid
    return dispatch_fits(n_wg, LibTile::THREADS);
}

bool mx_quant_grouped_launch_fits(int64_t M, int64_t K) {
    return dispatch_fits((M + WIN_ROWS - 1) / WIN_ROWS * ((K + 255) / 256), 256);
}

template <int SLOTS>
static void launch_mx_dequant_slots(const void* q, const void* s, int64_t rows, int64_t cols,
                                    void* y, hipStream_t stream) {
    const int64_t n_chunks = rows * cols / 8;
    const int64_t grid = (n_chunks + 256 * SLOTS - 1) / (256 * SLOTS);
    hipLaunchKernelGGL(mx_dequant_kernel<SLOTS>, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint2*)q, (const uint8_t*)s, (uint4*)y, n_chunks);
}

// Tensors of up to MX_DQ_SMALL_CHUNKS chunks (8 codes each) take 8 slots per thread: a
// quarter of the workgroups to dispatch and four times the loads in flight per wave.
// Measured: 8192 x 2048 12.6 -> 11.9 us, 2048 x 6144 10.2 -> 9.2 us; at 196608 x 2048 two
// slots stay faster (194 against 204 us), at 65536 x 2048 the two are level (67.0, 67.6).
constexpr int64_t MX_DQ_SMALL_CHUNKS = int64_t(1) << 22;

bool mx_dequant_launch_fits(int64_t rows, int64_t cols) {
    const int64_t n_chunks = rows * cols / 8;
    const int64_t slots = n_chunks <= MX_DQ_SMALL_CHUNKS ? 8 : MX_DQ_SLOTS;
    return dispatch_fits((n_chunks + 256 * slots - 1) / (256 * slots), 256);
}

hipError_t launch_mx_dequant(const void* q, const void* s, int64_t rows, int64_t cols,
                             void* y, hipStream_t stream) {
    if (rows * cols / 8 <= MX_DQ_SMALL_CHUNKS)
        launch_mx_dequant_slots<8>(q, s, rows, cols, y, stream);
    else
        launch_mx_dequant_slots<MX_DQ_SLOTS>(q, s, rows, cols, y, stream);
    return hipGetLastError();
}

}  // namespace bsq
