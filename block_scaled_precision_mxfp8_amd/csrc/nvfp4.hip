// nvfp4.hip -- per-token NVFP4 quantization (flat, grouped by expert, and quantize-then-
// scatter of routed rows), NVFP4 with one FP32 scale per row group (per tensor or expert)
// and with 16x16 weight tiles, and NVFP4 dequantization to BF16, for gfx950.
//
// Page "Towards Blackwell-native 8-bit and 4-bit RL":
//  * section "Format background": E2M1 values, one E4M3 scale per 16 values rounded to
//    the nearest representable value, and a coarse FP32 scale that maps the tensor or
//    token into the NVFP4 range; which range the FP32 scale covers is a recipe choice.
//  * section "Per-token activation scaling": one FP32 activation scale per token,
//    computed online, so that no token's bytes depend on other tokens of the batch; the
//    single call that emits packed FP4 and the E4M3 block scales also returns the
//    per-token FP32 scales (no separate calibration pass).
//  * section "High-precision and dequantized backward": BF16 dequantized operands.
//
// The per-token scale needs the whole row before any element can be encoded.  A wave
// owns a row (two rows when they are 768 elements or shorter) and keeps it in registers
// (16-byte loads, 8 BF16 per lane per slot), so the row is read from HBM exactly once:
// row maximum by a wave reduction, then each 1x16 block (a lane pair) is scaled and
// encoded from registers.
#include <float.h>

#include "bsq_device.h"

namespace bsq {

// Cache policy of each kernel family's one-touch accesses: bit 0 = non-temporal loads,
// bit 1 = non-temporal stores (see the measurements noted in mxfp8.hip).  The quantizer
// reads 2 bytes per element once: non-temporal loads take it from 477 to 437 us on
// 524288 x 2048 when timed alone.
#ifndef BSQ_POLICY_NVQ
#define BSQ_POLICY_NVQ 3
#endif
#ifndef BSQ_POLICY_NVDQ
#define BSQ_POLICY_NVDQ 2
#endif
constexpr bool NVQ_NT_LOAD = (BSQ_POLICY_NVQ & 1) != 0, NVQ_NT_STORE = (BSQ_POLICY_NVQ & 2) != 0;
constexpr bool NVDQ_NT_LOAD = (BSQ_POLICY_NVDQ & 1) != 0, NVDQ_NT_STORE = (BSQ_POLICY_NVDQ & 2) != 0;

// Eight E2M1 codes (one nibble each, element 2j in the low nibble of byte j) of the
// BF16 values of a 16-byte chunk multiplied by f: q = ENC_E2M1(fl(x * f)).  The binary32
// product is rounded by the multiply; the FP4 convert (scale 1.0) then rounds it to the
// nearest E2M1 value, ties to the even code, keeping the sign.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(bf16_lo_bits(w)); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(bf16_hi_bits(w)); }

__device__ __forceinline__ uint32_t nv_enc8(const uint4& v, float f) {
    uint32_t r = 0u;
    r = cvt_e2m1x2_f32<0>(r, bf16_lo(v.x) * f, bf16_hi(v.x) * f);
    r = cvt_e2m1x2_f32<1>(r, bf16_lo(v.y) * f, bf16_hi(v.y) * f);
    r = cvt_e2m1x2_f32<2>(r, bf16_lo(v.z) * f, bf16_hi(v.z) * f);
    r = cvt_e2m1x2_f32<3>(r, bf16_lo(v.w) * f, bf16_hi(v.w) * f);
    return r;
}

__device__ __forceinline__ uint32_t chunk_absmax8(const uint4& v) {
    return fold2(absmax2(absmax2(absmax2(absmax2(0u, v.x), v.y), v.z), v.w));
}

// Block scale code, and the element multiplier of the block, from the block maximum
// (BF16 magnitude bits) and the token scale s_t:
//   sb = ENC_E4M3(fl(amax_b / fl(6 s_t))) (0 if s_t == 0),  D = fl(DEC(sb) s_t),
//   f = 0 if D == 0 else min(fl(1 / D), FLT_MAX).
// Both divisions are IEEE binary32 divisions (correctly rounded, denormals kept).
__device__ __forceinline__ uint32_t nv_block_scale(uint32_t amax_b_bits, float s_t, float p, float& f) {
    const float amax_b = __uint_as_float(amax_b_bits << 16);
    const uint32_t code = (s_t == 0.0f) ? 0u : e4m3_code(amax_b / p);
    const float d = e4m3_decode_mag(code) * s_t;
    f = (d == 0.0f) ? 0.0f : fminf(1.0f / d, FLT_MAX);
    return code;
}

// Device-side check of the expert offsets of the grouped call, by one wave:
// offsets[0] == 0, offsets[E] == R, offsets[e] <= offsets[e+1].
__device__ void check_offsets(const int64_t* __restrict__ off, int64_t E, int64_t R,
                              int32_t* __restrict__ status, int64_t gran = 1) {
    const int lane = threadIdx.x & 63;
    bool bad = false;
    for (int64_t e = lane; e < E; e += 64) bad |= off[e] > off[e + 1] || (off[e + 1] % gran) != 0;
    if (lane == 0) bad |= (off[0] != 0) || (off[E] != R);
    const bool any_bad = __any(bad);
    if (lane == 0) *status = any_bad ? 6 /* BSQ_ERR_OFFSETS */ : 0;
}

__global__ __launch_bounds__(64)
void nv_check_offsets_kernel(const int64_t* __restrict__ off, int64_t E, int64_t R,
                             int32_t* __restrict__ status) {
    check_offsets(off, E, R, status);
}

// One wave per span of RPW consecutive rows (RPW = 1 or 2), the span held in registers:
// NS slots of 64 lanes x 8 BF16 (so spans of up to 512*NS elements).  Lane l of slot j
// holds chunk 64 j + l of the span (elements 8 (64 j + l) .. +7); a 1x16 block is the
// lane pair (2i, 2i+1), and since K % 16 == 0 no block straddles two rows.  Two short
// rows per wave keep every lane busy and twice the bytes in flight per wave (K = 768:
// 192 chunks fill 3 slots exactly, where one row would leave half of its second slot
// idle).
// Waves per workgroup of the row kernels (2 / 4 / 8: 449.6 / 442.5 / 439.4 us alone on
// 524288 x 2048, but 8 slower in the step, 6159-6178 against 6179-6188 GB/s); the per-token
// quantizer's and the scatter's one-row spans run one wave per workgroup instead (see
// launch_rows and launch_scatter).
#ifndef BSQ_NV_WAVES
#define BSQ_NV_WAVES 4
#endif
constexpr int NV_WAVES = BSQ_NV_WAVES;

// Wave index as a scalar: all address arithmetic of a span is then wave-uniform and the
// per-lane part is a 32-bit offset.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// Max over the whole wave of both 16-bit halves independently (two rows' maxima at once),
// returned uniform; same DPP pattern as wave_max.
__device__ __forceinline__ uint32_t wave_max_pk(uint32_t v) {
    v = pk_max_u16(v, dpp_xor1(v));
    v = pk_max_u16(v, dpp_xor2(v));
    v = pk_max_u16(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));  // row_half_mirror
    v = pk_max_u16(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true));  // row_mirror
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return pk_max_u16(pk_max_u16(a, b), pk_max_u16(c, d));
}

// FULL: the span is exactly NS slots long (RPW * K == 512 NS and all RPW rows exist), so
// no lane is ever out of range.
template <int NS, bool FULL>
__device__ __forceinline__ void load_span(uint4 (&v)[NS], const uint4* __restrict__ xs, int n_ch) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int ch = 64 * j + lane;
        v[j] = (FULL || ch < n_ch) ? ld_stream<NVQ_NT_LOAD>(xs + ch) : make_uint4(0u, 0u, 0u, 0u);
    }
}

// Largest magnitudes of the span's rows (BF16 bits; row a in the low half, row b in the
// high half for RPW = 2), uniform over the wave.
template <int NS, int RPW>
__device__ __forceinline__ uint32_t span_amax(const uint4 (&v)[NS], int cpr) {
    static_assert(RPW == 1 || RPW == 2, "one or two rows per wave");
    const int lane = threadIdx.x & 63;
    uint32_t m = 0u;
    if (RPW == 1) {
#pragma unroll
        for (int j = 0; j < NS; ++j) m = max(m, chunk_absmax8(v[j]));
        return wave_max(m);
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const uint32_t c = chunk_absmax8(v[j]);
        m = pk_max_u16(m, (64 * j + lane >= cpr) ? (c << 16) : c);
    }
    return wave_max_pk(m);
}

// FP32 decode scale of a row or group from its largest magnitude (BF16 bits):
// fl(amax / (6 * 448)).
__device__ __forceinline__ float nv_decode_scale(uint32_t amax_bf16) {
    return __uint_as_float(amax_bf16 << 16) / 2688.0f;
}

// Encode the span held in v (all lanes of the wave take part) under the FP32 decode
// scales s_a (row r0) and s_b (row r0+1, RPW = 2): packed[j] gets the 8 E2M1 codes of the
// lane's chunk in slot j, and the span's block-scale bytes are gathered in the wave's LDS
// slice `lsb` (32 NS bytes, byte i = block i of the span), ready when this returns.
template <int NS, int RPW>
__device__ __forceinline__ void encode_span(const uint4 (&v)[NS], int cpr, float s_a, float s_b,
                                            uint32_t (&packed)[NS], uint8_t* lsb) {
    const int lane = threadIdx.x & 63;
    // second row of the span for slot j? (RPW == 2 only; cpr is the row length in chunks)
    auto in_b = [&](int j) { return RPW == 2 && 64 * j + lane >= cpr; };
    const float p_a = 6.0f * s_a, p_b = 6.0f * s_b;                   // fl(6 s)
    const bool odd = (lane & 1) != 0;
    // Slots are taken two at a time: the two lanes of a block pair hold both blocks'
    // maxima, the even lane works out slot j's scale and multiplier, the odd lane slot
    // j+1's, and they swap results with one DPP move each (the two IEEE divisions per
    // block are done once, not twice).
#pragma unroll
    for (int j = 0; j < NS; j += 2) {
        const bool two = j + 1 < NS;
        const uint32_t a0 = pair_max(chunk_absmax8(v[j]));
        const uint32_t a1 = two ? pair_max(chunk_absmax8(v[j + 1])) : 0u;
        const int jj = (two && odd) ? j + 1 : j;                      // slot this lane works out
        const bool b = in_b(jj);
        float f;
        const uint32_t code = nv_block_scale((two && odd) ? a1 : a0, b ? s_b : s_a, b ? p_b : p_a, f);
        uint32_t code0 = code, code1 = code;
        float f0 = f, f1 = f;
        if (two) {
            const uint32_t oc = dpp_xor1(code);
            const float of = __uint_as_float(dpp_xor1(__float_as_uint(f)));
            code0 = odd ? oc : code;
            f0 = odd ? of : f;
            code1 = odd ? code : oc;
            f1 = odd ? f : of;
        }
        packed[j] = nv_enc8(v[j], f0);
        if (!odd) lsb[32 * j + (lane >> 1)] = (uint8_t)code0;
        if (two) {
            packed[j + 1] = nv_enc8(v[j + 1], f1);
            if (!odd) lsb[32 * (j + 1) + (lane >> 1)] = (uint8_t)code1;
        }
    }
    // the wave's LDS slice: written above by even lanes, read after this by any lane
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Quantize the span held in v into rows r0 .. of q and sb (n_ch valid chunks); the scale
// bytes leave as 16-byte stores when the span's run is 16-byte aligned.
template <int NS, int RPW, bool FULL>
__device__ __forceinline__ void quant_span(const uint4 (&v)[NS], int64_t r0, int n_ch, int cpr,
                                           float s_a, float s_b,
                                           uint32_t* __restrict__ q, uint8_t* __restrict__ sb,
                                           uint8_t* lsb) {
    const int lane = threadIdx.x & 63;
    uint32_t packed[NS];
    encode_span<NS, RPW>(v, cpr, s_a, s_b, packed, lsb);
    uint32_t* qs = q + r0 * cpr;                      // 4 bytes of q per chunk
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int ch = 64 * j + lane;
        if (FULL || ch < n_ch) st_stream<NVQ_NT_STORE>(qs + ch, packed[j]);
    }
    uint8_t* sbs = sb + r0 * (cpr >> 1);              // one scale byte per chunk pair
    const int nsb = n_ch >> 1;                        // scale bytes of the span
    if ((nsb & 15) == 0 && ((r0 * (cpr >> 1)) & 15) == 0) {
        if (lane < (nsb >> 4))
            st_stream<NVQ_NT_STORE>(reinterpret_cast<uint4*>(sbs) + lane, reinterpret_cast<const uint4*>(lsb)[lane]);
    } else {
        for (int i = lane; i < nsb; i += 64) sbs[i] = lsb[i];
    }
}

// Workgroup index that workgroup b of n takes when the rows are dealt to the XCDs in chunks
// of NV_XCD_CHUNK_ROWS consecutive rows (CH workgroups).  Workgroups go to the eight XCDs
// in turn (b % 8), so workgroup b takes index (8 (c / CH) + b % 8) CH + c % CH with c = b /
// 8: each XCD walks contiguous chunks of the tensor.  The workgroups past the last whole
// round of 8 chunks keep index b, so the map is a bijection of [0, n).  Measured on the
// per-token quantizer with the following read (one box, interleaved): one-row spans,
// 524288 x 2048 442.1 -> 434.1 us (the layer step 1111.6 -> 1103.8 us), 262144 x 4096 459.7
// -> 448.9, 196608 x 2048 165.0 -> 163.4, and with the rows starting 37 or 300 rows into an
// allocation 440.0 -> 436.8 and 442.7 -> 442.0; two-row spans, 262144 x 768 80.9 -> 79.9,
// 524288 x 512 104.2 -> 102.7, 1048576 x 256 151.4 -> 146.2.  Other chunk sizes were not
// monotone: 64 / 128 / 256 / 1024 rows took 447.3 / 435.3 / 440.5 / 444.2 us on 524288 x
// 2048 (the memory-only pattern behaves alike), and 128 lost on 262144 x 4096.  The
// quantize-then-scatter (one token per workgroup, writes scattered by the routing) became
// 4% slower with it, and the dequantizer's pattern too; they keep b.
constexpr int64_t NV_XCD_CHUNK_ROWS = 512;
template <int64_t CH>
__device__ __forceinline__ int64_t xcd_chunk(int64_t b, int64_t n) {
    const int64_t full = n / (8 * CH) * (8 * CH);
    if (b >= full) return b;
    const int64_t c = b >> 3;
    return ((c / CH) * 8 + (b & 7)) * CH + c % CH;
}

// One span per wave, WAVES waves per workgroup, per-token scales.
template <int NS, int RPW, bool FULL, int WAVES>
__global__ __launch_bounds__(64 * WAVES)
void nv_quant_rows_kernel(const uint4* __restrict__ x, uint32_t* __restrict__ q,
                          uint8_t* __restrict__ sb, float* __restrict__ st,
                          int64_t R, int64_t K,
                          const int64_t* __restrict__ offsets, int64_t E,
                          int32_t* __restrict__ status) {
    const int wave = wave_id();
    const int lane = threadIdx.x & 63;
    if (status != nullptr && blockIdx.x == 0 && wave == 0) check_offsets(offsets, E, R, status);
    const int64_t wg = xcd_chunk<NV_XCD_CHUNK_ROWS / (WAVES * RPW)>(blockIdx.x, gridDim.x);
    const int64_t r0 = (wg * WAVES + wave) * RPW;
    if (r0 >= R) return;
    __shared__ __align__(16) uint8_t lds_sb[WAVES][32 * NS];
    const int cpr = (int)(K >> 3);                    // 8-element chunks per row
    const int n_ch = (RPW == 2 && r0 + 1 >= R) ? cpr : RPW * cpr;
    uint4 v[NS];
    // The wave issues its loads at raised priority, so that waves that have just started
    // get their reads out ahead of the others' arithmetic and stores: 458 -> 447 us on
    // 524288 x 2048; with the same in the dequantizers and the MXFP8 tile kernel, the step
    // 6123 -> 6191 GB/s (means of three interleaved runs).  (Measured and not kept, as
    // slower: the same in the 16x16-tile quantizer.)
    __builtin_amdgcn_s_setprio(3);
    load_span<NS, FULL>(v, x + r0 * cpr, n_ch);
    __builtin_amdgcn_s_setprio(0);
    const uint32_t mm = span_amax<NS, RPW>(v, cpr);
    const float s_a = nv_decode_scale(mm & 0xFFFFu);
    const float s_b = nv_decode_scale(mm >> 16);
    quant_span<NS, RPW, FULL>(v, r0, n_ch, cpr, s_a, s_b, q, sb, lds_sb[wave]);
    if (lane == 0) st[r0] = s_a;
    if (RPW == 2 && lane == 1 && n_ch > cpr) st[r0 + 1] = s_b;
}

// ----------------------------------------------------------------------------- scatter

// Quantize-then-scatter of routed rows.  Page "Towards Blackwell-native 8-bit and 4-bit
// RL", section "Per-token activation scaling": a token's bytes depend on that token only.
// So the routed rows X[i] = H[t] (a token appears once per expert it is routed to) need
// not be gathered in BF16 and quantized one by one: each token row of H is quantized once
// and its bytes are written to every routed row it lands in, bit-identical to quantizing
// X, while reading H once instead of X (top_k times the bytes).  dst[t][j] is the routed
// row of token t's j-th choice; a negative entry is a dropped choice, an entry >= N is
// reported in *status and skipped.
// Ordinary stores look faster for the scattered writes when the kernel is timed alone,
// 172 -> 143 us on 65536 tokens x 2048 to top 8 of 128, but leave the dirty lines for
// whatever runs next: timed together with the 512 MiB read that follows, 168 us with
// non-temporal stores against 198 us with ordinary ones (since then 159 us, with the launch
// shape below).  A memory-only kernel with the same loads and stores and no arithmetic,
// launched the same way, takes as long (156 us kernel-only on that workload).

__global__ __launch_bounds__(64)
void nv_status_clear_kernel(int32_t* __restrict__ status) {
    if (threadIdx.x == 0) *status = 0;
}

// Lane i's 64-bit value, read as a wave-uniform one.
__device__ __forceinline__ int64_t readlane_i64(int64_t v, int i) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, i);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), i);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

template <int NS, int RPW, bool FULL, int WAVES>
__global__ __launch_bounds__(64 * WAVES)
void nv_quant_scatter_kernel(const uint4* __restrict__ h, int64_t T, int64_t K,
                             const int64_t* __restrict__ dst, int64_t top_k, int64_t N,
                             uint32_t* __restrict__ q, uint8_t* __restrict__ sb, float* __restrict__ st,
                             int32_t* __restrict__ status) {
    const int wave = wave_id();
    const int lane = threadIdx.x & 63;
    const int64_t r0 = ((int64_t)blockIdx.x * WAVES + wave) * RPW;
    if (r0 >= T) return;
    __shared__ __align__(16) uint8_t lds_sb[WAVES][32 * NS];
    const int cpr = (int)(K >> 3);
    const int n_ch = (RPW == 2 && r0 + 1 >= T) ? cpr : RPW * cpr;
    const bool has_b = RPW == 2 && n_ch > cpr;
    uint4 v[NS];
    // Single-row spans (one wave per workgroup) load at raised priority, as in the row
    // kernel: the two together 166.1 -> 158.8 us on 65536 tokens x 2048 to 524288
    // Zipf-routed rows (174.1 -> 165.4 us on a random map), timed with the following read,
    // where one wave per workgroup alone measured 166.7 us and the priority alone, with
    // four waves per workgroup, 173.8.  Two-row spans keep four waves and ordinary
    // priority (with it 131072 tokens x 768: 173.2 -> 177.3 us).
    if (RPW == 1) __builtin_amdgcn_s_setprio(3);
    load_span<NS, FULL>(v, h + r0 * cpr, n_ch);
    if (RPW == 1) __builtin_amdgcn_s_setprio(0);
    // The destination rows, 32 entries at a time, loaded together with the span: lane l < 32
    // holds entry c0 + l of token r0, lane 32 + l the same entry of token r0 + 1 (-1 where
    // there is none); the loop below reads them back as wave-uniform values.  Loading each
    // entry inside the loop made every destination wait for a load and, with it, for the
    // previous destination's stores (one counter covers both): 171.1 -> 167.5 us on 65536
    // tokens x 2048 to 524288 Zipf-routed rows, timed with the following read.
    const auto load_dst = [&](int64_t c0) -> int64_t {
        const int64_t c = c0 + (lane & 31);
        const bool second = lane >= 32;
        return (c < top_k && (!second || has_b)) ? dst[(r0 + (second ? 1 : 0)) * top_k + c] : -1;
    };
    int64_t dl = load_dst(0);
    const uint32_t mm = span_amax<NS, RPW>(v, cpr);
    const float s_a = nv_decode_scale(mm & 0xFFFFu);
    const float s_b = nv_decode_scale(mm >> 16);
    uint32_t packed[NS];
    uint8_t* lsb = lds_sb[wave];
    encode_span<NS, RPW>(v, cpr, s_a, s_b, packed, lsb);
    const int sbr = cpr >> 1;                         // scale bytes per row
    const bool sb16 = (sbr & 15) == 0;                // a row's scale run is whole 16-byte units
    for (int64_t c0 = 0; c0 < top_k; c0 += 32) {
        if (c0 > 0) dl = load_dst(c0);
        const int n_c = (int)min<int64_t>(32, top_k - c0);
        for (int i = 0; i < n_c; ++i) {
            const int64_t da = readlane_i64(dl, i);
            const int64_t db = has_b ? readlane_i64(dl, 32 + i) : -1;
            const bool va = da >= 0 && da < N, vb = db >= 0 && db < N;
            if (status != nullptr && lane == 0 && (da >= N || db >= N)) *status = 6;   // BSQ_ERR_OFFSETS
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const int ch = 64 * j + lane;
                const bool inb = RPW == 2 && ch >= cpr;
                if ((FULL || ch < n_ch) && (inb ? vb : va))
                    st_stream<NVQ_NT_STORE>(q + (inb ? db : da) * cpr + (inb ? ch - cpr : ch), packed[j]);
            }
            if (sb16) {
                const int units = sbr >> 4;               // 16-byte units per row
                const bool inb = lane >= units;
                if (lane < (has_b ? 2 : 1) * units && (inb ? vb : va))
                    st_stream<NVQ_NT_STORE>(reinterpret_cast<uint4*>(sb + (inb ? db : da) * sbr) + (inb ? lane - units : lane),
                                            reinterpret_cast<const uint4*>(lsb)[lane]);
            } else {
                for (int k = lane; k < (has_b ? 2 : 1) * sbr; k += 64) {
                    const bool inb = k >= sbr;
                    if (inb ? vb : va) sb[(inb ? db : da) * sbr + (inb ? k - sbr : k)] = lsb[k];
                }
            }
            if (lane == 0 && va) st[da] = s_a;
            if (lane == 1 && vb) st[db] = s_b;
        }
    }
}

// Tokens longer than the register-resident variants: one wave per token, the row streamed
// twice, each chunk's codes written to every destination.
__global__ __launch_bounds__(64 * NV_WAVES)
void nv_quant_scatter_long_kernel(const uint4* __restrict__ h, int64_t T, int64_t K,
                                  const int64_t* __restrict__ dst, int64_t top_k, int64_t N,
                                  uint32_t* __restrict__ q, uint8_t* __restrict__ sb, float* __restrict__ st,
                                  int32_t* __restrict__ status) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * NV_WAVES + (threadIdx.x >> 6);
    if (t >= T) return;
    const int64_t cpr = K >> 3;
    const uint4* xr = h + t * cpr;
    uint32_t m = 0u;
    for (int64_t base = 0; base < cpr; base += 64) {
        const int64_t ch = base + lane;
        if (ch < cpr) m = max(m, chunk_absmax8(xr[ch]));
    }
    const float s = nv_decode_scale(wave_max(m));
    const float p = 6.0f * s;
    for (int64_t c = 0; c < top_k; ++c) {
        const int64_t d = dst[t * top_k + c];
        if (status != nullptr && lane == 0 && d >= N) *status = 6;
        if (lane == 0 && d >= 0 && d < N) st[d] = s;
    }
    for (int64_t base = 0; base < cpr; base += 64) {
        const int64_t ch = base + lane;
        const uint4 v = (ch < cpr) ? xr[ch] : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t amax_b = pair_max(chunk_absmax8(v));
        float f;
        const uint32_t code = nv_block_scale(amax_b, s, p, f);
        const uint32_t packed = nv_enc8(v, f);
        if (ch < cpr) {
            for (int64_t c = 0; c < top_k; ++c) {
                const int64_t d = dst[t * top_k + c];
                if (d < 0 || d >= N) continue;
                q[d * cpr + ch] = packed;
                if ((lane & 1) == 0) sb[d * (K >> 4) + (ch >> 1)] = (uint8_t)code;
            }
        }
    }
}

// ----------------------------------------------------------------------------- per group

// Standard NVFP4 with one FP32 scale per group of rows (a tensor, or an expert's tensor
// with its gate and up projections together).  Page "Towards Blackwell-native 8-bit and
// 4-bit RL", section "Format background": the scope of the coarse FP32 scale is a recipe
// choice; section "Per-token activation scaling": gate and up share one FP32 scale in
// conversion and weight export.  s_g = fl(amax_g / 2688) over the group, then every row
// is encoded as a per-token row with s_t = s_g.  The group maximum needs the whole group
// before any element is encoded, so this takes two passes over x: the maxima are
// accumulated with atomicMax on their binary32 bit patterns (non-negative, so unsigned
// order is value order) in the caller's s_group array itself, which the last launch turns
// into the scales in place.

// Group of row r: the g in [0, G) with off[g] <= r < off[g+1] (clamped into [0, G) so
// that invalid offsets still index inside s_group).  Called with a wave-uniform row the
// search runs on scalar loads, which the scalar cache serves after the first workgroup.
__device__ __forceinline__ int64_t group_of(int64_t r, const int64_t* off, int64_t G) {
    int64_t lo = 0, hi = G;                           // off[lo] <= r < off[hi] (if valid)
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (off[mid] <= r) lo = mid; else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(256)
void nv_group_init_kernel(uint32_t* __restrict__ amax_bits, int64_t G, const int64_t* __restrict__ off,
                          int64_t R, int32_t* __restrict__ status, int64_t gran) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g < G) amax_bits[g] = 0u;
    if (status != nullptr && blockIdx.x == 0 && threadIdx.x < 64) check_offsets(off, G, R, status, gran);
}

// Pass 1: group maxima.  The tensor is read as one flat run of 16-byte pieces (eight BF16
// elements; a row holds K/8 of them) in a grid-stride sweep: at any moment the workgroups
// read one contiguous band, each wave 64 lanes x NV_AMAX_PIECES neighbouring pieces.  The
// band ends at the tensor's tail, which the quantize pass (walking backwards) then finds in
// the Infinity Cache.  A wave's pieces nearly always lie in one group; a wave that straddles
// group boundaries takes one masked maximum per group touched.  Maxima are kept as binary32
// bits (non-negative, so unsigned order is value order).  With LDS_TABLE each workgroup
// gathers its maxima in an LDS table of all G groups and sends each nonzero entry to the
// global array with one atomicMax at its end: the waves in flight all work in the same few
// groups, so an atomic per wave and piece run would serialise on those few addresses.
// (Measured on the 128-expert weight stacks: 4 to 16 pieces a lane and 4 to 16 workgroups a
// compute unit lie within 3% of each other; the sweep reads at about the pure-read rate.)
#ifndef BSQ_NV_AMAX_PIECES
#define BSQ_NV_AMAX_PIECES 8
#endif
#ifndef BSQ_NV_AMAX_WGS_PER_CU
#define BSQ_NV_AMAX_WGS_PER_CU 4
#endif
constexpr int NV_AMAX_PIECES = BSQ_NV_AMAX_PIECES;
constexpr int64_t NV_AMAX_LDS_GROUPS = 8192;          // 32 KiB of LDS per workgroup at most
// Up to this many groups the workgroup also keeps every group's first piece in LDS (16 KiB),
// so the two searches of each step read LDS instead of global memory: each of their seven
// dependent steps was a round trip to the caches, in the way of the step's loads.
constexpr int64_t NV_AMAX_LDS_STARTS = 2048;

// Group of the piece p: largest g with off[g] * cpr <= p (clamped to [0, G)); uniform.
// `starts` holds off[g] * cpr, in LDS or read from global memory.
template <bool LDS_STARTS>
__device__ __forceinline__ int64_t group_of_piece(int64_t p, const int64_t* off, const int64_t* starts,
                                                  int64_t G, int64_t cpr) {
    int64_t lo = 0, hi = G;
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if ((LDS_STARTS ? starts[mid] : off[mid] * cpr) <= p) lo = mid; else hi = mid;
    }
    return lo;
}

template <bool LDS_TABLE>
__device__ __forceinline__ void amax_put(uint32_t* table, uint32_t* amax_bits, int64_t g, uint32_t m, int lane) {
    if (lane != 0) return;
    if (LDS_TABLE) atomicMax(table + g, m << 16);
    else atomicMax(amax_bits + g, m << 16);
}

template <bool LDS_TABLE, bool LDS_STARTS>
__global__ __launch_bounds__(64 * NV_WAVES)
void nv_group_amax_kernel(const uint4* __restrict__ x, int64_t R, int64_t K,
                          const int64_t* __restrict__ off, int64_t G, uint32_t* __restrict__ amax_bits) {
    // dynamic LDS: the G + 1 group starts (in pieces) when LDS_STARTS, then the G table
    // entries when LDS_TABLE
    extern __shared__ __align__(8) uint64_t lds_dyn[];
    int64_t* starts = reinterpret_cast<int64_t*>(lds_dyn);
    uint32_t* table = reinterpret_cast<uint32_t*>(lds_dyn + (LDS_STARTS ? G + 1 : 0));
    constexpr int64_t WAVE_PIECES = 64 * NV_AMAX_PIECES;
    const int lane = threadIdx.x & 63;
    const int64_t cpr = K >> 3;
    const int64_t n = R * cpr;
    const int64_t stride = (int64_t)gridDim.x * NV_WAVES * WAVE_PIECES;
    if (LDS_STARTS) {
        for (int64_t g = threadIdx.x; g <= G; g += 64 * NV_WAVES) starts[g] = off[g] * cpr;
    }
    if (LDS_TABLE) {
        for (int64_t g = threadIdx.x; g < G; g += 64 * NV_WAVES) table[g] = 0u;
    }
    if (LDS_STARTS || LDS_TABLE) __syncthreads();
    for (int64_t wb = ((int64_t)blockIdx.x * NV_WAVES + wave_id()) * WAVE_PIECES; wb < n; wb += stride) {
        const int64_t we = min(n, wb + WAVE_PIECES);
        uint32_t a[NV_AMAX_PIECES];
        if (we - wb == WAVE_PIECES) {
            uint4 v[NV_AMAX_PIECES];
#pragma unroll
            for (int u = 0; u < NV_AMAX_PIECES; ++u) v[u] = x[wb + 64 * u + lane];
#pragma unroll
            for (int u = 0; u < NV_AMAX_PIECES; ++u) a[u] = chunk_absmax8(v[u]);
        } else {
#pragma unroll
            for (int u = 0; u < NV_AMAX_PIECES; ++u) {
                const int64_t q = wb + 64 * u + lane;
                a[u] = q < we ? chunk_absmax8(x[q]) : 0u;
            }
        }
        const int64_t g0 = group_of_piece<LDS_STARTS>(wb, off, starts, G, cpr);
        const int64_t g1 = group_of_piece<LDS_STARTS>(we - 1, off, starts, G, cpr);
        if (g0 == g1) {
            uint32_t m = a[0];
#pragma unroll
            for (int u = 1; u < NV_AMAX_PIECES; ++u) m = max(m, a[u]);
            amax_put<LDS_TABLE>(table, amax_bits, g0, wave_max(m), lane);
        } else {
            for (int64_t g = g0; g <= g1; ++g) {       // g1 < g0 only for invalid offsets
                const int64_t lo = g == g0 ? wb : (LDS_STARTS ? starts[g] : off[g] * cpr);
                const int64_t hi = g == g1 ? we : (LDS_STARTS ? starts[g + 1] : off[g + 1] * cpr);
                uint32_t m = 0u;
#pragma unroll
                for (int u = 0; u < NV_AMAX_PIECES; ++u) {
                    const int64_t q = wb + 64 * u + lane;
                    if (q >= lo && q < hi) m = max(m, a[u]);
                }
                amax_put<LDS_TABLE>(table, amax_bits, g, wave_max(m), lane);
            }
        }
    }
    if (LDS_TABLE) {
        __syncthreads();
        for (int64_t g = threadIdx.x; g < G; g += 64 * NV_WAVES) {
            const uint32_t m = table[g];
            if (m != 0u) atomicMax(amax_bits + g, m);
        }
    }
}

// Pass 2: quantize every span under its rows' group scales.
template <int NS, int RPW, bool FULL>
__global__ __launch_bounds__(64 * NV_WAVES)
void nv_group_quant_kernel(const uint4* __restrict__ x, uint32_t* __restrict__ q, uint8_t* __restrict__ sb,
                           int64_t R, int64_t K, const int64_t* __restrict__ off, int64_t G,
                           const uint32_t* __restrict__ amax_bits) {
    __shared__ __align__(16) uint8_t lds_sb[NV_WAVES][32 * NS];
    const int wave = wave_id();
    // workgroups in reverse row order: the first spans read are the rows the maximum pass
    // read last, still in the Infinity Cache when the tensor is not much larger than it
    const int64_t wg = (int64_t)gridDim.x - 1 - blockIdx.x;
    const int64_t r0 = (wg * NV_WAVES + wave) * RPW;
    const int cpr = (int)(K >> 3);
    const int n_ch = r0 >= R ? 0 : (RPW == 2 && r0 + 1 >= R) ? cpr : RPW * cpr;
    uint4 v[NS];
    if (n_ch > 0) load_span<NS, FULL>(v, x + r0 * cpr, n_ch);
    if (n_ch == 0) return;
    const float s_a = nv_decode_scale(amax_bits[group_of(r0, off, G)] >> 16);
    const float s_b = (RPW == 2 && n_ch > cpr) ? nv_decode_scale(amax_bits[group_of(r0 + 1, off, G)] >> 16) : 0.0f;
    quant_span<NS, RPW, FULL>(v, r0, n_ch, cpr, s_a, s_b, q, sb, lds_sb[wave]);
}

__global__ __launch_bounds__(256)
void nv_group_finalize_kernel(float* __restrict__ s_group, int64_t G) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g < G) s_group[g] = nv_decode_scale(__float_as_uint(s_group[g]) >> 16);
}

// Rows longer than the register-resident variants: two passes over the row (the second
// read of a row is served by the caches), same arithmetic.
__global__ __launch_bounds__(64 * NV_WAVES)
void nv_quant_rows_long_kernel(const uint4* __restrict__ x, uint32_t* __restrict__ q,
                               uint8_t* __restrict__ sb, float* __restrict__ st,
                               int64_t R, int64_t K,
                               const int64_t* __restrict__ offsets, int64_t E,
                               int32_t* __restrict__ status) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (status != nullptr && blockIdx.x == 0 && wave == 0) check_offsets(offsets, E, R, status);
    const int64_t row = (int64_t)blockIdx.x * NV_WAVES + wave;
    if (row >= R) return;
    const int64_t cpr = K >> 3;
    const uint4* xr = x + row * cpr;
    uint32_t m = 0u;
    for (int64_t base = 0; base < cpr; base += 64) {
        const int64_t ch = base + lane;
        if (ch < cpr) m = max(m, chunk_absmax8(xr[ch]));
    }
    const uint32_t amax_t = wave_max(m);
    const float s_t = __uint_as_float(amax_t << 16) / 2688.0f;
    const float p = 6.0f * s_t;
    uint32_t* qr = q + row * cpr;
    uint8_t* sbr = sb + row * (K >> 4);
    for (int64_t base = 0; base < cpr; base += 64) {
        const int64_t ch = base + lane;
        const uint4 v = (ch < cpr) ? xr[ch] : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t amax_b = pair_max(chunk_absmax8(v));
        float f;
        const uint32_t code = nv_block_scale(amax_b, s_t, p, f);
        const uint32_t packed = nv_enc8(v, f);
        if (ch < cpr) {
            qr[ch] = packed;
            if ((lane & 1) == 0) sbr[ch >> 1] = (uint8_t)code;
        }
    }
    if (lane == 0) st[row] = s_t;
}

// Quantize pass for rows longer than the register-resident variants (one wave per row,
// the row streamed twice; same arithmetic).
__global__ __launch_bounds__(64 * NV_WAVES)
void nv_group_quant_long_kernel(const uint4* __restrict__ x, uint32_t* __restrict__ q, uint8_t* __restrict__ sb,
                                int64_t R, int64_t K, const int64_t* __restrict__ off, int64_t G,
                                const uint32_t* __restrict__ amax_bits) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * NV_WAVES + (threadIdx.x >> 6);
    if (row >= R) return;
    const int64_t cpr = K >> 3;
    const uint4* xr = x + row * cpr;
    const float s = nv_decode_scale(amax_bits[group_of(row, off, G)] >> 16);
    const float p = 6.0f * s;
    uint32_t* qr = q + row * cpr;
    uint8_t* sbr = sb + row * (K >> 4);
    for (int64_t base = 0; base < cpr; base += 64) {
        const int64_t ch = base + lane;
        const uint4 v = (ch < cpr) ? xr[ch] : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t amax_b = pair_max(chunk_absmax8(v));
        float f;
        const uint32_t code = nv_block_scale(amax_b, s, p, f);
        const uint32_t packed = nv_enc8(v, f);
        if (ch < cpr) {
            qr[ch] = packed;
            if ((lane & 1) == 0) sbr[ch >> 1] = (uint8_t)code;
        }
    }
}

// ----------------------------------------------------------------------------- 16x16 tiles

// NVFP4 with 16x16 weight tiles: two-dimensional block scaling of the weights, one of the
// four parts of NVIDIA's NVFP4 pretraining recipe (page "NVIDIA verified the 4-bit NVFP4
// format on a Mamba-Transformer (12B) at 10 trillion tokens"; Miles turns it off, "Towards
// Blackwell-native 8-bit and 4-bit RL", section "Try the NVFP4 recipe in Miles").  Every
// 16x16 tile shares one E4M3 scale under its row group's FP32 scale s_g (the group maxima
// come from the per-group pass above), so one copy serves the weight and its transpose:
//   sb = ENC_E4M3(fl(amax_tile / fl(6 s_g))),  f from sb as in the per-token steps,
//   q = ENC_E2M1(fl(x f)).
// One wave owns a strip of 16 rows x 256 columns: lane l = 32 h + c holds rows 8h .. 8h+7
// of chunk column c (8 BF16 each), so a tile is the four lanes {2t, 2t+1, 32+2t, 33+2t}:
// its maximum is a lane-local max, one DPP pair exchange and one exchange 32 lanes apart.
// Each load instruction reads 512 contiguous bytes of two rows and each q store writes a
// whole 128-byte line of two rows.
constexpr int NV2D_COLS = 256;

template <bool FULL>
__global__ __launch_bounds__(64 * NV_WAVES)
void nv_quant_2d_kernel(const uint16_t* __restrict__ x, uint32_t* __restrict__ q, uint8_t* __restrict__ sb,
                        int64_t R, int64_t K, const int64_t* __restrict__ off, int64_t G,
                        const uint32_t* __restrict__ amax_bits, int64_t col_strips) {
    const int wave = wave_id();
    const int lane = threadIdx.x & 63;
    const int64_t strip = (int64_t)blockIdx.x * NV_WAVES + wave;
    const int64_t n_strips = (R >> 4) * col_strips;
    const int64_t rs = strip / col_strips;
    const int64_t r0 = rs * 16;
    const int64_t kw = (strip - rs * col_strips) * NV2D_COLS;
    const int c = lane & 31, hrow = lane >> 5;
    const int64_t col = kw + 8 * c;
    const bool ok = FULL || col < K;
    uint4 v[8];
    if (strip < n_strips) {
        const uint16_t* src = x + (r0 + 8 * hrow) * K + (ok ? col : kw);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = ld_stream<NVQ_NT_LOAD>(reinterpret_cast<const uint4*>(src + i * K));

    }
    if (strip >= n_strips) return;
    const float s = nv_decode_scale(amax_bits[group_of(r0, off, G)] >> 16);
    const float p = 6.0f * s;
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, chunk_absmax8(v[i]));
    m = pair_max(m);
    m = max(m, (uint32_t)__shfl_xor((int)m, 32, 64));
    float f;
    const uint32_t code = nv_block_scale(m, s, p, f);
    const int64_t cpr = K >> 3;
    if (ok) {
        uint32_t* qr = q + (r0 + 8 * hrow) * cpr + (col >> 3);
#pragma unroll
        for (int i = 0; i < 8; ++i) st_stream<NVQ_NT_STORE>(qr + i * cpr, nv_enc8(v[i], f));
        if (hrow == 0 && (c & 1) == 0) sb[rs * (K >> 4) + (col >> 4)] = (uint8_t)code;
    }
}

// ----------------------------------------------------------------------------- dequant

// NVFP4 -> BF16, a 1-D stream over half blocks (8 elements = 4 bytes of q = 16 bytes of
// BF16): thread t of a workgroup owns half block blockIdx*256*NVDQ_SLOTS + 256 j + t in
// slot j, so loads read 256 contiguous bytes and stores write 1 KiB contiguous per
// instruction.  The row of half block h is h / (K/8), an exact multiply-high division.
// y = RNE_BF16(fl(exact(DEC_E2M1(q) DEC_E4M3(sb)) s_t)).
// Re-measured with the loads at raised priority: 1 / 2 / 4 slots 584 / 434 / 457 us on
// 524288 x 2048 (the MXFP8 dequant: 71.8 / 65.4 / 68.2 us on 65536 x 2048).
#ifndef BSQ_NV_DQ_SLOTS
#define BSQ_NV_DQ_SLOTS 2
#endif
constexpr int NV_DQ_SLOTS = BSQ_NV_DQ_SLOTS;

// Two BF16 (one dword) of the E2M1 codes in byte `sel` of `word`; the inner product is
// exact, the product with s_t is one binary32 rounding, the convert is RNE to BF16.
template <int sel>
__device__ __forceinline__ uint32_t nv_dec2(uint32_t word, float bscale, float s_t) {
    const float2_t e = cvt_f32x2_e2m1<sel>(word);
    return cvt_bf16x2_f32((e.x * bscale) * s_t, (e.y * bscale) * s_t);
}

// The same with NaN results written as 0x7FC0 (only reachable when the block scale is a
// NaN code or s_t is not finite).
template <int sel>
__device__ __forceinline__ uint32_t nv_dec2_nan(uint32_t word, float bscale, float s_t) {
    const float2_t e = cvt_f32x2_e2m1<sel>(word);
    const float p0 = (e.x * bscale) * s_t, p1 = (e.y * bscale) * s_t;
    const uint32_t y = cvt_bf16x2_f32(p0, p1);
    const uint32_t lo = (p0 != p0) ? 0x7FC0u : (y & 0xFFFFu);
    const uint32_t hi = (p1 != p1) ? 0x7FC00000u : (y & 0xFFFF0000u);
    return lo | hi;
}

// GROUPED: st holds one scale per row group (offsets off[0..G], rows counted from row0);
// each row's scale is that of its group.
template <int NVDQ_SLOTS, bool GROUPED, bool TWO_D = false>
__global__ __launch_bounds__(256)
void nv_dequant_kernel(const uint32_t* __restrict__ q, const uint8_t* __restrict__ sb,
                       const float* __restrict__ st, uint4* __restrict__ y,
                       uint32_t n_half, FastDiv halves_per_row,
                       const int64_t* __restrict__ off, int64_t G, int64_t row0) {
    const uint32_t base = blockIdx.x * (256u * NVDQ_SLOTS) + threadIdx.x;
    uint32_t w[NVDQ_SLOTS], code[NVDQ_SLOTS];
    float s_t[NVDQ_SLOTS];
    __builtin_amdgcn_s_setprio(3);                   // loads at raised priority (see nv_quant_rows_kernel)
#pragma unroll
    for (int j = 0; j < NVDQ_SLOTS; ++j) {
        const uint32_t h = base + 256u * j;
        const bool ok = h < n_half;
        w[j] = ok ? ld_stream<NVDQ_NT_LOAD>(q + h) : 0u;
        if (TWO_D) {
            // half block h = row r, columns 8 (h - r hpr) ..: tile (r / 16, (h - r hpr) / 2)
            const uint32_t r = fastdiv(h, halves_per_row);
            const uint32_t hpr = halves_per_row.d;
            code[j] = ok ? sb[(uint64_t)(r >> 4) * (hpr >> 1) + ((h - r * hpr) >> 1)] : 0u;
        } else {
            code[j] = ok ? sb[h >> 1] : 0u;
        }
        if (!GROUPED) s_t[j] = ok ? st[fastdiv(h, halves_per_row)] : 0.0f;
    }
    if (GROUPED) {
        // groups of the workgroup's first and last rows (uniform searches, done while the
        // codes are in flight); the threads walk from the first one only when the workgroup
        // straddles a group boundary
        const uint32_t h0 = blockIdx.x * (256u * NVDQ_SLOTS);
        const uint32_t h1 = min(h0 + 256u * NVDQ_SLOTS, n_half) - 1u;
        const int64_t g_first = group_of(row0 + fastdiv(h0, halves_per_row), off, G);
        const int64_t g_last = group_of(row0 + fastdiv(h1, halves_per_row), off, G);
#pragma unroll
        for (int j = 0; j < NVDQ_SLOTS; ++j) {
            const uint32_t h = base + 256u * j;
            int64_t g = g_first;
            if (g_last != g_first) {
                const int64_t r = row0 + fastdiv(h, halves_per_row);
                while (g < g_last && off[g + 1] <= r) ++g;
            }
            s_t[j] = h < n_half ? st[g] : 0.0f;
        }
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int j = 0; j < NVDQ_SLOTS; ++j) {
        const uint32_t h = base + 256u * j;
        const uint32_t mag = code[j] & 0x7Fu;
        const float bm = e4m3_decode_mag(mag);
        const float bscale = (mag == 0x7Fu) ? __uint_as_float(0x7FC00000u)
                                            : ((code[j] & 0x80u) ? -bm : bm);
        const float t = s_t[j];
        uint4 o;
        if (mag != 0x7Fu && fabsf(t) <= FLT_MAX) {
            o = make_uint4(nv_dec2<0>(w[j], bscale, t), nv_dec2<1>(w[j], bscale, t),
                           nv_dec2<2>(w[j], bscale, t), nv_dec2<3>(w[j], bscale, t));
        } else {
            o = make_uint4(nv_dec2_nan<0>(w[j], bscale, t), nv_dec2_nan<1>(w[j], bscale, t),
                           nv_dec2_nan<2>(w[j], bscale, t), nv_dec2_nan<3>(w[j], bscale, t));
        }
        if (h < n_half) st_stream<NVDQ_NT_STORE>(y + h, o);
    }
}

// ----------------------------------------------------------------------------- launch

// Spans of RPW rows per wave; FULL when every span fills its NS slots exactly (the last
// span of an odd row count under RPW = 2 takes the bounds-checked kernel).  One-row spans
// run one wave per workgroup: 450-451 -> 444.5-445 us on the 524288 x 2048 routed rows
// inside the step (the step 6172-6186 -> 6210-6219 GB/s), 168.7 -> 166.3 us on 196608 x
// 2048 timed with the following read, then with consecutive rows on different XCDs; the
// same change made two-row spans slower (262144 x 768: 82.3 -> 88.7 us), which keep
// NV_WAVES.  Both now take their rows in XCD chunks of 512 rows (xcd_chunk, which needs the
// grid to be exactly one workgroup per WAVES spans, as here).  Either way the grid has one wave per
// span, so nv_quant_launch_fits (which counts NV_WAVES-wave workgroups, the stricter count)
// covers both.
template <int NS, int RPW>
static void launch_rows(const void* x, int64_t R, int64_t K, void* q, void* sb, float* st,
                        const int64_t* off, int64_t E, int32_t* status, hipStream_t stream) {
    constexpr int WAVES = RPW == 1 ? 1 : NV_WAVES;
    const int64_t spans = (R + RPW - 1) / RPW;
    const int64_t grid = (spans + WAVES - 1) / WAVES;
    const bool full = RPW * K == 512 * NS && R % RPW == 0;
    if (full)
        hipLaunchKernelGGL((nv_quant_rows_kernel<NS, RPW, true, WAVES>), dim3((unsigned)grid), dim3(64 * WAVES), 0,
                           stream, (const uint4*)x, (uint32_t*)q, (uint8_t*)sb, st, R, K, off, E, status);
    else
        hipLaunchKernelGGL((nv_quant_rows_kernel<NS, RPW, false, WAVES>), dim3((unsigned)grid), dim3(64 * WAVES), 0,
                           stream, (const uint4*)x, (uint32_t*)q, (uint8_t*)sb, st, R, K, off, E, status);
}

// Rows of at most this many elements go two to a wave.
#ifndef BSQ_NV_PAIR_MAX_K
#define BSQ_NV_PAIR_MAX_K 768
#endif
constexpr int64_t NV_PAIR_MAX_K = BSQ_NV_PAIR_MAX_K;

// Workgroups of NV_WAVES waves for the per-row quantizers (per-token, grouped, per-group
// pass 2, scatter): one wave per span of two rows up to NV_PAIR_MAX_K, of one row above
// (the per-token quantizer and the scatter launch their one-row spans as one-wave
// workgroups: the same waves, and a grid that fits whenever this one does).
static int64_t nv_rows_grid(int64_t R, int64_t K) {
    const int64_t rpw = K <= NV_PAIR_MAX_K ? 2 : 1;
    return ((R + rpw - 1) / rpw + NV_WAVES - 1) / NV_WAVES;
}

// The grids of the launchers below fit one dispatch?
bool nv_quant_launch_fits(int64_t R, int64_t K) { return dispatch_fits(nv_rows_grid(R, K), 64 * NV_WAVES); }

bool nv_group_launch_fits(int64_t R, int64_t K, int64_t G) {
    return nv_quant_launch_fits(R, K) && dispatch_fits((G + 255) / 256, 256);
}

bool nv_2d_launch_fits(int64_t R, int64_t K, int64_t G) {
    const int64_t strips = (R / 16) * ((K + NV2D_COLS - 1) / NV2D_COLS);
    return dispatch_fits((strips + NV_WAVES - 1) / NV_WAVES, 64 * NV_WAVES) && dispatch_fits((G + 255) / 256, 256);
}

// The dequantizers index half blocks (8 codes) with 32 bits and split a tensor into row
// ranges of at most 2^31 half blocks: a row must fit in one range (whole 16-row tiles for
// the 16x16 layout).
bool nv_dequant_launch_fits(int64_t R, int64_t K) {
    (void)R;
    return K / 8 <= (int64_t(1) << 31);
}

bool nv_dequant_2d_launch_fits(int64_t R, int64_t K) {
    (void)R;
    return 16 * (K / 8) <= (int64_t(1) << 31);
}

hipError_t launch_nv_quant(const void* x, int64_t R, int64_t K, void* q, void* sb, float* st,
                           const int64_t* offsets, int64_t E, int32_t* status,
                           hipStream_t stream) {
    const int64_t slots = (K / 8 + 63) / 64;
    const int64_t grid = (R + NV_WAVES - 1) / NV_WAVES;
    if (R == 0 || K == 0) {
        // nothing to quantize; still report on the offsets when asked to
        if (status != nullptr)
            hipLaunchKernelGGL(nv_check_offsets_kernel, dim3(1), dim3(64), 0, stream, offsets, E, R,
                               status);
        return hipGetLastError();
    }
    if (K <= NV_PAIR_MAX_K) {
        switch ((2 * (K / 8) + 63) / 64) {
            case 1: launch_rows<1, 2>(x, R, K, q, sb, st, offsets, E, status, stream); break;
            case 2: launch_rows<2, 2>(x, R, K, q, sb, st, offsets, E, status, stream); break;
            case 3: launch_rows<3, 2>(x, R, K, q, sb, st, offsets, E, status, stream); break;
            default: launch_rows<4, 2>(x, R, K, q, sb, st, offsets, E, status, stream); break;
        }
        return hipGetLastError();
    }
    switch (slots) {
        case 1: launch_rows<1, 1>(x, R, K, q, sb, st, offsets, E, status, stream); break;
        case 2: launch_rows<2, 1>(x, R, K, q, sb, st, offsets, E, status, stream); break;
        case 3: launch_rows<3, 1>(x, R, K, q, sb, st, offsets, E, status, stream); break;
        case 4: launch_rows<4, 1>(x, R, K, q, sb, st, offsets, E, status, stream); break;
        case 5: case 6: launch_rows<6, 1>(x, R, K, q, sb, st, offsets, E, status, stream); break;
        case 7: case 8: launch_rows<8, 1>(x, R, K, q, sb, st, offsets, E, status, stream); break;
        default:
            hipLaunchKernelGGL(nv_quant_rows_long_kernel, dim3((unsigned)grid), dim3(64 * NV_WAVES), 0,
                               stream, (const uint4*)x, (uint32_t*)q, (uint8_t*)sb, st, R, K,
                               offsets, E, status);
    }
    return hipGetLastError();
}

template <int SLOTS, bool GROUPED>
static hipError_t launch_nv_dequant_slots(const void* q, const void* sb, const float* st, int64_t R,
                                          int64_t K, void* y, const int64_t* off, int64_t G,
                                          hipStream_t stream) {
    // 32-bit half-block indices: launch row ranges of fewer than 2^31 half blocks each
    const int64_t hpr = K / 8;
    const int64_t rows_per_launch = ((int64_t)1 << 31) / hpr;
    const FastDiv div = make_fastdiv((uint32_t)hpr);
    for (int64_t r0 = 0; r0 < R; r0 += rows_per_launch) {
        const int64_t rows = (R - r0 < rows_per_launch) ? R - r0 : rows_per_launch;
        const int64_t n_half = rows * hpr;
        const int64_t grid = (n_half + 256 * SLOTS - 1) / (256 * SLOTS);
        hipLaunchKernelGGL((nv_dequant_kernel<SLOTS, GROUPED>), dim3((unsigned)grid), dim3(256),
                           0, stream,
                           (const uint32_t*)q + r0 * hpr, (const uint8_t*)sb + r0 * (K / 16),
                           GROUPED ? st : st + r0, (uint4*)y + r0 * hpr, (uint32_t)n_half, div,
                           off, G, r0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_nv_dequant(const void* q, const void* sb, const float* st, int64_t R, int64_t K,
                             void* y, hipStream_t stream) {
    return launch_nv_dequant_slots<NV_DQ_SLOTS, false>(q, sb, st, R, K, y, nullptr, 0, stream);
}

// Slots per thread of the per-group dequant (each workgroup first finds the groups of its
// first and last rows).  Measured on the 128-expert weights: gate_up 212 / 167 / 178 us and
// down 110 / 88 / 92 us with 2 / 4 / 8 slots.
#ifndef BSQ_NV_DQ_GROUP_SLOTS
#define BSQ_NV_DQ_GROUP_SLOTS 4
#endif

hipError_t launch_nv_dequant_group(const void* q, const void* sb, const float* s_group, const int64_t* off,
                                   int64_t G, int64_t R, int64_t K, void* y, hipStream_t stream) {
    return launch_nv_dequant_slots<BSQ_NV_DQ_GROUP_SLOTS, true>(q, sb, s_group, R, K, y, off, G, stream);
}

template <int NS, int RPW>
static void launch_group_passes(const void* x, int64_t R, int64_t K, void* q, void* sb, uint32_t* bits,
                                const int64_t* off, int64_t G, hipStream_t stream) {
    const int64_t spans = (R + RPW - 1) / RPW;
    const int64_t grid = (spans + NV_WAVES - 1) / NV_WAVES;
    const bool full = RPW * K == 512 * NS && R % RPW == 0;
    if (full)
        hipLaunchKernelGGL((nv_group_quant_kernel<NS, RPW, true>), dim3((unsigned)grid), dim3(64 * NV_WAVES),
                           0, stream, (const uint4*)x, (uint32_t*)q, (uint8_t*)sb, R, K, off, G, bits);
    else
        hipLaunchKernelGGL((nv_group_quant_kernel<NS, RPW, false>), dim3((unsigned)grid), dim3(64 * NV_WAVES),
                           0, stream, (const uint4*)x, (uint32_t*)q, (uint8_t*)sb, R, K, off, G, bits);
}

// Pass 1 of the per-group scales: a few workgroups per compute unit, grid-stride; the LDS
// table of group maxima when G fits in it.
static void launch_group_amax(const void* x, int64_t R, int64_t K, const int64_t* off, int64_t G,
                              uint32_t* bits, hipStream_t stream) {
    const int64_t per_wg = (int64_t)NV_WAVES * 64 * NV_AMAX_PIECES;
    const int64_t need = (R * (K >> 3) + per_wg - 1) / per_wg;
    const int64_t agrid = std::min<int64_t>(need, 256 * BSQ_NV_AMAX_WGS_PER_CU);
    if (G <= NV_AMAX_LDS_STARTS)
        hipLaunchKernelGGL((nv_group_amax_kernel<true, true>), dim3((unsigned)agrid), dim3(64 * NV_WAVES),
                           (size_t)(G + 1) * sizeof(int64_t) + (size_t)G * sizeof(uint32_t), stream,
                           (const uint4*)x, R, K, off, G, bits);
    else if (G <= NV_AMAX_LDS_GROUPS)
        hipLaunchKernelGGL((nv_group_amax_kernel<true, false>), dim3((unsigned)agrid), dim3(64 * NV_WAVES),
                           (size_t)G * sizeof(uint32_t), stream, (const uint4*)x, R, K, off, G, bits);
    else
        hipLaunchKernelGGL((nv_group_amax_kernel<false, false>), dim3((unsigned)agrid), dim3(64 * NV_WAVES), 0, stream,
                           (const uint4*)x, R, K, off, G, bits);
}

hipError_t launch_nv_quant_2d(const void* x, int64_t R, int64_t K, const int64_t* off, int64_t G,
                              void* q, void* sb, float* s_group, int32_t* status, hipStream_t stream) {
    uint32_t* bits = reinterpret_cast<uint32_t*>(s_group);
    const unsigned gg = (unsigned)((G + 255) / 256);
    hipLaunchKernelGGL(nv_group_init_kernel, dim3(gg), dim3(256), 0, stream, bits, G, off, R, status, (int64_t)16);
    if (R > 0 && K > 0) {
        launch_group_amax(x, R, K, off, G, bits, stream);
        const int64_t col_strips = (K + NV2D_COLS - 1) / NV2D_COLS;
        const int64_t strips = (R / 16) * col_strips;
        const int64_t grid = (strips + NV_WAVES - 1) / NV_WAVES;
        if (K % NV2D_COLS == 0)
            hipLaunchKernelGGL(nv_quant_2d_kernel<true>, dim3((unsigned)grid), dim3(64 * NV_WAVES), 0, stream,
                               (const uint16_t*)x, (uint32_t*)q, (uint8_t*)sb, R, K, off, G, bits, col_strips);
        else
            hipLaunchKernelGGL(nv_quant_2d_kernel<false>, dim3((unsigned)grid), dim3(64 * NV_WAVES), 0, stream,
                               (const uint16_t*)x, (uint32_t*)q, (uint8_t*)sb, R, K, off, G, bits, col_strips);
    }
    hipLaunchKernelGGL(nv_group_finalize_kernel, dim3(gg), dim3(256), 0, stream, s_group, G);
    return hipGetLastError();
}

hipError_t launch_nv_dequant_2d(const void* q, const void* sb, const float* s_group, const int64_t* off,
                                int64_t G, int64_t R, int64_t K, void* y, hipStream_t stream) {
    // 32-bit half-block indices: row ranges of fewer than 2^31 half blocks, whole tiles each
    const int64_t hpr = K / 8;
    const int64_t rows_per_launch = (((int64_t)1 << 31) / hpr) / 16 * 16;
    const FastDiv div = make_fastdiv((uint32_t)hpr);
    for (int64_t r0 = 0; r0 < R; r0 += rows_per_launch) {
        const int64_t rows = (R - r0 < rows_per_launch) ? R - r0 : rows_per_launch;
        const int64_t n_half = rows * hpr;
        const int64_t grid = (n_half + 256 * BSQ_NV_DQ_GROUP_SLOTS - 1) / (256 * BSQ_NV_DQ_GROUP_SLOTS);
        hipLaunchKernelGGL((nv_dequant_kernel<BSQ_NV_DQ_GROUP_SLOTS, true, true>), dim3((unsigned)grid), dim3(256),
                           0, stream, (const uint32_t*)q + r0 * hpr, (const uint8_t*)sb + (r0 / 16) * (K / 16),
                           s_group, (uint4*)y + r0 * hpr, (uint32_t)n_half, div, off, G, r0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_nv_quant_group(const void* x, int64_t R, int64_t K, const int64_t* off, int64_t G,
                                 void* q, void* sb, float* s_group, int32_t* status, hipStream_t stream) {
    uint32_t* bits = reinterpret_cast<uint32_t*>(s_group);   // group maxima, then the scales
    const unsigned gg = (unsigned)((G + 255) / 256);
    hipLaunchKernelGGL(nv_group_init_kernel, dim3(gg), dim3(256), 0, stream, bits, G, off, R, status, (int64_t)1);
    if (R > 0 && K > 0) {
        launch_group_amax(x, R, K, off, G, bits, stream);
        if (K <= NV_PAIR_MAX_K) {
            switch ((2 * (K / 8) + 63) / 64) {
                case 1: launch_group_passes<1, 2>(x, R, K, q, sb, bits, off, G, stream); break;
                case 2: launch_group_passes<2, 2>(x, R, K, q, sb, bits, off, G, stream); break;
                default: launch_group_passes<3, 2>(x, R, K, q, sb, bits, off, G, stream); break;
            }
        } else {
            switch ((K / 8 + 63) / 64) {
                case 2: launch_group_passes<2, 1>(x, R, K, q, sb, bits, off, G, stream); break;
                case 3: launch_group_passes<3, 1>(x, R, K, q, sb, bits, off, G, stream); break;
                case 4: launch_group_passes<4, 1>(x, R, K, q, sb, bits, off, G, stream); break;
                case 5: case 6: launch_group_passes<6, 1>(x, R, K, q, sb, bits, off, G, stream); break;
                case 7: case 8: launch_group_passes<8, 1>(x, R, K, q, sb, bits, off, G, stream); break;
                default: {
                    const int64_t grid = (R + NV_WAVES - 1) / NV_WAVES;
                    hipLaunchKernelGGL(nv_group_quant_long_kernel, dim3((unsigned)grid), dim3(64 * NV_WAVES),
                                       0, stream, (const uint4*)x, (uint32_t*)q, (uint8_t*)sb, R, K, off, G, bits);
                }
            }
        }
    }
    hipLaunchKernelGGL(nv_group_finalize_kernel, dim3(gg), dim3(256), 0, stream, s_group, G);
    return hipGetLastError();
}

template <int NS, int RPW>
static void launch_scatter(const void* h, int64_t T, int64_t K, const int64_t* dst, int64_t top_k, int64_t N,
                           void* q, void* sb, float* st, int32_t* status, hipStream_t stream) {
    // One wave per workgroup for single-row spans, as in the row kernel.
    constexpr int WAVES = RPW == 1 ? 1 : NV_WAVES;
    const int64_t spans = (T + RPW - 1) / RPW;
    const int64_t grid = (spans + WAVES - 1) / WAVES;
    const bool full = RPW * K == 512 * NS && T % RPW == 0;
    if (full)
        hipLaunchKernelGGL((nv_quant_scatter_kernel<NS, RPW, true, WAVES>), dim3((unsigned)grid), dim3(64 * WAVES),
                           0, stream, (const uint4*)h, T, K, dst, top_k, N, (uint32_t*)q, (uint8_t*)sb, st, status);
    else
        hipLaunchKernelGGL((nv_quant_scatter_kernel<NS, RPW, false, WAVES>), dim3((unsigned)grid), dim3(64 * WAVES),
                           0, stream, (const uint4*)h, T, K, dst, top_k, N, (uint32_t*)q, (uint8_t*)sb, st, status);
}

hipError_t launch_nv_quant_scatter(const void* h, int64_t T, int64_t K, const int64_t* dst, int64_t top_k,
                                   int64_t N, void* q, void* sb, float* st, int32_t* status,
                                   hipStream_t stream) {
    if (status != nullptr)
        hipLaunchKernelGGL(nv_status_clear_kernel, dim3(1), dim3(64), 0, stream, status);
    if (T == 0 || K == 0 || N == 0) {
        if (T > 0 && K > 0 && status != nullptr) {   // no rows to write, but report bad entries
            hipLaunchKernelGGL(nv_quant_scatter_long_kernel, dim3((unsigned)((T + NV_WAVES - 1) / NV_WAVES)),
                               dim3(64 * NV_WAVES), 0, stream, (const uint4*)h, T, K, dst, top_k, N,
                               (uint32_t*)q, (uint8_t*)sb, st, status);
        }
        return hipGetLastError();
    }
    if (K <= NV_PAIR_MAX_K) {
        switch ((2 * (K / 8) + 63) / 64) {
            case 1: launch_scatter<1, 2>(h, T, K, dst, top_k, N, q, sb, st, status, stream); break;
            case 2: launch_scatter<2, 2>(h, T, K, dst, top_k, N, q, sb, st, status, stream); break;
            default: launch_scatter<3, 2>(h, T, K, dst, top_k, N, q, sb, st, status, stream); break;
        }
        return hipGetLastError();
    }
    switch ((K / 8 + 63) / 64) {
        case 2: launch_scatter<2, 1>(h, T, K, dst, top_k, N, q, sb, st, status, stream); break;
        case 3: launch_scatter<3, 1>(h, T, K, dst, top_k, N, q, sb, st, status, stream); break;
        case 4: launch_scatter<4, 1>(h, T, K, dst, top_k, N, q, sb, st, status, stream); break;
        case 5: case 6: launch_scatter<6, 1>(h, T, K, dst, top_k, N, q, sb, st, status, stream); break;
        case 7: case 8: launch_scatter<8, 1>(h, T, K, dst, top_k, N, q, sb, st, status, stream); break;
        default:
            hipLaunchKernelGGL(nv_quant_scatter_long_kernel, dim3((unsigned)((T + NV_WAVES - 1) / NV_WAVES)),
                               dim3(64 * NV_WAVES), 0, stream, (const uint4*)h, T, K, dst, top_k, N,
                               (uint32_t*)q, (uint8_t*)sb, st, status);
    }
    return hipGetLastError();
}

}  // namespace bsq
