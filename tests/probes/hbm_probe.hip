// hbm_probe.hip -- measurement-only kernels that move bytes the way the library's kernels
// do, with no arithmetic, so that a kernel's time can be set against what its access
// pattern costs on the device: plain 16-byte streams (read, write, copy) and the access
// patterns of the per-token NVFP4 quantizer on rows of 2048 BF16, of its dequantizer, of the
// quantize-then-scatter, and of the MXFP8 dual quantizer on 128 x 256 tiles.  Not part of
// the library; `bench.py --hbm-ceiling` times them.  The streams take one 16-byte piece per lane, the
// NVFP4 quantizer pattern one row per wave, the dequantizer two output pieces a thread, the
// scatter one token per wave, the MXFP8 pattern one tile per workgroup (no grid-stride
// loops); the host wrappers below size the grids and check the sizes.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }

template <bool NT>
__device__ __forceinline__ void st(u32x4* p, u32x4 v) {
    if (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Read-only: the XOR of each lane's piece is stored only if it equals a value the inputs
// never produce, which keeps the loads alive without writing anything.
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ x, uint32_t* __restrict__ sink) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const u32x4 v = ld_nt(x + i);
    const uint32_t h = v.x ^ v.y ^ v.z ^ v.w;
    if (h == 0x5EEDF00Du) sink[0] = h;
}

template <bool NT>
__global__ __launch_bounds__(256) void write_kernel(u32x4* __restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const uint32_t t = (uint32_t)i;
    st<NT>(y + i, u32x4{t, t ^ 1u, t ^ 2u, t ^ 3u});
}

template <bool NT>
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ x, u32x4* __restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    st<NT>(y + i, ld_nt(x + i));
}

// Row of workgroup b of n when rows are dealt to the eight XCDs (b % 8) in chunks of 512
// consecutive rows, as the per-token quantizer deals them; rows past the last whole round of
// eight chunks keep row = b.
__device__ __forceinline__ int64_t chunk_row(int64_t b, int64_t n) {
    const int64_t full = n / 4096 * 4096;
    if (b >= full) return b;
    const int64_t c = b >> 3;
    return ((c / 512) * 8 + (b & 7)) * 512 + c % 512;
}

// The per-token NVFP4 quantizer's traffic on rows of 2048 BF16 (256 pieces): one wave per
// row and per workgroup, the rows dealt to the XCDs as the quantizer deals them (chunk_row),
// four 16-byte loads a lane at raised wave priority, then per row
// 1 KiB of codes as 4-byte stores (256 bytes per store instruction), 128 scale bytes gathered
// in LDS and written as eight 16-byte stores, and one 4-byte token scale.  The stored values
// are XORs of the loaded ones, not codes.
__global__ __launch_bounds__(64) void nv_pattern_kernel(const u32x4* __restrict__ x, uint32_t* __restrict__ q,
                                                        uint8_t* __restrict__ sb, float* __restrict__ s) {
    __shared__ __align__(16) uint8_t lsb[1][128];
    const int lane = threadIdx.x & 63, wave = 0;
    const int64_t row = chunk_row(blockIdx.x, gridDim.x);
    const u32x4* xr = x + row * 256;
    u32x4 v[4];
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = ld_nt(xr + 64 * j + lane);
    __builtin_amdgcn_s_setprio(0);
    uint32_t* qr = q + row * 256;
#pragma unroll
    for (int j = 0; j < 4; ++j) __builtin_nontemporal_store(v[j].x ^ v[j].y ^ v[j].z ^ v[j].w, qr + 64 * j + lane);
    if ((lane & 1) == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) lsb[wave][32 * j + (lane >> 1)] = (uint8_t)v[j].x;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < 8)
        __builtin_nontemporal_store(reinterpret_cast<const u32x4*>(lsb[wave])[lane],
                                    reinterpret_cast<u32x4*>(sb + row * 128) + lane);
    if (lane == 0) s[row] = __uint_as_float(v[0].y);
}

// The MXFP8 dual quantizer's traffic (rowwise and columnwise copies) on 128 x 256 tiles, one
// workgroup of four waves a tile: lane 8g + c of wave w loads rows 16g .. 16g+15 of the
// tile's columns 64w + 8c .. +7 (sixteen 16-byte loads at raised priority), stages 8 bytes a
// row for q_row and 16 bytes a column for q_col in LDS, and after a barrier writes whole
// 256-byte tile rows of q_row and whole 128-byte lines of q_col with 16-byte non-temporal
// stores, then the 8 s_row bytes of each tile row and the 4 s_col bytes of each tile column
// with ordinary stores.  The bytes written are XORs of the loaded ones, not codes.
constexpr int MXT_ROWS = 128, MXT_COLS = 256;
__global__ __launch_bounds__(256) void mx_dual_pattern_kernel(const uint8_t* __restrict__ x, int64_t M, int64_t K,
                                                              uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                                                              uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col,
                                                              int64_t col_groups) {
    __shared__ __align__(16) uint8_t lq[MXT_ROWS][MXT_COLS + 16];
    __shared__ __align__(16) uint8_t lc[MXT_COLS][MXT_ROWS + 16];
    __shared__ __align__(16) uint8_t lsr[MXT_ROWS][8];
    __shared__ __align__(16) uint8_t lsc[MXT_COLS][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 3, c = lane & 7;
    const int64_t stripe = blockIdx.x / col_groups;
    const int64_t rw = stripe * MXT_ROWS, kw = (blockIdx.x - stripe * col_groups) * MXT_COLS;
    const int lrow = 16 * g, lcol = 64 * wave + 8 * c;
    const uint8_t* base = x + 2 * ((rw + lrow) * K + kw + lcol);
    u32x4 v[16];
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = ld_nt(reinterpret_cast<const u32x4*>(base + 2 * i * K));
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        *reinterpret_cast<uint2*>(&lq[lrow + i][lcol]) = make_uint2(v[i].x ^ v[i].y, v[i].z ^ v[i].w);
        if ((c & 3) == 0) lsr[lrow + i][lcol >> 5] = (uint8_t)v[i].x;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const u32x4 cc = {v[0].x ^ v[4 + (e & 3)].y, v[1].z ^ v[8].w, v[2 + (e >> 2)].x ^ v[12].y, v[3].w ^ v[15].x};
        *reinterpret_cast<u32x4*>(&lc[lcol + e][lrow]) = cc;
        if ((g & 1) == 0) lsc[lcol + e][lrow >> 5] = (uint8_t)cc.x;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {                     // 128 tile rows x 16 pieces
        const int idx = j * 256 + (int)threadIdx.x, r = idx >> 4, c16 = idx & 15;
        st<true>(reinterpret_cast<u32x4*>(q_row + (rw + r) * K + kw + 16 * c16),
                 *reinterpret_cast<const u32x4*>(&lq[r][16 * c16]));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {                     // 256 tile columns x 8 pieces
        const int idx = j * 256 + (int)threadIdx.x, col = idx >> 3, part = idx & 7;
        st<true>(reinterpret_cast<u32x4*>(q_col + (kw + col) * M + rw + 16 * part),
                 *reinterpret_cast<const u32x4*>(&lc[col][16 * part]));
    }
    if (threadIdx.x < MXT_ROWS)
        *reinterpret_cast<uint2*>(s_row + (rw + threadIdx.x) * (K / 32) + kw / 32) =
            *reinterpret_cast<const uint2*>(lsr[threadIdx.x]);
    *reinterpret_cast<uint32_t*>(s_col + (kw + threadIdx.x) * (M / 32) + rw / 32) =
        *reinterpret_cast<const uint32_t*>(lsc[threadIdx.x]);
}

// The per-token NVFP4 dequantizer's traffic: 256 threads a workgroup, two slots a thread;
// for half block h (8 elements) a thread loads the code dword h, scale byte h / 2 and token
// scale h / hpr, and writes 16 bytes of output at h.  The stored dwords are a, a+1, a+2, a+3
// for a = code ^ scale byte ^ token-scale bits, not BF16 values.
__global__ __launch_bounds__(256) void nv_dq_pattern_kernel(const uint32_t* __restrict__ q, const uint8_t* __restrict__ sb,
                                                            const float* __restrict__ s, u32x4* __restrict__ y,
                                                            uint32_t n_half, uint32_t hpr) {
    const uint32_t base = blockIdx.x * 512u + threadIdx.x;
    uint32_t w[2], c[2], t[2];
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t h = base + 256u * j;
        const bool ok = h < n_half;
        w[j] = ok ? q[h] : 0u;
        c[j] = ok ? sb[h >> 1] : 0u;
        t[j] = ok ? __float_as_uint(s[h / hpr]) : 0u;
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t h = base + 256u * j;
        const uint32_t a = w[j] ^ c[j] ^ t[j];
        if (h < n_half) st<true>(y + h, u32x4{a, a + 1u, a + 2u, a + 3u});
    }
}

// The quantize-then-scatter's traffic on tokens of 2048 BF16: one wave per token and per
// workgroup reads the token (four 16-byte loads a lane at raised priority) and its
// destination rows (one load, entries 0..top_k-1 in lanes 0..top_k-1, top_k <= 64), then for
// each destination writes the row's 1 KiB of codes as 4-byte stores, its 128 scale bytes
// (eight 16-byte stores, gathered in LDS) and its 4-byte token scale.  Values are XORs of
// the loaded ones.  Entries outside [0, N) are skipped.
__global__ __launch_bounds__(64) void scatter_pattern_kernel(const u32x4* __restrict__ x, const int64_t* __restrict__ dst,
                                                             int top_k, int64_t N, uint32_t* __restrict__ q,
                                                             uint8_t* __restrict__ sb, float* __restrict__ s) {
    __shared__ __align__(16) uint8_t lsb[128];
    const int lane = threadIdx.x & 63;
    const int64_t t = blockIdx.x;
    const u32x4* xr = x + t * 256;
    u32x4 v[4];
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = ld_nt(xr + 64 * j + lane);
    __builtin_amdgcn_s_setprio(0);
    const int64_t dl = lane < top_k ? dst[t * top_k + lane] : -1;
    uint32_t p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    if ((lane & 1) == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) lsb[32 * j + (lane >> 1)] = (uint8_t)v[j].x;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const u32x4 sv = reinterpret_cast<const u32x4*>(lsb)[lane & 7];
    for (int i = 0; i < top_k; ++i) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)dl, i);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)dl >> 32), i);
        const int64_t d = (int64_t)(((uint64_t)hi << 32) | lo);
        if (d < 0 || d >= N) continue;
        uint32_t* qr = q + d * 256;
#pragma unroll
        for (int j = 0; j < 4; ++j) __builtin_nontemporal_store(p[j], qr + 64 * j + lane);
        if (lane < 8) __builtin_nontemporal_store(sv, reinterpret_cast<u32x4*>(sb + d * 128) + lane);
        if (lane == 0) s[d] = __uint_as_float(p[0]);
    }
}

bool pieces_ok(int64_t n16) { return n16 > 0 && n16 % 256 == 0 && n16 / 256 < (int64_t(1) << 31); }

}  // namespace

extern "C" {
// n16: number of 16-byte pieces (a positive multiple of 256); buffers hold n16 * 16 bytes,
// 16-byte aligned; sink: one device dword.  Enqueued on `stream`; 0 or a hipError_t.
int hbm_probe_read(const void* x, int64_t n16, void* sink, void* stream) {
    if (!pieces_ok(n16)) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_kernel, dim3((unsigned)(n16 / 256)), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4*)x, (uint32_t*)sink);
    return (int)hipGetLastError();
}
int hbm_probe_write(void* y, int64_t n16, int nt, void* stream) {
    if (!pieces_ok(n16)) return (int)hipErrorInvalidValue;
    if (nt) hipLaunchKernelGGL(write_kernel<true>, dim3((unsigned)(n16 / 256)), dim3(256), 0, (hipStream_t)stream, (u32x4*)y);
    else hipLaunchKernelGGL(write_kernel<false>, dim3((unsigned)(n16 / 256)), dim3(256), 0, (hipStream_t)stream, (u32x4*)y);
    return (int)hipGetLastError();
}
int hbm_probe_copy(const void* x, void* y, int64_t n16, int nt, void* stream) {
    if (!pieces_ok(n16)) return (int)hipErrorInvalidValue;
    if (nt) hipLaunchKernelGGL(copy_kernel<true>, dim3((unsigned)(n16 / 256)), dim3(256), 0, (hipStream_t)stream,
                               (const u32x4*)x, (u32x4*)y);
    else hipLaunchKernelGGL(copy_kernel<false>, dim3((unsigned)(n16 / 256)), dim3(256), 0, (hipStream_t)stream,
                            (const u32x4*)x, (u32x4*)y);
    return (int)hipGetLastError();
}
// x: R rows of 2048 BF16; q: R * 1024 bytes; sb: R * 128 bytes; s: R floats; 0 < R < 2^26.
int hbm_probe_nv_pattern(const void* x, int64_t R, void* q, void* sb, void* s, void* stream) {
    if (R <= 0 || R >= (int64_t(1) << 26)) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(nv_pattern_kernel, dim3((unsigned)R), dim3(64), 0, (hipStream_t)stream,
                       (const u32x4*)x, (uint32_t*)q, (uint8_t*)sb, (float*)s);
    return (int)hipGetLastError();
}
// x: T tokens of 2048 BF16; dst: int64 [T][top_k], 1 <= top_k <= 64; q: N * 1024 bytes,
// sb: N * 128 bytes, s: N floats; 0 < T < 2^31.
int hbm_probe_scatter_pattern(const void* x, int64_t T, const int64_t* dst, int top_k, int64_t N, void* q,
                              void* sb, void* s, void* stream) {
    if (T <= 0 || T >= (int64_t(1) << 31) || top_k < 1 || top_k > 64 || N < 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(scatter_pattern_kernel, dim3((unsigned)T), dim3(64), 0, (hipStream_t)stream,
                       (const u32x4*)x, dst, top_k, N, (uint32_t*)q, (uint8_t*)sb, (float*)s);
    return (int)hipGetLastError();
}
// q: R * K / 2 bytes, sb: R * K / 16 bytes, s: R floats, y: R * K BF16; K a positive
// multiple of 16, 0 < R * K / 8 < 2^32.
int hbm_probe_nv_dequant_pattern(const void* q, const void* sb, const void* s, int64_t R, int64_t K, void* y,
                                 void* stream) {
    if (R <= 0 || K <= 0 || K % 16 != 0 || R * (K / 8) >= (int64_t(1) << 32)) return (int)hipErrorInvalidValue;
    const uint32_t n_half = (uint32_t)(R * (K / 8));
    hipLaunchKernelGGL(nv_dq_pattern_kernel, dim3((n_half + 511u) / 512u), dim3(256), 0, (hipStream_t)stream,
                       (const uint32_t*)q, (const uint8_t*)sb, (const float*)s, (u32x4*)y, n_half, (uint32_t)(K / 8));
    return (int)hipGetLastError();
}
// x: M x K BF16; q_row M * K, s_row M * K / 32, q_col K * M, s_col K * M / 32 bytes;
// M a positive multiple of 128, K of 256, (M / 128) * (K / 256) < 2^23.
int hbm_probe_mx_dual_pattern(const void* x, int64_t M, int64_t K, void* q_row, void* s_row, void* q_col,
                              void* s_col, void* stream) {
    if (M <= 0 || K <= 0 || M % MXT_ROWS != 0 || K % MXT_COLS != 0) return (int)hipErrorInvalidValue;
    const int64_t col_groups = K / MXT_COLS, wgs = (M / MXT_ROWS) * col_groups;
    if (wgs >= (int64_t(1) << 23)) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mx_dual_pattern_kernel, dim3((unsigned)wgs), dim3(256), 0, (hipStream_t)stream,
                       (const uint8_t*)x, M, K, (uint8_t*)q_row, (uint8_t*)s_row, (uint8_t*)q_col, (uint8_t*)s_col,
                       col_groups);
    return (int)hipGetLastError();
}
}
