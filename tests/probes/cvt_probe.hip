// cvt_probe.hip -- test-only kernels that apply the library's conversion helpers
// (block_scaled_precision_mxfp8_amd/csrc/bsq_device.h) to every binary32 bit pattern of
// a range, so the tests can compare them with the CPU oracle over all 2^32 inputs.
// Built with the library's own compiler flags.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsq_device.h"

// Thread i converts the patterns start + 2i and start + 2i + 1 (n is even).
__global__ void sweep_e2m1_kernel(uint32_t start, int64_t n, uint8_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (2 * i >= n) return;
    const float a = __uint_as_float(start + (uint32_t)(2 * i));
    const float b = __uint_as_float(start + (uint32_t)(2 * i + 1));
    out[i] = (uint8_t)bsq::cvt_e2m1x2_f32<0>(0u, a, b);
}

__global__ void sweep_bf16_kernel(uint32_t start, int64_t n, uint32_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (2 * i >= n) return;
    const float a = __uint_as_float(start + (uint32_t)(2 * i));
    const float b = __uint_as_float(start + (uint32_t)(2 * i + 1));
    out[i] = bsq::cvt_bf16x2_f32(a, b);
}

extern "C" {
// out: device buffer of n/2 bytes (E2M1) or n/2 dwords (BF16 pairs); n even, > 0.
int probe_sweep_e2m1(uint32_t start, int64_t n, void* out) {
    const int64_t threads = n / 2;
    hipLaunchKernelGGL(sweep_e2m1_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, 0,
                       start, n, (uint8_t*)out);
    return (int)hipDeviceSynchronize();
}
int probe_sweep_bf16(uint32_t start, int64_t n, void* out) {
    const int64_t threads = n / 2;
    hipLaunchKernelGGL(sweep_bf16_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, 0,
                       start, n, (uint32_t*)out);
    return (int)hipDeviceSynchronize();
}
}
