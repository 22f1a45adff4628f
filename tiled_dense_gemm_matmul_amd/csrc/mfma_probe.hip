// MFMA ceiling probe (measurement support, not part of the GEMM path).
//
// Streams of independent v_mfma_f32_16x16x4_f32 with random operands and no
// memory traffic inside the timed loop, so that a timing harness can check
// how much of the fp32 matrix-core peak (256 CUs x 256 flop per clock at
// 2.4 GHz = 157.3 TFLOP/s) the chip sustains, and at which engine clock.  Each wave records its start and end on the shader
// clock (s_memtime) and on the 100 MHz constant clock (s_memrealtime); their
// ratio is the engine clock while the MFMAs ran.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mfma_probe.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float hash_to_unit(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return (float)(x & 0xffffffu) * (1.0f / 16777216.0f) - 0.5f;
}

// Every wave runs `iters` x 8 MFMAs over four accumulators (two dependent
// MFMAs per accumulator per iteration, eight independent operand pairs).
__global__ __launch_bounds__(256) void mfma_probe_kernel(float *sink, unsigned long long *clocks, int iters) {
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    float a[8], b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = hash_to_unit(t * 16u + j);
        b[j] = hash_to_unit(t * 16u + 8u + j);
    }
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc[j & 3], 0, 0, 0);
    }
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    sink[t] = s;
    if (threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = c1 - c0;
        clocks[2 * blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace

extern "C" int mfma_probe_launch(float *sink, unsigned long long *clocks, int blocks, int iters, void *stream) {
    if (sink == nullptr || clocks == nullptr || blocks <= 0 || blocks > (1 << 20) || iters <= 0 || iters > (1 << 24))
        return -1;
    hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream), sink,
                       clocks, iters);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

extern "C" long long mfma_probe_flops(int blocks, int iters) {
    // 4 waves per block, 8 MFMAs per iteration, 2 * 16 * 16 * 4 flops each
    return (long long)blocks * 4 * iters * 8 * 2048;
}
