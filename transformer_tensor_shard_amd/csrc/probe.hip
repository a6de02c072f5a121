// Measurement support, not part of the method: a register-only MFMA loop that
// gives the matrix-core throughput this GPU sustains right now (clock and
// power limits included), the ceiling against which the GEMM's roofline
// fraction can be read.  Each SIMD runs two waves of back-to-back independent
// MFMA 16x16x32 bf16 on values held in registers; nothing is loaded.
#include "tp_kernels.h"

namespace tpk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(512, 1) void mfma_probe_kernel(float* __restrict__ out, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[0][i] = (__bf16)(0.01f * (lane + i));
        b[0][i] = (__bf16)(0.01f * (lane - i));
        a[1][i] = (__bf16)(0.01f * (lane * i));
        b[1][i] = (__bf16)(0.01f * (3 - i));
    }
    f32x4 acc[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 32; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j & 1], b[(j >> 1) & 1], acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) s += acc[j][0] + acc[j][3];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;   // keeps the loop alive
}

}  // namespace

hipError_t mfma_probe(float* out, int blocks, int iters, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(512), 0, stream, out, iters);
    return hipGetLastError();
}

}  // namespace tpk
