// Measurement kernel: the MFMA throughput this GPU sustains with no memory
// traffic at all (register operands only), the ceiling against which the
// expert GEMMs' rate is also reported.  Each wave runs 8 independent
// accumulator chains of v_mfma_f32_32x32x16_bf16 (enough in flight to keep
// its SIMD's matrix core busy); 4 waves per workgroup, one per SIMD.
#include "device_util.h"
#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 pk_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float pk_f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* __restrict__ sink) {
    pk_bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = static_cast<__bf16>(static_cast<float>((threadIdx.x + i) & 7) * 0.125f);
        b[i] = static_cast<__bf16>(static_cast<float>((threadIdx.x * 3 + i) & 7) * 0.0625f);
    }
    pk_f32x16_t acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    // one value per workgroup keeps the chains live
    if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_peak(int workgroups, int iters, float* sink, hipStream_t s) {
    mfma_peak_kernel<<<static_cast<unsigned>(workgroups), 256, 0, s>>>(iters, sink);
    return hipGetLastError();
}

}  // namespace moe
