// Measurement kernels, not part of the layer:
//   - the MFMA throughput this GPU sustains with no memory traffic at all
//     (register operands only), the ceiling against which the expert GEMMs'
//     rate is also reported.  Each wave runs 8 independent accumulator chains
//     of v_mfma_f32_32x32x16_bf16 (enough in flight to keep its SIMD's matrix
//     core busy); 4 waves per workgroup, one per SIMD;
//   - a plain device copy in 16-byte words, the streaming ceiling against
//     which the dispatch and combine bandwidths are also reported (and the
//     reference that calibrates the HBM byte counters).
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

// dst[i] = src[i] over n16 16-byte words: each workgroup copies 2048-word
// (32 KB) blocks, 8 loads in flight per thread, blocks strided by the grid.
constexpr int kCopyUnroll = 8;
constexpr int64_t kCopyBlockWords = 256 * kCopyUnroll;

__global__ __launch_bounds__(256) void stream_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                          int64_t n16) {
    const int64_t step = static_cast<int64_t>(gridDim.x) * kCopyBlockWords;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kCopyBlockWords; base < n16; base += step) {
        uint4 v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int64_t i = base + u * 256 + threadIdx.x;
            if (i < n16) v[u] = src[i];
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int64_t i = base + u * 256 + threadIdx.x;
            if (i < n16) dst[i] = v[u];
        }
    }
}

}  // namespace

hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
    const int64_t n16 = static_cast<int64_t>(bytes / 16);
    const int64_t blocks = ceil_div(n16, kCopyBlockWords);
    const unsigned grid = static_cast<unsigned>(blocks < 65536 ? blocks : 65536);
    stream_copy_kernel<<<grid, 256, 0, s>>>(static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16);
    return hipGetLastError();
}

hipError_t launch_mfma_peak(int workgroups, int iters, float* sink, hipStream_t s) {
    mfma_peak_kernel<<<static_cast<unsigned>(workgroups), 256, 0, s>>>(iters, sink);
    return hipGetLastError();
}

}  // namespace moe
