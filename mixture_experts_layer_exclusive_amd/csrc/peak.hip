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

// dst[i] = src[i] over n16 16-byte words.  A workgroup copies 1024-word
// (16 KB) blocks strided by the grid: each thread first loads its 4 words
// (all in flight together), then stores them, with non-temporal loads and
// stores (the data is touched once).  Measured on one MI355X, 1 GiB: 6.0
// TB/s on 4096 workgroups, against 5.3 TB/s for hipMemcpyAsync and 5.3-5.6
// TB/s with 8 or 16 words per thread or temporal accesses.
constexpr int kCopyUnroll = 4;
constexpr int64_t kCopyBlockWords = 256 * kCopyUnroll;
constexpr int64_t kCopyGrid = 4096;

__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                          int64_t n16) {
    const int64_t step = static_cast<int64_t>(gridDim.x) * kCopyBlockWords;
    int64_t base = static_cast<int64_t>(blockIdx.x) * kCopyBlockWords;
    // whole blocks: no bounds checks between the loads, so all 4 are in flight
    for (; base + kCopyBlockWords <= n16; base += step) {
        const u32x4_t* s = src + base + threadIdx.x;
        u32x4_t* d = dst + base + threadIdx.x;
        u32x4_t v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) v[u] = __builtin_nontemporal_load(s + u * 256);
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(v[u], d + u * 256);
    }
    // the last, partial block
    if (base < n16) {
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int64_t i = base + u * 256 + threadIdx.x;
            if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
        }
    }
}

}  // namespace

hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
    const int64_t n16 = static_cast<int64_t>(bytes / 16);
    const int64_t blocks = ceil_div(n16, kCopyBlockWords);
    const unsigned grid = static_cast<unsigned>(blocks < kCopyGrid ? blocks : kCopyGrid);
    stream_copy_kernel<<<grid, 256, 0, s>>>(static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), n16);
    return hipGetLastError();
}

hipError_t launch_mfma_peak(int workgroups, int iters, float* sink, hipStream_t s) {
    mfma_peak_kernel<<<static_cast<unsigned>(workgroups), 256, 0, s>>>(iters, sink);
    return hipGetLastError();
}

}  // namespace moe
