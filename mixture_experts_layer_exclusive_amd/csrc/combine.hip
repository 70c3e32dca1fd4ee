// Gate-weighted combine (reverse dispatch; MoEBlaze summary, Methodology 2):
//   y[t, :] = sum_j gates[t, j] * y_perm[assign_pos[t*k + j], :]
// One workgroup per token; each thread owns 16-byte column chunks, reads the
// k expert rows of its token and accumulates in fp32 in ascending j, then
// rounds once.  Every y row is written exactly once, so the result does not
// depend on scheduling.
#include "device_util.h"
#include "moe_internal.h"

namespace moe {

namespace {

// KM > 0: k <= KM, the k row loads of a chunk issued together (the token's
// positions and gates read once, into LDS); KM = 0: any k, one row at a time.
template <int KM>
__global__ __launch_bounds__(256) void combine_bf16_kernel(const uint4* __restrict__ y_perm,
                                                          const int32_t* __restrict__ assign_pos,
                                                          const float* __restrict__ gates, int k,
                                                          int chunks_per_row,
                                                          uint4* __restrict__ y) {
    const int64_t t = blockIdx.x;
    if constexpr (KM > 0) {
        __shared__ int s_pos[KM];
        __shared__ float s_g[KM];
        if (threadIdx.x < KM) {
            const int j = threadIdx.x;
            s_pos[j] = j < k ? assign_pos[t * k + j] : -1;
            s_g[j] = j < k ? gates[t * k + j] : 0.f;
        }
        __syncthreads();
        int pos[KM];
        float g[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            pos[j] = s_pos[j];
            g[j] = s_g[j];
        }
        for (int c = threadIdx.x; c < chunks_per_row; c += 256) {
            uint4 v[KM];
#pragma unroll
            for (int j = 0; j < KM; ++j)
                v[j] = pos[j] >= 0 ? load_nt(y_perm + static_cast<int64_t>(pos[j]) * chunks_per_row + c)
                                   : make_uint4(0u, 0u, 0u, 0u);
            float acc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
            for (int j = 0; j < KM; ++j) {
                if (pos[j] < 0) continue;
                const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = fmaf(g[j], lo_bf16(w[i]), acc[2 * i]);
                    acc[2 * i + 1] = fmaf(g[j], hi_bf16(w[i]), acc[2 * i + 1]);
                }
            }
            uint4 o;
            o.x = pack_bf16x2(acc[0], acc[1]);
            o.y = pack_bf16x2(acc[2], acc[3]);
            o.z = pack_bf16x2(acc[4], acc[5]);
            o.w = pack_bf16x2(acc[6], acc[7]);
            y[t * chunks_per_row + c] = o;
        }
        return;
    }
    for (int c = threadIdx.x; c < chunks_per_row; c += 256) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
        for (int j = 0; j < k; ++j) {
            const int pos = assign_pos[t * k + j];
            if (pos < 0) continue;
            const float g = gates[t * k + j];
            const uint4 v = load_nt(y_perm + static_cast<int64_t>(pos) * chunks_per_row + c);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = fmaf(g, lo_bf16(w[i]), acc[2 * i]);
                acc[2 * i + 1] = fmaf(g, hi_bf16(w[i]), acc[2 * i + 1]);
            }
        }
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        y[t * chunks_per_row + c] = o;
    }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(const float* __restrict__ y_perm,
                                                         const int32_t* __restrict__ assign_pos,
                                                         const float* __restrict__ gates, int k,
                                                         int d, float* __restrict__ y) {
    const int64_t t = blockIdx.x;
    for (int c = threadIdx.x; c < d; c += 256) {
        float acc = 0.f;
        for (int j = 0; j < k; ++j) {
            const int pos = assign_pos[t * k + j];
            if (pos < 0) continue;
            acc = fmaf(gates[t * k + j], y_perm[static_cast<int64_t>(pos) * d + c], acc);
        }
        y[t * d + c] = acc;
    }
}

}  // namespace

hipError_t launch_combine(const moe_problem_t& p, const void* y_perm, const int32_t* assign_pos,
                          const float* gates, void* y, hipStream_t s) {
    const unsigned grid = static_cast<unsigned>(p.T);
    const uint4* yp = static_cast<const uint4*>(y_perm);
    uint4* yo = static_cast<uint4*>(y);
    if (p.dtype == MOE_DTYPE_BF16 && p.k <= 2)
        combine_bf16_kernel<2><<<grid, 256, 0, s>>>(yp, assign_pos, gates, p.k, p.d / 8, yo);
    else if (p.dtype == MOE_DTYPE_BF16 && p.k <= 4)
        combine_bf16_kernel<4><<<grid, 256, 0, s>>>(yp, assign_pos, gates, p.k, p.d / 8, yo);
    else if (p.dtype == MOE_DTYPE_BF16 && p.k <= 8)
        combine_bf16_kernel<8><<<grid, 256, 0, s>>>(yp, assign_pos, gates, p.k, p.d / 8, yo);
    else if (p.dtype == MOE_DTYPE_BF16)
        combine_bf16_kernel<0><<<grid, 256, 0, s>>>(yp, assign_pos, gates, p.k, p.d / 8, yo);
    else
        combine_f32_kernel<<<grid, 256, 0, s>>>(static_cast<const float*>(y_perm), assign_pos, gates,
                                                p.k, p.d, static_cast<float*>(y));
    return hipGetLastError();
}

}  // namespace moe
