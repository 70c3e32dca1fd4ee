// Router GEMM and static top-k gating.
//
// The router picks a few experts per token (Piper, Japanese explainer,
// opening section); the policy is static top-k (MoEBlaze summary,
// Limitations).  Selection is exact on fp32 logits with ties broken toward
// the lower expert id; gates are the softmax renormalised over the k chosen
// logits.
#include <float.h>
#include <limits.h>

#include "device_util.h"
#include "moe_internal.h"

namespace moe {

namespace {

// ---- router GEMM: logits[T, E] = x[T, d] * W_r[E, d]^T, fp32 accumulate ----
//
// 64 tokens x 64 experts per workgroup, 32-wide reduction chunks staged in
// LDS, 4 x 4 outputs per thread.
constexpr int RT_M = 64;
constexpr int RT_N = 64;
constexpr int RT_K = 32;

template <typename TIn>
__device__ __forceinline__ float load_in(const TIn* p, int64_t i);
template <>
__device__ __forceinline__ float load_in<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_in<bf16_t>(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

template <typename TIn>
__global__ __launch_bounds__(256) void router_logits_kernel(const TIn* __restrict__ x,
                                                           const TIn* __restrict__ w,
                                                           float* __restrict__ logits,
                                                           int64_t T, int d, int E) {
    __shared__ float xs[RT_K][RT_M + 4];
    __shared__ float ws[RT_K][RT_N + 4];
    const int tid = threadIdx.x;
    const int tx = tid & 15;   // expert group
    const int ty = tid >> 4;   // token group
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * RT_M;
    const int e0 = blockIdx.y * RT_N;

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    for (int k0 = 0; k0 < d; k0 += RT_K) {
#pragma unroll
        for (int i = 0; i < (RT_M * RT_K) / 256; ++i) {
            const int idx = tid + 256 * i;
            const int r = idx / RT_K, c = idx % RT_K;
            const int64_t t = t0 + r;
            const int kk = k0 + c;
            xs[c][r] = (t < T && kk < d) ? load_in(x, t * d + kk) : 0.f;
            const int e = e0 + r;
            ws[c][r] = (e < E && kk < d) ? load_in(w, static_cast<int64_t>(e) * d + kk) : 0.f;
        }
        __syncthreads();
#pragma unroll 8
        for (int c = 0; c < RT_K; ++c) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = xs[c][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = ws[c][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + ty * 4 + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + tx * 4 + j;
            if (e < E) logits[t * E + e] = acc[i][j];
        }
    }
}

// ---- bf16 router GEMM on MFMA ------------------------------------------------
//
// A workgroup takes 32 tokens and all experts; its 4 waves split the hidden
// dimension in four.  Each wave computes logits^T blocks of 32 experts x 32
// tokens with v_mfma_f32_32x32x16_bf16, loading its fragments straight from
// global memory (x rows stream from HBM once; the small router weight stays
// in L2).  The partial sums of the four waves are added in LDS in a fixed
// order, so the result does not depend on scheduling.  The kernel is bound by
// the HBM read of x.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int EB>
__global__ __launch_bounds__(256) void router_logits_mfma_kernel(const bf16_t* __restrict__ x,
                                                                const bf16_t* __restrict__ w,
                                                                float* __restrict__ logits,
                                                                int64_t T, int d, int E) {
    __shared__ float part[3][EB][16][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 32;
    int64_t tok = t0 + (lane & 31);
    if (tok >= T) tok = T - 1;  // clamped rows compute discarded outputs
    const int kq = 8 * (lane >> 5);
    const bf16_t* xr = x + tok * d + kq;
    const bf16_t* wr[EB];
#pragma unroll
    for (int b = 0; b < EB; ++b) {
        int e = b * 32 + (lane & 31);
        if (e >= E) e = E - 1;
        wr[b] = w + static_cast<int64_t>(e) * d + kq;
    }
    f32x16_t acc[EB];
#pragma unroll
    for (int b = 0; b < EB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;

    const int kspan = d / 4;  // multiple of 16
    const int k1 = (wave + 1) * kspan;
    int k = wave * kspan;
    // 8 K steps per round so that 8 x-row loads are in flight per wave
    for (; k + 128 <= k1; k += 128) {
        bf16x8_t xf[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) xf[s] = *reinterpret_cast<const bf16x8_t*>(xr + k + 16 * s);
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int b = 0; b < EB; ++b) {
                const bf16x8_t wf = *reinterpret_cast<const bf16x8_t*>(wr[b] + k + 16 * s);
                acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, xf[s], acc[b], 0, 0, 0);
            }
    }
    for (; k < k1; k += 16) {
        const bf16x8_t xf = *reinterpret_cast<const bf16x8_t*>(xr + k);
#pragma unroll
        for (int b = 0; b < EB; ++b) {
            const bf16x8_t wf = *reinterpret_cast<const bf16x8_t*>(wr[b] + k);
            acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, xf, acc[b], 0, 0, 0);
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int b = 0; b < EB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) part[wave - 1][b][r][lane] = acc[b][r];
    }
    __syncthreads();
    if (wave != 0) return;
    const int64_t t = t0 + (lane & 31);
    if (t >= T) return;
#pragma unroll
    for (int b = 0; b < EB; ++b) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // fixed order: wave 0 + wave 1 + wave 2 + wave 3
            const float v = ((acc[b][r] + part[0][b][r][lane]) + part[1][b][r][lane]) + part[2][b][r][lane];
            // lane holds token (lane & 31); register r holds expert
            // b*32 + 8*(r/4) + 4*(lane/32) + r%4
            const int e = b * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (e < E) logits[t * E + e] = v;
        }
    }
}

// ---- top-k selection and gates: one 64-lane wave per token -----------------
//
// Lane l holds the logits of experts l, l + 64, ... (EPL of them).  Each of
// the k rounds takes every lane's best unchosen (value, id) and reduces it
// across the wave with the order "larger value first, then lower id".  Lane j
// keeps the winner of round j.
__device__ __forceinline__ bool better(float v, int e, float bv, int be) {
    return v > bv || (v == bv && e < be);
}

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                        int64_t T, int E, int k,
                                                        int32_t* __restrict__ ids,
                                                        float* __restrict__ gates) {
    const int lane = lane_id();
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (t >= T) return;

    float v[EPL];
    bool live[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        live[i] = e < E;
        v[i] = live[i] ? logits[t * E + e] : -FLT_MAX;
    }

    float my_v = 0.f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -FLT_MAX;
        int be = INT_MAX;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            if (live[i] && (be == INT_MAX || better(v[i], e, bv, be))) {
                bv = v[i];
                be = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int oe = __shfl_xor(be, off, 64);
            if (oe != INT_MAX && (be == INT_MAX || better(ov, oe, bv, be))) {
                bv = ov;
                be = oe;
            }
        }
        // be is the same on every lane now; its owner retires it.
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane + 64 * i == be) live[i] = false;
        if (lane == j) {
            my_v = bv;
            my_e = be;
        }
    }

    // gates: softmax over the k chosen logits, shifted by the largest (slot 0)
    const float m = __shfl(my_v, 0, 64);
    const float pj = (lane < k) ? expf(my_v - m) : 0.f;
    float s = pj;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane < k) {
        ids[t * k + lane] = my_e;
        gates[t * k + lane] = pj / s;
    }
}

}  // namespace

hipError_t launch_router_logits(const moe_problem_t& p, const void* x, const void* w_router,
                                float* logits, hipStream_t s) {
    if (p.dtype == MOE_DTYPE_F32) {
        dim3 grid(static_cast<unsigned>(ceil_div(p.T, RT_M)), static_cast<unsigned>(ceil_div(p.E, RT_N)));
        router_logits_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x),
                                                         static_cast<const float*>(w_router), logits,
                                                         p.T, p.d, p.E);
        return hipGetLastError();
    }
    const unsigned grid = static_cast<unsigned>(ceil_div(p.T, 32));
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* wb = static_cast<const bf16_t*>(w_router);
    switch (ceil_div(p.E, 32)) {
        case 1: router_logits_mfma_kernel<1><<<grid, 256, 0, s>>>(xb, wb, logits, p.T, p.d, p.E); break;
        case 2: router_logits_mfma_kernel<2><<<grid, 256, 0, s>>>(xb, wb, logits, p.T, p.d, p.E); break;
        case 3: router_logits_mfma_kernel<3><<<grid, 256, 0, s>>>(xb, wb, logits, p.T, p.d, p.E); break;
        case 4: router_logits_mfma_kernel<4><<<grid, 256, 0, s>>>(xb, wb, logits, p.T, p.d, p.E); break;
        case 5: router_logits_mfma_kernel<5><<<grid, 256, 0, s>>>(xb, wb, logits, p.T, p.d, p.E); break;
        case 6: router_logits_mfma_kernel<6><<<grid, 256, 0, s>>>(xb, wb, logits, p.T, p.d, p.E); break;
        case 7: router_logits_mfma_kernel<7><<<grid, 256, 0, s>>>(xb, wb, logits, p.T, p.d, p.E); break;
        default: router_logits_mfma_kernel<8><<<grid, 256, 0, s>>>(xb, wb, logits, p.T, p.d, p.E); break;
    }
    return hipGetLastError();
}

hipError_t launch_route_topk(const moe_problem_t& p, const float* logits, int32_t* ids,
                             float* gates, hipStream_t s) {
    const unsigned grid = static_cast<unsigned>(ceil_div(p.T, 4));
    const int epl = static_cast<int>(ceil_div(p.E, 64));
    switch (epl) {
        case 1: route_topk_kernel<1><<<grid, 256, 0, s>>>(logits, p.T, p.E, p.k, ids, gates); break;
        case 2: route_topk_kernel<2><<<grid, 256, 0, s>>>(logits, p.T, p.E, p.k, ids, gates); break;
        case 3: route_topk_kernel<3><<<grid, 256, 0, s>>>(logits, p.T, p.E, p.k, ids, gates); break;
        default: route_topk_kernel<4><<<grid, 256, 0, s>>>(logits, p.T, p.E, p.k, ids, gates); break;
    }
    return hipGetLastError();
}

}  // namespace moe
