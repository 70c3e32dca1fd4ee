// Per-row FP8 quantisation for the fp8 expert FFN.
//
// Quantised experts are named as future work in the MoEBlaze summary
// (euno.news, "MoEBlaze: breaking the memory wall for efficient MoE training
// on modern GPUs"), Limitations and future work; the scheme is this
// library's reading: each row r of a bf16 matrix gets the power-of-two scale
// 2^a_r, the smallest with max|row| <= 448 * 2^a_r (a_r = 0 for a zero row),
// and each element becomes the OCP FP8 E4M3 code of value / 2^a_r, rounded
// to nearest even by the hardware conversion.  Scaling by a power of two is
// exact, so the conversion is the only rounding.
#include "device_util.h"
#include "moe_internal.h"

namespace moe {

namespace {

// One workgroup per row: the row's absolute maximum, its scale exponent,
// and the codes.  Rows of at most 256 * RC 16-byte chunks stay in registers
// between the two steps (one read of the row); longer rows (RC = 0) are read
// twice, the second time from the caches.
template <int RC>
__global__ __launch_bounds__(256) void quant_rows_fp8_kernel(const uint4* __restrict__ src, int chunks,
                                                            uint2* __restrict__ dst, int32_t* __restrict__ exps) {
    __shared__ float s_max[4];
    const int64_t r = blockIdx.x;
    const uint4* row = src + r * chunks;
    uint4 keep[RC > 0 ? RC : 1];
    float m = 0.f;
    if (RC > 0) {
#pragma unroll
        for (int i = 0; i < RC; ++i) {
            const int c = threadIdx.x + 256 * i;
            keep[RC > 0 ? i : 0] = c < chunks ? row[c] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < RC; ++i) {
            const uint32_t w[4] = {keep[i].x, keep[i].y, keep[i].z, keep[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(lo_bf16(w[j])), fabsf(hi_bf16(w[j]))));
        }
    } else {
        for (int c = threadIdx.x; c < chunks; c += 256) {
            const uint4 v = row[c];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(lo_bf16(w[j])), fabsf(hi_bf16(w[j]))));
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    // amax = mm 2^e with mm in [0.5, 1); 448 = 0.875 * 2^9
    int a = 0;
    if (amax > 0.f) {
        int e = 0;
        const float mm = frexpf(amax, &e);
        a = mm <= 0.875f ? e - 9 : e - 8;
    }
    if (threadIdx.x == 0) exps[r] = a;
    uint2* out = dst + r * chunks;
    auto convert = [&](const uint4 v) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __builtin_amdgcn_ldexpf(lo_bf16(w[i]), -a);
            f[2 * i + 1] = __builtin_amdgcn_ldexpf(hi_bf16(w[i]), -a);
        }
        // element 0 in the lowest byte
        int p0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        p0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], p0, true);
        int p1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
        p1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], p1, true);
        return make_uint2(static_cast<uint32_t>(p0), static_cast<uint32_t>(p1));
    };
    if (RC > 0) {
#pragma unroll
        for (int i = 0; i < RC; ++i) {
            const int c = threadIdx.x + 256 * i;
            if (c < chunks) out[c] = convert(keep[RC > 0 ? i : 0]);
        }
    } else {
        for (int c = threadIdx.x; c < chunks; c += 256) out[c] = convert(row[c]);
    }
}

// Short rows (at most 64 * RW 16-byte chunks): one 64-lane wave per row, 4
// rows per workgroup, the row kept in registers and its maximum taken with
// wave shuffles alone.  (One 256-thread workgroup per row left most of its
// threads idle on rows of 768 columns: 2.6 TB/s.)  The maximum is exact in
// any order, so the scale and the codes equal the one-workgroup kernel's.
template <int RW>
__global__ __launch_bounds__(256) void quant_rows_fp8_wave_kernel(const uint4* __restrict__ src, int64_t rows,
                                                                 int chunks, uint2* __restrict__ dst,
                                                                 int32_t* __restrict__ exps) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;  // whole waves leave together
    const int lane = threadIdx.x & 63;
    const uint4* row = src + r * chunks;
    uint4 keep[RW];
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const int c = lane + 64 * i;
        keep[i] = c < chunks ? row[c] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const uint32_t w[4] = {keep[i].x, keep[i].y, keep[i].z, keep[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(lo_bf16(w[j])), fabsf(hi_bf16(w[j]))));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    // amax = mm 2^e with mm in [0.5, 1); 448 = 0.875 * 2^9
    int a = 0;
    if (m > 0.f) {
        int e = 0;
        const float mm = frexpf(m, &e);
        a = mm <= 0.875f ? e - 9 : e - 8;
    }
    if (lane == 0) exps[r] = a;
    uint2* out = dst + r * chunks;
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const int c = lane + 64 * i;
        if (c >= chunks) continue;
        const uint32_t w[4] = {keep[i].x, keep[i].y, keep[i].z, keep[i].w};
        float f[8];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            f[2 * h] = __builtin_amdgcn_ldexpf(lo_bf16(w[h]), -a);
            f[2 * h + 1] = __builtin_amdgcn_ldexpf(hi_bf16(w[h]), -a);
        }
        // element 0 in the lowest byte
        int p0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        p0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], p0, true);
        int p1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
        p1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], p1, true);
        out[c] = make_uint2(static_cast<uint32_t>(p0), static_cast<uint32_t>(p1));
    }
}

}  // namespace

hipError_t launch_quant_rows_fp8(const void* src, int64_t rows, int cols, void* codes, int32_t* exps,
                                 hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const int chunks = cols / 8;
    const unsigned g = static_cast<unsigned>(rows);
    const unsigned gw = static_cast<unsigned>(ceil_div(rows, 4));
    if (chunks <= 64)
        quant_rows_fp8_wave_kernel<1><<<gw, 256, 0, s>>>(static_cast<const uint4*>(src), rows, chunks,
                                                         static_cast<uint2*>(codes), exps);
    else if (chunks <= 128)
        quant_rows_fp8_wave_kernel<2><<<gw, 256, 0, s>>>(static_cast<const uint4*>(src), rows, chunks,
                                                         static_cast<uint2*>(codes), exps);
    else if (chunks <= 256)
        quant_rows_fp8_wave_kernel<4><<<gw, 256, 0, s>>>(static_cast<const uint4*>(src), rows, chunks,
                                                         static_cast<uint2*>(codes), exps);
    else if (chunks <= 256 * 2)
        quant_rows_fp8_kernel<2><<<g, 256, 0, s>>>(static_cast<const uint4*>(src), chunks, static_cast<uint2*>(codes),
                                                   exps);
    else if (chunks <= 256 * 8)
        quant_rows_fp8_kernel<8><<<g, 256, 0, s>>>(static_cast<const uint4*>(src), chunks, static_cast<uint2*>(codes),
                                                   exps);
    else
        quant_rows_fp8_kernel<0><<<g, 256, 0, s>>>(static_cast<const uint4*>(src), chunks, static_cast<uint2*>(codes),
                                                   exps);
    return hipGetLastError();
}

}  // namespace moe
