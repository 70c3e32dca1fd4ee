// Device helpers shared by the kernels: bf16 conversion and wave-level
// primitives for 64-lane CDNA wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bf16 bit pattern in memory

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even, with gfx950's packed conversion
// (v_cvt_pk_bf16_f32, two values per instruction; NaN stays a NaN).
typedef __bf16 hw_bf16x2_t __attribute__((ext_vector_type(2)));

// Two bf16 packed into one 32-bit word, element 0 in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    hw_bf16x2_t v;
    v[0] = static_cast<__bf16>(lo);
    v[1] = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x & 63); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = lane_id();
    return (l == 0) ? 0ull : (~0ull >> (64 - l));
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) loads for data read exactly once.
template <typename T>
__device__ __forceinline__ T load_nt(const T* p) {
    return __builtin_nontemporal_load(p);
}
template <>
__device__ __forceinline__ uint4 load_nt<uint4>(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace moe
