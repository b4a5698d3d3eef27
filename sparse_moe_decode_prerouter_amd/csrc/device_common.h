// Device helpers shared by the gfx950 kernels of the MoE block library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float f16_to_f32(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (unsigned short)h); }

// fp32 -> bf16, round to nearest even (no NaN inputs here)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// fp64 -> bf16 with a single rounding (to nearest even): round the fp64
// significand to 8 bits in place, then the value converts to fp32 exactly.
__device__ __forceinline__ uint32_t f64_to_bf16(double x) {
    uint64_t b = (uint64_t)__double_as_longlong(x);
    const uint64_t lsb = (b >> 45) & 1ull;
    b += 0x00000FFFFFFFFFFFull + lsb;
    b &= ~0x00001FFFFFFFFFFFull;
    const float f = (float)__longlong_as_double((long long)b);
    return __float_as_uint(f) >> 16;
}

// (128 + q) for two int4 codes placed at bits [0,4) and [16,20): a pair of
// bf16 values with exponent 2^7, so the code lands in the units place.
__device__ __forceinline__ uint32_t nib_pair_bf16(uint32_t w, int p) {
    return ((w >> (4 * p)) & 0x000F000Fu) | 0x43004300u;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// device-scope (coherent across XCDs) scalar stores / loads; used for data
// published to other workgroups inside one kernel
__device__ __forceinline__ void st_dev(float* p, float v) {
    __hip_atomic_store((__attribute__((address_space(1))) float*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(double* p, double v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_dev(int* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ float ld_dev(const float* p) {
    return __hip_atomic_load((__attribute__((address_space(1))) const float*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double ld_dev(const double* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ int ld_dev(const int* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ unsigned ld_dev(const unsigned* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

__device__ __forceinline__ void set_err(int* err, int bit) {
    if (err) __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// sum over groups of `width` consecutive lanes (width a power of two <= 64)
template <typename T>
__device__ __forceinline__ T group_sum(T v, int width) {
    for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float silu_f32(float a) { return a / (1.0f + __expf(-a)); }

// top-k comparison: (value desc, index asc)
__device__ __forceinline__ bool better(double va, int ia, double vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

}  // namespace moe
