// device_common.hpp -- small gfx950 device helpers shared by the attention
// kernels: 16-bit element traits, MFMA wrappers, conversions, lane exchange.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;

// Element traits: storage is raw 16-bit patterns; arithmetic is fp32.
struct Bf16 {
    using vec8 = bf16x8;
    static __device__ __forceinline__ float to_f32(uint16_t b) {
        return __uint_as_float(static_cast<uint32_t>(b) << 16);
    }
    // round to nearest even (v_cvt_pk_bf16_f32)
    static __device__ __forceinline__ uint16_t from_f32(float x) {
        __bf16 h = static_cast<__bf16>(x);
        return __builtin_bit_cast(uint16_t, h);
    }
    // 32x32x16 MFMA: D = A * B + C (A: 32 rows x 16 k, B: 16 k x 32 cols)
    static __device__ __forceinline__ f32x16 mfma32(s16x8 a, s16x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

struct Fp16 {
    using vec8 = f16x8;
    static __device__ __forceinline__ float to_f32(uint16_t b) {
        return static_cast<float>(__builtin_bit_cast(_Float16, b));
    }
    // round to nearest even (v_cvt_f16_f32)
    static __device__ __forceinline__ uint16_t from_f32(float x) {
        _Float16 h = static_cast<_Float16>(x);
        return __builtin_bit_cast(uint16_t, h);
    }
    static __device__ __forceinline__ f32x16 mfma32(s16x8 a, s16x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};

// Packs two fp32 values into one dword of two 16-bit elements (lo first).
template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return static_cast<uint32_t>(T::from_f32(lo)) | (static_cast<uint32_t>(T::from_f32(hi)) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor_shfl(float v, int mask) { return __shfl_xor(v, mask, 64); }

// 16-byte global load / store of raw bits.
__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void st16(void *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }

}  // namespace attn
