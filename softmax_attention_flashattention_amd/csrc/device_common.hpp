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
    // 16x16x32 MFMA: D = A * B + C (A: 16 rows x 32 k, B: 32 k x 16 cols); lane l
    // holds row / col l % 16 and k 8 (l / 16) .. +7 of A / B, and rows
    // 4 (l / 16) .. +3 of column l % 16 of C
    static __device__ __forceinline__ f32x4 mfma16(s16x8 a, s16x8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    // acc + a.lo * b.lo + a.hi * b.hi for two packed pairs (v_dot2_f32_bf16)
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                               acc, false);
    }
    // acc + lo(w) + hi(w): the two packed 16-bit values of w summed in fp32
    static __device__ __forceinline__ float sum2(uint32_t w, float acc) { return dot2(w, 0x3F803F80u, acc); }
    // two fp32 -> two bf16 (lo first), round to nearest even, one v_cvt_pk_bf16_f32
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
        return __builtin_bit_cast(uint32_t, v);
    }
    static constexpr uint32_t one_bits = 0x3F80u;
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
    static __device__ __forceinline__ f32x4 mfma16(s16x8 a, s16x8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
    }
    static __device__ __forceinline__ float sum2(uint32_t w, float acc) { return dot2(w, 0x3C003C00u, acc); }
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        const f16x2 v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
        return __builtin_bit_cast(uint32_t, v);
    }
    static constexpr uint32_t one_bits = 0x3C00u;
};

// Buffer resource for raw 16-byte loads of [base, base + num_bytes): loads
// past num_bytes return zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                             static_cast<int>(num_bytes), 0x00020000);
}
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), 0, 0));
}

// Packs two fp32 values into one dword of two 16-bit elements (lo first).
template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return T::pack2(lo, hi);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor_shfl(float v, int mask) { return __shfl_xor(v, mask, 64); }

// The value of lane l ^ 32, without going through LDS (v_permlane32_swap).
__device__ __forceinline__ float swap_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    // r[0]: lanes 32..63 now hold lanes 0..31; r[1]: lanes 0..31 now hold lanes 32..63
    return __uint_as_float(__lane_id() < 32 ? r[1] : r[0]);
}
// v + (value of lane l ^ 32), the same bits in both lanes
__device__ __forceinline__ float sum_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// v + (value of lane l ^ 16) (v_permlane16_swap exchanges rows 0<->1, 2<->3)
__device__ __forceinline__ float sum_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// DPP moves inside rows of 16 lanes (every source lane is in the row)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within each half row
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within the row
// Reductions over the 16 lanes of each row; every lane of the row gets the
// same bits (each step combines two equal partial results commutatively).
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_mov<kDppXor1>(v));
    v = fmaxf(v, dpp_mov<kDppXor2>(v));
    v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
    return fmaxf(v, dpp_mov<kDppMirror>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_mov<kDppXor1>(v);
    v += dpp_mov<kDppXor2>(v);
    v += dpp_mov<kDppHalfMirror>(v);
    return v + dpp_mov<kDppMirror>(v);
}

// max(v, value of lane l ^ 32)
__device__ __forceinline__ float max_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// 16-byte global load / store of raw bits.
__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
// 16-byte load of data read once: marked non-temporal, so it streams
// through the caches instead of displacing what other waves still reuse
__device__ __forceinline__ uint4 ld16_stream(const void *p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return uint4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ void st16(void *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }

}  // namespace attn
