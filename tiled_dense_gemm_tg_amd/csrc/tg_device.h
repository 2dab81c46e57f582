// tg_device.h -- device helpers shared by the GEMM kernels (gfx950 only).
//
// 16-bit element traits with their MFMA instructions, 16-byte vector views,
// and the register-resident epilogue (bias + GELU(tanh) + round to the output
// format) that the fourth TileLang page ("Designing high-performance GPU
// kernels with TileLang", part 3 "Epilogue fusion") describes as running
// while the product still sits in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum Epi { EPI_NONE = 0, EPI_BIAS = 1, EPI_BIAS_GELU_TANH = 2 };

// fp16: IEEE binary16 inputs, v_mfma_f32_{32x32x16,16x16x32}_f16.
struct F16 {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    static __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b),
                                                      c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b),
                                                      c, 0, 0, 0);
    }
    static __device__ __forceinline__ float to_f32(uint16_t bits) {
        return (float)__builtin_bit_cast(_Float16, bits);
    }
    // round to nearest even (v_cvt_f16_f32)
    static __device__ __forceinline__ uint16_t from_f32(float x) {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    }
};

// bf16: upper half of IEEE binary32, v_mfma_f32_{32x32x16,16x16x32}_bf16.
struct BF16 {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    static __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b),
                                                       c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b),
                                                       c, 0, 0, 0);
    }
    static __device__ __forceinline__ float to_f32(uint16_t bits) {
        return __builtin_bit_cast(float, (uint32_t)bits << 16);
    }
    // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
    static __device__ __forceinline__ uint16_t from_f32(float x) {
        return __builtin_bit_cast(uint16_t, (__bf16)x);
    }
};

// GELU, tanh form, via the identity 0.5*y*(1 + tanh(z)) = y * sigmoid(2z)
// = y / (1 + exp(-2z)), z = sqrt(2/pi) * (y + 0.044715 * y^3).  exp(-2z) is
// taken as exp2(t) on the hardware exp2, with t = -2*log2(e)*z evaluated as
// y * (k0 + k1 * y^2) (one multiply, one fma, one multiply); for z -> -inf
// the reciprocal of +inf gives 0 and the result -0, for z -> +inf it gives y.
static __device__ __forceinline__ float gelu_tanh(float y) {
    const float k0 = -2.0f * 1.4426950408889634f * 0.7978845608028654f;  // -2*log2(e)*sqrt(2/pi)
    const float k1 = k0 * 0.044715f;
    const float t = y * __builtin_fmaf(y * y, k1, k0);
    const float e = __builtin_amdgcn_exp2f(t);
    return y * __builtin_amdgcn_rcpf(1.0f + e);
}

template <int EPI>
static __device__ __forceinline__ float epilogue(float acc, float bias) {
    if constexpr (EPI == EPI_NONE) {
        return acc;
    } else if constexpr (EPI == EPI_BIAS) {
        return acc + bias;
    } else {
        return gelu_tanh(acc + bias);
    }
}

// Pack two 16-bit patterns into one dword, first in the low half.
static __device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
    return (uint32_t)lo | ((uint32_t)hi << 16);
}

// Select two 16-bit halves from a pair of dwords (v_perm_b32): with lo and
// hi each holding two elements, sel 0x05040100 keeps the low halves
// (lo.h0, hi.h0) and sel 0x07060302 the high halves (lo.h1, hi.h1).
static __device__ __forceinline__ uint32_t perm_lo(uint32_t lo, uint32_t hi) {
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}
static __device__ __forceinline__ uint32_t perm_hi(uint32_t lo, uint32_t hi) {
    return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

}  // namespace tg
