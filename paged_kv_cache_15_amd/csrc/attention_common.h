// Device-side helpers shared by the decode attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "common.h"

namespace pkv_dev {

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;

constexpr int kBS = pkv::kKernelBlockSize;  // tokens per block
constexpr int kWaves = 4;                   // waves per partition workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -INFINITY;
constexpr float kRescaleSlack = 8.f;        // log2 units: weights stay below 2^8

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-bit storage bits -> float
template <int DT>
__device__ __forceinline__ float bits_to_f32(uint32_t b) {
    if constexpr (DT == DT_BF16) return __uint_as_float(b << 16);
    else if constexpr (DT == DT_F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
    else return __uint_as_float(b);
}

// float -> 16-bit storage bits, round to nearest even
template <int DT>
__device__ __forceinline__ uint16_t f32_to_bits16(float f) {
    if constexpr (DT == DT_BF16) return __builtin_bit_cast(uint16_t, (__bf16)f);
    else return __builtin_bit_cast(uint16_t, (_Float16)f);
}

template <int OUT_DT>
__device__ __forceinline__ void store_out(void* out, int64_t i, float v) {
    if constexpr (OUT_DT == DT_F32) static_cast<float*>(out)[i] = v;
    else static_cast<uint16_t*>(out)[i] = f32_to_bits16<OUT_DT>(v);
}

// max over the lanes that share lane % 16 (xor 16, 32)
__device__ __forceinline__ float max_across_quads(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}
__device__ __forceinline__ float sum_across_quads(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

}  // namespace pkv_dev
