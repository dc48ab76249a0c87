// Device-side helpers shared by the libmla kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(8 * sizeof(unsigned short)))) unsigned short u16x8;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned int)))) unsigned int u32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned short)))) unsigned short u16x4;

#define MLA_LDS __attribute__((address_space(3)))

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Cache layout: blocks of bs token rows, token-major for every dtype, so
// element (slot = block * bs + t, channel c) sits at slot * D + c.
__host__ __device__ __forceinline__ size_t cache_offset(size_t slot, int c, int D) {
    return slot * (size_t)D + c;
}

// ---- scalar conversions ---------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(unsigned short b) {
    return __uint_as_float(static_cast<unsigned int>(b) << 16);
}

// float -> bfloat16 bits, round to nearest even (NaN kept quiet).
// IEEE binary16 bit patterns (the conversion rounds to nearest even)
__device__ __forceinline__ unsigned short f32_to_f16_bits(float f) {
    return __builtin_bit_cast(unsigned short, (_Float16)f);
}
__device__ __forceinline__ float f16_bits_to_f32(unsigned short b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ unsigned short f32_to_bf16_bits(float f) {
    __bf16 h = static_cast<__bf16>(f);   // v_cvt_pk_bf16_f32 on gfx950: RNE
    return __builtin_bit_cast(unsigned short, h);
}

// Two floats -> packed bf16 pair (round to nearest even), low half first.
__device__ __forceinline__ unsigned int pack_bf16x2(float lo, float hi) {
    const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(unsigned int, v);
}

// max(a, b, c) in one instruction.  (fmaxf on matrix-core results first
// quiets each input in IEEE mode, one extra instruction per value; the
// callers pass scores that are never NaN: masked ones are -inf.)
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// OCP e4m3 code -> float (bias 7, subnormals, 0x7F / 0xFF NaN).
__device__ __forceinline__ float e4m3_to_f32(unsigned int code) {
    const unsigned int mag = code & 0x7Fu;
    const float sign = (code & 0x80u) ? -1.0f : 1.0f;
    if (mag == 0x7Fu) return __builtin_nanf("");
    const unsigned int e = mag >> 3, m = mag & 7u;
    float v = (e == 0) ? static_cast<float>(m) * 0.001953125f            // m * 2^-9
                       : __uint_as_float(((e + 120u) << 23) | (m << 20)); // (1+m/8) 2^(e-7)
    return sign * v;
}

// float -> OCP e4m3 code, round to nearest even, finite values beyond 448
// saturate to +-448, NaN -> 0x7F.
__device__ __forceinline__ unsigned int f32_to_e4m3_rne_sat(float x) {
    if (x != x) return 0x7Fu;
    const unsigned int sign = (__float_as_uint(x) >> 24) & 0x80u;
    float a = fminf(fabsf(x), 448.0f);
    unsigned int code;
    if (a < 0.015625f) {                        // below 2^-6: subnormal grid 2^-9
        code = static_cast<unsigned int>(rintf(a * 512.0f));   // 8 -> min normal 0x08
    } else {
        int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xFF) - 127;  // -6 .. 8
        float frac = a * __uint_as_float(static_cast<unsigned int>(127 - e) << 23) - 1.0f;
        unsigned int mm = static_cast<unsigned int>(rintf(frac * 8.0f));
        if (mm == 8u) { mm = 0u; ++e; }
        code = (static_cast<unsigned int>(e + 7) << 3) | mm;
    }
    return code | sign;
}

// ---- generic element loads ------------------------------------------------

template <int DT>
__device__ __forceinline__ float load_act(const void* p, size_t i) {
    if constexpr (DT == MLA_BF16) {
        return bf16_bits_to_f32(static_cast<const unsigned short*>(p)[i]);
    } else {
        return static_cast<const float*>(p)[i];
    }
}

template <int DT>
__device__ __forceinline__ void store_act(void* p, size_t i, float v) {
    if constexpr (DT == MLA_BF16) {
        static_cast<unsigned short*>(p)[i] = f32_to_bf16_bits(v);
    } else {
        static_cast<float*>(p)[i] = v;
    }
}

// ---- block reductions (blockDim.x multiple of 64, <= 1024) -----------------

__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// scratch: >= 16 floats of shared memory.
__device__ __forceinline__ float block_sum(float v, float* scratch) {
    v = wave_sum(v);
    const int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < nw; ++i) t += scratch[i];
    return t;
}
__device__ __forceinline__ float block_max(float v, float* scratch) {
    v = wave_max(v);
    const int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
    __syncthreads();
    float t = kNegInf;
    for (int i = 0; i < nw; ++i) t = fmaxf(t, scratch[i]);
    return t;
}

}  // namespace mla
