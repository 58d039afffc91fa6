// Device helpers shared by the kernels of libttt_la.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// learning-rate encodings of the mode bits
enum EtaKind : int { ETA_SCALAR = 0, ETA_PER_TOKEN = 1, ETA_SOFTPLUS = 2 };

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    __bf16 h = (__bf16)x;
    return __builtin_bit_cast(uint16_t, h);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// packs two fp32 into one dword of two bf16 (lo = a, hi = b), round to nearest
// even: one v_cvt_pk_bf16_f32 on gfx950
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2 r = __builtin_convertvector(f32x2{a, b}, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// softplus(a) = ln(1 + e^a), stable form max(a, 0) + log1p(x), x = e^-|a| in
// (0, 1].  log1p(x) is taken as ln(u) x / (u - 1) with u = 1 + x rounded (the
// correction of the rounding of 1 + x from Goldberg, "What every computer
// scientist should know about floating-point arithmetic", 1991; x itself when u
// rounds to 1), on the hardware exp2 and log2: a few ulp, without a library call.
__device__ __forceinline__ float softplus_f32(float a) {
    const float x = __builtin_amdgcn_exp2f(-fabsf(a) * 1.4426950408889634f);
    const float u = 1.0f + x;
    const float l = u == 1.0f ? x : __builtin_amdgcn_logf(u) * 0.6931471805599453f * (x / (u - 1.0f));
    return fmaxf(a, 0.0f) + l;
}

__device__ __forceinline__ float silu_f32(float u) {
    return u / (1.0f + __expf(-u));
}

template <typename TI> __device__ __forceinline__ float load_as_f32(const TI* p, size_t i);
template <> __device__ __forceinline__ float load_as_f32<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p, size_t i) {
    return bf16_bits_to_f32(p[i]);
}

template <typename TO> __device__ __forceinline__ void store_from_f32(TO* p, size_t i, float x);
template <> __device__ __forceinline__ void store_from_f32<float>(float* p, size_t i, float x) { p[i] = x; }
template <> __device__ __forceinline__ void store_from_f32<uint16_t>(uint16_t* p, size_t i, float x) {
    p[i] = f32_to_bf16_bits(x);
}

__device__ __forceinline__ float eta_at(int kind, const float* eta, float eta_scalar, size_t idx) {
    if (kind == ETA_SCALAR) return eta_scalar;
    float a = eta[idx];
    return kind == ETA_SOFTPLUS ? softplus_f32(a) : a;
}

}  // namespace ttt
