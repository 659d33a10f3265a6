// Device helpers shared by the gfx950 kernels: vector types, bf16 packing,
// the matrix-core wrappers and small wave-level utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

namespace hla {

constexpr float kLog2e = 1.4426950408889634f;

// bf16 (stored as the high half of an fp32) -> fp32, exact.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return (uint16_t)(pack_bf16(x, 0.f) & 0xffffu);
}

// ReLU on two packed bf16: a bf16 is negative exactly when its int16 view is
// negative, so max(int16, 0) zeroes negatives (and -0) and keeps the rest.
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t w) {
  s16x2 v = __builtin_bit_cast(s16x2, w);
  v = __builtin_elementwise_max(v, (s16x2){0, 0});
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ u32x4 relu_bf16x8(u32x4 w) {
  return (u32x4){relu_bf16x2(w[0]), relu_bf16x2(w[1]), relu_bf16x2(w[2]), relu_bf16x2(w[3])};
}

// D = A(32x16) * B(16x32) + C on the matrix cores; operands as 8 packed bf16.
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// D = A(16x32) * B(32x16) + C.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Logistic gate 1 / (1 + e^-x): exactly 0 at -inf, exactly 1 at +inf, 0.5 at 0.
__device__ __forceinline__ float sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + exp2_fast(-x * kLog2e));
}

// Value of lane (lane ^ 32): the other half of a wave64.
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void stg16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace hla
