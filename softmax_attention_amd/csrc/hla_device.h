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

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
// D = A(32x64) * B(64x32) + C with OCP fp8 e4m3 operands: lane l holds row
// (A) or column (B) l % 32, k = 32 (l / 32) + byte index of the 8 dwords. The
// products are exact in fp32; the zero format/scale arguments select the
// plain (unscaled) fp8 instruction.
__device__ __forceinline__ f32x16 mfma32x32x64_fp8(u32x8 a, u32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a),
                                                         __builtin_bit_cast(i32x8, b), c, 0, 0, 0,
                                                         0, 0, 0);
}
__device__ __forceinline__ u32x8 concat(u32x4 lo, u32x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Logistic gate 1 / (1 + e^-x): exactly 0 at -inf, exactly 1 at +inf, 0.5 at 0.
__device__ __forceinline__ float sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + exp2_fast(-x * kLog2e));
}

// Combine x with the value of lane (lane ^ 32), the other half of the wave64,
// through v_permlane32_swap (no LDS round trip): the swap leaves the two
// halves' values in its two results, in an order that depends on the lane, so
// only symmetric combinations are offered.
__device__ __forceinline__ float max_halves(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float add_halves(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Raw buffer access: a 32-bit byte offset from a per-tensor base; reads past
// num_bytes return 0 and never touch memory. Resource word 3 is the gfx9-family
// raw-buffer format (32-bit data format, no swizzle).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes,
                                           0x00020000);
}
// Same, for a base and size the compiler cannot prove wave-uniform although
// they are (readfirstlane keeps the descriptor in scalar registers).
__device__ __forceinline__ rsrc_t make_rsrc_uniform(const void* base, uint32_t num_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(num_bytes);
  return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), n);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}

// 16 bytes per lane from a raw buffer straight into LDS: lane i of the wave
// writes lds_base + 16 i (lds_base is wave-uniform); past num_bytes it writes 0.
__device__ __forceinline__ void buf_load16_lds(rsrc_t r, uint32_t byte_off, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16,
                                           (int)byte_off, 0, 0, 0);
}

// Wait until every outstanding memory operation of this wave has completed.
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Row sum helper: a + lo(p) + hi(p) for a packed bf16 pair p (v_dot2 with ones).
__device__ __forceinline__ float add_bf16x2(uint32_t p, float a) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p),
                                         (bf16x2){(__bf16)1.0f, (__bf16)1.0f}, a, false);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// Non-temporal 16-byte load (streaming cache policy), for data read exactly
// once: on the linear state pass it measured 5-10 % faster than a plain load.
__device__ __forceinline__ u32x4 ldg16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void stg16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// ---- fp8 (OCP e4m3) inputs ---------------------------------------------------
// Every e4m3 value is exactly representable in bf16 (4-bit exponent, 3-bit
// mantissa), so fp8 inputs convert losslessly into the bf16 operands the
// kernels already use.

// four fp8 bytes -> four floats (bytes 0,1 then 2,3), exact
__device__ __forceinline__ f32x4 fp8x4_to_f32(uint32_t w) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  return (f32x4){lo[0], lo[1], hi[0], hi[1]};
}
__device__ __forceinline__ float fp8_to_f32(uint8_t b) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((uint32_t)b, false)[0];
}
// ReLU on four packed e4m3 values: a byte is negative exactly when its top
// bit is set. v_perm_b32 selectors 8-11 yield 0xff or 0x00 from the top bit
// of bytes 1, 3, 5 and 7 of {first operand : second operand}; with x << 8 as
// the first operand those are the sign bits of x's bytes 0 and 2, with x as
// the second, of bytes 1 and 3. The mask then clears every negative byte
// (-0 included; a NaN with the sign bit set becomes 0, as the bf16 route does).
__device__ __forceinline__ uint32_t relu_fp8x4(uint32_t x) {
  const uint32_t neg = __builtin_amdgcn_perm(x << 8, x, 0x090B080Au);
  return x & ~neg;
}

// eight fp8 values (8 bytes) -> eight bf16 (one 16-byte MFMA operand), exact:
// v_cvt_scalef32_pk_bf16_fp8 with scale 1 converts two values per instruction
// (every e4m3 value is a bf16 value; checked equal to the fp32 route on all
// 65536 byte pairs)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4 fp8x8_to_bf16(u32x2 w) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
  return (u32x4){__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                 __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
}

// Four floats -> four OCP e4m3 bytes (v_cvt_pk_fp8_f32: round to nearest even),
// a in byte 0 .. d in byte 3.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}
// four e4m3 bytes -> four bf16 as two packed pairs (bytes 0,1 then 2,3), exact
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return (u32x2){__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}

// Eight consecutive elements of a bf16 or fp8 tensor as eight bf16 values.
template <typename T>
__device__ __forceinline__ u32x4 load8_bf16(const T* p) {
  if constexpr (sizeof(T) == 1) return fp8x8_to_bf16(*reinterpret_cast<const u32x2*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}
// Same, with a non-temporal (streaming) load.
template <typename T>
__device__ __forceinline__ u32x4 load8_bf16_stream(const T* p) {
  if constexpr (sizeof(T) == 1)
    return fp8x8_to_bf16(__builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p)));
  else return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
// Eight / sixteen consecutive elements of a bf16 or fp8 tensor as floats.
template <typename T>
__device__ __forceinline__ void load8_f32(const T* p, float* o) {
  if constexpr (sizeof(T) == 1) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const f32x4 f = fp8x4_to_f32(w[q]);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[4 * q + e] = f[e];
    }
  } else {
    const u32x4 w = ldg16(p);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[2 * q] = bf_lo(w[q]);
      o[2 * q + 1] = bf_hi(w[q]);
    }
  }
}
template <typename T>
__device__ __forceinline__ void load16_f32(const T* p, float* o) {
  if constexpr (sizeof(T) == 1) {
    const u32x4 w = ldg16(p);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 f = fp8x4_to_f32(w[q]);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[4 * q + e] = f[e];
    }
  } else {
    load8_f32(p, o);
    load8_f32(p + 8, o + 8);
  }
}
// One element of a bf16 or fp8 tensor as float.
template <typename T>
__device__ __forceinline__ float elem_f32(T x) {
  if constexpr (sizeof(T) == 1) return fp8_to_f32(x);
  else return bf16_to_f32(x);
}

}  // namespace hla
