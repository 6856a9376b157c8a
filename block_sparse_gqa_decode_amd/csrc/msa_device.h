// Device-side helpers for gfx950: vector types, the bf16 MFMA tile, fp8
// e4m3fn -> bf16 conversion and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// D = A(16x32) * B(32x16) + C with bf16 operands and fp32 accumulate.
// Operand layout (wave64): lane l holds row/column (l % 16) and eight
// contraction slots selected by (l / 16); the accumulator holds rows
// 4*(l/16) .. 4*(l/16)+3 of column (l % 16).
__device__ __forceinline__ f32x4_t mfma_bf16_16x16x32(bf16x8_t a, bf16x8_t b,
                                                       f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// Two OCP fp8 e4m3fn codes (bytes 2*hi, 2*hi+1 of w) -> two bf16 packed in a
// dword, low half from the lower byte.  Exact: every e4m3fn value is a bf16.
template <bool kHi>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi);
  return __builtin_bit_cast(uint32_t, r);
}

// Eight fp8 codes (two dwords, little-endian byte order) -> eight bf16.
__device__ __forceinline__ u32x4_t fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4_t r;
  r.x = fp8x2_to_bf16x2<false>(lo);
  r.y = fp8x2_to_bf16x2<true>(lo);
  r.z = fp8x2_to_bf16x2<false>(hi);
  r.w = fp8x2_to_bf16x2<true>(hi);
  return r;
}

// fp32 -> bf16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// Byte permute: bytes of {src0 (bytes 4..7), src1 (bytes 0..3)} by selector.
__device__ __forceinline__ uint32_t byte_perm(uint32_t src0, uint32_t src1,
                                              uint32_t sel) {
  return __builtin_amdgcn_perm(src0, src1, sel);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// Reductions across the four 16-lane rows of a wavefront (lanes l, l^16,
// l^32, l^48).  (The gfx950 row-swap permutes would avoid the LDS crossbar,
// but this compiler folds max(swap.a, swap.b) to swap.a when both inputs are
// one value, so the plain lane shuffles stay.)
__device__ __forceinline__ float wave_max_xor_16_32(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float wave_sum_xor_16_32(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

}  // namespace msa
