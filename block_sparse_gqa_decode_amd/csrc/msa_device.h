// Device-side helpers for gfx950: vector types, the bf16, fp8 and fp4 x fp8
// MFMA tiles, fp8 (e4m3fn / e5m2) and MXFP4 -> bf16 conversion and wavefront
// reductions.
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
typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

// D = A(16x32) * B(32x16) + C with bf16 operands and fp32 accumulate.
// Operand layout (wave64): lane l holds row/column (l % 16) and eight
// contraction slots selected by (l / 16); the accumulator holds rows
// 4*(l/16) .. 4*(l/16)+3 of column (l % 16).
__device__ __forceinline__ f32x4_t mfma_bf16_16x16x32(bf16x8_t a, bf16x8_t b,
                                                       f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D = A(16x128) * B(128x16) + C with 8-bit float operands (32 per lane) and
// fp32 accumulate; kAFmt / kBFmt: 0 = e4m3fn, 1 = e5m2.  The block scales are
// 2^0 (E8M0 code 127), so the products are the plain fp8 values.  A and B
// share one lane / byte -> contraction index map, so any fixed assignment of
// head dims to (lane group, byte) that both operands follow gives the full
// dot product.
template <int kAFmt, int kBFmt>
__device__ __forceinline__ f32x4_t mfma_f8_16x16x128(i32x8_t a, i32x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, kAFmt, kBFmt, 0, 127, 0,
                                                          127);
}

// D = A(16x128) * B(128x16) + C with an MXFP4 A (32 e2m1 codes per lane in
// the low four dwords) and an fp8 e4m3fn B.  The fp4 A lane (n, g) holds row n,
// contraction indexes 32g..32g+31 in order, and its E8M0 scale code a_scale
// multiplies exactly those 32; the fp8 B lane (n, g) holds column n,
// contraction indexes 16g..16g+15 (bytes 0..15) and 64+16g..64+16g+15 (bytes
// 16..31), at unit scale (both layouts measured on gfx950).
__device__ __forceinline__ f32x4_t mfma_f4f8_16x16x128(u32x4_t a, int a_scale, i32x8_t b,
                                                        f32x4_t c) {
  const i32x8_t a8 = i32x8_t{(int32_t)a.x, (int32_t)a.y, (int32_t)a.z, (int32_t)a.w,
                             0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, c, 4, 0, 0, a_scale, 0, 127);
}

__device__ __forceinline__ i32x8_t cat_i32x8(u32x4_t lo, u32x4_t hi) {
  return i32x8_t{(int32_t)lo.x, (int32_t)lo.y, (int32_t)lo.z, (int32_t)lo.w,
                 (int32_t)hi.x, (int32_t)hi.y, (int32_t)hi.z, (int32_t)hi.w};
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

// The same for OCP fp8 e5m2 codes (exact too: e5m2 values, +-inf and NaN
// included, are bf16 values).
template <bool kHi>
__device__ __forceinline__ uint32_t bf8x2_to_bf16x2(uint32_t w) {
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, kHi);
  return __builtin_bit_cast(uint32_t, r);
}

// Eight 8-bit codes (two dwords, little-endian byte order) -> eight bf16;
// kFmt: 1 = e4m3fn, 2 = e5m2 (the KV format values).
template <int kFmt>
__device__ __forceinline__ u32x4_t f8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4_t r;
  if constexpr (kFmt == 2) {
    r.x = bf8x2_to_bf16x2<false>(lo);
    r.y = bf8x2_to_bf16x2<true>(lo);
    r.z = bf8x2_to_bf16x2<false>(hi);
    r.w = bf8x2_to_bf16x2<true>(hi);
  } else {
    r.x = fp8x2_to_bf16x2<false>(lo);
    r.y = fp8x2_to_bf16x2<true>(lo);
    r.z = fp8x2_to_bf16x2<false>(hi);
    r.w = fp8x2_to_bf16x2<true>(hi);
  }
  return r;
}

// OCP E8M0 block-scale code -> fp32 2^(code-127): code 0 is the subnormal
// 2^-127, code 255 NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t code) {
  const uint32_t bits = code == 0u ? 0x00400000u : (code == 255u ? 0x7fc00000u : code << 23);
  return __builtin_bit_cast(float, bits);
}

// The block scale of byte `shift / 8` of a row's scale dword, as the fp32
// bit pattern code << 23: exactly 2^(code-127) for codes 1..254.  Code 0
// (2^-127) reads as 0 and code 255 (NaN) as +inf, a difference of at most
// 6 * 2^-127 per element, or a non-finite result either way; two operations
// where the exact e8m0_to_f32 takes six, on the per-page path.
__device__ __forceinline__ float e8m0_scale_of(uint32_t word, uint32_t shift) {
  return __builtin_bit_cast(float, ((word >> shift) & 0xffu) << 23);
}

// Eight OCP e2m1 codes (one dword; element 2i is the low nibble of byte i)
// times a block scale -> eight bf16, in element order.  Exact: an e2m1 value
// times a power of two is a bf16 value.
__device__ __forceinline__ u32x4_t f4x8_to_bf16x8(uint32_t w, float scale) {
  u32x4_t r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
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

// The Q^T (B) operand of an S^T = K Q^T tile for one q row per lane: four
// bf16 chunks (format 0), or the 32 fp8 e4m3fn bytes of the row's two 16-dim
// runs (format 1).
template <int kQ>
struct QRegs;

template <>
struct QRegs<0> {
  bf16x8_t f[4];
};

template <>
struct QRegs<1> {
  i32x8_t b;
};

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
