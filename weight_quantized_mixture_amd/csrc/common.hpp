// Internal helpers shared by the gfx950 kernels of the MoE library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---- 16-bit float conversions ------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Two fp32 -> packed bf16x2 by taking the high halves.  Exact when both values
// have at most 8 significant bits (small integers, e.g. int8 codes).
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Two fp32 -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Split four fp32 values into bf16 hi + lo parts (hi = rne(v), lo = rne(v - hi)),
// 16 significant bits in total; v - hi is exact in fp32.
__device__ __forceinline__ void split_bf16x4(float4 v, u32x2& hi, u32x2& lo) {
  hi.x = pack_bf16_rne(v.x, v.y);
  hi.y = pack_bf16_rne(v.z, v.w);
  const float h0 = __uint_as_float(hi.x << 16), h1 = __uint_as_float(hi.x & 0xffff0000u);
  const float h2 = __uint_as_float(hi.y << 16), h3 = __uint_as_float(hi.y & 0xffff0000u);
  lo.x = pack_bf16_rne(v.x - h0, v.y - h1);
  lo.y = pack_bf16_rne(v.z - h2, v.w - h3);
}

// ---- int8 -> 16-bit float, exact ----------------------------------------------

// Four signed int8 codes in one dword -> four bf16 values (two dwords), exact:
// each byte is sign-extended and converted to fp32 in one instruction
// (v_cvt_f32_i32 with an SDWA byte select), and pairs are packed with
// v_cvt_pk_bf16_f32 (integers |q| <= 128 are exact in bf16).
__device__ __forceinline__ u32x2 i8x4_to_bf16x4(uint32_t w) {
  const float f0 = static_cast<float>(static_cast<int8_t>(w & 0xffu));
  const float f1 = static_cast<float>(static_cast<int8_t>((w >> 8) & 0xffu));
  const float f2 = static_cast<float>(static_cast<int8_t>((w >> 16) & 0xffu));
  const float f3 = static_cast<float>(static_cast<int32_t>(w) >> 24);
  u32x2 r;
  r.x = pack_bf16_rne(f0, f1);
  r.y = pack_bf16_rne(f2, f3);
  return r;
}

// Four signed int8 codes -> four fp16 values.  0x6400 | b is the half
// 1024 + b for a byte b, so (q + 128) becomes 1152 + q and one packed
// subtraction of 1152 leaves q exactly.
__device__ __forceinline__ u32x2 i8x4_to_f16x4(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t magic = 0x64646464u;
  const uint32_t p0 = __builtin_amdgcn_perm(magic, u, 0x04010400u);
  const uint32_t p1 = __builtin_amdgcn_perm(magic, u, 0x04030402u);
  const f16x2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
  const f16x2 h0 = __builtin_bit_cast(f16x2, p0) - off;
  const f16x2 h1 = __builtin_bit_cast(f16x2, p1) - off;
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, h0);
  r.y = __builtin_bit_cast(uint32_t, h1);
  return r;
}

// ---- wave reductions (deterministic butterfly order) ----------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  return v;
}

// ---- MFMA wrappers -------------------------------------------------------------
// 16x16x32: lane l holds A[l%16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l%16];
// the 16x16 fp32 result sits in lane l at rows 4*(l/16) .. +3, column l%16.

__device__ __forceinline__ f32x4 mfma16_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <bool kF16>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (kF16) return mfma16_f16(a, b, c);
  else return mfma16_bf16(a, b, c);
}

// 16 int8 codes (one dwordx4) -> two 8-wide 16-bit MFMA operands.
template <bool kF16>
__device__ __forceinline__ void i8x16_to_operands(u32x4 w, u32x4& lo, u32x4& hi) {
  u32x2 p0, p1, p2, p3;
  if constexpr (kF16) {
    p0 = i8x4_to_f16x4(w.x); p1 = i8x4_to_f16x4(w.y); p2 = i8x4_to_f16x4(w.z); p3 = i8x4_to_f16x4(w.w);
  } else {
    p0 = i8x4_to_bf16x4(w.x); p1 = i8x4_to_bf16x4(w.y); p2 = i8x4_to_bf16x4(w.z); p3 = i8x4_to_bf16x4(w.w);
  }
  lo = u32x4{p0.x, p0.y, p1.x, p1.y};
  hi = u32x4{p2.x, p2.y, p3.x, p3.y};
}

// 16 OCP e4m3fn codes (one dwordx4) -> two 8-wide 16-bit MFMA operands in
// natural K order, exact (e4m3 values have 4 significant bits and exponents
// in [-9, 8], inside both bf16 and fp16).  gfx950's conversion instructions
// take a code pair from the low (false) or high (true) half of a dword.
template <bool kF16, bool kHi>
__device__ __forceinline__ uint32_t fp8x2_to_16x2(uint32_t w) {
  if constexpr (kF16) return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHi));
  else return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
}

template <bool kF16>
__device__ __forceinline__ void fp8x16_to_operands(u32x4 w, u32x4& lo, u32x4& hi) {
  lo = u32x4{fp8x2_to_16x2<kF16, false>(w.x), fp8x2_to_16x2<kF16, true>(w.x), fp8x2_to_16x2<kF16, false>(w.y),
             fp8x2_to_16x2<kF16, true>(w.y)};
  hi = u32x4{fp8x2_to_16x2<kF16, false>(w.z), fp8x2_to_16x2<kF16, true>(w.z), fp8x2_to_16x2<kF16, false>(w.w),
             fp8x2_to_16x2<kF16, true>(w.w)};
}

// 16 weight codes (int8 or e4m3fn) -> two 8-wide MFMA operands.
template <bool kF16, bool kFP8>
__device__ __forceinline__ void w8_operands(u32x4 w, u32x4& lo, u32x4& hi) {
  if constexpr (kFP8) fp8x16_to_operands<kF16>(w, lo, hi);
  else i8x16_to_operands<kF16>(w, lo, hi);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

__device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe
