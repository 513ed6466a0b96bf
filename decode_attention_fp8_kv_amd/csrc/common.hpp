// Device-side building blocks shared by the gfx950 kernels: vector types,
// exact e4m3 -> bf16/f16/f32 conversion, the saturating fp32 -> e4m3
// encoder, byte/half transposes for MFMA operands and wave reductions.
//
// e4m3 is the OCP OFP8 E4M3 format (bias 7, no infinities, NaN = S.1111.111,
// largest finite 448), the cache format named by the source pages
// ("Cloudflare tối ưu hóa Kimi và GLM trên Workers AI", section "Lượng tử hóa
// KV cache").  gfx950's conversion instructions implement exactly that
// format; every e4m3 value is exactly representable in bf16, f16 and f32, so
// the conversions below lose nothing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8kv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

constexpr float kE4M3Max = 448.0f;

// ---------------------------------------------------------------- decode --
// Two e4m3 codes (bytes 0,1 or 2,3 of `w`) -> two bf16 / f16 values.
template <bool HIGH>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH));
}
template <bool HIGH>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HIGH));
}

// Eight e4m3 codes (two dwords, byte order = element order) -> bf16x8.
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4_t r = {e4m3x2_to_bf16x2<false>(lo), e4m3x2_to_bf16x2<true>(lo),
               e4m3x2_to_bf16x2<false>(hi), e4m3x2_to_bf16x2<true>(hi)};
  return __builtin_bit_cast(bf16x8_t, r);
}
__device__ __forceinline__ f16x8_t e4m3x8_to_f16x8(uint32_t lo, uint32_t hi) {
  u32x4_t r = {e4m3x2_to_f16x2<false>(lo), e4m3x2_to_f16x2<true>(lo),
               e4m3x2_to_f16x2<false>(hi), e4m3x2_to_f16x2<true>(hi)};
  return __builtin_bit_cast(f16x8_t, r);
}
// Four e4m3 codes -> four f32 values.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* o) {
  f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  o[0] = a[0]; o[1] = a[1]; o[2] = b[0]; o[3] = b[1];
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// ---------------------------------------------------------------- encode --
// fp32 -> e4m3: nearest value, ties to the even code, saturating at +-448
// (+-inf too), any NaN -> 0x7F.  The hardware conversion rounds to
// nearest-even but does not saturate, so magnitudes are clamped to 448
// first; NaN is mapped explicitly (fmin/fmax would turn it into a number).
__device__ __forceinline__ uint32_t e4m3_encode_pair(float a, float b) {
  const float ca = __builtin_fminf(__builtin_fmaxf(a, -kE4M3Max), kE4M3Max);
  const float cb = __builtin_fminf(__builtin_fmaxf(b, -kE4M3Max), kE4M3Max);
  uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
  if (__builtin_isnan(a)) r = (r & 0xFF00u) | 0x007Fu;
  if (__builtin_isnan(b)) r = (r & 0x00FFu) | 0x7F00u;
  return r;
}

// -------------------------------------------------------------- permutes --
// v_perm_b32: result byte i = byte sel[i] of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// 4x4 byte transpose: in r[t] = bytes (d0,d1,d2,d3) of token t;
// out o[d] = bytes (t0,t1,t2,t3) of element d.  Eight v_perm_b32.
__device__ __forceinline__ void transpose4x4_bytes(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                                   uint32_t& o0, uint32_t& o1, uint32_t& o2, uint32_t& o3) {
  const uint32_t t0 = perm(r1, r0, 0x05010400u);  // r0.b0 r1.b0 r0.b1 r1.b1
  const uint32_t t1 = perm(r1, r0, 0x07030602u);  // r0.b2 r1.b2 r0.b3 r1.b3
  const uint32_t t2 = perm(r3, r2, 0x05010400u);  // r2.b0 r3.b0 r2.b1 r3.b1
  const uint32_t t3 = perm(r3, r2, 0x07030602u);  // r2.b2 r3.b2 r2.b3 r3.b3
  o0 = perm(t2, t0, 0x05040100u);
  o1 = perm(t2, t0, 0x07060302u);
  o2 = perm(t3, t1, 0x05040100u);
  o3 = perm(t3, t1, 0x07060302u);
}

// Pair the 16-bit halves of two tokens' dwords: low halves or high halves.
__device__ __forceinline__ uint32_t pair_lo16(uint32_t t0, uint32_t t1) { return perm(t1, t0, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi16(uint32_t t0, uint32_t t1) { return perm(t1, t0, 0x07060302u); }

// ------------------------------------------------------- wave reductions --
__device__ __forceinline__ float xor_max(float v, int mask) { return __builtin_fmaxf(v, __shfl_xor(v, mask)); }
__device__ __forceinline__ float xor_sum(float v, int mask) { return v + __shfl_xor(v, mask); }

// Sum over the 8 lanes of an aligned octet (lanes differing in bits 0..2),
// with DPP moves: swap neighbours, swap pairs, then mirror the half-row.
__device__ __forceinline__ float octet_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave max / sum of a float through DPP (register-to-register lane moves,
// no LDS round trips): row_shr:1,2,4,8 give running results inside each row
// of 16 lanes, row_bcast:15 and row_bcast:31 carry them into the rows
// above; lane 63 then holds the wave's result, which every lane reads.
// Lanes the pattern gives no source combine with the identity.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max(float v) {
  const int t = __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, -__builtin_huge_valf()), __builtin_bit_cast(int, v), CTRL, ROW_MASK,
                                            0xF, false);
  return __builtin_fmaxf(v, __builtin_bit_cast(float, t));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_sum(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF,
                                                                   false));
}
__device__ __forceinline__ float wave_max(float v) {
  v = dpp_max<0x111, 0xF>(v);
  v = dpp_max<0x112, 0xF>(v);
  v = dpp_max<0x114, 0xF>(v);
  v = dpp_max<0x118, 0xF>(v);
  v = dpp_max<0x142, 0xA>(v);
  v = dpp_max<0x143, 0xC>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_sum<0x111, 0xF>(v);
  v = dpp_sum<0x112, 0xF>(v);
  v = dpp_sum<0x114, 0xF>(v);
  v = dpp_sum<0x118, 0xF>(v);
  v = dpp_sum<0x142, 0xA>(v);
  v = dpp_sum<0x143, 0xC>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}


// bf16 round-to-nearest-even of an fp32 value, as bits.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

}  // namespace fp8kv
