// kvq_device.h -- device helpers for the libkvq kernels (gfx950).
//
// Number formats ([P1] "KV Cache 量化深度解析", §2.1-2.3; [P5] "NVFP4 KV Cache：
// Blackwell 上的 4-bit 缓存量化", §NVFP4 中的 4 bit 表示什么 and
// §双层缩放怎样恢复动态范围):
//   E4M3: OCP FP8, exponent bias 7, largest finite 448, subnormals 2^-9 apart.
//   E2M1: grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}, sign in bit 3.
// Encoders round to nearest with ties to even and saturate at the top value;
// they take the magnitude and the sign separately so that a signed zero input
// keeps its sign.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Correctly rounded division by a value shared by many numerators.
//
// For a divisor s, make_recip stores hi = RN(1/s) (the compiler's correctly
// rounded division) and lo = (1 - s*hi) * hi, the Newton correction, so that
// hi + lo approximates 1/s to about 2^-47.  div_rn then forms a faithful
// quotient q0 = RN(x*hi + RN(x*lo)), the exact remainder r = x - s*q0 with one
// FMA, and returns RN(q0 + r*hi), which equals RN(x / s) by Markstein's
// theorem (faithful quotient + correctly rounded reciprocal).  Valid while
// x / s and the remainder stay normal, which the validated scale ranges
// guarantee.  4 VALU operations per quotient instead of the ~10 of a full
// division sequence.
// ---------------------------------------------------------------------------
struct Recip {
  float hi, lo;
};

__device__ __forceinline__ Recip make_recip(float s) {
  float hi = 1.0f / s;
  float e = __builtin_fmaf(-s, hi, 1.0f);
  return Recip{hi, e * hi};
}

__device__ __forceinline__ float div_rn(float x, float s, Recip r) {
  float q0 = __builtin_fmaf(x, r.hi, x * r.lo);
  float rem = __builtin_fmaf(-s, q0, x);
  return __builtin_fmaf(rem, r.hi, q0);
}

// ---------------------------------------------------------------------------
// Encoders (integer ALU on the binary32 bit pattern)
// ---------------------------------------------------------------------------

// |y| -> E4M3 magnitude code 0..126.
__device__ __forceinline__ uint32_t e4m3_mag(float a) {
  uint32_t b = __float_as_uint(a);
  // below 2^-6 the grid is the multiples of 2^-9 (codes 0..8 continue into
  // the normal range without a seam)
  uint32_t sub = (uint32_t)__builtin_rintf(a * 512.0f);
  // normal range: keep three mantissa bits with round-to-nearest-even, then
  // rebias the exponent from 127 to 7
  uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
  uint32_t nor = (r >> 20) - (120u << 3);
  uint32_t c = b < 0x3C800000u ? sub : nor;
  return b >= 0x43E00000u ? 0x7Eu : c;  // >= 448 saturates
}

// E4M3 magnitude code 0..126 -> value.
__device__ __forceinline__ float e4m3_val(uint32_t c) {
  uint32_t e = c >> 3, m = c & 7u;
  float nor = __uint_as_float(((e + 120u) << 23) | (m << 20));
  float sub = (float)m * 0.001953125f;
  return e ? nor : sub;
}

// |y| -> E2M1 magnitude code 0..7.
__device__ __forceinline__ uint32_t e2m1_mag(float a) {
  uint32_t b = __float_as_uint(a);
  uint32_t sub = (uint32_t)__builtin_rintf(a * 2.0f);  // below 1: 0, 0.5 (and 1.0)
  uint32_t r = b + 0x1FFFFFu + ((b >> 22) & 1u);     // one mantissa bit, RNE
  uint32_t nor = (r >> 22) - 252u;                     // rebias 127 -> 1
  uint32_t c = b < 0x3F800000u ? sub : (nor > 7u ? 7u : nor);
  return b >= 0x40C00000u ? 7u : c;  // >= 6 saturates
}

// E2M1 magnitude code 0..7 -> value.
__device__ __forceinline__ float e2m1_val(uint32_t c) {
  uint32_t e = c >> 1, m = c & 1u;
  float nor = __uint_as_float(((e + 126u) << 23) | (m << 22));
  return e ? nor : 0.5f * (float)m;
}

__device__ __forceinline__ uint32_t sign_bit(float x) { return __float_as_uint(x) >> 31; }

// ---------------------------------------------------------------------------
// 8-bit K and V layout inside a chunk.  Each group of 16 tokens (u = t/16,
// s = t%16) takes 16*D bytes, ordered so that the decode's k-th 16-byte load
// (B-byte for D = 32) of all 64 lanes is one contiguous 64*B-byte run:
//   K: lane (token s, quarter g) holds channels (D/4)*g .. +D/4, in pieces
//      of B = min(16, D/4) bytes; piece h of all lanes is contiguous.
//   V: lane (channel group n, token quad s/4) holds channels (D/16)*n + c of
//      tokens s/4*4 .. +3 as 4 bytes per channel; pieces of B bytes likewise.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int64_t k8_offset(int t, int d) {
  constexpr int B = D / 4 < 16 ? D / 4 : 16;
  const int g = d / (D / 4), r = d % (D / 4), h = r / B, e = r % B;
  return (int64_t)16 * D * (t / 16) + 64 * B * h + 16 * B * g + B * (t % 16) + e;
}

template <int D>
__device__ __forceinline__ int64_t v8_offset(int t, int d) {
  constexpr int B = D / 4 < 16 ? D / 4 : 16;
  const int n = d / (D / 16), c = d % (D / 16), h = c / (B / 4), j = c % (B / 4);
  const int s = t % 16;
  return (int64_t)16 * D * (t / 16) + 64 * B * h + 16 * B * (s / 4) + B * n + 4 * j + s % 4;
}

// ---------------------------------------------------------------------------
// Exact code -> binary16 conversions for the decode operands.  Every value of
// every format is exactly representable in binary16 (INT8 codes, E4M3 values,
// E2M1 values times an E4M3 block scale, KVarN integers 0..15), so these
// conversions introduce no error.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t perm(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
  return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// Four signed bytes -> two binary16 pairs (b0, b1), (b2, b3).  Offset to
// unsigned, place each byte under the 0x64 exponent byte (binary16 1024 + u),
// subtract 1024 + 128.
__device__ __forceinline__ void i8x4_to_h(uint32_t w, half2_t& lo, half2_t& hi) {
  uint32_t u = w ^ 0x80808080u;
  const half2_t bias = {(half_t)1152.0f, (half_t)1152.0f};
  lo = as_h2(perm(0x64646464u, u, 0x04010400u)) - bias;
  hi = as_h2(perm(0x64646464u, u, 0x04030402u)) - bias;
}

// ---------------------------------------------------------------------------
// gfx950 hardware conversions, issued directly: the compiler's lowering of the
// matching builtins repacks the two binary16 results when they are used one by
// one (the high half is replaced by a copy of the low half).  With scale 1.0
// both conversions are exact for every finite code.  Each block ends with two
// wait states: the compiler does not see these instructions' latency inside
// an asm statement and may otherwise place an MFMA that reads their results
// too close behind (observed as wrong FP8 products).  Reading their source
// right after a VALU write needs no wait state (the compiler's own code for
// the builtins does it back to back).
// ---------------------------------------------------------------------------

// Eight E2M1 codes (two per byte, low nibble first) -> four binary16 pairs in
// code order.
__device__ __forceinline__ void e2m1x8_to_h(uint32_t w, uint32_t (&h)[4]) {
  asm("v_cvt_scalef32_pk_f16_fp4 %0, %4, 1.0\n\t"
      "v_cvt_scalef32_pk_f16_fp4 %1, %4, 1.0 op_sel:[1,0,0]\n\t"
      "v_cvt_scalef32_pk_f16_fp4 %2, %4, 1.0 op_sel:[0,1,0]\n\t"
      "v_cvt_scalef32_pk_f16_fp4 %3, %4, 1.0 op_sel:[1,1,0]\n\t"
      "s_nop 1"
      : "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3])
      : "v"(w));
}

// The same with a power-of-two scale: the conversion multiplies by the
// scale's binary32 exponent, so E2M1 value * 2^k comes out exact while it is
// a binary16 number (k in [-23, 13]).
__device__ __forceinline__ void e2m1x8_to_h_scaled(uint32_t w, float scale, uint32_t (&h)[4]) {
  asm("v_cvt_scalef32_pk_f16_fp4 %0, %4, %5\n\t"
      "v_cvt_scalef32_pk_f16_fp4 %1, %4, %5 op_sel:[1,0,0]\n\t"
      "v_cvt_scalef32_pk_f16_fp4 %2, %4, %5 op_sel:[0,1,0]\n\t"
      "v_cvt_scalef32_pk_f16_fp4 %3, %4, %5 op_sel:[1,1,0]\n\t"
      "s_nop 1"
      : "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3])
      : "v"(w), "v"(scale));
}

// Byte i of w (two E2M1 codes) with its own power-of-two scale s[i].
__device__ __forceinline__ void e2m1x8_to_h_scaled4(uint32_t w, const float (&s)[4], uint32_t (&h)[4]) {
  asm("v_cvt_scalef32_pk_f16_fp4 %0, %4, %5\n\t"
      "v_cvt_scalef32_pk_f16_fp4 %1, %4, %6 op_sel:[1,0,0]\n\t"
      "v_cvt_scalef32_pk_f16_fp4 %2, %4, %7 op_sel:[0,1,0]\n\t"
      "v_cvt_scalef32_pk_f16_fp4 %3, %4, %8 op_sel:[1,1,0]\n\t"
      "s_nop 1"
      : "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3])
      : "v"(w), "v"(s[0]), "v"(s[1]), "v"(s[2]), "v"(s[3]));
}

// Eight E2M1 codes of w (low nibble of byte 0 first) -> binary32 values,
// exact (gfx950's scaled conversion at scale 1, one byte per instruction;
// checked code by code in tests/test_gpu_probes.py).
__device__ __forceinline__ void e2m1x8_to_f32(uint32_t w, float (&v)[8]) {
  const float2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const float2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const float2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const float2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  v[0] = a.x, v[1] = a.y, v[2] = b.x, v[3] = b.y, v[4] = c.x, v[5] = c.y, v[6] = d.x, v[7] = d.y;
}

// E8M0 byte e -> 2^(e - 127) as a binary32 scale operand (e = 0 gives +0,
// used only by all-zero blocks).
__device__ __forceinline__ float e8m0_scale(uint32_t e) { return __uint_as_float((e & 0xFFu) << 23); }

// Four E4M3 codes -> two binary16 pairs in code order.
__device__ __forceinline__ void e4m3x4_to_h_hw(uint32_t w, uint32_t& lo, uint32_t& hi) {
  asm("v_cvt_scalef32_pk_f16_fp8 %0, %2, 1.0\n\t"
      "v_cvt_scalef32_pk_f16_fp8 %1, %2, 1.0 op_sel:[1,0,0]\n\t"
      "s_nop 1"
      : "=&v"(lo), "=&v"(hi)
      : "v"(w));
}

// The two low E4M3 bytes of w as one binary16 pair, exact (scale 1.0).
__device__ __forceinline__ uint32_t e4m3x2_to_h_hw(uint32_t w) {
  uint32_t lo;
  asm("v_cvt_scalef32_pk_f16_fp8 %0, %1, 1.0\n\t"
      "s_nop 1"
      : "=&v"(lo)
      : "v"(w));
  return lo;
}

// The same with a power-of-two scale.
__device__ __forceinline__ void e4m3x4_to_h_scaled(uint32_t w, float scale, uint32_t& lo, uint32_t& hi) {
  asm("v_cvt_scalef32_pk_f16_fp8 %0, %2, %3\n\t"
      "v_cvt_scalef32_pk_f16_fp8 %1, %2, %3 op_sel:[1,0,0]\n\t"
      "s_nop 1"
      : "=&v"(lo), "=&v"(hi)
      : "v"(w), "v"(scale));
}

}  // namespace kvq
