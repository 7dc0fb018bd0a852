// row_encode.h -- quantise one token-head row (the write path's per-row
// encoders), shared by the write kernels and by the decode kernels that also
// store and attend a step's new token (gfx950).
//
// Write path of [P5] "NVFP4 KV Cache：Blackwell 上的 4-bit 缓存量化",
// §KV 的写入与读取路径 (compute scales, round and clip, pack, write payload and
// scale metadata into the page) and of [P4] "KV 量化", §写和读.
//
// Every function with binary32 arithmetic opens with
// `#pragma clang fp contract(off)`: its operations round exactly as written
// (no fused multiply-add is formed) whatever the including file's setting, so
// the bytes it produces are the same in every kernel that uses it.
#pragma once

#include "decode_common.h"

namespace kvq {
namespace {

// Maps a lane to its row; returns false when the row is out of range or its
// slot is skipped (the whole lane group agrees).
struct RowCtx {
  int side;
  int64_t r;  // row within its side: token * H + head
  int h, t;
  uint8_t* chunk;
};

__device__ __forceinline__ bool row_ctx(const WriteArgs& a, int64_t row, RowCtx& c) {
  const int64_t per_side = a.n_tok * a.H;
  if (row >= 2 * per_side) return false;
  c.side = row >= per_side;
  c.r = c.side ? row - per_side : row;
  const int64_t tok = c.r / a.H;
  c.h = (int)(c.r - tok * a.H);
  const int64_t slot = a.slots[tok];
  if (slot < 0 || slot >= (int64_t)a.num_pages * a.P) return false;
  const int64_t page = slot / a.P;
  c.t = (int)(slot - page * a.P);
  c.chunk = a.cache + (page * a.H + c.h) * a.geom.chunk_bytes;
  return true;
}

// Eight binary16 input values of row `row` (both sides stacked, as for
// row_ctx) starting at channel d0, requested without waiting for the row's
// slot (the address does not depend on it); zero past the last row.
__device__ __forceinline__ uint4 load_row_piece(const WriteArgs& a, int64_t row, int D, int d0) {
  const int64_t per_side = a.n_tok * a.H;
  if (row >= 2 * per_side) return uint4{0u, 0u, 0u, 0u};
  const bool side = row >= per_side;
  const int64_t r = side ? row - per_side : row;
  return *reinterpret_cast<const uint4*>((side ? a.v : a.k) + r * D + d0);
}

template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = W / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, W));
  return v;
}

__device__ __forceinline__ void halves8_to_f32(uint4 raw, float* x) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    half2_t h = as_h2(w[i]);
    x[2 * i] = (float)h[0];
    x[2 * i + 1] = (float)h[1];
  }
}

// The codes one lane of the per-row path produced, for a caller that also
// attends the row it wrote: 8-bit formats, the codes of channels 8j .. 8j+7
// (byte i = channel 8j+i); 4-bit formats, values 16j .. 16j+15 packed two per
// byte (low nibble first).  s is the row scale (per-token-head formats) or the
// layout scale (FP8 per-tensor), sb the block-scale byte (NVFP4, MXFP4).
struct RowCodes {
  uint32_t w[2];
  float s;
  uint32_t sb;
};

// ---------------------------------------------------------------------------
// 8-bit formats: FMT 1 = FP8 per-tensor, 2 = INT8 per-token-head,
// 3 = FP8 per-token-head.
// ---------------------------------------------------------------------------
// Row scale of the 8-bit formats ([P3] §可运行 fake-quant 实验: floor the max
// at 1e-8, then divide by the top code: 127 for INT8, FP8_MAX = 448 for E4M3,
// [P1] §2.2).
template <int FMT>
__device__ __forceinline__ float row_scale(float amax) {
#pragma clang fp contract(off)
  return fmaxf(amax, 1e-8f) / (FMT == 2 ? 127.0f : 448.0f);
}

// Four codes of x[0..3] packed into a dword (code i in byte i).  INT8:
// clip(rne(x / s)).  E4M3: x / s, its sign forced to x's (a zero quotient of
// -0 keeps its sign), clamped to +-448 (saturation), then gfx950's packed
// binary32 -> E4M3 conversion, which rounds to nearest even like the
// encoder's definition for every |y| <= 448 (checked code by code in
// tests/test_gpu_probes.py).
template <int FMT>
__device__ __forceinline__ uint32_t encode8x4(const float* x, float s, Recip rc) {
#pragma clang fp contract(off)
  if constexpr (FMT == 2) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float q = fminf(fmaxf(__builtin_rintf(div_rn(x[i], s, rc)), -127.0f), 127.0f);
      w |= ((uint32_t)(int32_t)q & 0xFFu) << (8 * i);
    }
    return w;
  } else {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      y[i] = __builtin_amdgcn_fmed3f(__builtin_copysignf(div_rn(x[i], s, rc), x[i]), -448.0f, 448.0f);
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], r, true);
    return (uint32_t)r;
  }
}

// One token-head row by D/8 lanes (lane j: channels 8j .. 8j+7), any slot.
// With `out`, the lane's codes are also returned; `store` = false quantises
// without writing the cache.
template <int FMT, int D>
__device__ __forceinline__ void write_row_8bit(const WriteArgs& a, int64_t row, int j, bool store = true,
                                               RowCodes* out = nullptr) {
#pragma clang fp contract(off)
  constexpr int LPR = D / 8;
  const uint4 raw = load_row_piece(a, row, D, 8 * j);  // requested before the slot is read
  RowCtx c;
  if (!row_ctx(a, row, c)) return;

  float x[8];
  halves8_to_f32(raw, x);

  float s;
  if constexpr (FMT == 1) {
    s = c.side ? a.v_scale : a.k_scale;
  } else {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    s = row_scale<FMT>(group_max<LPR>(amax));
  }
  const Recip rc = make_recip(s);
  uint2 packed;
  packed.x = encode8x4<FMT>(x, s, rc);
  packed.y = encode8x4<FMT>(x + 4, s, rc);
  if (out) {
    out->w[0] = packed.x;
    out->w[1] = packed.y;
    out->s = s;
  }
  if (!store) return;

  // 16-token groups of K and V are laid out in the decode's operand order
  // (see k8_offset / v8_offset)
  if (c.side == 0) {
    *reinterpret_cast<uint2*>(c.chunk + k8_offset<D>(c.t, 8 * j)) = packed;
  } else {
    uint8_t* vp = c.chunk + a.geom.v_codes;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      vp[v8_offset<D>(c.t, 8 * j + i)] = (uint8_t)((i < 4 ? packed.x : packed.y) >> (8 * (i & 3)));
  }
  if (FMT != 1 && j == 0) {
    float* sp = reinterpret_cast<float*>(c.chunk + a.geom.k_scales) + c.side * a.P + c.t;
    *sp = s;
  }
}


// ---------------------------------------------------------------------------
// NVFP4 ([P5] §双层缩放怎样恢复动态范围): one lane per 16-value block.
// ---------------------------------------------------------------------------

// Sixteen E2M1 codes of y[0..15] (already divided by the block divisor)
// with gfx950's scaled packed conversion at scale 1, which rounds to the
// nearest value with ties to the even code and saturates at 6 like the
// encoder's definition (checked nibble by nibble in tests/test_gpu_probes.py):
// byte i of the result holds values 2i (low nibble) and 2i+1.
__device__ __forceinline__ void e2m1_encode16(const float* y, uint32_t (&w)[2]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float* p = y + 8 * h;
    uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, p[0], p[1], 1.0f, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, p[2], p[3], 1.0f, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, p[4], p[5], 1.0f, 2);
    w[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, p[6], p[7], 1.0f, 3);
  }
}

// Codes of one block for block-scale code sb and, when ERR (the 4over6
// choice needs it), the squared reconstruction error summed by the balanced
// tree over the block's index order.  The quotients keep x's sign on zero;
// the reconstructions come back exactly through the hardware E2M1 -> binary16
// conversion.
template <bool ERR>
__device__ __forceinline__ float nvfp4_block(const float* x, float st, uint32_t sb, uint32_t (&w)[2]) {
#pragma clang fp contract(off)
  const float sbv = e4m3_val(sb);
  float e2[16];
  if (sbv == 0.0f) {
    w[0] = w[1] = 0u;
    if constexpr (!ERR) return 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) e2[i] = x[i] * x[i];
  } else {
    const float d = st * sbv;
    const Recip rc = make_recip(d);
    float y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = __builtin_copysignf(div_rn(x[i], d, rc), x[i]);
    e2m1_encode16(y, w);
    if constexpr (!ERR) return 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float v[8];
      e2m1x8_to_f32(w[h], v);  // values 8h .. 8h+7 in order
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float err = x[8 * h + k] - d * v[k];
        e2[8 * h + k] = err * err;
      }
    }
  }
#pragma unroll
  for (int wd = 1; wd < 16; wd <<= 1)
#pragma unroll
    for (int i = 0; i < 16; i += 2 * wd) e2[i] = e2[i] + e2[i + wd];
  return e2[0];
}

// Codes and block-scale code of one 16-value block (lane j of a row): the
// block max lands near 6, the top of the E2M1 grid; with 4over6 ([P5]
// §用一组数直观看缩放的作用) the max/4 candidate is kept if strictly better.
// byte[i] packs values 2i (low nibble) and 2i+1.
__device__ __forceinline__ uint32_t nvfp4_encode_block(const float* x, float st, int flags, uint32_t* byte) {
#pragma clang fp contract(off)
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  uint32_t sb = e4m3_mag((amax / 6.0f) / st);
  uint32_t w[2];
  if (flags & 1) {
    const float err6 = nvfp4_block<true>(x, st, sb, w);
    const uint32_t sb4 = e4m3_mag((amax / 4.0f) / st);
    uint32_t w4[2];
    const float err4 = nvfp4_block<true>(x, st, sb4, w4);
    if (err4 < err6) {
      sb = sb4;
      w[0] = w4[0];
      w[1] = w4[1];
    }
  } else {
    nvfp4_block<false>(x, st, sb, w);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) byte[i] = (w[i >> 2] >> (8 * (i & 3))) & 0xFFu;
  return sb;
}

// INT4 per-token-head codes of one lane's 16 values: the INT8 rule at 4 bits,
// s = max(max|x|, 1e-8) / 7 over the whole row (NB lanes), q = clip(rne(x /
// s), -7, 7) as a two's-complement nibble.  byte[i] packs values 2i (low
// nibble) and 2i+1.  Returns s.
template <int NB>
__device__ __forceinline__ float int4_encode_block(const float* x, uint32_t* byte) {
#pragma clang fp contract(off)
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const float s = fmaxf(group_max<NB>(amax), 1e-8f) / 7.0f;
  const Recip rc = make_recip(s);
  // The clamp to [-7, 7] comes first (integer bounds, so it commutes with
  // the rounding); adding 1.5 * 2^23 then rounds to an integer with ties to
  // even and leaves it, in two's complement, in the low mantissa bits of the
  // sum, whose low 4 bits are the nibble.
  uint32_t nib[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float yc = __builtin_amdgcn_fmed3f(div_rn(x[i], s, rc), -7.0f, 7.0f);
    nib[i] = __float_as_uint(yc + 12582912.0f) & 15u;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) byte[i] = nib[2 * i] | (nib[2 * i + 1] << 4);
  return s;
}

// MXFP4 codes of one lane's 16 values; lanes j and j ^ 1 hold the two halves
// of a 32-value block and share its scale.  The block's E8M0 exponent is
// floor(log2 max|x|) - 2 (OCP Microscaling conversion; [P5]
// §双层缩放怎样恢复动态范围 gives the block size and the E8M0 scale), read off
// the binary32 exponent field of the max: byte = field - 2 and x / 2^k is the
// exact product x * 2^-k, with 2^-k's field 256 - field.  Values in the top
// binade [6, 8) * 2^k saturate to 6.  An all-zero block stores byte 0.
// byte[i] packs values 2i (low nibble) and 2i+1.  Returns the scale byte.
__device__ __forceinline__ uint32_t mxfp4_encode_half(const float* x, uint32_t* byte) {
#pragma clang fp contract(off)
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = group_max<2>(amax);
  const uint32_t field = __float_as_uint(amax) >> 23;
  const float inv = amax > 0.0f ? __uint_as_float((256u - field) << 23) : 1.0f;
  float y[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = x[i] * inv;  // exact, sign kept on zero
  uint32_t w[2];
  e2m1_encode16(y, w);
#pragma unroll
  for (int i = 0; i < 8; ++i) byte[i] = (w[i >> 2] >> (8 * (i & 3))) & 0xFFu;
  return amax > 0.0f ? field - 2u : 0u;
}

// One token-head row of a 4-bit format (FMT 4 = NVFP4, 6 = INT4
// per-token-head, 7 = MXFP4) by D/16 lanes (lane j: values 16j .. 16j+15),
// any slot.  All share the code layout; NVFP4 stores an E4M3 scale per 16
// values, MXFP4 an E8M0 scale per 32 values (lane pairs), INT4 one fp32 scale
// per row.
template <int FMT, int D>
__device__ __forceinline__ void write_row_4bit(const WriteArgs& a, int64_t row, int j, bool store = true,
                                               RowCodes* out = nullptr) {
#pragma clang fp contract(off)
  constexpr int NB = D / 16;
  constexpr int NS = FMT == 7 ? D / 32 : D / 16;  // block-scale bytes per row
  constexpr int SL = FMT == 7 ? 2 : 1;            // lanes per block scale
  const uint4 raw0 = load_row_piece(a, row, D, 16 * j), raw1 = load_row_piece(a, row, D, 16 * j + 8);
  RowCtx c;
  if (!row_ctx(a, row, c)) return;
  float x[16];
  halves8_to_f32(raw0, x);
  halves8_to_f32(raw1, x + 8);
  uint32_t byte[8];
  uint32_t sb = 0;
  float s = 0.0f;
  if constexpr (FMT == 4)
    sb = nvfp4_encode_block(x, c.side ? a.v_scale : a.k_scale, a.flags, byte);
  else if constexpr (FMT == 7)
    sb = mxfp4_encode_half(x, byte);
  else
    s = int4_encode_block<NB>(x, byte);
  const bool scale_lane = (FMT == 4 || FMT == 7) && j % SL == 0;
  uint2 packed;
  packed.x = byte[0] | (byte[1] << 8) | (byte[2] << 16) | (byte[3] << 24);
  packed.y = byte[4] | (byte[5] << 8) | (byte[6] << 16) | (byte[7] << 24);
  if (out) {
    out->w[0] = packed.x;
    out->w[1] = packed.y;
    out->s = s;
    out->sb = sb;
  }
  if (!store) return;
  if (c.side == 0) {
    *reinterpret_cast<uint2*>(c.chunk + (int64_t)c.t * (D / 2) + 8 * j) = packed;
    if (scale_lane) c.chunk[a.geom.k_scales + (int64_t)c.t * NS + j / SL] = (uint8_t)sb;
  } else {
    // V: byte (quad, channel pair, token) so that each byte belongs to one token
    uint8_t* vp = c.chunk + a.geom.v_codes + 2 * D * (c.t / 4) + 32 * j + (c.t % 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) vp[4 * i] = (uint8_t)byte[i];
    if (scale_lane) c.chunk[a.geom.v_scales + (int64_t)(j / SL) * a.P + c.t] = (uint8_t)sb;
  }
  if constexpr (FMT == 6)
    if (j == 0) reinterpret_cast<float*>(c.chunk + a.geom.k_scales)[c.side * a.P + c.t] = s;
}


template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = W / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, W);
  return v;
}

// The lane's code values with the block scales applied (exact in binary32)
// and the row scale not: INT8 and INT4 integers, E4M3 values, E2M1 values
// times the E4M3 (NVFP4) or E8M0 (MXFP4) block scale.
template <int FMT, int VPL>
__device__ __forceinline__ void lane_values(const RowCodes& rc, float (&c)[VPL]) {
#pragma clang fp contract(off)
  if constexpr (FMT == 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = (float)(int32_t)(int8_t)(uint8_t)(rc.w[i / 4] >> (8 * (i % 4)));
  } else if constexpr (FMT == 1 || FMT == 3) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t lo, hi;
      e4m3x4_to_h_hw(rc.w[h], lo, hi);
      const half2_t a = as_h2(lo), b = as_h2(hi);
      c[4 * h] = (float)a[0];
      c[4 * h + 1] = (float)a[1];
      c[4 * h + 2] = (float)b[0];
      c[4 * h + 3] = (float)b[1];
    }
  } else if constexpr (FMT == 6) {
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = (float)((int32_t)(rc.w[i / 8] << (28 - 4 * (i % 8))) >> 28);
  } else {
    const float bs = FMT == 4 ? e4m3_val(rc.sb) : __uint_as_float((rc.sb & 0xFFu) << 23);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t v[4];
      e2m1x8_to_h(rc.w[h], v);  // values 8h .. 8h+7 in order
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const half2_t pr = as_h2(v[k]);
        c[8 * h + 2 * k] = (float)pr[0] * bs;
        c[8 * h + 2 * k + 1] = (float)pr[1] * bs;
      }
    }
  }
}


}  // namespace
}  // namespace kvq
