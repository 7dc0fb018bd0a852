/*
 * kvq_oracle.c -- plain CPU reference ("oracle") for KV-cache quantisation
 * and dequant-fused paged decode attention.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test-suite, the smoke check
 * and the benchmark's CPU-baseline leg may load this library.  The GPU library
 * shares no code with it: every format, page-layout rule and algorithm below is
 * written out again here, slowly and literally, so that the two can be compared.
 *
 * Arithmetic rules (apply to every function in this file):
 *   - inputs are IEEE binary16, widened exactly to binary32;
 *   - quantisation runs in binary32 with round-to-nearest-even, correctly
 *     rounded '/' and sqrtf, and no FMA contraction (built with
 *     -ffp-contract=off, no fast-math);
 *   - every float sum uses the balanced pairwise tree over index order,
 *     S(x[0..n)) = S(x[0..n/2)) + S(x[n/2..n)), n a power of two;
 *   - max/min are exact;
 *   - dequantisation for attention, and attention itself, run in binary64.
 *
 * Sources (cited by page title and section only):
 *   [P1] "KV Cache 量化深度解析：Per-Tensor、Per-Token-Head 与 NVFP4"
 *   [P2] "KVarN：华为推出的原生 vLLM KV-cache 量化后端"
 *   [P3] "KV Cache 量化 · LLM Glossary"
 *   [P4] "KV 量化" (vLLM / SGLang source walk-through)
 *   [P5] "NVFP4 KV Cache：Blackwell 上的 4-bit 缓存量化"
 *
 * Pins live in tests/test_oracle_pins.py.  The KVarN pipeline is pinned by
 * invariants only (orthogonality and involution of the rotation, unit column
 * deviation after normalisation, the half-step rounding bound, capacity):
 * the pages print no KVarN code or output, so agreement with Huawei's own
 * kernels is "parity unpinned"; the constants are readings of [P2] §技术原理.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Formats                                                                   */
/* ------------------------------------------------------------------------ */

enum {
  O_FP8_PER_TENSOR = 1,  /* [P1] §2.1; [P4] §FP8 per-tensor */
  O_INT8_PTH = 2,        /* [P1] §2.2; [P3] §它改变缓存表示 formula */
  O_FP8_PTH = 3,         /* [P1] §2.2 pseudo-code */
  O_NVFP4 = 4,           /* [P1] §2.3; [P5] §双层缩放怎样恢复动态范围 */
  O_KVARN_K4V2_G128 = 5, /* [P2] §技术原理, §配置与部署 */
  O_INT4_PTH = 6,        /* [P4] §scale 和数据放在一起 (int4_per_token_head) */
  O_MXFP4 = 7            /* [P5] §双层缩放怎样恢复动态范围 (the MXFP4 comparison) */
};
enum { O_FLAG_NVFP4_4OVER6 = 1 }; /* [P5] §用一组数直观看缩放的作用 */

/* Field order matches the library's kvq_layout (an ABI contract written out
 * again here, not shared code). */
typedef struct {
  int32_t format, flags;
  int32_t num_kv_heads, head_dim;
  int32_t page_size, num_pages;
  float k_scale, v_scale;
} kvqo_layout;

enum { O_OK = 0, O_BAD_ARG = 1 };

/* Normalisation sweeps of the KVarN preset (one sweep = token pass, then
 * channel pass). */
#define KVARN_ITERS 4
/* One KVarN tile (128 tokens x 128 channels): 4-bit K codes, 2-bit V codes,
 * 6 x 128 fp32 metadata. */
#define KVARN_TILE_BYTES (128 * 64 + 128 * 32 + 4 * 6 * 128)

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* IEEE binary16 bits -> binary32 value (exact).  Pinned against numpy. */
float kvqo_half_to_float(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  float v;
  if (e == 0)
    v = ldexpf((float)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexpf((float)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

/* E4M3 ("fn": exponent bias 7, no infinities, S.1111.111 = NaN) -> value.
 * Pinned against torch.float8_e4m3fn for all 256 codes. */
double kvqo_e4m3_decode(uint8_t c) {
  int sign = c >> 7;
  int e = (c >> 3) & 15;
  int m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9); /* subnormal: (m/8) * 2^-6 */
  else
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return sign ? -v : v;
}

/* Round a >= 0 onto an ascending grid (grid[0] = 0) with round-to-nearest,
 * ties to the even code.  Callers saturate values above the top first.
 * Every grid value and midpoint is exact in binary64, so the comparisons are
 * exact. */
static int round_to_grid(double a, const double* grid, int n) {
  int lo = 0;
  for (int c = 1; c < n; c++)
    if (grid[c] <= a) lo = c;
  if (lo == n - 1) return lo;
  int hi = lo + 1;
  double mid = 0.5 * grid[lo] + 0.5 * grid[hi];
  if (a < mid) return lo;
  if (a > mid) return hi;
  return (lo % 2 == 0) ? lo : hi;
}

/* binary32 -> E4M3 code.  Readings: OCP E4M3 (largest finite 448);
 * magnitudes >= 448 saturate to 448 rather than becoming NaN; otherwise
 * nearest value with ties to even, subnormals included; the sign is kept,
 * also on zero.  Pinned against torch.float8_e4m3fn for |y| < 464. */
uint8_t kvqo_e4m3_encode(float y) {
  double grid[127];
  for (int c = 0; c < 127; c++) grid[c] = kvqo_e4m3_decode((uint8_t)c);
  if (isnan(y)) return 0x7F;
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  double a = fabs((double)y);
  if (a >= 448.0) return sign | 0x7E;
  return sign | (uint8_t)round_to_grid(a, grid, 127);
}

/* E2M1 magnitudes of codes 0..7, [P5] §NVFP4 中的 4 bit 表示什么; bit 3 is the
 * sign. */
static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double kvqo_e2m1_decode(uint8_t c) {
  double v = E2M1_GRID[c & 7];
  return (c & 8) ? -v : v;
}

/* binary32 -> E2M1 nibble: nearest grid value with ties to the even code;
 * magnitudes above 6 saturate to 6 (the page asks that out-of-range inputs be
 * handled, [P5] §双层缩放怎样恢复动态范围); sign kept on zero.
 * Pinned by brute force over the 15 signed grid values. */
uint8_t kvqo_e2m1_encode(float y) {
  if (isnan(y)) return 0x7;
  uint8_t sign = signbit(y) ? 8 : 0;
  double a = fabs((double)y);
  if (a >= 6.0) return sign | 7;
  return sign | (uint8_t)round_to_grid(a, E2M1_GRID, 8);
}

/* Balanced pairwise sum over index order, n a power of two. */
static float sum_tree(const float* x, int n) {
  if (n == 1) return x[0];
  return sum_tree(x, n / 2) + sum_tree(x + n / 2, n / 2);
}

static float clampf(float v, float lo, float hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

/* ------------------------------------------------------------------------ */
/* Row quantisers (one token-head row of D values, binary32)                 */
/* ------------------------------------------------------------------------ */

/* INT8 per-token-head, [P3] §它改变缓存表示 and §可运行 fake-quant 实验:
 * s = max(max|x|, 1e-8) / 127 (the script clamps the max before dividing),
 * q = clip(rne(x / s), -127, 127).  Codes are stored as signed bytes. */
static void quant_row_int8(const float* x, int D, uint8_t* codes, float* s_out) {
  float a = 0.0f;
  for (int d = 0; d < D; d++) a = fmaxf(a, fabsf(x[d]));
  float s = fmaxf(a, 1e-8f) / 127.0f;
  for (int d = 0; d < D; d++) {
    float y = x[d] / s;
    float r = clampf(rintf(y), -127.0f, 127.0f);
    codes[d] = (uint8_t)(int8_t)r;
  }
  *s_out = s;
}

/* INT4 per-token-head.  [P4] §scale 和数据放在一起 lists int4_per_token_head
 * beside the INT8 and FP8 modes: half-width data (two values per byte) and one
 * fp32 scale per token-head side.  The pages give no INT4 formula; reading:
 * the INT8 rule at 4 bits, s = max(max|x|, 1e-8) / 7, q = clip(rne(x / s),
 * -7, 7) (symmetric, like INT8's +-127), stored as two's-complement nibbles. */
static void quant_row_int4(const float* x, int D, uint8_t* codes, float* s_out) {
  float a = 0.0f;
  for (int d = 0; d < D; d++) a = fmaxf(a, fabsf(x[d]));
  float s = fmaxf(a, 1e-8f) / 7.0f;
  for (int d = 0; d < D; d++) {
    float y = x[d] / s;
    float r = clampf(rintf(y), -7.0f, 7.0f);
    codes[d] = (uint8_t)((int)r & 15);
  }
  *s_out = s;
}

/* FP8 per-token-head, [P1] §2.2: scale = max|x| / FP8_MAX with FP8_MAX = 448
 * (E4M3), codes = E4M3(x / scale).  The 1e-8 floor on the max is borrowed
 * from the INT8 script so an all-zero row has a finite scale. */
static void quant_row_fp8_pth(const float* x, int D, uint8_t* codes, float* s_out) {
  float a = 0.0f;
  for (int d = 0; d < D; d++) a = fmaxf(a, fabsf(x[d]));
  float s = fmaxf(a, 1e-8f) / 448.0f;
  for (int d = 0; d < D; d++) codes[d] = kvqo_e4m3_encode(x[d] / s);
  *s_out = s;
}

/* FP8 per-tensor, [P1] §2.1 and [P4] §写和读: divide by the layer's scale,
 * convert to E4M3, keep the bits as bytes.  No scale is stored in the page. */
static void quant_row_fp8_pt(const float* x, int D, float scale, uint8_t* codes) {
  for (int d = 0; d < D; d++) codes[d] = kvqo_e4m3_encode(x[d] / scale);
}

/* Codes of one 16-value block for a given E4M3 block-scale code, and the
 * block's squared reconstruction error (balanced tree sum, binary32). */
static float nvfp4_block_codes(const float* x, float st, uint8_t sb, uint8_t* codes) {
  float sbv = (float)kvqo_e4m3_decode(sb); /* exact in binary32 */
  float err[16];
  if (sbv == 0.0f) {
    for (int i = 0; i < 16; i++) {
      codes[i] = 0;
      err[i] = x[i] * x[i];
    }
  } else {
    float dsc = st * sbv; /* the divisor s_t * s_b, rounded to binary32 */
    for (int i = 0; i < 16; i++) {
      codes[i] = kvqo_e2m1_encode(x[i] / dsc);
      float rec = dsc * (float)kvqo_e2m1_decode(codes[i]);
      float e = x[i] - rec;
      err[i] = e * e;
    }
  }
  return sum_tree(err, 16);
}

/* NVFP4, [P5] §双层缩放怎样恢复动态范围: per 16 contiguous channels one E4M3
 * block scale s_b and one per-layer binary32 global scale s_t;
 * q_i = Q_E2M1(x_i / (s_t s_b)).  Reading: s_b = E4M3((max|x_b| / 6) / s_t),
 * i.e. the block maximum lands near 6, the top of the grid.
 * 4over6 ([P5] §用一组数直观看缩放的作用): also try s_b = E4M3((max/4) / s_t)
 * and keep it only if its squared reconstruction error is strictly smaller. */
static void quant_row_nvfp4(const float* x, int D, float st, int four_over_six,
                            uint8_t* codes, uint8_t* bscales) {
  for (int b = 0; b < D / 16; b++) {
    const float* xb = x + 16 * b;
    float a = 0.0f;
    for (int i = 0; i < 16; i++) a = fmaxf(a, fabsf(xb[i]));
    uint8_t s6 = kvqo_e4m3_encode((a / 6.0f) / st);
    uint8_t c6[16];
    float e6 = nvfp4_block_codes(xb, st, s6, c6);
    uint8_t chosen = s6;
    const uint8_t* cc = c6;
    uint8_t c4[16];
    if (four_over_six) {
      uint8_t s4 = kvqo_e4m3_encode((a / 4.0f) / st);
      float e4 = nvfp4_block_codes(xb, st, s4, c4);
      if (e4 < e6) {
        chosen = s4;
        cc = c4;
      }
    }
    bscales[b] = chosen;
    memcpy(codes + 16 * b, cc, 16);
  }
}

/* MXFP4.  [P5] §双层缩放怎样恢复动态范围 contrasts NVFP4 with MXFP4: blocks
 * of 32 values sharing one E8M0 scale, a pure power of two, and E2M1
 * elements.  The page gives no rule for choosing the scale; reading: the
 * format's published definition (OCP Microscaling Formats v1.0, conversion
 * of a block), i.e. X = 2^(floor(log2(max|x|)) - 2), 2 being the exponent of
 * E2M1's largest power of two (4), and q_i = E2M1(x_i / X) with values above
 * 6 saturated (the top binade of the block, [6, 8) * X, clips).  The scale
 * byte is the biased exponent floor(log2(max|x|)) - 2 + 127.  A block whose
 * values are all zero has no exponent; it takes the smallest scale, byte 0
 * (any scale reconstructs zeros).  x_i / X is exact (a power of two). */
static void quant_row_mxfp4(const float* x, int D, uint8_t* codes, uint8_t* bscales) {
  for (int b = 0; b < D / 32; b++) {
    const float* xb = x + 32 * b;
    float a = 0.0f;
    for (int i = 0; i < 32; i++) a = fmaxf(a, fabsf(xb[i]));
    if (a == 0.0f) {
      bscales[b] = 0;
      for (int i = 0; i < 32; i++) codes[32 * b + i] = kvqo_e2m1_encode(xb[i]);
      continue;
    }
    int ex;
    frexpf(a, &ex); /* a = m * 2^ex, m in [0.5, 1): floor(log2(a)) = ex - 1 */
    int k = (ex - 1) - 2;
    bscales[b] = (uint8_t)(k + 127);
    for (int i = 0; i < 32; i++) codes[32 * b + i] = kvqo_e2m1_encode(ldexpf(xb[i], -k));
  }
}

/* Exported row quantiser for pins: x is D binary16 values; codes gets one
 * unpacked code per element (INT8 as a signed byte, E4M3 byte, or E2M1
 * nibble); scales gets the fp32 per-token-head scale (as 4 bytes), the D/16
 * NVFP4 block-scale bytes or the D/32 MXFP4 E8M0 bytes.  scale is the per-tensor / global scale. */
int kvqo_quantize_row(int format, int flags, float scale, const uint16_t* x16, int D,
                      uint8_t* codes, uint8_t* scales) {
  if (D <= 0 || D % 32 != 0 || D > 4096) return O_BAD_ARG;
  float x[4096];
  for (int d = 0; d < D; d++) x[d] = kvqo_half_to_float(x16[d]);
  float s;
  switch (format) {
    case O_INT8_PTH: quant_row_int8(x, D, codes, &s); memcpy(scales, &s, 4); return O_OK;
    case O_INT4_PTH: quant_row_int4(x, D, codes, &s); memcpy(scales, &s, 4); return O_OK;
    case O_FP8_PTH: quant_row_fp8_pth(x, D, codes, &s); memcpy(scales, &s, 4); return O_OK;
    case O_FP8_PER_TENSOR: quant_row_fp8_pt(x, D, scale, codes); return O_OK;
    case O_NVFP4:
      quant_row_nvfp4(x, D, scale, flags & O_FLAG_NVFP4_4OVER6, codes, scales);
      return O_OK;
    case O_MXFP4: quant_row_mxfp4(x, D, codes, scales); return O_OK;
  }
  return O_BAD_ARG;
}

/* ------------------------------------------------------------------------ */
/* KVarN k4v2 g128 tile pipeline, [P2] §技术原理 (four stages)                */
/* ------------------------------------------------------------------------ */

/* RN(1/sqrt(128)) in binary32 (bit pattern 0x3DB504F3). */
static const float INV_SQRT128_F = 0x1.6a09e6p-4f;

/* Stage 2, rotation along channels: 128-point Walsh-Hadamard transform in
 * Sylvester order as in-place butterflies (a, b) -> (a + b, a - b) on pairs
 * (j, j + h), j & h = 0, for h = 1, 2, 4, ..., 64, then one multiplication by
 * RN(1/sqrt(128)).  The result is H x / sqrt(128) with H symmetric and
 * H H = 128 I, so the normalised transform is orthogonal and its own inverse. */
void kvqo_kvarn_rotate_f32(float* y) {
  for (int h = 1; h < 128; h <<= 1)
    for (int j = 0; j < 128; j++)
      if ((j & h) == 0) {
        float a = y[j], b = y[j + h];
        y[j] = a + b;
        y[j + h] = a - b;
      }
  for (int j = 0; j < 128; j++) y[j] = y[j] * INV_SQRT128_F;
}

/* The same transform in binary64 (used to go back to the original basis when
 * dequantising; the normalised transform is its own inverse). */
static void rotate_f64(double* y) {
  for (int h = 1; h < 128; h <<= 1)
    for (int j = 0; j < 128; j++)
      if ((j & h) == 0) {
        double a = y[j], b = y[j + h];
        y[j] = a + b;
        y[j + h] = a - b;
      }
  double c = 1.0 / sqrt(128.0);
  for (int j = 0; j < 128; j++) y[j] = y[j] * c;
}

/* Population standard deviation of 128 values (mean and mean square by the
 * balanced tree, 1/128 applied as an exact power of two); a zero or non-finite
 * result is replaced by 1 so the division that follows is harmless. */
static float dev128(const float* v) {
  float mean = sum_tree(v, 128) * 0.0078125f;
  float sq[128];
  for (int i = 0; i < 128; i++) {
    float dv = v[i] - mean;
    sq[i] = dv * dv;
  }
  float sd = sqrtf(sum_tree(sq, 128) * 0.0078125f);
  if (!(sd > 0.0f) || !isfinite(sd)) sd = 1.0f;
  return sd;
}

/* One KVarN tile of one kv head and one side.
 *   x16:   128 tokens x 128 channels of binary16, token t at x16 + t*stride.
 *   side:  0 = keys (4-bit codes, per-channel scale/zero),
 *          1 = values (2-bit codes, per-token scale/zero).
 * Outputs (any may be NULL): y_rot / y_norm [128*128] token-major, r[128]
 * (token factors), c[128] (channel factors), codes [128*128] token-major one
 * code per byte, qs / qm [128] quantiser step and zero (per channel for keys,
 * per token for values), meta [3*128] the stored metadata:
 *   keys:   alpha_j = c_j s_j, beta_j = c_j m_j, rho_t = r_t
 *   values: alpha_t = r_t s_t, beta_t = r_t m_t, gamma_j = c_j
 * so that the rotated tile is rebuilt as
 *   K_tj = rho_t (alpha_j code + beta_j),  V_tj = gamma_j (alpha_t code + beta_t)
 * which folds the scales back per channel for keys and per token for values
 * ([P2] §技术原理, stage 4).
 * Readings: the normalisation alternates a pass over tokens and a pass over
 * channels, 4 sweeps; a pass multiplies the values by RN(1 / sigma), sigma
 * the population deviation, and the running factor by sigma (the page's
 * log-domain update, subtracting log sigma, done in the linear domain with
 * one rounding of the reciprocal, as the rotation's x RN(1/sqrt(128)));
 * quantisation is asymmetric round-to-nearest with zero = group minimum and
 * step = (max - min) / (2^bits - 1), codes clipped to the range. */
void kvqo_kvarn_tile(const uint16_t* x16, int64_t stride, int side, float* y_rot,
                     float* y_norm, float* r_out, float* c_out, uint8_t* codes,
                     float* qs, float* qm, float* meta) {
  static const int N = 128;
  float* Y = (float*)malloc(sizeof(float) * N * N);
  float r[128], c[128], col[128];
  uint8_t* cd = (uint8_t*)malloc((size_t)N * N);
  float s_q[128], m_q[128];

  /* stage 1 (the raw tile) and stage 2 (rotation of every token row) */
  for (int t = 0; t < N; t++) {
    for (int j = 0; j < N; j++) Y[t * N + j] = kvqo_half_to_float(x16[t * stride + j]);
    kvqo_kvarn_rotate_f32(Y + t * N);
  }
  if (y_rot) memcpy(y_rot, Y, sizeof(float) * N * N);

  /* stage 3: alternating deviation normalisation */
  for (int i = 0; i < N; i++) r[i] = c[i] = 1.0f;
  for (int it = 0; it < KVARN_ITERS; it++) {
    for (int t = 0; t < N; t++) {
      float sd = dev128(Y + t * N);
      float inv = 1.0f / sd;
      for (int j = 0; j < N; j++) Y[t * N + j] = Y[t * N + j] * inv;
      r[t] = r[t] * sd;
    }
    for (int j = 0; j < N; j++) {
      for (int t = 0; t < N; t++) col[t] = Y[t * N + j];
      float sd = dev128(col);
      float inv = 1.0f / sd;
      for (int t = 0; t < N; t++) Y[t * N + j] = Y[t * N + j] * inv;
      c[j] = c[j] * sd;
    }
  }
  if (y_norm) memcpy(y_norm, Y, sizeof(float) * N * N);

  /* stage 4: asymmetric round-to-nearest */
  const float levels = side == 0 ? 15.0f : 3.0f;
  for (int g = 0; g < N; g++) { /* g = channel for keys, token for values */
    float mn = INFINITY, mx = -INFINITY;
    for (int e = 0; e < N; e++) {
      float v = side == 0 ? Y[e * N + g] : Y[g * N + e];
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
    float s = (mx - mn) / levels;
    for (int e = 0; e < N; e++) {
      int idx = side == 0 ? e * N + g : g * N + e;
      uint8_t q = 0;
      if (s != 0.0f) q = (uint8_t)clampf(rintf((Y[idx] - mn) / s), 0.0f, levels);
      cd[idx] = q;
    }
    s_q[g] = s;
    m_q[g] = mn;
  }

  if (r_out) memcpy(r_out, r, sizeof r);
  if (c_out) memcpy(c_out, c, sizeof c);
  if (codes) memcpy(codes, cd, (size_t)N * N);
  if (qs) memcpy(qs, s_q, sizeof s_q);
  if (qm) memcpy(qm, m_q, sizeof m_q);
  if (meta) {
    for (int i = 0; i < N; i++) {
      if (side == 0) {
        meta[i] = c[i] * s_q[i];
        meta[N + i] = c[i] * m_q[i];
        meta[2 * N + i] = r[i];
      } else {
        meta[i] = r[i] * s_q[i];
        meta[N + i] = r[i] * m_q[i];
        meta[2 * N + i] = c[i];
      }
    }
  }
  free(Y);
  free(cd);
}

/* ------------------------------------------------------------------------ */
/* Page layout (the library's documented cache contract)                     */
/* ------------------------------------------------------------------------ */
/*
 * cache = num_pages pages; a page holds num_kv_heads chunks; the chunk of
 * (page p, head h) starts at byte (p*H + h) * chunk_bytes.  Inside a chunk
 * (P = page_size, D = head_dim, t = token offset in the page, d = channel):
 *
 *  8-bit formats (FP8 per-tensor, INT8 / FP8 per-token-head): K and V each
 *  take 16*D bytes per group of 16 tokens (u = t/16, s = t%16), at 16*D*u
 *  inside their region; with B = min(16, D/4):
 *    K codes  at 0:     d = (D/4)*g + B*h + e  ->  64*B*h + 16*B*g + B*s + e
 *    V codes  at P*D:   d = (D/16)*n + c, c = (B/4)*h + j  ->
 *                       64*B*h + 16*B*(s/4) + B*n + 4*j + s%4
 *    per-token-head only: K scales fp32 [P] at 2*P*D, V scales fp32 [P] after
 *  NVFP4 (in a byte the low nibble holds the first element):
 *    K codes  [P][D/2]      at 0:            byte t*D/2 + d/2, nibble d%2
 *    V codes  [P/4][D/2][4] at P*D/2:        byte 2*D*(t/4) + 4*(d/2) + t%4,
 *                                            nibble d%2
 *    K block scales [P][D/16]  at P*D:       byte t*D/16 + d/16
 *    V block scales [D/16][P]  after:        byte (d/16)*P + t
 *  MXFP4: the NVFP4 code layout, with E8M0 bytes per 32 channels
 *    K block scales [P][D/32]  at P*D:       byte t*D/32 + d/32
 *    V block scales [D/32][P]  after:        byte (d/32)*P + t
 *  INT4 per-token-head (two's-complement nibbles, low nibble first):
 *    K codes  [P][D/2]      at 0:            byte t*D/2 + d/2, nibble d%2
 *    V codes  [P/4][D/2][4] at P*D/2:        byte 2*D*(t/4) + 4*(d/2) + t%4,
 *                                            nibble d%2
 *    K scales fp32 [P] at P*D, V scales fp32 [P] after
 *  KVarN k4v2 (D = 128, P = 128 or 256): a page holds P/128 tiles of 128
 *  tokens back to back, KVARN_TILE_BYTES each; tile k holds tokens
 *  128k .. 128k+127 of the page, t below is the token's offset in its tile:
 *    K codes  [P][D/2] 4-bit at 0:           byte t*D/2 + d/2, nibble d%2
 *    V codes  [P/4][D] 2-bit at P*D/2:       byte D*(t/4) + d, bits 2(t%4)+1..2(t%4)
 *    fp32 K alpha[D], K beta[D], K rho[P], V alpha[P], V beta[P], V gamma[D]
 */

static int valid_layout(const kvqo_layout* L) {
  if (!L) return 0;
  int D = L->head_dim, P = L->page_size;
  if (L->num_kv_heads <= 0 || L->num_pages <= 0) return 0;
  switch (L->format) {
    case O_FP8_PER_TENSOR:
    case O_INT8_PTH:
    case O_FP8_PTH:
    case O_NVFP4:
    case O_INT4_PTH:
    case O_MXFP4:
      return D > 0 && D % 32 == 0 && D <= 4096 && P > 0 && P % 16 == 0;
    case O_KVARN_K4V2_G128:
      return D == 128 && (P == 128 || P == 256);
    default:
      return 0;
  }
}

static int valid_scale(float s) {
  return isfinite(s) && s >= 0x1p-64f && s <= 0x1p64f;
}

int64_t kvqo_chunk_bytes(const kvqo_layout* L) {
  if (!valid_layout(L)) return -1;
  int64_t D = L->head_dim, P = L->page_size;
  switch (L->format) {
    case O_FP8_PER_TENSOR: return 2 * P * D;
    case O_INT8_PTH:
    case O_FP8_PTH: return 2 * P * D + 2 * 4 * P;
    case O_INT4_PTH: return 2 * (P * D / 2) + 2 * 4 * P;
    case O_NVFP4: return 2 * (P * D / 2) + 2 * (P * D / 16);
    case O_MXFP4: return 2 * (P * D / 2) + 2 * (P * D / 32);
    case O_KVARN_K4V2_G128: return (P / 128) * KVARN_TILE_BYTES;
  }
  return -1;
}

int64_t kvqo_page_bytes(const kvqo_layout* L) {
  int64_t c = kvqo_chunk_bytes(L);
  return c < 0 ? -1 : c * L->num_kv_heads;
}

static uint8_t* chunk_at(const kvqo_layout* L, const uint8_t* cache, int64_t page, int h) {
  return (uint8_t*)cache + (page * L->num_kv_heads + h) * kvqo_chunk_bytes(L);
}

/* Byte offsets of element (t, d) in the 8-bit K and V regions. */
static int64_t k8_off(int D, int t, int d) {
  int B = D / 4 < 16 ? D / 4 : 16;
  int g = d / (D / 4), r = d % (D / 4), h = r / B, e = r % B;
  int u = t / 16, s = t % 16;
  return 16LL * D * u + 64 * B * h + 16 * B * g + B * s + e;
}
static int64_t v8_off(int D, int t, int d) {
  int B = D / 4 < 16 ? D / 4 : 16;
  int n = d / (D / 16), c = d % (D / 16), h = c / (B / 4), j = c % (B / 4);
  int u = t / 16, s = t % 16;
  return 16LL * D * u + 64 * B * h + 16 * B * (s / 4) + B * n + 4 * j + s % 4;
}

static void put_nibble(uint8_t* p, int hi, uint8_t v) {
  if (hi)
    *p = (uint8_t)((*p & 0x0F) | ((v & 15) << 4));
  else
    *p = (uint8_t)((*p & 0xF0) | (v & 15));
}
static uint8_t get_nibble(const uint8_t* p, int hi) { return hi ? (*p >> 4) : (*p & 15); }

/* Store one token-head row (K and V) at token offset t of a chunk. */
static void store_row(const kvqo_layout* L, uint8_t* ch, int t, const float* xk,
                      const float* xv) {
  int D = L->head_dim, P = L->page_size;
  uint8_t ck[4096], cv[4096], bk[256], bv[256];
  float sk = 0, sv = 0;
  switch (L->format) {
    case O_INT8_PTH:
      quant_row_int8(xk, D, ck, &sk);
      quant_row_int8(xv, D, cv, &sv);
      break;
    case O_FP8_PTH:
      quant_row_fp8_pth(xk, D, ck, &sk);
      quant_row_fp8_pth(xv, D, cv, &sv);
      break;
    case O_FP8_PER_TENSOR:
      quant_row_fp8_pt(xk, D, L->k_scale, ck);
      quant_row_fp8_pt(xv, D, L->v_scale, cv);
      break;
    case O_NVFP4: {
      int f = L->flags & O_FLAG_NVFP4_4OVER6;
      quant_row_nvfp4(xk, D, L->k_scale, f, ck, bk);
      quant_row_nvfp4(xv, D, L->v_scale, f, cv, bv);
      break;
    }
    case O_INT4_PTH:
      quant_row_int4(xk, D, ck, &sk);
      quant_row_int4(xv, D, cv, &sv);
      break;
    case O_MXFP4:
      quant_row_mxfp4(xk, D, ck, bk);
      quant_row_mxfp4(xv, D, cv, bv);
      break;
  }
  if (L->format == O_INT4_PTH) {
    uint8_t* kc = ch;
    uint8_t* vc = ch + (int64_t)P * D / 2;
    float* ksc = (float*)(ch + (int64_t)P * D);
    for (int d = 0; d < D; d++) {
      put_nibble(kc + (int64_t)t * D / 2 + d / 2, d % 2, ck[d]);
      put_nibble(vc + 2LL * D * (t / 4) + 4 * (d / 2) + t % 4, d % 2, cv[d]);
    }
    ksc[t] = sk;
    ksc[P + t] = sv;
  } else if (L->format == O_NVFP4 || L->format == O_MXFP4) {
    const int BL = L->format == O_NVFP4 ? 16 : 32; /* values per block scale */
    uint8_t* kc = ch;
    uint8_t* vc = ch + (int64_t)P * D / 2;
    uint8_t* ks = ch + (int64_t)P * D;
    uint8_t* vs = ks + (int64_t)P * D / BL;
    for (int d = 0; d < D; d++) {
      put_nibble(kc + (int64_t)t * D / 2 + d / 2, d % 2, ck[d]);
      put_nibble(vc + 2LL * D * (t / 4) + 4 * (d / 2) + t % 4, d % 2, cv[d]);
    }
    for (int b = 0; b < D / BL; b++) {
      ks[(int64_t)t * (D / BL) + b] = bk[b];
      vs[(int64_t)b * P + t] = bv[b];
    }
  } else {
    uint8_t* kc = ch;
    uint8_t* vc = ch + (int64_t)P * D;
    for (int d = 0; d < D; d++) {
      kc[k8_off(D, t, d)] = ck[d];
      vc[v8_off(D, t, d)] = cv[d];
    }
    if (L->format != O_FP8_PER_TENSOR) {
      float* ksc = (float*)(ch + 2LL * P * D);
      ksc[t] = sk;
      ksc[P + t] = sv;
    }
  }
}

/* Read one token-head row back in binary64 (x_hat = code value times scales;
 * the products are exact in binary64).  KVarN rows are returned in the
 * original (unrotated) basis. */
static void load_row(const kvqo_layout* L, const uint8_t* ch, int t, double* k, double* v) {
  int D = L->head_dim, P = L->page_size;
  switch (L->format) {
    case O_INT8_PTH:
    case O_FP8_PTH:
    case O_FP8_PER_TENSOR: {
      const uint8_t* kc = ch;
      const uint8_t* vc = ch + (int64_t)P * D;
      double sk, sv;
      if (L->format == O_FP8_PER_TENSOR) {
        sk = L->k_scale;
        sv = L->v_scale;
      } else {
        float tmp[2];
        memcpy(&tmp[0], ch + 2LL * P * D + 4LL * t, 4);
        memcpy(&tmp[1], ch + 2LL * P * D + 4LL * (P + t), 4);
        sk = tmp[0];
        sv = tmp[1];
      }
      for (int d = 0; d < D; d++) {
        uint8_t a = kc[k8_off(D, t, d)];
        uint8_t b = vc[v8_off(D, t, d)];
        double qa, qb;
        if (L->format == O_INT8_PTH) {
          qa = (double)(int8_t)a;
          qb = (double)(int8_t)b;
        } else {
          qa = kvqo_e4m3_decode(a);
          qb = kvqo_e4m3_decode(b);
        }
        k[d] = qa * sk;
        v[d] = qb * sv;
      }
      break;
    }
    case O_NVFP4: {
      const uint8_t* kc = ch;
      const uint8_t* vc = ch + (int64_t)P * D / 2;
      const uint8_t* ks = ch + (int64_t)P * D;
      const uint8_t* vs = ks + (int64_t)P * D / 16;
      for (int d = 0; d < D; d++) {
        uint8_t a = get_nibble(kc + (int64_t)t * D / 2 + d / 2, d % 2);
        uint8_t b = get_nibble(vc + 2LL * D * (t / 4) + 4 * (d / 2) + t % 4, d % 2);
        double sbk = kvqo_e4m3_decode(ks[(int64_t)t * (D / 16) + d / 16]);
        double sbv = kvqo_e4m3_decode(vs[(int64_t)(d / 16) * P + t]);
        /* x_hat = s_t * s_b * q, [P5] §双层缩放怎样恢复动态范围 */
        k[d] = (double)L->k_scale * sbk * kvqo_e2m1_decode(a);
        v[d] = (double)L->v_scale * sbv * kvqo_e2m1_decode(b);
      }
      break;
    }
    case O_MXFP4: {
      const uint8_t* kc = ch;
      const uint8_t* vc = ch + (int64_t)P * D / 2;
      const uint8_t* ks = ch + (int64_t)P * D;
      const uint8_t* vs = ks + (int64_t)P * D / 32;
      for (int d = 0; d < D; d++) {
        uint8_t a = get_nibble(kc + (int64_t)t * D / 2 + d / 2, d % 2);
        uint8_t b = get_nibble(vc + 2LL * D * (t / 4) + 4 * (d / 2) + t % 4, d % 2);
        /* x_hat = 2^(E - 127) * q, E the block's E8M0 byte */
        k[d] = ldexp(kvqo_e2m1_decode(a), (int)ks[(int64_t)t * (D / 32) + d / 32] - 127);
        v[d] = ldexp(kvqo_e2m1_decode(b), (int)vs[(int64_t)(d / 32) * P + t] - 127);
      }
      break;
    }
    case O_INT4_PTH: {
      const uint8_t* kc = ch;
      const uint8_t* vc = ch + (int64_t)P * D / 2;
      float tmp[2];
      memcpy(&tmp[0], ch + (int64_t)P * D + 4LL * t, 4);
      memcpy(&tmp[1], ch + (int64_t)P * D + 4LL * (P + t), 4);
      for (int d = 0; d < D; d++) {
        int a = get_nibble(kc + (int64_t)t * D / 2 + d / 2, d % 2);
        int b = get_nibble(vc + 2LL * D * (t / 4) + 4 * (d / 2) + t % 4, d % 2);
        /* two's-complement nibble -> -8..7 */
        k[d] = (double)((a ^ 8) - 8) * (double)tmp[0];
        v[d] = (double)((b ^ 8) - 8) * (double)tmp[1];
      }
      break;
    }
    case O_KVARN_K4V2_G128: {
      ch += (int64_t)(t / 128) * KVARN_TILE_BYTES; /* the token's tile in the page */
      t %= 128;
      const uint8_t* kc = ch;
      const uint8_t* vc = ch + 128 * 64;
      const float* meta = (const float*)(ch + 128 * 64 + 128 * 32);
      const float *ka = meta, *kb = meta + 128, *kr = meta + 256;
      const float *va = meta + 384, *vb = meta + 512, *vg = meta + 640;
      for (int j = 0; j < 128; j++) {
        uint8_t a = get_nibble(kc + t * 64 + j / 2, j % 2);
        uint8_t b = (uint8_t)((vc[128 * (t / 4) + j] >> (2 * (t % 4))) & 3);
        k[j] = (double)kr[t] * ((double)ka[j] * a + (double)kb[j]);
        v[j] = (double)vg[j] * ((double)va[t] * b + (double)vb[t]);
      }
      rotate_f64(k);
      rotate_f64(v);
      break;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Entry points                                                              */
/* ------------------------------------------------------------------------ */

/* Quantise-on-write: k16, v16 are [n_tok][H][D] binary16; token i goes to
 * slot slots[i] = page * P + offset.  Negative slots and slots past the pool
 * are skipped.  KVarN: n_tok % 128 == 0 and each run of 128 tokens must
 * fill one tile of a page in order (slots s0 + 0..127, s0 a multiple of
 * 128). */
int kvqo_quantize_write(const kvqo_layout* L, const uint16_t* k16, const uint16_t* v16,
                        const int64_t* slots, int64_t n_tok, uint8_t* cache) {
  if (!valid_layout(L) || n_tok < 0) return O_BAD_ARG;
  if ((L->format == O_FP8_PER_TENSOR || L->format == O_NVFP4) &&
      !(valid_scale(L->k_scale) && valid_scale(L->v_scale)))
    return O_BAD_ARG;
  int H = L->num_kv_heads, D = L->head_dim, P = L->page_size;
  int64_t pool = (int64_t)L->num_pages * P;
  if (L->format == O_KVARN_K4V2_G128) {
    if (n_tok % 128) return O_BAD_ARG;
    uint8_t* codes = (uint8_t*)malloc(128 * 128);
    float meta[384];
    for (int64_t tile = 0; tile < n_tok / 128; tile++) {
      int64_t s0 = slots[tile * 128];
      if (s0 < 0 || s0 >= pool) continue;
      if (s0 % 128) { free(codes); return O_BAD_ARG; }
      for (int t = 1; t < 128; t++)
        if (slots[tile * 128 + t] != s0 + t) { free(codes); return O_BAD_ARG; }
      int64_t page = s0 / P;
      for (int h = 0; h < H; h++) {
        uint8_t* ch = chunk_at(L, cache, page, h) + (s0 % P) / 128 * KVARN_TILE_BYTES;
        const int64_t row0 = (tile * 128 * H + h) * (int64_t)D;
        float* mbase = (float*)(ch + 128 * 64 + 128 * 32);
        /* keys */
        kvqo_kvarn_tile(k16 + row0, (int64_t)H * D, 0, NULL, NULL, NULL, NULL, codes, NULL,
                        NULL, meta);
        for (int t = 0; t < 128; t++)
          for (int j = 0; j < 128; j++) put_nibble(ch + t * 64 + j / 2, j % 2, codes[t * 128 + j]);
        memcpy(mbase, meta, 384 * sizeof(float));
        /* values */
        kvqo_kvarn_tile(v16 + row0, (int64_t)H * D, 1, NULL, NULL, NULL, NULL, codes, NULL,
                        NULL, meta);
        uint8_t* vc = ch + 128 * 64;
        memset(vc, 0, 128 * 32);
        for (int t = 0; t < 128; t++)
          for (int j = 0; j < 128; j++)
            vc[128 * (t / 4) + j] |= (uint8_t)(codes[t * 128 + j] << (2 * (t % 4)));
        memcpy(mbase + 384, meta, 384 * sizeof(float));
      }
    }
    free(codes);
    return O_OK;
  }
  float xk[4096], xv[4096];
  for (int64_t i = 0; i < n_tok; i++) {
    int64_t s = slots[i];
    if (s < 0 || s >= pool) continue;
    int64_t page = s / P;
    int t = (int)(s % P);
    for (int h = 0; h < H; h++) {
      const uint16_t* kr = k16 + (i * H + h) * (int64_t)D;
      const uint16_t* vr = v16 + (i * H + h) * (int64_t)D;
      for (int d = 0; d < D; d++) {
        xk[d] = kvqo_half_to_float(kr[d]);
        xv[d] = kvqo_half_to_float(vr[d]);
      }
      store_row(L, chunk_at(L, cache, page, h), t, xk, xv);
    }
  }
  return O_OK;
}

/* Dequantise the tokens at the given slots into binary64 [n_tok][H][D]
 * (KVarN in the original basis).  Rows of skipped slots are left untouched. */
int kvqo_dequantize(const kvqo_layout* L, const uint8_t* cache, const int64_t* slots,
                    int64_t n_tok, double* k_out, double* v_out) {
  if (!valid_layout(L) || n_tok < 0) return O_BAD_ARG;
  int H = L->num_kv_heads, D = L->head_dim, P = L->page_size;
  int64_t pool = (int64_t)L->num_pages * P;
  for (int64_t i = 0; i < n_tok; i++) {
    int64_t s = slots[i];
    if (s < 0 || s >= pool) continue;
    for (int h = 0; h < H; h++)
      load_row(L, chunk_at(L, cache, s / P, h), (int)(s % P), k_out + (i * H + h) * D,
               v_out + (i * H + h) * D);
  }
  return O_OK;
}

/* Single-query attention in binary64 over explicit rows:
 * out = softmax(scale * K q) V, [P5] §K 与 V 的量化误差进入 attention 的位置不同
 * (mask M = 0: every cached token precedes the decoding query). */
void kvqo_attention_dense(const double* q, const double* k, const double* v, int64_t T, int D,
                          double scale, double* out) {
  for (int d = 0; d < D; d++) out[d] = 0.0;
  if (T <= 0) return;
  double* lg = (double*)malloc(sizeof(double) * T);
  double mx = -INFINITY;
  for (int64_t t = 0; t < T; t++) {
    double acc = 0.0;
    for (int d = 0; d < D; d++) acc += q[d] * k[t * D + d];
    lg[t] = acc * scale;
    if (lg[t] > mx) mx = lg[t];
  }
  double den = 0.0;
  for (int64_t t = 0; t < T; t++) {
    lg[t] = exp(lg[t] - mx);
    den += lg[t];
  }
  for (int64_t t = 0; t < T; t++)
    for (int d = 0; d < D; d++) out[d] += lg[t] * v[t * D + d];
  for (int d = 0; d < D; d++) out[d] /= den;
  free(lg);
}

/* Paged decode attention, [P5] §Prefill 写一次，Decode 反复读 and the attention
 * equation of §K 与 V 的量化误差进入 attention 的位置不同, reading the cache
 * through block tables ([P4] §写和读 flowchart).
 *   q16 [B][Hq][D] binary16; q head h reads kv head h / (Hq/H) (consecutive
 *   grouping); block_tables [B][max_pages]; ctx_lens [B].
 *   KVarN: the last ctx % 128 tokens of a sequence are read as binary16 from
 *   tail16 [B][2][H][128][D] (keys then values, row j = token
 *   ctx - ctx%128 + j); the complete tiles come from the cache.
 *   pairs [n_pairs][2] = (b, q head) selects the outputs computed;
 *   out [n_pairs][D] binary64.  An empty context gives a zero row. */
int kvqo_decode_attention(const kvqo_layout* L, const uint8_t* cache, const uint16_t* q16,
                          int32_t num_q_heads, const int32_t* block_tables, int32_t max_pages,
                          const int32_t* ctx_lens, int32_t batch, float sm_scale,
                          const uint16_t* tail16, const int32_t* pairs, int32_t n_pairs,
                          double* out) {
  if (!valid_layout(L)) return O_BAD_ARG;
  int H = L->num_kv_heads, D = L->head_dim, P = L->page_size;
  if (num_q_heads <= 0 || num_q_heads % H) return O_BAD_ARG;
  int G = num_q_heads / H;
  for (int32_t i = 0; i < n_pairs; i++) {
    int b = pairs[2 * i], h = pairs[2 * i + 1];
    if (b < 0 || b >= batch || h < 0 || h >= num_q_heads) return O_BAD_ARG;
    int64_t ctx = ctx_lens[b];
    if (ctx < 0 || ctx > (int64_t)max_pages * P) return O_BAD_ARG;
    int64_t n_cached = ctx, n_tail = 0;
    if (L->format == O_KVARN_K4V2_G128) {
      n_tail = ctx % 128;
      n_cached = ctx - n_tail;
      if (n_tail && !tail16) return O_BAD_ARG;
    }
    int kvh = h / G;
    double* K = (double*)malloc(sizeof(double) * (ctx ? ctx : 1) * D);
    double* V = (double*)malloc(sizeof(double) * (ctx ? ctx : 1) * D);
    for (int64_t t = 0; t < n_cached; t++) {
      int32_t page = block_tables[(int64_t)b * max_pages + t / P];
      if (page < 0 || page >= L->num_pages) {
        free(K);
        free(V);
        return O_BAD_ARG;
      }
      load_row(L, chunk_at(L, cache, page, kvh), (int)(t % P), K + t * D, V + t * D);
    }
    for (int64_t j = 0; j < n_tail; j++) {
      const uint16_t* kt = tail16 + ((((int64_t)b * 2 + 0) * H + kvh) * 128 + j) * D;
      const uint16_t* vt = tail16 + ((((int64_t)b * 2 + 1) * H + kvh) * 128 + j) * D;
      for (int d = 0; d < D; d++) {
        K[(n_cached + j) * D + d] = kvqo_half_to_float(kt[d]);
        V[(n_cached + j) * D + d] = kvqo_half_to_float(vt[d]);
      }
    }
    double qd[4096];
    for (int d = 0; d < D; d++) qd[d] = kvqo_half_to_float(q16[((int64_t)b * num_q_heads + h) * D + d]);
    kvqo_attention_dense(qd, K, V, ctx, D, (double)sm_scale, out + (int64_t)i * D);
    free(K);
    free(V);
  }
  return O_OK;
}
