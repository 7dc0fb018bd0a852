// decode_attn.hip -- dequant-fused paged GQA decode attention for FP8
// per-tensor, INT8 / FP8 / INT4 per-token-head, NVFP4 and MXFP4 caches
// (gfx950).
//
// Computes O = softmax(q K^T * sm_scale) V for every (sequence, q head) with
// the cache read through block tables ([P5] "NVFP4 KV Cache：Blackwell 上的
// 4-bit 缓存量化", §K 与 V 的量化误差进入 attention 的位置不同 and §KV 的写入与
// 读取路径: unpack, apply scales, feed the attention math inside the tile
// load, never materialise a full-precision copy).
//
// Decomposition.  A workgroup of W wavefronts (4, or 8 when one workgroup
// per (sequence, kv head) fills the GPU) owns one (sequence, kv head,
// context split); wave w walks pages w, w+W, ... of the split.  Per 16-token
// sub-page a wave computes
//   S^T[16 tok][16 cols] = K[16 tok][D] * Q^T[D][16 cols]   (D/32 MFMA 16x16x32 f16)
//   O[16 rows][D]       += P[16 rows][16 tok] * V[16 tok][D] (D/16 MFMA 16x16x16 f16)
// With K as the A operand the score tile lands in the registers in exactly
// the layout the second MFMA wants for P (lane l: head l%16, tokens
// 4*(l/16)..+3), so softmax needs no data movement between the two products.
// The G query heads of the group occupy MFMA rows 0..G-1; rows G..2G-1 carry
// the binary16 rounding remainder of P (P = hi + lo), which makes the PV
// product accurate to ~2^-22 at no extra MFMA cost.  Codes are converted to
// binary16 exactly (every format's values are binary16 numbers); per-token
// scales fold into the scores (K) and into P (V), per-tensor / global scales
// into the score scale and the final output.
//
// Cache layout in HBM is chosen for these operands: each lane's K bytes are
// one contiguous run of D/4 codes of one token, and each lane's V bytes are
// one contiguous run holding four consecutive tokens per channel, so loads
// are 16-byte vectors that together cover whole 128-byte lines and need no
// LDS staging.  Loads are raw buffer loads from a per-chunk resource.
//
// Splits: with more than one, each workgroup writes its partial (m, l, O) to
// the workspace and a second, small kernel merges the partials of every
// (sequence, kv head); a single split writes the output directly.  In a
// decode step (kvq_decode_attention_append) the split-0 workgroup of each
// (sequence, kv head) also quantises and stores the new token and folds it
// into its own partial: the step is the split kernel, plus the merge when
// there are several splits.
#include "row_encode.h"

namespace kvq {
namespace {

constexpr int kDepth = 2;  // 16-token units per wave: 1 in compute, kDepth-1 in flight

// Formats with 4-bit codes in the nibble layout (NVFP4, INT4 per-token-head,
// MXFP4) and formats with per-token-head fp32 scales.
template <int FMT> constexpr bool kNibble = FMT == 4 || FMT == 6 || FMT == 7;
template <int FMT> constexpr bool kPth = FMT == 2 || FMT == 3 || FMT == 6;

// INT4 keys enter the QK product with their channels in the order
// 0, 2, 4, 6, 1, 3, 5, 7 within each group of 8 (the byte permute unpack);
// the query columns are permuted to match.
__host__ __device__ constexpr int int4_slot_channel(int i) { return i < 4 ? 2 * i : 2 * (i - 4) + 1; }

// Raw bytes of one 16-token unit for one lane, as loaded from the chunk.
template <int FMT, int D>
struct Raw {
  static constexpr int KW = kNibble<FMT> ? D / 32 : D / 16;  // dwords of K codes
  static constexpr int VW = kNibble<FMT> ? D / 32 : D / 16;  // dwords of V codes
  uint32_t k[KW];
  uint32_t v[VW];
  uint32_t ksc, vsc;  // block-scale bytes (K: this token's blocks; V: 4 tokens)
  float4 ks, vs;      // per-token-head scales of the lane's 4 score tokens
};

template <int FMT, int D>
__device__ __forceinline__ void zero_raw(Raw<FMT, D>& r) {
#pragma unroll
  for (int i = 0; i < Raw<FMT, D>::KW; ++i) r.k[i] = 0u;
#pragma unroll
  for (int i = 0; i < Raw<FMT, D>::VW; ++i) r.v[i] = 0u;
  r.ksc = r.vsc = 0u;
  r.ks = r.vs = float4{0.f, 0.f, 0.f, 0.f};
}

// Per-lane byte offsets of a unit's loads within its chunk, fixed for the
// whole kernel: the chunk (page, kv head) is a buffer resource in scalar
// registers and the 16-token group a scalar offset, so a load's only vector
// operand is this 32-bit offset and no address arithmetic runs per unit.
struct LaneOffs {
  uint32_t k, v, ks, vs;
};

template <int FMT, int D>
__device__ __forceinline__ LaneOffs lane_offsets(int gq, int n, int P) {
  constexpr int DL = D / 4;
  constexpr int NV = D / 16;
  LaneOffs o;
  if constexpr (!kNibble<FMT>) {
    constexpr int B = DL < 16 ? DL : 16;
    o.k = 16 * B * gq + B * n;
    o.v = o.k;
    o.ks = o.vs = 16 * gq;  // per-token-head scales of tokens 4gq .. 4gq+3
  } else {
    o.k = n * (D / 2) + (DL / 2) * gq;
    o.v = 2 * D * gq + 4 * ((NV * n) / 2);
    if constexpr (FMT == 4) {
      o.ks = n * (D / 16) + (DL * gq) / 16;
      o.vs = ((NV * n) / 16) * P + 4 * gq;
    } else if constexpr (FMT == 7) {
      o.ks = n * (D / 32) + (DL * gq) / 32;
      o.vs = ((NV * n) / 32) * P + 4 * gq;
    } else {
      o.ks = o.vs = 16 * gq;
    }
  }
  return o;
}

// Issue the loads of unit `sub` (16 tokens) of a chunk.  K: D/4 channels of
// token row n starting at channel (D/4)*gq; V: channels (D/16)*n .. +D/16 of
// tokens 4*gq .. 4*gq+3.  The unit's position within the chunk is a scalar
// offset.
template <int FMT, int D>
__device__ __forceinline__ void load_unit(const uint8_t* chunk, const ChunkGeom& g, int sub, const LaneOffs& lo,
                                          Raw<FMT, D>& r) {
  constexpr int DL = D / 4;
  constexpr int NV = D / 16;
  const __amdgpu_buffer_rsrc_t rs = chunk_rsrc(chunk, g.chunk_bytes);
  if constexpr (!kNibble<FMT>) {
    // coalesced 8-bit layout: piece h of all 64 lanes is one contiguous run
    constexpr int B = DL < 16 ? DL : 16;
    const int kb = 16 * D * sub;
    const int vb = (int)g.v_codes + 16 * D * sub;
#pragma unroll
    for (int h = 0; h < DL / B; ++h) buf_dwords<B / 4>(rs, lo.k, kb + 64 * B * h, r.k + (B / 4) * h);
#pragma unroll
    for (int h = 0; h < (4 * NV) / B; ++h) buf_dwords<B / 4>(rs, lo.v, vb + 64 * B * h, r.v + (B / 4) * h);
    if constexpr (FMT == 2 || FMT == 3) {
      r.ks = buf_f4(rs, lo.ks, (int)g.k_scales + 64 * sub);
      r.vs = buf_f4(rs, lo.vs, (int)g.v_scales + 64 * sub);
    }
  } else {
    buf_dwords<Raw<FMT, D>::KW>(rs, lo.k, sub * 16 * (D / 2), r.k);
    buf_dwords<Raw<FMT, D>::VW>(rs, lo.v, (int)g.v_codes + sub * 8 * D, r.v);
    if constexpr (FMT == 4) {
      const int so = (int)g.k_scales + sub * 16 * (D / 16);
      if constexpr (DL >= 32)
        r.ksc = __builtin_amdgcn_raw_buffer_load_b16(rs, lo.ks, so, kLoadNt);
      else
        r.ksc = __builtin_amdgcn_raw_buffer_load_b8(rs, lo.ks, so, kLoadNt);
      r.vsc = __builtin_amdgcn_raw_buffer_load_b32(rs, lo.vs, (int)g.v_scales + 16 * sub, kLoadNt);
    } else if constexpr (FMT == 7) {
      // the lane's D/4 key channels and D/16 value channels each lie in one
      // 32-channel block: one E8M0 byte for the key, one per token for V
      r.ksc = __builtin_amdgcn_raw_buffer_load_b8(rs, lo.ks, (int)g.k_scales + sub * 16 * (D / 32), kLoadNt);
      r.vsc = __builtin_amdgcn_raw_buffer_load_b32(rs, lo.vs, (int)g.v_scales + 16 * sub, kLoadNt);
    } else {
      r.ks = buf_f4(rs, lo.ks, (int)g.k_scales + 64 * sub);
      r.vs = buf_f4(rs, lo.vs, (int)g.v_scales + 64 * sub);
    }
  }
}

// K operand for QK MFMA kk: 8 channels (D/4)*gq + 8*kk .. +7 of token row n.
template <int FMT, int D>
__device__ __forceinline__ half8_t k_operand(const Raw<FMT, D>& r, int kk, half2_t ksc, float kmx) {
  if constexpr (FMT == 7) {
    // E2M1 * 2^k in binary16, the block scale applied by the conversion
    uint32_t h[4];
    e2m1x8_to_h_scaled(r.k[kk], kmx, h);
    return cat(as_h2(h[0]), as_h2(h[1]), as_h2(h[2]), as_h2(h[3]));
  } else if constexpr (FMT == 6) {
    // two's-complement nibble ^ 8 = code + 8 in 0..15.  A byte holding it is
    // the E4M3 encoding of (code + 8) * 2^-9, so the scaled conversion at 2^9
    // returns code + 8 exactly, two per instruction; the offset 8 * sum(q) is
    // removed from the scores once per head.  (An offset of 1032, as a byte
    // permute under the 0x64 exponent byte gives, would cost accuracy: the
    // biased sums would be ~100x larger than the scores.)
    const uint32_t w = r.k[kk] ^ 0x88888888u;
    const uint32_t x = w & 0x0F0F0F0Fu, y = (w >> 4) & 0x0F0F0F0Fu;
    uint32_t a, b, c, d;
    e4m3x4_to_h_scaled(x, 512.0f, a, b);
    e4m3x4_to_h_scaled(y, 512.0f, c, d);
    return cat(as_h2(a), as_h2(b), as_h2(c), as_h2(d));
  } else if constexpr (FMT != 4) {
    half2_t a, b, c, d;
    if constexpr (FMT == 2) {
      // signed codes, exact in binary16.  (Feeding 1152 + code and removing
      // 1152 * sum(q) from the scores afterwards saves the subtraction, but
      // the bias then dominates the binary32 sums: with a query of mean 16
      // the scores lose ~1e-2 to cancellation.)
      i8x4_to_h(r.k[2 * kk], a, b);
      i8x4_to_h(r.k[2 * kk + 1], c, d);
    } else {
      uint32_t p0, p1, p2, p3;
      e4m3x4_to_h_hw(r.k[2 * kk], p0, p1);
      e4m3x4_to_h_hw(r.k[2 * kk + 1], p2, p3);
      a = as_h2(p0), b = as_h2(p1), c = as_h2(p2), d = as_h2(p3);
    }
    return cat(a, b, c, d);
  } else {
    constexpr int DL = D / 4;
    uint32_t h[4];
    e2m1x8_to_h(r.k[kk], h);  // channels 0..7 in order
    const half_t sc = ksc[(DL >= 32) ? (8 * kk) / 16 : 0];
    const half2_t s2 = {sc, sc};
    return cat(as_h2(h[0]) * s2, as_h2(h[1]) * s2, as_h2(h[2]) * s2, as_h2(h[3]) * s2);
  }
}

// V operand for PV MFMA nn: channel (D/16)*n + nn of tokens 4*gq .. +3.
// NVFP4: the dword holds the channel pair (nn & ~1, nn | 1) of the 4 tokens,
// one token per byte; `pairs` are its conversions, (even, odd) per token.
template <int FMT, int D>
__device__ __forceinline__ half4_t v_operand(const Raw<FMT, D>& r, int nn, half2_t s01, half2_t s23,
                                             const uint32_t (&pairs)[4]) {
  if constexpr (FMT == 6) {
    // the channel's nibble of each of the 4 token bytes as code + 8, the
    // same way as the keys, then the exact binary16 subtraction of 8: the
    // values enter the product signed (an offset removed after the sum would
    // cancel against it, which loses the small outputs of rows whose scale
    // is large)
    const uint32_t w = r.v[nn / 2] ^ 0x88888888u;
    const uint32_t x = (nn & 1) ? ((w >> 4) & 0x0F0F0F0Fu) : (w & 0x0F0F0F0Fu);
    uint32_t lo, hi;
    e4m3x4_to_h_scaled(x, 512.0f, lo, hi);
    const half2_t eight = {(half_t)8.0f, (half_t)8.0f};
    return cat4(as_h2(lo) - eight, as_h2(hi) - eight);
  } else if constexpr (FMT == 7) {
    // `pairs` already carry each token's block scale
    const uint32_t sel = (nn & 1) ? 0x07060302u : 0x05040100u;
    return cat4(as_h2(perm(pairs[1], pairs[0], sel)), as_h2(perm(pairs[3], pairs[2], sel)));
  } else if constexpr (FMT != 4) {
    half2_t a, b;
    if constexpr (FMT == 2) {
      i8x4_to_h(r.v[nn], a, b);
    } else {
      uint32_t p0, p1;
      e4m3x4_to_h_hw(r.v[nn], p0, p1);
      a = as_h2(p0), b = as_h2(p1);
    }
    return cat4(a, b);
  } else {
    const uint32_t sel = (nn & 1) ? 0x07060302u : 0x05040100u;
    return cat4(as_h2(perm(pairs[1], pairs[0], sel)) * s01, as_h2(perm(pairs[3], pairs[2], sel)) * s23);
  }
}

// Online-softmax state and accumulators of one wavefront.
template <int D>
struct WaveState {
  float4_t acc[D / 16];
  float m_run, l_run;
};

template <int FMT, int D, int G>
__device__ __forceinline__ void process_unit(const Raw<FMT, D>& r, bool valid, int tok0, int ctx, int n, int gq,
                                             const half8_t* qB, float kconst, float kbias, WaveState<D>& st) {
  constexpr int NK = D / 32;
  constexpr int NV = D / 16;
  constexpr bool PTH = kPth<FMT>;

  // the lane's two key block scales (its D/4 channels), E4M3 -> binary16, exact
  half2_t ksc01 = {0, 0};
  if constexpr (FMT == 4) ksc01 = as_h2(e4m3x2_to_h_hw(r.ksc));
  const float kmx = FMT == 7 ? e8m0_scale(r.ksc) : 0.0f;
  float4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
    s = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand<FMT, D>(r, kk, ksc01, kmx), qB[kk], s, 0, 0, 0);

  // scores in log2 units; a unit wholly inside the context and on a valid
  // page (the common case, uniform across the wave) needs no token masks.
  // Lanes n >= G hold no head: their values are computed but never used.
  float lg[4], vsc[4];
  const bool full = valid && (tok0 + 16 <= ctx);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float c = PTH ? r.ks[i] * kconst : kconst;
    lg[i] = (s[i] - kbias) * c;
    vsc[i] = PTH ? r.vs[i] : 1.0f;
  }
  if (!full) {
    // a masked token's score becomes -inf and, with per-token value scales,
    // its scale 0 (its scale slot may hold anything, including a NaN that a
    // zero weight would not cancel)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (!(valid && tok0 + 4 * gq + i < ctx)) {
        lg[i] = kNegInf;
        if constexpr (PTH) vsc[i] = 0.0f;
      }
  }
  // The reference m_run is always finite (it starts at kRefStart), so a
  // masked score (-inf) gives exactly 0 without a select.  The weights
  // P * v_scale enter the PV product as binary16 high halves h and
  // remainders lo, two tokens per register.
  float p[4];
  uint32_t h01, h23, lo01, lo23;
  auto weights = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(lg[i] - st.m_run);
    split_products(p[0], vsc[0], p[1], vsc[1], h01, lo01);
    split_products(p[2], vsc[2], p[3], vsc[3], h23, lo23);
  };
  weights();
  const bool over = pairs_exceed_tau(h01, h23) & (n < G);

  // P (high/low halves) times V into the output rows.  Both sides of the
  // rare rescale branch below run their own copy, so the accumulators are
  // never merged between the branches (which costs a register copy of every
  // accumulator on the common path).
  auto accumulate = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) st.l_run += p[i];
    const half4_t pA = cat4(as_h2(hi_lo_rows<G>(h01, lo01)), as_h2(hi_lo_rows<G>(h23, lo23)));
    half2_t vs01 = {0, 0}, vs23 = {0, 0};
    if constexpr (FMT == 4) {
      uint32_t lo, hi;
      e4m3x4_to_h_hw(r.vsc, lo, hi);
      vs01 = as_h2(lo);
      vs23 = as_h2(hi);
    }
    float vmx[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (FMT == 7)
#pragma unroll
      for (int i = 0; i < 4; ++i) vmx[i] = e8m0_scale(r.vsc >> (8 * i));
    uint32_t pairs[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int nn = 0; nn < NV; ++nn) {
      if constexpr (FMT == 4)
        if ((nn & 1) == 0) e2m1x8_to_h(r.v[nn / 2], pairs);
      if constexpr (FMT == 7)
        if ((nn & 1) == 0) e2m1x8_to_h_scaled4(r.v[nn / 2], vmx, pairs);
      st.acc[nn] = __builtin_amdgcn_mfma_f32_16x16x16f16(pA, v_operand<FMT, D>(r, nn, vs01, vs23, pairs),
                                                         st.acc[nn], 0, 0, 0);
    }
  };

  if (__builtin_amdgcn_ballot_w64(over) != 0) {
    // move the reference to the exact maximum of score + log2(v_scale)
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lg[i] != kNegInf && n < G) mx = fmaxf(mx, PTH ? lg[i] + __log2f(vsc[i]) : lg[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m_run, mx);
    const float alpha = (m_new > st.m_run) ? exp2f(st.m_run - m_new) : 1.0f;
    st.l_run *= alpha;
    float ar[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * gq + i;
      ar[i] = __shfl(alpha, row < G ? row : (row < 2 * G ? row - G : 0));
    }
#pragma unroll
    for (int nn = 0; nn < NV; ++nn)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.acc[nn][i] *= ar[i];
    st.m_run = m_new;
    weights();
    accumulate();
  } else {
    accumulate();
  }
}

// The step's new token of (sequence b, kv head) in a single-split call:
// wave 0 quantises and stores the key row, wave 1 the value row, with the
// write path's per-row encoders (so the bytes are kvq_quantize_write's).
// When the token is attended, the dequantised key row goes through s_k and
// wave 0's 64 lanes take its dot products with the G queries, leaving each
// head's score in s_lg (log2 units, as the kernel's scores); wave 1 leaves
// the value row (codes times the row scale; a per-tensor or global V scale
// follows at the output) in s_v.
template <int FMT, int D, int G>
__device__ __forceinline__ void new_token_row(const DecodeArgs& a, int b, int kvh, int w, int lane, bool attend,
                                              float* s_k, float* s_lg, float* s_v) {
  constexpr bool K8 = !kNibble<FMT>;
  constexpr int VPL = K8 ? 8 : 16;  // values per lane of the row encoders
  constexpr int LPR = D / VPL;      // lanes per row
  if (lane < LPR) {
    const WriteArgs& wa = a.wnew;
    RowCodes rc;
    const int64_t row = (int64_t)w * wa.n_tok * wa.H + (int64_t)b * wa.H + kvh;
    if constexpr (K8)
      write_row_8bit<FMT, D>(wa, row, lane, true, &rc);
    else
      write_row_4bit<FMT, D>(wa, row, lane, true, &rc);
    if (attend) {
      float c[VPL];
      lane_values<FMT, VPL>(rc, c);
      const float rs = kPth<FMT> ? rc.s : 1.0f;
      float* dst = w == 0 ? s_k : s_v;
#pragma unroll
      for (int i = 0; i < VPL; ++i) dst[VPL * lane + i] = c[i] * rs;
    }
  }
  if (w != 0 || !attend) return;
  // the wave's own LDS writes complete before its reads
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  constexpr int LPH = (64 / G) < (D / 2) ? (64 / G) : (D / 2);  // lanes per head
  constexpr int VH = D / LPH;                                     // channels per lane
  const int g = lane / LPH, ch = VH * (lane % LPH);
  float part = 0.0f;
  if (g < G) {
    const uint16_t* qp = a.q + ((int64_t)b * a.Hq + kvh * G + g) * D + ch;
#pragma unroll
    for (int i = 0; i < VH; ++i) part = __builtin_fmaf((float)__builtin_bit_cast(half_t, qp[i]), s_k[ch + i], part);
  }
#pragma unroll
  for (int m = LPH / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m);
  const float kconst = (FMT == 1 || FMT == 4) ? a.k_scale * a.qk_scale : a.qk_scale;
  if (g < G && lane % LPH == 0) s_lg[g] = part * kconst;
}

template <int FMT, int D, int G, int W>
__global__ __launch_bounds__(64 * W) void decode_kernel(DecodeArgs a) {
  constexpr int NK = D / 32;
  constexpr int NV = D / 16;
  constexpr int DL = D / 4;

  constexpr int NT = 64 * W;  // threads
  __shared__ float lds_o[W][2 * G][D];
  __shared__ float lds_m[W][16];
  __shared__ float lds_l[W][16];
  __shared__ int s_pages[kPageChunk];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, l = tid & 63, n = l & 15, gq = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar register
  const int P = a.P;
  const int S = a.num_splits;

  float* partials = reinterpret_cast<float*>(a.workspace);
  const int64_t rec_floats = ws_record_floats(D);

  // The first chunk's block-table entries are requested before the context
  // length arrives: entries p_begin .. p_begin + 255 of the split lie inside
  // the table's row whatever the length is, so the two round trips overlap.
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_pages;
  const int first_cap = min(kPageChunk, min(a.pages_per_split, a.max_pages - split * a.pages_per_split));
  const int bt_first = tid < first_cap ? bt[split * a.pages_per_split + tid] : 0;

  // wave-uniform bounds (kept in scalar registers)
  int ctx = __builtin_amdgcn_readfirstlane(a.ctx_lens[b]);
  ctx = ctx < 0 ? 0 : (ctx > a.max_pages * P ? a.max_pages * P : ctx);
  bool attend_new = false;
  if (a.new_slots != nullptr) {
    // append-and-decode: the last position is the new token, attended by
    // the split-0 workgroup below when its slot is in the pool
    const int64_t ns = a.new_slots[b];
    attend_new = ctx >= 1 && ns >= 0 && ns < (int64_t)a.num_pages * P;
    if (attend_new) ctx -= 1;
  }
  const int n_pages = (ctx + P - 1) / P;
  const int p_begin = split * a.pages_per_split;
  const int p_end = min(p_begin + a.pages_per_split, n_pages);

  // Q^T as the B operand: column n = head kvh*G + n, rows = channels DL*gq + 8kk + 0..7
  half8_t qB[NK];
  if (n < G) {
    const uint16_t* qp = a.q + ((int64_t)b * a.Hq + kvh * G + n) * D + DL * gq;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const half8_t qv = *reinterpret_cast<const half8_t*>(qp + 8 * kk);
      if constexpr (FMT == 6) {
#pragma unroll
        for (int i = 0; i < 8; ++i) qB[kk][i] = qv[int4_slot_channel(i)];
      } else {
        qB[kk] = qv;
      }
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) qB[kk] = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
  }

  const float kconst = (FMT == 1 || FMT == 4) ? a.k_scale * a.qk_scale : a.qk_scale;
  // INT4 keys enter the MFMA as code + 8: remove 8 * sum(q) from the scores
  // (small enough not to cost accuracy: 8 against codes up to 7)
  float kbias = 0.0f;
  if constexpr (FMT == 6) {
    float qs = 0.0f;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) qs += (float)qB[kk][e];
    qs += __shfl_xor(qs, 16);
    qs += __shfl_xor(qs, 32);
    kbias = 8.0f * qs;
  }
  WaveState<D> st;
#pragma unroll
  for (int nn = 0; nn < NV; ++nn) st.acc[nn] = float4_t{0.f, 0.f, 0.f, 0.f};
  st.m_run = kRefStart;
  st.l_run = 0.0f;

  // This wave's pages: p_begin + w + 4*j, j < n_it.  Their block-table
  // entries are fetched 64 at a time into one VGPR (lane j holds entry j) and
  // read with readlane, so no load sits between consecutive pages.  Units of
  // 16 tokens are double-buffered: the next unit's bytes are in flight while
  // the current one is computed.
  const LaneOffs lofs = lane_offsets<FMT, D>(gq, n, P);
  const int sp_shift = a.sp_shift;  // P / 16 == 1 << sp_shift
  const int sp_mask = (1 << sp_shift) - 1;
  const uint8_t* head_base = a.cache + (int64_t)kvh * a.geom.chunk_bytes;
  const int64_t page_stride = (int64_t)a.H * a.geom.chunk_bytes;

  // The split's block-table entries are staged in LDS, kPageChunk at a time,
  // by the whole workgroup; wave w then walks pages w, w+4, ... of the chunk.
  // Reading a page index from LDS involves no vector-memory counter, so it
  // never forces a wait on the data loads in flight.
  for (int c0 = p_begin; c0 < p_end; c0 += kPageChunk) {
    const int nc = min(kPageChunk, p_end - c0);  // <= first_cap for the first chunk
    static_assert(NT >= kPageChunk, "one block-table entry per thread and chunk");
    __syncthreads();
    if (tid < nc) {
      if (c0 == p_begin)  // uniform
        s_pages[tid] = bt_first;
      else
        s_pages[tid] = bt[c0 + tid];
    }
    __syncthreads();
    const int nj = w < nc ? (nc - w + W - 1) / W : 0;  // this wave's pages
    const int nu = nj << sp_shift;
    if (nu == 0) continue;
    // the unit count is padded to a whole number of ring turns; padded units
    // are masked out, so the loop body has no data-dependent branches
    const int nu_pad = (nu + kDepth - 1) / kDepth * kDepth;
    auto unit_page = [&](int u, bool& valid) {
      const int page = __builtin_amdgcn_readfirstlane(s_pages[w + W * (u >> sp_shift)]);
      valid = page >= 0 && page < a.num_pages;
      return head_base + (valid ? page : 0) * page_stride;
    };
    auto unit_tok0 = [&](int u) { return (c0 + w + W * (u >> sp_shift)) * P + (u & sp_mask) * 16; };

    // Units are prefetched kDepth-1 ahead into a ring of register buffers;
    // the loop is unrolled by kDepth so every ring slot is a fixed set of
    // registers.  There is no separate prologue: the ring starts zeroed and
    // the first kDepth-1 steps process masked placeholder units, so the only
    // loads pending at the loop header are the loop's own and the compiler
    // waits for exactly the unit about to be used.  Loads stay unconditional
    // (past the end they reload the last unit: in bounds, unused).
    Raw<FMT, D> rr[kDepth];
    bool vv[kDepth];
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      zero_raw(rr[k]);
      vv[k] = false;
    }
    for (int u = 0; u < nu_pad + kDepth; u += kDepth) {
#pragma unroll
      for (int k = 0; k < kDepth; ++k) {
        const int ul = min(u + k, nu - 1);      // unit loaded now
        const int up = u + k - (kDepth - 1);    // unit processed now
        const int ls = k;                        // its ring slots
        const int ps = (k + 1) % kDepth;
        load_unit<FMT, D>(unit_page(ul, vv[ls]), a.geom, ul & sp_mask, lofs, rr[ls]);
        const bool live = vv[ps] && up >= 0 && up < nu;
        process_unit<FMT, D, G>(rr[ps], live, unit_tok0(up < 0 ? 0 : up), ctx, n, gq, qB, kconst, kbias, st);
      }
    }
  }

  // ---- a decode step's new token: split 0 stores it and folds it into its
  // own partial
  __shared__ float s_new_lg[kMaxGroup];
  __shared__ float s_new_k[D], s_new_v[D];
  const bool fold_new = split == 0 && a.new_slots != nullptr;
  if (fold_new && w < 2) new_token_row<FMT, D, G>(a, b, kvh, w, l, attend_new, s_new_k, s_new_lg, s_new_v);

  // ---- combine the W waves (and the hi/lo rows) in LDS
  float l_tot = st.l_run + __shfl_xor(st.l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (gq == 0) {
    lds_m[w][n] = st.m_run;
    lds_l[w][n] = l_tot;
  }
#pragma unroll
  for (int nn = 0; nn < NV; ++nn)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * gq + i;
      if (row < 2 * G) lds_o[w][row][NV * n + nn] = st.acc[nn][i];
    }
  __syncthreads();

  const float post = (FMT == 1 || FMT == 4) ? a.v_scale : 1.0f;
  float* rec = partials + (((int64_t)b * a.H + kvh) * S + split) * rec_floats;
  for (int i = tid; i < G * D; i += NT) {
    const int g = i / D, d = i % D;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < W; ++ww) M = fmaxf(M, lds_m[ww][g]);
    float L = 0.0f, O = 0.0f;
    if (M != kNegInf) {
#pragma unroll
      for (int ww = 0; ww < W; ++ww) {
        const float f = exp2f(lds_m[ww][g] - M);
        L += f * lds_l[ww][g];
        const float o = lds_o[ww][g][d] + lds_o[ww][g + G][d];
        O += f * o;
      }
    }
    if (fold_new && attend_new) {
      // the new token as one more partial: m = its score, l = 1, o = its value row
      const float lg = s_new_lg[g];
      const float mc = fmaxf(M, lg);
      const float f = exp2f(lg - mc), sc = exp2f(M - mc);
      M = mc;
      L = L * sc + f;
      O = O * sc + f * s_new_v[d];
    }
    if (S == 1) {
      const float o = L > 0.0f ? O / L * post : 0.0f;
      a.out[((int64_t)b * a.Hq + kvh * G + g) * D + d] = __builtin_bit_cast(uint16_t, (half_t)o);
    } else {
      if (d == 0) {
        rec[g] = M;
        rec[kMaxGroup + g] = L;
      }
      rec[2 * kMaxGroup + g * D + d] = O;
    }
  }
}

// Merge of the context splits: m = max m_s, l = sum 2^(m_s - m) l_s,
// o = sum 2^(m_s - m) o_s / l.  A separate launch: the kernel boundary makes
// every split's partial visible on all XCDs without device-wide cache
// maintenance inside the split kernel (a count-and-merge by the split
// kernel's last workgroup measured slower than this launch: a device-scope
// release writes back the XCD's whole L2, and even with write-through record
// stores each workgroup waits for its stores and its count).  One thread per
// output element; every split's (m, l, o) is requested before any is used,
// 8 splits at a time, so the merge costs one memory round trip per 8 splits.
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a, int D, float post) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.B * a.Hq * D) return;
  const int d = (int)(idx % D);
  const int64_t bh = idx / D;
  const int hq = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  const int kvh = hq / a.G, g = hq - kvh * a.G;
  const int S = a.num_splits;
  const int64_t rf = ws_record_floats(D);
  const float* recs = reinterpret_cast<const float*>(a.workspace) + ((int64_t)b * a.H + kvh) * S * rf;
  float M = kNegInf, L = 0.0f, O = 0.0f;
  merge_splits(recs, rf, S, g, 2 * kMaxGroup + g * D + d, M, L, O);
  const float o = L > 0.0f ? O / L * post : 0.0f;
  a.out[idx] = __builtin_bit_cast(uint16_t, (half_t)o);
}

// Four-wave workgroups normally; eight waves when each (sequence, kv head)
// runs as a single workgroup that fills a compute unit by itself.
template <int FMT, int D, int G>
hipError_t launch_w(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  if (a.waves == 8)
    decode_kernel<FMT, D, G, 8><<<grid, 512, 0, s>>>(a);
  else
    decode_kernel<FMT, D, G, 4><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int FMT, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.num_splits, (unsigned)a.H, (unsigned)a.B);
  switch (a.G) {
    case 1: return launch_w<FMT, D, 1>(a, grid, s);
    case 2: return launch_w<FMT, D, 2>(a, grid, s);
    case 4: return launch_w<FMT, D, 4>(a, grid, s);
    case 8: return launch_w<FMT, D, 8>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const DecodeArgs& a, hipStream_t s) {
  switch (a.D) {
    case 32: return launch_d<FMT, 32>(a, s);
    case 64: return launch_d<FMT, 64>(a, s);
    case 128: return launch_d<FMT, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int FMT, int D, int G>
int occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&decode_kernel<FMT, D, G, 4>), 256,
                                                   0) != hipSuccess)
    return 0;
  return n;
}

template <int FMT, int D>
int occupancy_g(int G) {
  switch (G) {
    case 1: return occupancy<FMT, D, 1>();
    case 2: return occupancy<FMT, D, 2>();
    case 4: return occupancy<FMT, D, 4>();
    case 8: return occupancy<FMT, D, 8>();
  }
  return 0;
}

template <int FMT>
int occupancy_dg(int D, int G) {
  switch (D) {
    case 32: return occupancy_g<FMT, 32>(G);
    case 64: return occupancy_g<FMT, 64>(G);
    case 128: return occupancy_g<FMT, 128>(G);
  }
  return 0;
}

}  // namespace

int decode_blocks_per_cu(int fmt, int D, int G) {
  switch (fmt) {
    case 1: return occupancy_dg<1>(D, G);
    case 2: return occupancy_dg<2>(D, G);
    case 3: return occupancy_dg<3>(D, G);
    case 4: return occupancy_dg<4>(D, G);
    case 6: return occupancy_dg<6>(D, G);
    case 7: return occupancy_dg<7>(D, G);
  }
  return 0;
}

hipError_t launch_decode(int fmt, const DecodeArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  hipError_t e = hipErrorInvalidValue;
  switch (fmt) {
    case 1: e = launch_fmt<1>(a, s); break;
    case 2: e = launch_fmt<2>(a, s); break;
    case 3: e = launch_fmt<3>(a, s); break;
    case 4: e = launch_fmt<4>(a, s); break;
    case 6: e = launch_fmt<6>(a, s); break;
    case 7: e = launch_fmt<7>(a, s); break;
  }
  if (e != hipSuccess || a.num_splits == 1) return e;
  const float post = (fmt == 1 || fmt == 4) ? a.v_scale : 1.0f;
  const int64_t outs = (int64_t)a.B * a.Hq * a.D;
  decode_merge_kernel<<<dim3((unsigned)((outs + 255) / 256)), 256, 0, s>>>(a, a.D, post);
  return hipGetLastError();
}


}  // namespace kvq
