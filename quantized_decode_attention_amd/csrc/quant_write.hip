// quant_write.hip -- quantise-on-write for FP8 per-tensor, INT8 / FP8 / INT4
// per-token-head and NVFP4 (gfx950).
//
// Write path of [P5] "NVFP4 KV Cache：Blackwell 上的 4-bit 缓存量化",
// §KV 的写入与读取路径 (compute scales, round and clip, pack, write payload and
// scale metadata into the page) and of [P4] "KV 量化", §写和读 (divide by the
// scale, convert, keep the bits as bytes).
//
// Work mapping.  8-bit formats: one workgroup per (16 consecutive tokens, kv
// head); a run of tokens that fills one aligned 16-token group of a page is
// quantised by lanes of 16 values and written as contiguous 16-byte stores,
// any other slot pattern row by row (D/8 lanes of 8 values).  The 4-bit
// formats (NVFP4, MXFP4, INT4 per-token-head) use the same group / per-row
// split with one lane per 16 values.
// This file is built with -ffp-contract=off: every binary32 operation below
// rounds exactly as written.
#include "row_encode.h"

namespace kvq {
namespace {

constexpr int kBlock = 256;

// Whether tokens 16g .. 16g+15 fill one aligned 16-token group of a page, in
// order: then the group's K and V bytes are contiguous runs of the cache.
// Returns the group's first slot, or -1.  Uniform across the workgroup.
__device__ __forceinline__ int64_t group_slot(const WriteArgs& a, int64_t g, int* s_ok, int64_t* s_slot0) {
  const int tid = threadIdx.x;
  if (tid == 0) *s_ok = 1;
  __syncthreads();
  if (tid < 16) {
    const int64_t tok = 16 * g + tid;
    bool ok = tok < a.n_tok;
    int64_t sl = ok ? a.slots[tok] : -1;
    const int64_t s0 = ok ? a.slots[16 * g] : -1;
    ok = ok && s0 >= 0 && s0 < (int64_t)a.num_pages * a.P && (s0 & 15) == 0 && sl == s0 + tid;
    if (!ok) *s_ok = 0;
    if (tid == 0) *s_slot0 = s0;
  }
  __syncthreads();
  return *s_ok ? *s_slot0 : -1;
}

// One workgroup per (16 consecutive tokens, kv head): 128 lanes per side,
// lane (token s, chunk q) quantises channels 16q .. 16q+15 of token s.  When
// the 16 tokens fill one aligned page group (a prefill-style run) the codes
// are assembled in LDS in the cache's byte order and written as contiguous
// 16-byte stores; otherwise every row goes through the per-row path.
template <int FMT, int D>
__global__ __launch_bounds__(kBlock) void quant_write_8bit(WriteArgs a) {
  constexpr int GB = 16 * D;  // bytes of one 16-token group, one side
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[2][GB];
  __shared__ float s_scale[2][16];
  __shared__ int s_ok;
  __shared__ int64_t s_slot0;
  const int64_t g = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  constexpr int QPR = D / 16;               // lanes per token row
  constexpr int LPS = 16 * QPR;             // lanes per side
  const int side = tid / LPS;               // D = 128: 128 lanes per side
  const bool active = tid < 2 * LPS;
  const int lt = tid % LPS, sidx = lt / QPR, q = lt % QPR;
  // The group's inputs are requested before its slots are checked (they do
  // not depend on them), so the two round trips overlap.  A partial last
  // group never takes the contiguous path and loads nothing here.
  uint4 raw[2] = {};
  if (active && 16 * g + 16 <= a.n_tok) {
    const uint16_t* src = (side ? a.v : a.k) + ((16 * g + sidx) * a.H + h) * (int64_t)D + 16 * q;
    raw[0] = *reinterpret_cast<const uint4*>(src);
    raw[1] = *reinterpret_cast<const uint4*>(src + 8);
  }
  const int64_t slot0 = group_slot(a, g, &s_ok, &s_slot0);

  if (slot0 < 0) {
    // general slots: rows (side, token 16g + i, head h), D/8 lanes each
    constexpr int LPR = D / 8;
    for (int t = tid; t < 32 * LPR; t += kBlock) {
      const int rr = t / LPR, side = rr / 16, i = rr % 16;
      const int64_t tok = 16 * g + i;
      if (tok >= a.n_tok) continue;
      write_row_8bit<FMT, D>(a, (int64_t)side * a.n_tok * a.H + tok * a.H + h, t % LPR);
    }
    return;
  }

  if (active) {
    float x[16];
    halves8_to_f32(raw[0], x);
    halves8_to_f32(raw[1], x + 8);
    float s;
    if constexpr (FMT == 1) {
      s = side ? a.v_scale : a.k_scale;
    } else {
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
      s = row_scale<FMT>(group_max<QPR>(amax));
      if (q == 0) s_scale[side][sidx] = s;
    }
    const Recip rc = make_recip(s);
    uint8_t* dst = s_codes[side];
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = encode8x4<FMT>(x + 4 * k, s, rc);
    if (side == 0 && D >= 64) {
      // channels 16q .. 16q+15 of a key row are 16 consecutive bytes
      *reinterpret_cast<uint4*>(dst + k8_offset<D>(sidx, 16 * q)) = uint4{w[0], w[1], w[2], w[3]};
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = 16 * q + i;
        const int off = side == 0 ? (int)k8_offset<D>(sidx, d) : (int)v8_offset<D>(sidx, d);
        dst[off] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
      }
    }
  }
  __syncthreads();
  const int64_t page = slot0 / a.P;
  const int t0 = (int)(slot0 - page * a.P);
  uint8_t* chunk = a.cache + (page * a.H + h) * a.geom.chunk_bytes;
  for (int i = tid; i < 2 * GB / 16; i += kBlock) {
    const int sd = i / (GB / 16), o = 16 * (i % (GB / 16));
    uint8_t* base = chunk + (sd ? a.geom.v_codes : 0) + (int64_t)D * t0;
    *reinterpret_cast<uint4*>(base + o) = *reinterpret_cast<const uint4*>(&s_codes[sd][o]);
  }
  if (FMT != 1 && tid < 32) {
    float* sp = reinterpret_cast<float*>(chunk + a.geom.k_scales) + (tid / 16) * a.P + t0 + (tid % 16);
    *sp = s_scale[tid / 16][tid % 16];
  }
}

// One workgroup per (16 consecutive tokens, kv head), as for the 8-bit
// formats: an aligned run is assembled in LDS (K codes and V codes: one
// contiguous run each; NVFP4 / MXFP4 K block scales: one run, V block scales:
// one run of 16 bytes per block column; INT4: 16 fp32 scales per side) and
// written with 16-byte stores; other slot patterns go row by row.
template <int FMT, int D>
__global__ __launch_bounds__(kBlock) void quant_write_4bit(WriteArgs a) {
  constexpr int NB = D / 16;                      // 16-value lanes per row
  constexpr int NS = FMT == 7 ? D / 32 : D / 16;  // block-scale bytes per row
  constexpr int SL = FMT == 7 ? 2 : 1;            // lanes per block scale
  constexpr int CB = 16 * D / 2;                  // code bytes of 16 tokens, one side
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[2][CB];
  __shared__ __attribute__((aligned(16))) uint8_t s_sc[2][16 * NS];
  __shared__ float s_rs[2][16];
  __shared__ int s_ok;
  __shared__ int64_t s_slot0;
  const int64_t g = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  // lane (side, token s, block q); 2 * 16 * NB <= 256 lanes.  Inputs are
  // requested before the slot check, as for the 8-bit formats.
  const bool active = tid < 32 * NB;
  const int side = tid / (16 * NB), lt = tid % (16 * NB), sidx = lt / NB, q = lt % NB;
  uint4 raw[2] = {};
  if (active && 16 * g + 16 <= a.n_tok) {
    const uint16_t* src = (side ? a.v : a.k) + ((16 * g + sidx) * a.H + h) * (int64_t)D + 16 * q;
    raw[0] = *reinterpret_cast<const uint4*>(src);
    raw[1] = *reinterpret_cast<const uint4*>(src + 8);
  }
  const int64_t slot0 = group_slot(a, g, &s_ok, &s_slot0);

  if (slot0 < 0) {
    for (int t = tid; t < 32 * NB; t += kBlock) {
      const int rr = t / NB, side = rr / 16, i = rr % 16;
      const int64_t tok = 16 * g + i;
      if (tok >= a.n_tok) continue;
      write_row_4bit<FMT, D>(a, (int64_t)side * a.n_tok * a.H + tok * a.H + h, t % NB);
    }
    return;
  }

  if (active) {
    float x[16];
    halves8_to_f32(raw[0], x);
    halves8_to_f32(raw[1], x + 8);
    uint32_t byte[8];
    uint32_t sb = 0;
    if constexpr (FMT == 4) {
      sb = nvfp4_encode_block(x, side ? a.v_scale : a.k_scale, a.flags, byte);
    } else if constexpr (FMT == 7) {
      sb = mxfp4_encode_half(x, byte);
    } else {
      const float s = int4_encode_block<NB>(x, byte);
      if (q == 0) s_rs[side][sidx] = s;
    }
    const bool scale_lane = q % SL == 0;
    if (side == 0) {
      uint8_t* kp = s_codes[0] + sidx * (D / 2) + 8 * q;
#pragma unroll
      for (int i = 0; i < 8; ++i) kp[i] = (uint8_t)byte[i];
      if (scale_lane) s_sc[0][sidx * NS + q / SL] = (uint8_t)sb;
    } else {
      uint8_t* vp = s_codes[1] + 2 * D * (sidx / 4) + 32 * q + (sidx % 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) vp[4 * i] = (uint8_t)byte[i];
      if (scale_lane) s_sc[1][(q / SL) * 16 + sidx] = (uint8_t)sb;  // [block][token]
    }
  }
  __syncthreads();
  const int64_t page = slot0 / a.P;
  const int t0 = (int)(slot0 - page * a.P);
  uint8_t* chunk = a.cache + (page * a.H + h) * a.geom.chunk_bytes;
  for (int i = tid; i < 2 * CB / 16; i += kBlock) {
    const int sd = i / (CB / 16), o = 16 * (i % (CB / 16));
    uint8_t* base = chunk + (sd ? a.geom.v_codes : 0) + (int64_t)t0 * (D / 2);
    *reinterpret_cast<uint4*>(base + o) = *reinterpret_cast<const uint4*>(&s_codes[sd][o]);
  }
  if constexpr (FMT == 4 || FMT == 7) {
    // K block scales: 16 * NS contiguous bytes; V block scales: NS runs of 16
    if (tid < NS)
      *reinterpret_cast<uint4*>(chunk + a.geom.k_scales + (int64_t)t0 * NS + 16 * tid) =
          *reinterpret_cast<const uint4*>(&s_sc[0][16 * tid]);
    else if (tid < 2 * NS)
      *reinterpret_cast<uint4*>(chunk + a.geom.v_scales + (int64_t)(tid - NS) * a.P + t0) =
          *reinterpret_cast<const uint4*>(&s_sc[1][16 * (tid - NS)]);
  } else {
    if (tid < 32)
      reinterpret_cast<float*>(chunk + a.geom.k_scales)[(tid / 16) * a.P + t0 + (tid % 16)] =
          s_rs[tid / 16][tid % 16];
  }
}

// ---------------------------------------------------------------------------
// A decode step's new tokens, quantised and attended in the merge of the
// context splits (kvq_decode_attention_append).  The split kernel has read
// positions 0 .. ctx-2 of each sequence from the cache.  This kernel
// quantises the new token of every (sequence, kv head) with the per-row write
// path above, stores it into its slot, and adds it to each head's merge as
// one more partial: m = its score, l = 1, o = its dequantised value row.  The
// step then has no separate write launch ahead of the split kernel.
// ---------------------------------------------------------------------------

// Grid (ceil(G / HPW), H, B): workgroup x serves heads HPW*x .. of the kv
// head, one thread per output value.  Every workgroup quantises the new key
// and value rows (wave 0 and wave 1, D/8 or D/16 lanes); only x == 0 stores
// them.
template <int FMT, int D>
__global__ __launch_bounds__(256) void append_merge_kernel(WriteArgs wa, DecodeArgs a, float post) {
  constexpr bool K8 = FMT == 1 || FMT == 2 || FMT == 3;
  constexpr int VPL = K8 ? 8 : 16;  // values per lane
  constexpr int LPR = D / VPL;      // lanes per row
  constexpr int HPW = 256 / D;      // heads per workgroup
  constexpr bool PTH = FMT == 2 || FMT == 3 || FMT == 6;
  __shared__ float s_v[D];
  __shared__ float s_lg[HPW];

  const int kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.G, S = a.num_splits;
  const int g0 = blockIdx.x * HPW;
  const int g = g0 + tid / D, d = tid % D;
  const bool has_out = g < G;

  int ctx = a.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > a.max_pages * a.P ? a.max_pages * a.P : ctx);
  const int64_t slot = wa.slots[b];
  const bool attend = ctx >= 1 && slot >= 0 && slot < (int64_t)wa.num_pages * wa.P;

  // the splits' records are requested first, so their round trip overlaps
  // the quantisation
  const int64_t rf = ws_record_floats(D);
  const float* recs = reinterpret_cast<const float*>(a.workspace) + ((int64_t)b * a.H + kvh) * S * rf;
  const int gr = has_out ? g : g0;
  RecGroup r0;
  load_recs(recs, rf, S, 0, gr, 2 * kMaxGroup + gr * D + d, r0);

  if (wv < 2 && lane < LPR) {
    float qv[HPW][VPL];
    if (wv == 0) {
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        const int gh = g0 + h < G ? g0 + h : g0;
        const uint16_t* qp = a.q + ((int64_t)b * a.Hq + kvh * G + gh) * D + VPL * lane;
#pragma unroll
        for (int k = 0; k < VPL / 8; ++k) halves8_to_f32(*reinterpret_cast<const uint4*>(qp + 8 * k), qv[h] + 8 * k);
      }
    }
    RowCodes rc;
    const int64_t row = (int64_t)wv * wa.n_tok * wa.H + (int64_t)b * wa.H + kvh;
    if constexpr (K8)
      write_row_8bit<FMT, D>(wa, row, lane, blockIdx.x == 0, &rc);
    else
      write_row_4bit<FMT, D>(wa, row, lane, blockIdx.x == 0, &rc);
    if (attend) {
      float c[VPL];
      lane_values<FMT, VPL>(rc, c);
      const float rs = PTH ? rc.s : 1.0f;
      if (wv == 0) {
        const float kconst = (FMT == 1 || FMT == 4) ? a.k_scale * a.qk_scale : a.qk_scale;
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
          float part = 0.0f;
#pragma unroll
          for (int i = 0; i < VPL; ++i) part = __builtin_fmaf(qv[h][i], c[i], part);
          part = group_sum<LPR>(part);
          if (lane == 0) s_lg[h] = part * (rs * kconst);
        }
      } else {
#pragma unroll
        for (int i = 0; i < VPL; ++i) s_v[VPL * lane + i] = c[i] * rs;
      }
    }
  }
  __syncthreads();
  if (!has_out) return;

  float M = kNegInf, L = 0.0f, O = 0.0f;
  merge_recs(r0, M, L, O);
  for (int s0 = 8; s0 < S; s0 += 8) {
    RecGroup r;
    load_recs(recs, rf, S, s0, g, 2 * kMaxGroup + g * D + d, r);
    merge_recs(r, M, L, O);
  }
  if (attend) {
    const float lg = s_lg[g - g0];
    const float mc = fmaxf(M, lg);
    const float f = exp2f(lg - mc);
    const float sc = exp2f(M - mc);
    L = L * sc + f;
    O = O * sc + f * s_v[d];
  }
  const float o = L > 0.0f ? O / L * post : 0.0f;
  a.out[((int64_t)b * a.Hq + kvh * G + g) * D + d] = __builtin_bit_cast(uint16_t, (half_t)o);
}

template <int FMT>
hipError_t launch_append_merge_fmt(const WriteArgs& w, const DecodeArgs& a, hipStream_t s) {
  const float post = (FMT == 1 || FMT == 4) ? a.v_scale : 1.0f;
  const int hpw = 256 / a.D;
  const dim3 grid((unsigned)((a.G + hpw - 1) / hpw), (unsigned)a.H, (unsigned)a.B);
  switch (a.D) {
    case 32: append_merge_kernel<FMT, 32><<<grid, 256, 0, s>>>(w, a, post); break;
    case 64: append_merge_kernel<FMT, 64><<<grid, 256, 0, s>>>(w, a, post); break;
    case 128: append_merge_kernel<FMT, 128><<<grid, 256, 0, s>>>(w, a, post); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const WriteArgs& a, hipStream_t s) {
  if (a.n_tok == 0) return hipSuccess;
  const int64_t groups = (a.n_tok + 15) / 16;
  if (groups > 0x7FFFFFFF || a.H > 65535) return hipErrorInvalidValue;
  const dim3 g2((unsigned)groups, (unsigned)a.H);
  if constexpr (FMT == 4 || FMT == 6 || FMT == 7) {
    switch (a.D) {
      case 32: quant_write_4bit<FMT, 32><<<g2, kBlock, 0, s>>>(a); break;
      case 64: quant_write_4bit<FMT, 64><<<g2, kBlock, 0, s>>>(a); break;
      case 128: quant_write_4bit<FMT, 128><<<g2, kBlock, 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.D) {
      case 32: quant_write_8bit<FMT, 32><<<g2, kBlock, 0, s>>>(a); break;
      case 64: quant_write_8bit<FMT, 64><<<g2, kBlock, 0, s>>>(a); break;
      case 128: quant_write_8bit<FMT, 128><<<g2, kBlock, 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append_merge(int fmt, const WriteArgs& w, const DecodeArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  switch (fmt) {
    case 1: return launch_append_merge_fmt<1>(w, a, s);
    case 2: return launch_append_merge_fmt<2>(w, a, s);
    case 3: return launch_append_merge_fmt<3>(w, a, s);
    case 4: return launch_append_merge_fmt<4>(w, a, s);
    case 6: return launch_append_merge_fmt<6>(w, a, s);
    case 7: return launch_append_merge_fmt<7>(w, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_quant_write(int fmt, const WriteArgs& a, hipStream_t s) {
  switch (fmt) {
    case 1: return launch_fmt<1>(a, s);
    case 2: return launch_fmt<2>(a, s);
    case 3: return launch_fmt<3>(a, s);
    case 4: return launch_fmt<4>(a, s);
    case 6: return launch_fmt<6>(a, s);
    case 7: return launch_fmt<7>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
