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
