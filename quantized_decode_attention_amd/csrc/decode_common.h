// decode_common.h -- pieces shared by the decode kernels (gfx950): operand
// packing, streaming loads, lane shifts and the lazy-rescaling constants.
#pragma once

#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr int kWaves = 4;          // wavefronts per KVarN decode workgroup
constexpr int kPageChunk = 256;    // block-table entries staged in LDS at a time
constexpr float kNegInf = -INFINITY;

// Lazy rescaling: the weights P = 2^(score - m_run) * v_scale fed to the PV
// product are kept relative to a reference m_run that only moves when some
// weight would exceed 2^kTau, so the accumulators are rescaled a handful of
// times per split instead of every time the running maximum creeps up, and
// the common path needs no cross-lane maximum.  P <= 2^kTau keeps the binary16
// operands far from overflow.
constexpr float kTau = 8.0f;
constexpr float kTauPow = 256.0f;

// Starting reference of the running maximum: finite and far below any score
// (log2 units; scores of binary16 data stay below 2^40 in magnitude), so the
// first live score always triggers a rescale (its weight overflows to +inf,
// alpha = 2^(kRefStart - m) = 0) while masked scores (-inf) give weight 0.
constexpr float kRefStart = -0x1p100f;

__device__ __forceinline__ half8_t cat(half2_t a, half2_t b, half2_t c, half2_t d) {
  half8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ half4_t cat4(half2_t a, half2_t b) {
  half4_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  return r;
}

// Buffer resource of one (page, kv head) chunk: base and size live in scalar
// registers and a lane's load adds only its 32-bit byte offset, so no vector
// address arithmetic runs per load; a load past the chunk's size returns 0.
// Word 3 selects the raw 32-bit data format of CDNA buffer loads.
constexpr int kRsrcWord3 = 0x00020000;
// The cache is streamed once per decode step: nontemporal loads keep it from
// displacing reusable lines and measure ~8% faster than plain loads on MI355X.
constexpr int kLoadNt = 2;  // cache policy bits of the streaming loads: nontemporal
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const uint8_t* chunk, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(chunk), 0, (int)bytes, kRsrcWord3);
}
// N dwords (N = 1, 2 or a multiple of 4) at byte voff + soff of the chunk
template <int N>
__device__ __forceinline__ void buf_dwords(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff, uint32_t* w) {
  if constexpr (N == 1) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, kLoadNt);
  } else if constexpr (N == 2) {
    const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, kLoadNt);
    w[0] = x.x, w[1] = x.y;
  } else {
    static_assert(N % 4 == 0, "dword count");
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16 * i, soff, kLoadNt);
      w[4 * i] = x.x, w[4 * i + 1] = x.y, w[4 * i + 2] = x.z, w[4 * i + 3] = x.w;
    }
  }
}
__device__ __forceinline__ float4 buf_f4(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff) {
  const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kLoadNt);
  return float4{__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w)};
}

// Lane l receives lane l+G's value (within its 16-lane row): row_shl:G.
template <int G>
__device__ __forceinline__ uint32_t row_shl(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, 0x100 + G, 0xF, 0xF, false);
}

// Products x0 = a0 b0 and x1 = a1 b1 as binary16 pairs: h = (RN16 x0, RN16 x1)
// and the remainders r = (RN16(x0 - h0), RN16(x1 - h1)).  Each value is one
// mixed-precision fused multiply-add (binary32 inputs, binary16 result, the
// remainder's subtrahend read straight from h's half), four instructions per
// pair.
__device__ __forceinline__ void split_products(float a0, float b0, float a1, float b1, uint32_t& h, uint32_t& r) {
  asm("v_fma_mixlo_f16 %0, %2, %3, 0\n\t"
      "v_fma_mixhi_f16 %0, %4, %5, 0\n\t"
      "v_fma_mixlo_f16 %1, %2, %3, -%0 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %1, %4, %5, -%0 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
      : "=&v"(h), "=&v"(r)
      : "v"(a0), "v"(b0), "v"(a1), "v"(b1));
}

// P's MFMA A operand: rows 0..G-1 keep their own binary16 high halves, rows
// G..2G-1 take the remainders of rows 0..G-1 (one DPP move per register; rows
// past 2G hold values that no output row uses).
template <int G>
__device__ __forceinline__ uint32_t hi_lo_rows(uint32_t hi, uint32_t lo) {
  return __builtin_amdgcn_update_dpp(hi, lo, 0x110 + G, 0xF, 0xF, false);
}

// Whether a binary16 pair of non-negative weights P * v_scale, held in two
// registers, has a value above kTauPow.  Non-negative binary16 numbers order
// like their bit patterns (+inf, past the binary16 range, above every finite
// one; a NaN above +inf), so a saturating subtraction of kTauPow's pattern
// from the larger halves leaves a nonzero half exactly where one exceeds it.
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));
constexpr uint16_t kTauPowBits = 0x5C00;  // binary16 2^8
static_assert(kTauPow == 256.0f, "binary16 pattern of the weight bound");
__device__ __forceinline__ bool pairs_exceed_tau(uint32_t a, uint32_t b) {
  const u16x2_t m = __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a), __builtin_bit_cast(u16x2_t, b));
  const u16x2_t x = __builtin_elementwise_sub_sat(m, u16x2_t{kTauPowBits, kTauPowBits});
  return __builtin_bit_cast(uint32_t, x) != 0u;
}

// Online merge of split partial records into (M, L, O) for one output
// element: record s holds m at float g, l at kMaxGroup + g and the output row
// value at o_off.  Splits are read 8 at a time, all loads of a group issued
// before any is used; empty splits have m = -inf and contribute nothing.
struct RecGroup {
  float m[8], l[8], o[8];
};

// Loads of splits s0 .. s0+7.  Splits past S reread split 0 (in bounds) and
// are dropped by their max; every load is unconditional, so all of them are
// in flight before the first use.
__device__ __forceinline__ void load_recs(const float* recs, int64_t rf, int S, int s0, int g, int64_t o_off,
                                          RecGroup& r) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const bool in = s0 + k < S;
    const float* rec = recs + (int64_t)(in ? s0 + k : 0) * rf;
    const float mv = rec[g];
    r.m[k] = in ? mv : kNegInf;
    r.l[k] = rec[kMaxGroup + g];
    r.o[k] = rec[o_off];
  }
}

__device__ __forceinline__ void merge_recs(const RecGroup& r, float& M, float& L, float& O) {
  float mc = M;
#pragma unroll
  for (int k = 0; k < 8; ++k) mc = fmaxf(mc, r.m[k]);
  // No branch on an all-empty group (a branch would let the compiler sink
  // the l and o loads below it, a second round trip): with every m = -inf
  // any finite reference gives weights 0, and an empty split's l and o are
  // 0, so (L, O) stay (0, 0).
  const float mr = mc == kNegInf ? 0.0f : mc;
  const float sc = exp2f(M - mr);
  L *= sc;
  O *= sc;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float f = exp2f(r.m[k] - mr);
    L += f * r.l[k];
    O += f * r.o[k];
  }
  M = mc;
}

__device__ __forceinline__ void merge_splits(const float* recs, int64_t rf, int S, int g, int64_t o_off,
                                             float& M, float& L, float& O) {
  if (S > 8 && S <= 16) {  // uniform: both groups' loads in flight at once, one round trip
    RecGroup r0, r1;
    load_recs(recs, rf, S, 0, g, o_off, r0);
    load_recs(recs, rf, S, 8, g, o_off, r1);
    merge_recs(r0, M, L, O);
    merge_recs(r1, M, L, O);
    return;
  }
  for (int s0 = 0; s0 < S; s0 += 8) {
    RecGroup r;
    load_recs(recs, rf, S, s0, g, o_off, r);
    merge_recs(r, M, L, O);
  }
}

}  // namespace kvq
