// kvarn_write.hip -- KVarN k4v2 g128 tile quantisation on write (gfx950).
//
// [P2] "KVarN：华为推出的原生 vLLM KV-cache 量化后端", §技术原理: a tile of 128
// tokens of one kv head goes through four stages -- the raw tile, a Hadamard
// rotation along the channels, alternating normalisation of the token and
// channel deviations, and asymmetric round-to-nearest with the scales folded
// back (keys per channel, values per token).  Readings taken where the page
// is silent (the library's documented contract):
//   * rotation: 128-point Sylvester Walsh-Hadamard butterflies (a, b) ->
//     (a + b, a - b) on pairs (j, j + h), j & h = 0, h = 1, 2, ..., 64, then
//     one multiplication by RN(1/sqrt(128));
//   * normalisation: 4 sweeps, each a pass over the token rows followed by a
//     pass over the channel columns; a pass multiplies a row (column) by
//     RN(1 / sigma), sigma its population standard deviation (mean and mean
//     square by a balanced pairwise sum, 1/128 applied exactly), and the
//     row's (column's) running factor by sigma -- the page's log-domain
//     update, subtracting log sigma, in the linear domain with one rounding
//     of the reciprocal; a zero or non-finite deviation counts as 1;
//   * quantisation: zero = group minimum, step = (max - min) / (2^bits - 1),
//     code = clip(rne((y - min) / step), 0, 2^bits - 1), all-equal groups
//     give code 0; keys 4 bits per channel over the tile's tokens, values 2
//     bits per token over the channels;
//   * metadata (binary32): keys alpha_j = c_j s_j, beta_j = c_j m_j,
//     rho_t = r_t; values alpha_t = r_t s_t, beta_t = r_t m_t, gamma_j = c_j.
// All binary32 arithmetic rounds exactly as written (no contraction;
// correctly rounded square root, reciprocal and quantiser division; the
// rotation's fma(+-1, b, a) rounds exactly as a +- b), so the codes and
// metadata are a deterministic function of the binary16 input.
//
// Mapping.  One workgroup of 512 threads (8 wavefronts) per (tile, kv head,
// side).  The tile lives in LDS as binary32 with rows padded to 129 words.
// Lanes l, l + 16, l + 32 and l + 48 of wavefront w share index
// i = 16 w + (l & 15); quarter q = (l >> 4) & 3 holds elements
// [32 q, 32 q + 32) of token row i in a token pass and of channel column i
// in a channel pass.  A 128-value sum is the canonical tree
// (S0 + S1) + (S2 + S3) of its quarters' sums: each lane sums its quarter in
// registers, v_permlane16_swap and then v_permlane32_swap hand the partial
// sums across, with no LDS round trip or barrier.  Quarters 1 and 2 keep
// their values rotated by 16 in their registers.  That leaves every sum
// unchanged (it swaps the two 16-value subtrees of the quarter's tree, and
// binary32 addition commutes) and puts a row's four quarters 0, 48, 16 and 32
// banks apart (mod 64), so row and column accesses are free of LDS bank
// conflicts.  Two workgroups fit the LDS of a compute unit: 16 wavefronts,
// four per SIMD.
#include "kvq.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int N = 128;
constexpr int LDP = 129;  // padded LDS row (words)
constexpr int kSweeps = 4;
constexpr float kInvSqrt128 = (float)0.088388347648318440550;  // RN(1/sqrt(128))

// Chunk byte offsets (P = D = 128): K codes [128][64], V codes [32][128],
// then binary32 metadata K alpha, K beta, K rho, V alpha, V beta, V gamma.
constexpr int kVCodes = 128 * 64;
constexpr int kMeta = kVCodes + 128 * 32;
constexpr int kTileBytes = kMeta + 4 * 6 * 128;  // 15360; a page of P tokens holds P / 128 tiles
static_assert(kTileBytes == 15360, "KVarN tile size");

constexpr int kThreads = 512;
constexpr int Q = N / 4;  // values per lane and pass: a quarter of a row or column

// Balanced pairwise sum of 32 values in index order (one quarter of the
// canonical 128-value tree).
__device__ __forceinline__ float tree_sum32(const float (&v)[Q]) {
  float t[Q / 2];
#pragma unroll
  for (int i = 0; i < Q / 2; ++i) t[i] = v[2 * i] + v[2 * i + 1];
#pragma unroll
  for (int w = Q / 4; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = t[2 * i] + t[2 * i + 1];
  return t[0];
}

// The four quarters' partial values p0..p3 of one row or column, held by
// lanes l, l + 16, l + 32 and l + 48, combined as op(op(p0, p1), op(p2, p3))
// -- the top two levels of the canonical tree -- in all four lanes.
template <class Op>
__device__ __forceinline__ float combine4(float v, Op op) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float pair = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

struct Add {
  __device__ float operator()(float a, float b) const { return a + b; }
};
struct Min {
  __device__ float operator()(float a, float b) const { return fminf(a, b); }
};
struct Max {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

// Quarters 1 and 2 keep their 32 values rotated by 16 in their lane's
// registers (register j holds element (j + 16) mod 32 of the quarter);
// quarters 0 and 3 keep them in order.
__device__ __forceinline__ int rho(int q) { return 16 * ((q ^ (q >> 1)) & 1); }
// Column within the row (row within the column) of register j of quarter q.
__device__ __forceinline__ int pos(int j, int q) { return j < 16 ? 32 * q + j + rho(q) : 32 * q + j - rho(q); }

// Population standard deviation of 128 values (this lane's quarter v and
// the three partner lanes'); a zero or non-finite result becomes 1.
__device__ __forceinline__ float deviation(const float (&v)[Q]) {
  const float mean = combine4(tree_sum32(v), Add{}) * 0.0078125f;
  float sq[Q];
#pragma unroll
  for (int k = 0; k < Q; ++k) {
    const float d = v[k] - mean;
    sq[k] = d * d;
  }
  float sd = __builtin_sqrtf(combine4(tree_sum32(sq), Add{}) * 0.0078125f);
  if (!(sd > 0.0f) || !__builtin_isfinite(sd)) sd = 1.0f;
  return sd;
}

// Scale the 128 values by RN(1 / deviation) (one rounding of the reciprocal,
// one of each product; the sign of zero carries through the product);
// returns the deviation.
__device__ __forceinline__ float normalise(float (&v)[Q]) {
  const float sd = deviation(v);
  const float inv = 1.0f / sd;
#pragma unroll
  for (int k = 0; k < Q; ++k) v[k] = v[k] * inv;
  return sd;
}

// Butterfly stages h = 1 .. 16 of the rotation on this lane's quarter.
// Stages below 16 stay inside each 16-value block, so a rotated quarter's
// order does not matter to them; stage 16 puts each pair's sum and
// difference at the registers of their own elements.  a +- b is formed as
// fma(+-1, b, a): the product is exact, so the one rounding is that of the
// sum or difference, signed zeros included.
__device__ __forceinline__ void rotate_quarter(float (&y)[Q], bool rotated) {
#pragma unroll
  for (int h = 1; h < Q / 2; h <<= 1)
#pragma unroll
    for (int j = 0; j < Q; ++j)
      if ((j & h) == 0) {
        const float p = y[j], q = y[j + h];
        y[j] = p + q;
        y[j + h] = p - q;
      }
  // in order: register j holds element j, register j + 16 element j + 16
  // (sum to j, difference to j + 16); rotated: the reverse
  const float sg = rotated ? -1.0f : 1.0f;
#pragma unroll
  for (int j = 0; j < Q / 2; ++j) {
    const float u = rotated ? y[j + Q / 2] : y[j];  // element j
    const float v = rotated ? y[j] : y[j + Q / 2];  // element j + 16
    y[j] = __builtin_fmaf(sg, v, u);
    y[j + Q / 2] = __builtin_fmaf(-sg, v, u);
  }
}

// Asymmetric round-to-nearest of one group of 128 values (this lane's
// quarter and the partner lanes') into LEVELS + 1 codes; register j's code
// goes to LDS byte codes[stride * pos(j, q)].  Returns the step; *mn_out
// receives the zero point.
template <int LEVELS>
__device__ __forceinline__ float quantise_group(const float (&y)[Q], uint8_t* codes, int stride, int q,
                                                float* mn_out) {
  float mn = y[0], mx = y[0];
#pragma unroll
  for (int k = 1; k < Q; ++k) {
    mn = fminf(mn, y[k]);
    mx = fmaxf(mx, y[k]);
  }
  mn = combine4(mn, Min{});
  mx = combine4(mx, Max{});
  const float s = (mx - mn) / (float)LEVELS;
  // A zero step (all values equal, or a range so small that range / LEVELS
  // rounds to zero) gives code 0 throughout; dividing by 1 instead does that
  // with no select per value, since every y - mn is then below 1/2.
  const float sdiv = s != 0.0f ? s : 1.0f;
  const Recip rc = make_recip(sdiv);
  // clip(rne(.), 0, LEVELS): the clamp first (integer bounds, so it commutes
  // with the rounding), then adding 1.5 * 2^23 rounds to an integer with ties
  // to even and leaves it in the sum's low mantissa bits
#pragma unroll
  for (int k = 0; k < Q; ++k) {
    const float yc = __builtin_amdgcn_fmed3f(div_rn(y[k] - mn, sdiv, rc), 0.0f, (float)LEVELS);
    codes[stride * pos(k, q)] = (uint8_t)__float_as_uint(yc + 12582912.0f);
  }
  *mn_out = mn;
  return s;
}

// One tile-head side, by the 512 threads of a workgroup: token rows at
// src + t * row_stride (binary16), codes and metadata into chunk.  `tile`
// holds N * LDP floats of LDS.
__device__ __forceinline__ void kvarn_tile(const uint16_t* src, int64_t row_stride, uint8_t* chunk, int side,
                                           float* tile) {
  uint8_t* cb = reinterpret_cast<uint8_t*>(tile);  // codes [token][channel], after the last pass
  const int t = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int q = (t >> 4) & 3;        // quarter: elements [32 q, 32 q + 32)
  const int i = 16 * wv + (t & 15);  // token row / channel column

  // stage 1: the tile, binary16 -> binary32 (exact), coalesced 16-byte loads
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int p = t + kThreads * k, row = p >> 4, c8 = (p & 15) * 8;
    const half8_t x = *reinterpret_cast<const half8_t*>(src + row * row_stride + c8);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[row * LDP + c8 + e] = (float)x[e];
  }
  __syncthreads();

  float y[Q];
  float r = 1.0f, c = 1.0f;  // running token factor r_i, channel factor c_i
#pragma unroll 1
  for (int it = 0; it < kSweeps; ++it) {
    // token pass (token row i, this quarter); stage 2 on the first visit
#pragma unroll
    for (int j = 0; j < Q; ++j) y[j] = tile[i * LDP + pos(j, q)];
    if (it == 0) {
      // stages h = 1 .. 16 in registers; stages 32 and 64 across the
      // quarters through the tile: with a0..a3 the elements e, e + 32,
      // e + 64, e + 96 after stage 16, quarter k takes
      // (a0 +- a1) +- (a2 +- a3), the inner sign minus for odd k, the outer
      // for k >= 2, each as fma(+-1, b, a)
      rotate_quarter(y, rho(q) != 0);
#pragma unroll
      for (int j = 0; j < Q; ++j) tile[i * LDP + pos(j, q)] = y[j];
      __syncthreads();
      const float s1 = (q & 1) ? -1.0f : 1.0f, s2 = (q & 2) ? -1.0f : 1.0f;
#pragma unroll
      for (int j = 0; j < Q; ++j) {
        const float* a = tile + i * LDP + (pos(j, q) - 32 * q);
        const float lower = __builtin_fmaf(s1, a[32], a[0]);
        const float upper = __builtin_fmaf(s1, a[96], a[64]);
        y[j] = __builtin_fmaf(s2, upper, lower) * kInvSqrt128;
      }
      __syncthreads();  // every quarter has read the others' values
    }
    r = r * normalise(y);
#pragma unroll
    for (int j = 0; j < Q; ++j) tile[i * LDP + pos(j, q)] = y[j];
    __syncthreads();
    // channel pass (channel column i, this quarter)
#pragma unroll
    for (int k = 0; k < Q; ++k) y[k] = tile[pos(k, q) * LDP + i];
    c = c * normalise(y);
    if (it + 1 < kSweeps) {
#pragma unroll
      for (int k = 0; k < Q; ++k) tile[pos(k, q) * LDP + i] = y[k];
      __syncthreads();
    }
  }

  float* meta = reinterpret_cast<float*>(chunk + kMeta) + side * 3 * N;
  if (side == 0) {
    // keys: 4-bit codes per channel over the tile's tokens
    __syncthreads();  // every column has been read: the tile memory is free
    float mn;
    const float s = quantise_group<15>(y, cb + i, N, q, &mn);
    if (q == 0) {
      meta[i] = c * s;
      meta[N + i] = c * mn;
      meta[2 * N + i] = r;
    }
    __syncthreads();
    // pack: output byte t*64 + j/2 holds channel j (low nibble) and j+1
    {
      const int o0 = 16 * t;
      const uint32_t* w = reinterpret_cast<const uint32_t*>(cb + (o0 >> 6) * N + 2 * (o0 & 63));
      uint32_t out[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t x0 = w[2 * m] | (w[2 * m] >> 4);
        const uint32_t x1 = w[2 * m + 1] | (w[2 * m + 1] >> 4);
        out[m] = __builtin_amdgcn_perm(x1, x0, 0x06040200u);
      }
      *reinterpret_cast<uint4*>(chunk + o0) = uint4{out[0], out[1], out[2], out[3]};
    }
  } else {
    // values: back to token rows, 2-bit codes per token over the channels
#pragma unroll
    for (int k = 0; k < Q; ++k) tile[pos(k, q) * LDP + i] = y[k];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < Q; ++j) y[j] = tile[i * LDP + pos(j, q)];
    __syncthreads();  // every row has been read: the tile memory is free
    float mn;
    const float s = quantise_group<3>(y, cb + i * N, 1, q, &mn);
    if (q == 0) {
      meta[i] = r * s;
      meta[N + i] = r * mn;
      meta[2 * N + i] = c;
    }
    __syncthreads();
    // pack: output byte 128*(t/4) + j holds token 4*(t/4) + k in bits 2k..2k+1
    if (t < 256) {
      const int o0 = 16 * t;
      const int quad = o0 >> 7, j0 = o0 & 127;
      uint32_t out[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t v = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          v |= *reinterpret_cast<const uint32_t*>(cb + (4 * quad + k) * N + j0 + 4 * m) << (2 * k);
        out[m] = v;
      }
      *reinterpret_cast<uint4*>(chunk + kVCodes + o0) = uint4{out[0], out[1], out[2], out[3]};
    }
  }
}

constexpr int kLdsFloats = N * LDP;

// Contract violations found in device-resident arguments (KVQ_DEVERR_* bits of
// kvq.h), one word per device: raised with a vector atomic OR, read and
// cleared by kvq_take_device_errors.
__device__ uint32_t g_device_errors;

__device__ __forceinline__ void raise_error(uint32_t bit) { atomicOr(&g_device_errors, bit); }

__global__ __launch_bounds__(kThreads) void kvarn_write_kernel(WriteArgs a) {
  __shared__ float lds[kLdsFloats];
  const int ti = blockIdx.x, h = blockIdx.y, side = blockIdx.z;
  // The run's first slot places the tile: one outside the pool skips it (as
  // for every format), and otherwise all 128 slots must be that tile of its
  // page, in order.  A run that is not is skipped and reported.
  const int64_t s0 = a.slots[(int64_t)ti * N];
  if (s0 < 0) return;
  const int tid = threadIdx.x;
  const bool bad_slot = tid < N && a.slots[(int64_t)ti * N + tid] != s0 + tid;
  if (s0 >= (int64_t)a.num_pages * a.P) return;  // outside the pool: skipped, as for every format
  if (__syncthreads_or(bad_slot || s0 % N != 0)) {
    if (tid == 0 && h == 0 && side == 0) raise_error(KVQ_DEVERR_KVARN_TILE_SLOTS);
    return;
  }
  const int64_t page = s0 / a.P;
  uint8_t* chunk = a.cache + (page * a.H + h) * a.geom.chunk_bytes + (s0 - page * a.P) / N * kTileBytes;
  const uint16_t* src = (side ? a.v : a.k) + ((int64_t)ti * N * a.H + h) * N;
  kvarn_tile(src, (int64_t)a.H * N, chunk, side, lds);
}

// Incremental path ([P2] §配置与部署: the decode keeps the not yet quantised
// tokens of the last tile in a small fixed buffer).  Append: token i goes to
// row pos[i] % 128 of its sequence's binary16 tail.
__global__ __launch_bounds__(64) void kvarn_append_kernel(KvarnAppendArgs a) {
  const int64_t i = blockIdx.x;  // token
  const int hs = blockIdx.y;     // head * 2 + side
  const int h = hs >> 1, side = hs & 1;
  const int b = a.seq[i], pos = a.pos[i];
  if (b < 0 || b >= a.batch || pos < 0) return;
  if (hs == 0) {
    // the call's other tokens of this sequence must share this token's tile
    // and not its position (rows of the tail would be overwritten before the
    // tile is quantised); a violation is reported, not repaired
    bool bad = false;
    for (int64_t j = threadIdx.x; j < a.n_tok; j += 64)
      bad |= j != i && a.seq[j] == b && a.pos[j] >= 0 && ((a.pos[j] >> 7) != (pos >> 7) || a.pos[j] == pos);
    if (__builtin_amdgcn_ballot_w64(bad) != 0 && threadIdx.x == 0) raise_error(KVQ_DEVERR_KVARN_APPEND_SPAN);
  }
  const uint16_t* src = (side ? a.v : a.k) + (i * a.H + h) * N;
  uint16_t* dst = a.tail + ((((int64_t)b * 2 + side) * a.H + h) * N + (pos & (N - 1))) * N;
  if (threadIdx.x < N / 8)
    reinterpret_cast<uint4*>(dst)[threadIdx.x] = reinterpret_cast<const uint4*>(src)[threadIdx.x];
}

// Tile completion: a token at position 127 mod 128 completes its sequence's
// tile, which is quantised from the tail into the page of that tile.
__global__ __launch_bounds__(kThreads) void kvarn_complete_kernel(KvarnAppendArgs a) {
  __shared__ float lds[kLdsFloats];
  const int64_t i = blockIdx.x;
  const int h = blockIdx.y, side = blockIdx.z;
  const int b = a.seq[i], pos = a.pos[i];
  if (b < 0 || b >= a.batch || pos < 0 || (pos & (N - 1)) != N - 1) return;
  const int ti = pos / N;  // tile index in the sequence
  const int tpp = a.P / N;  // tiles per page
  if (ti / tpp >= a.max_pages) return;
  const int page = a.block_tables[(int64_t)b * a.max_pages + ti / tpp];
  if (page < 0 || page >= a.num_pages) return;
  uint8_t* chunk = a.cache + ((int64_t)page * a.H + h) * a.chunk_bytes + (ti % tpp) * kTileBytes;
  const uint16_t* src = a.tail + (((int64_t)b * 2 + side) * a.H + h) * N * N;
  kvarn_tile(src, N, chunk, side, lds);
}

}  // namespace

hipError_t take_device_errors(uint32_t* flags) {
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_device_errors));
  if (e != hipSuccess) return e;
  uint32_t v = 0;
  if ((e = hipMemcpy(&v, p, sizeof v, hipMemcpyDeviceToHost)) != hipSuccess) return e;
  const uint32_t zero = 0;
  if ((e = hipMemcpy(p, &zero, sizeof zero, hipMemcpyHostToDevice)) != hipSuccess) return e;
  *flags = v;
  return hipSuccess;
}

hipError_t launch_kvarn_write(const WriteArgs& a, hipStream_t s) {
  const int64_t tiles = a.n_tok / N;
  if (tiles == 0) return hipSuccess;
  if (tiles > 0x7FFFFFFF || a.H > 65535) return hipErrorInvalidValue;
  kvarn_write_kernel<<<dim3((unsigned)tiles, (unsigned)a.H, 2u), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_kvarn_append(const KvarnAppendArgs& a, hipStream_t s) {
  if (a.n_tok == 0) return hipSuccess;
  if (a.n_tok > 0x7FFFFFFF || a.H > 32767) return hipErrorInvalidValue;
  kvarn_append_kernel<<<dim3((unsigned)a.n_tok, (unsigned)(2 * a.H)), 64, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  kvarn_complete_kernel<<<dim3((unsigned)a.n_tok, (unsigned)a.H, 2u), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvq
