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
//     pass over the channel columns; a pass divides a row (column) by its
//     population standard deviation (mean and mean square by a balanced
//     pairwise sum, 1/128 applied exactly) and multiplies the row's (column's)
//     running factor by it; a zero or non-finite deviation counts as 1;
//   * quantisation: zero = group minimum, step = (max - min) / (2^bits - 1),
//     code = clip(rne((y - min) / step), 0, 2^bits - 1), all-equal groups
//     give code 0; keys 4 bits per channel over the tile's tokens, values 2
//     bits per token over the channels;
//   * metadata (binary32): keys alpha_j = c_j s_j, beta_j = c_j m_j,
//     rho_t = r_t; values alpha_t = r_t s_t, beta_t = r_t m_t, gamma_j = c_j.
// All binary32 arithmetic rounds exactly as written (no contraction,
// correctly rounded division and square root), so the codes and metadata are
// a deterministic function of the binary16 input.
//
// Mapping.  One workgroup of 128 threads per (tile, kv head, side).  The tile
// lives in LDS as binary32 with rows padded to 129 words; in a token pass
// thread t holds token row t in registers, in a channel pass thread t holds
// channel column t, so every sum and every division is in-thread and in the
// canonical order, and both access patterns are free of bank conflicts.
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

// Balanced pairwise sum of 128 values in index order.
__device__ __forceinline__ float tree_sum(const float (&v)[N]) {
  float t[N / 2];
#pragma unroll
  for (int i = 0; i < N / 2; ++i) t[i] = v[2 * i] + v[2 * i + 1];
#pragma unroll
  for (int w = N / 4; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = t[2 * i] + t[2 * i + 1];
  return t[0];
}

// Population standard deviation; a zero or non-finite result becomes 1.
__device__ __forceinline__ float deviation(const float (&v)[N]) {
  const float mean = tree_sum(v) * 0.0078125f;
  float sq[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float d = v[i] - mean;
    sq[i] = d * d;
  }
  float sd = __builtin_sqrtf(tree_sum(sq) * 0.0078125f);
  if (!(sd > 0.0f) || !__builtin_isfinite(sd)) sd = 1.0f;
  return sd;
}

// x / s correctly rounded, zero kept with its sign.
__device__ __forceinline__ float div_rn_z(float x, float s, Recip r) {
  const float q = div_rn(x, s, r);
  return x == 0.0f ? x : q;
}

// Divide the 128 values by their deviation; returns the deviation.
__device__ __forceinline__ float normalise(float (&v)[N]) {
  const float sd = deviation(v);
  const Recip rc = make_recip(sd);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = div_rn_z(v[i], sd, rc);
  return sd;
}

__device__ __forceinline__ void rotate(float (&y)[N]) {
#pragma unroll
  for (int h = 1; h < N; h <<= 1)
#pragma unroll
    for (int j = 0; j < N; ++j)
      if ((j & h) == 0) {
        const float p = y[j], q = y[j + h];
        y[j] = p + q;
        y[j + h] = p - q;
      }
#pragma unroll
  for (int j = 0; j < N; ++j) y[j] = y[j] * kInvSqrt128;
}

// Asymmetric round-to-nearest of one group of 128 values into `levels` + 1
// codes (one byte each, written to LDS at codes[stride * i]).  Returns the
// step; *mn receives the zero point.
template <int LEVELS>
__device__ __forceinline__ float quantise_group(const float (&y)[N], uint8_t* codes, int stride, float* mn_out) {
  float mn = y[0], mx = y[0];
#pragma unroll
  for (int i = 1; i < N; ++i) {
    mn = fminf(mn, y[i]);
    mx = fmaxf(mx, y[i]);
  }
  const float s = (mx - mn) / (float)LEVELS;
  const Recip rc = make_recip(s);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float q = __builtin_rintf(div_rn(y[i] - mn, s, rc));
    q = fminf(fmaxf(q, 0.0f), (float)LEVELS);
    codes[stride * i] = s != 0.0f ? (uint8_t)q : (uint8_t)0;
  }
  *mn_out = mn;
  return s;
}

// One tile-head side, by the 128 threads of a workgroup: token rows at
// src + t * row_stride (binary16), codes and metadata into chunk.  `tile` is
// the workgroup's LDS.
__device__ __forceinline__ void kvarn_tile(const uint16_t* src, int64_t row_stride, uint8_t* chunk, int side,
                                           float* tile) {
  uint8_t* cb = reinterpret_cast<uint8_t*>(tile);  // codes [token][channel], after the last pass
  const int t = threadIdx.x;

  // stage 1: the tile, binary16 -> binary32 (exact), coalesced 16-byte loads
#pragma unroll 4
  for (int k = 0; k < 16; ++k) {
    const int p = t + 128 * k, row = p >> 4, c8 = (p & 15) * 8;
    const half8_t x = *reinterpret_cast<const half8_t*>(src + row * row_stride + c8);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[row * LDP + c8 + e] = (float)x[e];
  }
  __syncthreads();

  float y[N];
  float r = 1.0f, c = 1.0f;  // running token factor r_t, channel factor c_t
#pragma unroll 1
  for (int it = 0; it < kSweeps; ++it) {
    // token pass (thread t: token row t); stage 2 on the first visit
#pragma unroll
    for (int j = 0; j < N; ++j) y[j] = tile[t * LDP + j];
    if (it == 0) rotate(y);
    r = r * normalise(y);
#pragma unroll
    for (int j = 0; j < N; ++j) tile[t * LDP + j] = y[j];
    __syncthreads();
    // channel pass (thread t: channel column t)
#pragma unroll
    for (int i = 0; i < N; ++i) y[i] = tile[i * LDP + t];
    c = c * normalise(y);
    if (it + 1 < kSweeps) {
#pragma unroll
      for (int i = 0; i < N; ++i) tile[i * LDP + t] = y[i];
      __syncthreads();
    }
  }

  float* meta = reinterpret_cast<float*>(chunk + kMeta) + side * 3 * N;
  if (side == 0) {
    // keys: 4-bit codes per channel over the tile's tokens
    __syncthreads();  // every column has been read: the tile memory is free
    float mn;
    const float s = quantise_group<15>(y, cb + t, N, &mn);
    meta[t] = c * s;
    meta[N + t] = c * mn;
    meta[2 * N + t] = r;
    __syncthreads();
    // pack: output byte t*64 + j/2 holds channel j (low nibble) and j+1
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int o0 = 16 * (t + 128 * k);
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
    for (int i = 0; i < N; ++i) tile[i * LDP + t] = y[i];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < N; ++j) y[j] = tile[t * LDP + j];
    __syncthreads();  // every row has been read: the tile memory is free
    float mn;
    const float s = quantise_group<3>(y, cb + t * N, 1, &mn);
    meta[t] = r * s;
    meta[N + t] = r * mn;
    meta[2 * N + t] = c;
    __syncthreads();
    // pack: output byte 128*(t/4) + j holds token 4*(t/4) + k in bits 2k..2k+1
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int o0 = 16 * (t + 128 * k);
      const int quad = o0 >> 7, j0 = o0 & 127;
      uint32_t out[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t v = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v |= *reinterpret_cast<const uint32_t*>(cb + (4 * quad + q) * N + j0 + 4 * m) << (2 * q);
        out[m] = v;
      }
      *reinterpret_cast<uint4*>(chunk + kVCodes + o0) = uint4{out[0], out[1], out[2], out[3]};
    }
  }
}

__global__ __launch_bounds__(128) void kvarn_write_kernel(WriteArgs a) {
  __shared__ float tile[N * LDP];
  const int ti = blockIdx.x, h = blockIdx.y, side = blockIdx.z;
  // only the first slot of a tile is read: the tile fills that page in order
  const int64_t s0 = a.slots[(int64_t)ti * N];
  if (s0 < 0 || s0 >= (int64_t)a.num_pages * N) return;
  uint8_t* chunk = a.cache + ((s0 / N) * a.H + h) * a.geom.chunk_bytes;
  const uint16_t* src = (side ? a.v : a.k) + ((int64_t)ti * N * a.H + h) * N;
  kvarn_tile(src, (int64_t)a.H * N, chunk, side, tile);
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
  const uint16_t* src = (side ? a.v : a.k) + (i * a.H + h) * N;
  uint16_t* dst = a.tail + ((((int64_t)b * 2 + side) * a.H + h) * N + (pos & (N - 1))) * N;
  if (threadIdx.x < N / 8)
    reinterpret_cast<uint4*>(dst)[threadIdx.x] = reinterpret_cast<const uint4*>(src)[threadIdx.x];
}

// Tile completion: a token at position 127 mod 128 completes its sequence's
// tile, which is quantised from the tail into the page of that tile.
__global__ __launch_bounds__(128) void kvarn_complete_kernel(KvarnAppendArgs a) {
  __shared__ float tile[N * LDP];
  const int64_t i = blockIdx.x;
  const int h = blockIdx.y, side = blockIdx.z;
  const int b = a.seq[i], pos = a.pos[i];
  if (b < 0 || b >= a.batch || pos < 0 || (pos & (N - 1)) != N - 1) return;
  const int pi = pos / N;
  if (pi >= a.max_pages) return;
  const int page = a.block_tables[(int64_t)b * a.max_pages + pi];
  if (page < 0 || page >= a.num_pages) return;
  uint8_t* chunk = a.cache + ((int64_t)page * a.H + h) * a.chunk_bytes;
  const uint16_t* src = a.tail + (((int64_t)b * 2 + side) * a.H + h) * N * N;
  kvarn_tile(src, N, chunk, side, tile);
}

}  // namespace

hipError_t launch_kvarn_write(const WriteArgs& a, hipStream_t s) {
  const int64_t tiles = a.n_tok / N;
  if (tiles == 0) return hipSuccess;
  if (tiles > 0x7FFFFFFF || a.H > 65535) return hipErrorInvalidValue;
  kvarn_write_kernel<<<dim3((unsigned)tiles, (unsigned)a.H, 2u), 128, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_kvarn_append(const KvarnAppendArgs& a, hipStream_t s) {
  if (a.n_tok == 0) return hipSuccess;
  if (a.n_tok > 0x7FFFFFFF || a.H > 32767) return hipErrorInvalidValue;
  kvarn_append_kernel<<<dim3((unsigned)a.n_tok, (unsigned)(2 * a.H)), 64, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  kvarn_complete_kernel<<<dim3((unsigned)a.n_tok, (unsigned)a.H, 2u), 128, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvq
