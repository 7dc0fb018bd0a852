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
// All binary32 arithmetic rounds exactly as written (no contraction,
// correctly rounded division and square root), so the codes and metadata are
// a deterministic function of the binary16 input.
//
// Mapping.  One workgroup of 256 threads (4 wavefronts) per (tile, kv head,
// side).  The tile lives in LDS as binary32 with rows padded to 129 words.
// Lanes l and l + 32 of wavefront w share index i = 32 w + (l & 31): the
// lower lane holds the left half [0, 64) of token row i in a token pass and
// of channel column i in a channel pass, the upper lane the right half
// [64, 128).  A 128-value sum is the canonical tree of its two 64-value
// halves, S = S(left) + S(right): each lane sums its half in registers and
// v_permlane32_swap hands both halves' sums to both lanes, with no LDS round
// trip or barrier.  The upper lane keeps its 64 values rotated by 32 in its
// registers: value j is element (j + 32) mod 64 of its half.  That leaves
// every sum unchanged (it swaps the two 32-value subtrees of the half's tree,
// and binary32 addition commutes) and makes both access patterns free of LDS
// bank conflicts (the two lanes of a pair sit 32 banks apart).  Two
// workgroups fit the LDS of a compute unit: 8 wavefronts.
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

constexpr int H = N / 2;  // values per thread and pass

// Balanced pairwise sum of 64 values in index order (one half of the
// canonical 128-value tree).
__device__ __forceinline__ float tree_sum64(const float (&v)[H]) {
  float t[H / 2];
#pragma unroll
  for (int i = 0; i < H / 2; ++i) t[i] = v[2 * i] + v[2 * i + 1];
#pragma unroll
  for (int w = H / 4; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = t[2 * i] + t[2 * i + 1];
  return t[0];
}

// The two halves' partial results for index i, from lanes l and l + 32:
// returns the left half's and the right half's values in both lanes.
struct Halves {
  float left, right;
};
__device__ __forceinline__ Halves exchange(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return Halves{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Column within the row (row within the column) of value j of this lane's
// half, the right half rotated by 32.
__device__ __forceinline__ int pos(int j, int half) { return j < 32 ? j + 96 * half : j + 32 * half; }
// ... and of the same element of the other half.
__device__ __forceinline__ int partner_pos(int j, int half) {
  return j < 32 ? j + 64 - 32 * half : j + 64 - 96 * half;
}

// Population standard deviation of 128 values (this thread's half v and the
// partner's); a zero or non-finite result becomes 1.
__device__ __forceinline__ float deviation(const float (&v)[H]) {
  const Halves s = exchange(tree_sum64(v));
  const float mean = (s.left + s.right) * 0.0078125f;
  float sq[H];
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const float d = v[k] - mean;
    sq[k] = d * d;
  }
  const Halves q = exchange(tree_sum64(sq));
  float sd = __builtin_sqrtf((q.left + q.right) * 0.0078125f);
  if (!(sd > 0.0f) || !__builtin_isfinite(sd)) sd = 1.0f;
  return sd;
}

// Scale the 128 values by RN(1 / deviation) (one rounding of the reciprocal,
// one of each product; the sign of zero carries through the product);
// returns the deviation.
__device__ __forceinline__ float normalise(float (&v)[H]) {
  const float sd = deviation(v);
  const float inv = 1.0f / sd;
#pragma unroll
  for (int k = 0; k < H; ++k) v[k] = v[k] * inv;
  return sd;
}

// Butterfly stages h = 1 .. 32 of the rotation on this lane's half.  Stages
// below 32 stay inside each 32-value block, so the right half's rotated order
// does not matter to them; stage 32 puts each pair's sum and difference at
// the registers of their own elements.
__device__ __forceinline__ void rotate_half(float (&y)[H], int half) {
#pragma unroll
  for (int h = 1; h < H / 2; h <<= 1)
#pragma unroll
    for (int j = 0; j < H; ++j)
      if ((j & h) == 0) {
        const float p = y[j], q = y[j + h];
        y[j] = p + q;
        y[j + h] = p - q;
      }
#pragma unroll
  for (int j = 0; j < H / 2; ++j) {
    // left half: p = element j, q = element j + 32; right half: the reverse
    const float p = y[j], q = y[j + H / 2];
    const float sum = p + q;
    y[j] = half == 0 ? sum : q - p;
    y[j + H / 2] = half == 0 ? p - q : sum;
  }
}

// Asymmetric round-to-nearest of one group of 128 values (this lane's half
// and the partner lane's) into LEVELS + 1 codes; value j's code goes to LDS
// byte codes[stride * pos(j, half)].  Returns the step; *mn_out receives the
// zero point.
template <int LEVELS>
__device__ __forceinline__ float quantise_group(const float (&y)[H], uint8_t* codes, int stride, int half,
                                                float* mn_out) {
  float mn = y[0], mx = y[0];
#pragma unroll
  for (int k = 1; k < H; ++k) {
    mn = fminf(mn, y[k]);
    mx = fmaxf(mx, y[k]);
  }
  const Halves a = exchange(mn);
  const Halves b = exchange(mx);
  mn = fminf(a.left, a.right);
  mx = fmaxf(b.left, b.right);
  const float s = (mx - mn) / (float)LEVELS;
  const Recip rc = make_recip(s);
  // clip(rne(.), 0, LEVELS): the clamp first (integer bounds, so it commutes
  // with the rounding), then adding 1.5 * 2^23 rounds to an integer with ties
  // to even and leaves it in the sum's low mantissa bits
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const float yc = __builtin_amdgcn_fmed3f(div_rn(y[k] - mn, s, rc), 0.0f, (float)LEVELS);
    codes[stride * pos(k, half)] = s != 0.0f ? (uint8_t)__float_as_uint(yc + 12582912.0f) : (uint8_t)0;
  }
  *mn_out = mn;
  return s;
}

// One tile-head side, by the 256 threads of a workgroup: token rows at
// src + t * row_stride (binary16), codes and metadata into chunk.  `tile`
// holds N * LDP floats of LDS.
__device__ __forceinline__ void kvarn_tile(const uint16_t* src, int64_t row_stride, uint8_t* chunk, int side,
                                           float* tile) {
  uint8_t* cb = reinterpret_cast<uint8_t*>(tile);  // codes [token][channel], after the last pass
  const int t = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int half = (t >> 5) & 1;
  const int i = 32 * wv + (t & 31);  // token row / channel column

  // stage 1: the tile, binary16 -> binary32 (exact), coalesced 16-byte loads
#pragma unroll 4
  for (int k = 0; k < 8; ++k) {
    const int p = t + 256 * k, row = p >> 4, c8 = (p & 15) * 8;
    const half8_t x = *reinterpret_cast<const half8_t*>(src + row * row_stride + c8);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[row * LDP + c8 + e] = (float)x[e];
  }
  __syncthreads();

  float y[H];
  float r = 1.0f, c = 1.0f;  // running token factor r_i, channel factor c_i
#pragma unroll 1
  for (int it = 0; it < kSweeps; ++it) {
    // token pass (token row i, this half); stage 2 on the first visit
#pragma unroll
    for (int j = 0; j < H; ++j) y[j] = tile[i * LDP + pos(j, half)];
    if (it == 0) {
      // stages h = 1 .. 32 in registers, stage 64 across the halves:
      // (a, b) -> (a + b, a - b) with a in the left half, b in the right
      rotate_half(y, half);
#pragma unroll
      for (int j = 0; j < H; ++j) tile[i * LDP + pos(j, half)] = y[j];
      __syncthreads();
#pragma unroll
      for (int j = 0; j < H; ++j) {
        const float z = tile[i * LDP + partner_pos(j, half)];
        y[j] = half == 0 ? y[j] + z : z - y[j];
      }
#pragma unroll
      for (int j = 0; j < H; ++j) y[j] = y[j] * kInvSqrt128;
      __syncthreads();  // both halves have read their partner's values
    }
    r = r * normalise(y);
#pragma unroll
    for (int j = 0; j < H; ++j) tile[i * LDP + pos(j, half)] = y[j];
    __syncthreads();
    // channel pass (channel column i, this half)
#pragma unroll
    for (int k = 0; k < H; ++k) y[k] = tile[pos(k, half) * LDP + i];
    c = c * normalise(y);
    if (it + 1 < kSweeps) {
#pragma unroll
      for (int k = 0; k < H; ++k) tile[pos(k, half) * LDP + i] = y[k];
      __syncthreads();
    }
  }

  float* meta = reinterpret_cast<float*>(chunk + kMeta) + side * 3 * N;
  if (side == 0) {
    // keys: 4-bit codes per channel over the tile's tokens
    __syncthreads();  // every column has been read: the tile memory is free
    float mn;
    const float s = quantise_group<15>(y, cb + i, N, half, &mn);
    if (half == 0) {
      meta[i] = c * s;
      meta[N + i] = c * mn;
      meta[2 * N + i] = r;
    }
    __syncthreads();
    // pack: output byte t*64 + j/2 holds channel j (low nibble) and j+1
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int o0 = 16 * (t + 256 * k);
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
    for (int k = 0; k < H; ++k) tile[pos(k, half) * LDP + i] = y[k];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < H; ++j) y[j] = tile[i * LDP + pos(j, half)];
    __syncthreads();  // every row has been read: the tile memory is free
    float mn;
    const float s = quantise_group<3>(y, cb + i * N, 1, half, &mn);
    if (half == 0) {
      meta[i] = r * s;
      meta[N + i] = r * mn;
      meta[2 * N + i] = c;
    }
    __syncthreads();
    // pack: output byte 128*(t/4) + j holds token 4*(t/4) + k in bits 2k..2k+1
    {
      const int o0 = 16 * t;
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

constexpr int kLdsFloats = N * LDP;

// Contract violations found in device-resident arguments (KVQ_DEVERR_* bits of
// kvq.h), one word per device: raised with a vector atomic OR, read and
// cleared by kvq_take_device_errors.
__device__ uint32_t g_device_errors;

__device__ __forceinline__ void raise_error(uint32_t bit) { atomicOr(&g_device_errors, bit); }

__global__ __launch_bounds__(256) void kvarn_write_kernel(WriteArgs a) {
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
__global__ __launch_bounds__(256) void kvarn_complete_kernel(KvarnAppendArgs a) {
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
  kvarn_write_kernel<<<dim3((unsigned)tiles, (unsigned)a.H, 2u), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_kvarn_append(const KvarnAppendArgs& a, hipStream_t s) {
  if (a.n_tok == 0) return hipSuccess;
  if (a.n_tok > 0x7FFFFFFF || a.H > 32767) return hipErrorInvalidValue;
  kvarn_append_kernel<<<dim3((unsigned)a.n_tok, (unsigned)(2 * a.H)), 64, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  kvarn_complete_kernel<<<dim3((unsigned)a.n_tok, (unsigned)a.H, 2u), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvq
