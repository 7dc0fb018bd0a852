// dequant.hip -- expand cached tokens back to binary32 (inspection / tests).
//
// x_hat = s * q ([P3] "KV Cache 量化 · LLM Glossary", §它改变缓存表示; INT4
// per-token-head codes are two's-complement nibbles), and for
// NVFP4 x_hat = s_t * s_b * q ([P5] "NVFP4 KV Cache：Blackwell 上的 4-bit 缓存
// 量化", §双层缩放怎样恢复动态范围); MXFP4 x_hat = 2^(e - 127) * q for the
// block's E8M0 byte e (exact).  KVarN ([P2] "KVarN：华为推出的原生 vLLM
// KV-cache 量化后端", §技术原理): the rotated tile is rebuilt from the folded
// metadata, K_tj = rho_t (alpha_j code + beta_j) and
// V_tj = gamma_j (alpha_t code + beta_t), and rotated back with the normalised
// Walsh-Hadamard transform (its own inverse), all in binary64 with one final
// rounding to binary32.  One thread per output element; this path is not
// performance-critical.  Built with -ffp-contract=off.
#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(WriteArgs a, float* k_out, float* v_out) {
  const int D = a.D, P = a.P;
  const int64_t row = blockIdx.x;  // token * H + head
  const int64_t tok = row / a.H;
  const int h = (int)(row - tok * a.H);
  const int64_t slot = a.slots[tok];
  if (slot < 0 || slot >= (int64_t)a.num_pages * P) return;
  const int64_t page = slot / P;
  const int t = (int)(slot - page * P);
  const uint8_t* chunk = a.cache + (page * a.H + h) * a.geom.chunk_bytes;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float kx, vx;
    if constexpr (FMT == 6) {
      const uint32_t kb = chunk[(int64_t)t * (D / 2) + d / 2];
      const uint32_t vb = chunk[a.geom.v_codes + 2 * D * (t / 4) + 4 * (d / 2) + (t % 4)];
      const int kc = (int)((d & 1) ? kb >> 4 : kb & 15u);
      const int vc = (int)((d & 1) ? vb >> 4 : vb & 15u);
      const float* sc = reinterpret_cast<const float*>(chunk + a.geom.k_scales);
      kx = (float)((kc ^ 8) - 8) * sc[t];  // two's-complement nibble times scale
      vx = (float)((vc ^ 8) - 8) * sc[P + t];
    } else if constexpr (FMT == 7) {
      const uint32_t kb = chunk[(int64_t)t * (D / 2) + d / 2];
      const uint32_t vb = chunk[a.geom.v_codes + 2 * D * (t / 4) + 4 * (d / 2) + (t % 4)];
      const uint32_t kc = (d & 1) ? kb >> 4 : kb & 15u;
      const uint32_t vc = (d & 1) ? vb >> 4 : vb & 15u;
      const int ke = chunk[a.geom.k_scales + (int64_t)t * (D / 32) + d / 32];
      const int ve = chunk[a.geom.v_scales + (int64_t)(d / 32) * P + t];
      const float kq = (kc & 8u) ? -e2m1_val(kc & 7u) : e2m1_val(kc & 7u);
      const float vq = (vc & 8u) ? -e2m1_val(vc & 7u) : e2m1_val(vc & 7u);
      kx = ldexpf(kq, ke - 127);
      vx = ldexpf(vq, ve - 127);
    } else if constexpr (FMT == 4) {
      const uint32_t kb = chunk[(int64_t)t * (D / 2) + d / 2];
      const uint32_t vb = chunk[a.geom.v_codes + 2 * D * (t / 4) + 4 * (d / 2) + (t % 4)];
      const uint32_t kc = (d & 1) ? kb >> 4 : kb & 15u;
      const uint32_t vc = (d & 1) ? vb >> 4 : vb & 15u;
      const float ksb = e4m3_val(chunk[a.geom.k_scales + (int64_t)t * (D / 16) + d / 16] & 0x7Fu);
      const float vsb = e4m3_val(chunk[a.geom.v_scales + (int64_t)(d / 16) * P + t] & 0x7Fu);
      const float kq = (kc & 8u) ? -e2m1_val(kc & 7u) : e2m1_val(kc & 7u);
      const float vq = (vc & 8u) ? -e2m1_val(vc & 7u) : e2m1_val(vc & 7u);
      kx = (kq * ksb) * a.k_scale;  // the first product is exact
      vx = (vq * vsb) * a.v_scale;
    } else {
      uint32_t kc, vc;
      switch (D) {
        case 32: kc = chunk[k8_offset<32>(t, d)]; vc = chunk[a.geom.v_codes + v8_offset<32>(t, d)]; break;
        case 64: kc = chunk[k8_offset<64>(t, d)]; vc = chunk[a.geom.v_codes + v8_offset<64>(t, d)]; break;
        default: kc = chunk[k8_offset<128>(t, d)]; vc = chunk[a.geom.v_codes + v8_offset<128>(t, d)]; break;
      }
      float kq, vq;
      if constexpr (FMT == 2) {
        kq = (float)(int8_t)kc;
        vq = (float)(int8_t)vc;
      } else {
        kq = (kc & 0x80u) ? -e4m3_val(kc & 0x7Fu) : e4m3_val(kc & 0x7Fu);
        vq = (vc & 0x80u) ? -e4m3_val(vc & 0x7Fu) : e4m3_val(vc & 0x7Fu);
      }
      float ks, vs;
      if constexpr (FMT == 1) {
        ks = a.k_scale;
        vs = a.v_scale;
      } else {
        ks = reinterpret_cast<const float*>(chunk + a.geom.k_scales)[t];
        vs = reinterpret_cast<const float*>(chunk + a.geom.v_scales)[t];
      }
      kx = kq * ks;
      vx = vq * vs;
    }
    k_out[row * D + d] = kx;
    v_out[row * D + d] = vx;
  }
}

// One workgroup of 128 threads per (token, kv head); thread j owns channel j.
__global__ __launch_bounds__(128) void dequant_kvarn_kernel(WriteArgs a, float* k_out, float* v_out,
                                                            double inv_sqrt128) {
  __shared__ double buf[2][2][128];  // [ping-pong][side][channel]
  const int64_t row = blockIdx.x;
  const int64_t tok = row / a.H;
  const int h = (int)(row - tok * a.H);
  const int j = threadIdx.x;
  const int64_t slot = a.slots[tok];
  if (slot < 0 || slot >= (int64_t)a.num_pages * a.P) return;
  const int64_t page = slot / a.P;
  const int tp = (int)(slot - page * a.P);  // token in the page: tile tp / 128, row t
  const int t = tp & 127;
  const uint8_t* chunk = a.cache + (page * a.H + h) * a.geom.chunk_bytes + (int64_t)(tp >> 7) * (a.geom.chunk_bytes / (a.P / 128));
  const float* meta = reinterpret_cast<const float*>(chunk + a.geom.k_scales);
  const uint32_t kb = chunk[t * 64 + j / 2];
  const uint32_t kc = (j & 1) ? kb >> 4 : kb & 15u;
  const uint32_t vc = (chunk[a.geom.v_codes + 128 * (t / 4) + j] >> (2 * (t % 4))) & 3u;
  buf[0][0][j] = (double)meta[256 + t] * ((double)meta[j] * (double)kc + (double)meta[128 + j]);
  buf[0][1][j] = (double)meta[640 + j] * ((double)meta[384 + t] * (double)vc + (double)meta[512 + t]);
  int cur = 0;
  for (int hb = 1; hb < 128; hb <<= 1) {
    __syncthreads();
#pragma unroll
    for (int sd = 0; sd < 2; ++sd) {
      const double* y = buf[cur][sd];
      buf[cur ^ 1][sd][j] = (j & hb) ? y[j - hb] - y[j] : y[j] + y[j + hb];
    }
    cur ^= 1;
  }
  k_out[row * 128 + j] = (float)(buf[cur][0][j] * inv_sqrt128);
  v_out[row * 128 + j] = (float)(buf[cur][1][j] * inv_sqrt128);
}

}  // namespace

hipError_t launch_dequant(int fmt, const WriteArgs& a, float* k_out, float* v_out, hipStream_t s) {
  const int64_t rows = a.n_tok * a.H;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)rows);
  const int threads = a.D < 256 ? a.D : 256;
  switch (fmt) {
    case 1: dequant_kernel<1><<<grid, threads, 0, s>>>(a, k_out, v_out); break;
    case 2: dequant_kernel<2><<<grid, threads, 0, s>>>(a, k_out, v_out); break;
    case 3: dequant_kernel<3><<<grid, threads, 0, s>>>(a, k_out, v_out); break;
    case 4: dequant_kernel<4><<<grid, threads, 0, s>>>(a, k_out, v_out); break;
    case 6: dequant_kernel<6><<<grid, threads, 0, s>>>(a, k_out, v_out); break;
    case 7: dequant_kernel<7><<<grid, threads, 0, s>>>(a, k_out, v_out); break;
    case 5: dequant_kvarn_kernel<<<grid, 128, 0, s>>>(a, k_out, v_out, 1.0 / sqrt(128.0)); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
