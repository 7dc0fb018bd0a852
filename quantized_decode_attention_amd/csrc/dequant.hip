// dequant.hip -- expand cached tokens back to binary32 (inspection / tests).
//
// x_hat = s * q ([P3] "KV Cache 量化 · LLM Glossary", §它改变缓存表示), and for
// NVFP4 x_hat = s_t * s_b * q ([P5] "NVFP4 KV Cache：Blackwell 上的 4-bit 缓存
// 量化", §双层缩放怎样恢复动态范围).  One thread per output element; this path
// is not performance-critical.  Built with -ffp-contract=off.
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
    if constexpr (FMT == 4) {
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
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
