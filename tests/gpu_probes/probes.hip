// probes.hip -- test-only kernels that record what gfx950 conversion
// builtins return for every input of interest, so the tests can compare
// them with exact values before the library relies on them.  Not part of
// libkvq.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// E4M3 pairs -> binary16 with a binary32 scale: out[2i], out[2i+1] for the
// bytes (i, i) of word i (low word).
__global__ void k_cvt_fp8_f16(const float* scales, int n_scales, uint16_t* out) {
  const int c = threadIdx.x;  // code 0..255
  const int si = blockIdx.x;
  if (c >= 256 || si >= n_scales) return;
  const uint32_t src = (uint32_t)c | ((uint32_t)c << 8);
  const half2_t h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src, scales[si], false);
  out[((int64_t)si * 256 + c) * 2] = __builtin_bit_cast(uint16_t, h[0]);
  out[((int64_t)si * 256 + c) * 2 + 1] = __builtin_bit_cast(uint16_t, h[1]);
}

// E2M1 nibble pairs -> binary16 with a binary32 scale: byte = lo | hi << 4.
__global__ void k_cvt_fp4_f16(const float* scales, int n_scales, uint16_t* out) {
  const int c = threadIdx.x;  // byte 0..255
  const int si = blockIdx.x;
  if (c >= 256 || si >= n_scales) return;
  const half2_t h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((uint32_t)c, scales[si], 0);
  out[((int64_t)si * 256 + c) * 2] = __builtin_bit_cast(uint16_t, h[0]);
  out[((int64_t)si * 256 + c) * 2 + 1] = __builtin_bit_cast(uint16_t, h[1]);
}

// binary32 -> E4M3 with the gfx950 packed conversion (input pre-clamped to
// +-448 by the caller's data).
__global__ void k_cvt_f32_fp8(const float* x, int64_t n, uint8_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int r = __builtin_amdgcn_cvt_pk_fp8_f32(x[i], 0.0f, 0, false);
  out[i] = (uint8_t)(r & 0xFF);
}

// binary32 -> E2M1 with the gfx950 scaled packed conversion, scale 1.
__global__ void k_cvt_f32_fp4(const float* x, int64_t n, uint8_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[i], 0.0f, 1.0f, 0);
  out[i] = (uint8_t)(r & 0xF);
}

extern "C" {
int probe_cvt_fp8_f16(const float* scales, int n_scales, uint16_t* out) {
  k_cvt_fp8_f16<<<n_scales, 256>>>(scales, n_scales, out);
  return (int)hipGetLastError();
}
int probe_cvt_fp4_f16(const float* scales, int n_scales, uint16_t* out) {
  k_cvt_fp4_f16<<<n_scales, 256>>>(scales, n_scales, out);
  return (int)hipGetLastError();
}
int probe_cvt_f32_fp8(const float* x, int64_t n, uint8_t* out) {
  if (n <= 0) return 0;
  k_cvt_f32_fp8<<<(unsigned)((n + 255) / 256), 256>>>(x, n, out);
  return (int)hipGetLastError();
}
int probe_cvt_f32_fp4(const float* x, int64_t n, uint8_t* out) {
  if (n <= 0) return 0;
  k_cvt_f32_fp4<<<(unsigned)((n + 255) / 256), 256>>>(x, n, out);
  return (int)hipGetLastError();
}
}

// ---- bandwidth references ---------------------------------------------------

// Streams n16 16-byte words, 4 independent loads in flight per thread.
__global__ __launch_bounds__(256) void k_read_stream(const uint4* p, int64_t n16, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads alive
}

// Reads chunks of `chunk` bytes (a multiple of 1024) at the given byte offsets,
// one wavefront per chunk at a time, two chunks in flight per wavefront.
__global__ __launch_bounds__(256) void k_read_chunks(const uint8_t* base, const int64_t* offs, int64_t n_chunks,
                                                     int chunk, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t n_waves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  uint32_t acc = 0;
  for (int64_t c = wave; c < n_chunks; c += n_waves) {
    const uint4* q = reinterpret_cast<const uint4*>(base + offs[c]);
    for (int k = lane; k < chunk / 16; k += 64) {
      const uint4 a = q[k];
      acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

extern "C" {
int probe_read_stream(const void* p, int64_t bytes, uint32_t* sink, int blocks) {
  k_read_stream<<<blocks, 256>>>(reinterpret_cast<const uint4*>(p), bytes / 16, sink);
  return (int)hipGetLastError();
}
int probe_read_chunks(const void* base, const int64_t* offs, int64_t n_chunks, int chunk, uint32_t* sink,
                      int blocks) {
  k_read_chunks<<<blocks, 256>>>(reinterpret_cast<const uint8_t*>(base), offs, n_chunks, chunk, sink);
  return (int)hipGetLastError();
}
}

// Each wavefront reads `per_wave` consecutive 16-byte words per step with all
// loads issued before any is used (U words per lane in flight); optionally
// nontemporal.
template <int U, bool NT>
__global__ __launch_bounds__(256) void k_read_deep(const uint4* p, int64_t n16, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t n_waves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  uint32_t acc = 0;
  for (int64_t base = wave * 64 * U; base < n16; base += n_waves * 64 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * 64 + lane;
      const int64_t j = i < n16 ? i : n16 - 1;
      if (NT) {
        v[u].x = __builtin_nontemporal_load(&p[j].x);
        v[u].y = __builtin_nontemporal_load(&p[j].y);
        v[u].z = __builtin_nontemporal_load(&p[j].z);
        v[u].w = __builtin_nontemporal_load(&p[j].w);
      } else {
        v[u] = p[j];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

extern "C" int probe_read_deep(const void* p, int64_t bytes, uint32_t* sink, int blocks, int unroll, int nt) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  if (unroll == 4 && !nt) k_read_deep<4, false><<<blocks, 256>>>(q, bytes / 16, sink);
  else if (unroll == 8 && !nt) k_read_deep<8, false><<<blocks, 256>>>(q, bytes / 16, sink);
  else if (unroll == 16 && !nt) k_read_deep<16, false><<<blocks, 256>>>(q, bytes / 16, sink);
  else if (unroll == 4 && nt) k_read_deep<4, true><<<blocks, 256>>>(q, bytes / 16, sink);
  else if (unroll == 8 && nt) k_read_deep<8, true><<<blocks, 256>>>(q, bytes / 16, sink);
  else if (unroll == 16 && nt) k_read_deep<16, true><<<blocks, 256>>>(q, bytes / 16, sink);
  else return -1;
  return (int)hipGetLastError();
}
