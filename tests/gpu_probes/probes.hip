// probes.hip -- test-only kernels that record what gfx950 conversion
// builtins return for every input of interest, so the tests can compare
// them with exact values before the library relies on them.  Not part of
// libkvq.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

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

// Pairs (x[2i], x[2i+1]) -> E4M3 with the packed conversion into both words
// of one dword, as an encoder would pack four values: out[i] holds pair 2i
// in bytes 0-1 and pair 2i+1 in bytes 2-3.
__global__ void k_cvt_f32_fp8_pairs(const float* x, int64_t n4, uint32_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * i], x[4 * i + 1], 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * i + 2], x[4 * i + 3], r, true);
  out[i] = (uint32_t)r;
}

// Eight values -> E2M1 nibbles with the scaled packed conversion (scale 1),
// value 2k in the low nibble of byte k, as an encoder would pack them.
__global__ void k_cvt_f32_fp4_x8(const float* x, int64_t n8, uint32_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const float* p = x + 8 * i;
  uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, p[0], p[1], 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, p[2], p[3], 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, p[4], p[5], 1.0f, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, p[6], p[7], 1.0f, 3);
  out[i] = r;
}

// E2M1 pairs -> binary16, issued directly as the library does (the
// compiler's lowering of the builtin repacks the two results when they are
// used one by one), byte selector k = 0..3.
template <int K>
__device__ __forceinline__ uint32_t cvt_fp4_byte(uint32_t w, float scale) {
  uint32_t r;
  if constexpr (K == 0)
    asm volatile("v_cvt_scalef32_pk_f16_fp4 %0, %1, %2\n\ts_nop 1" : "=v"(r) : "v"(w), "v"(scale));
  else if constexpr (K == 1)
    asm volatile("v_cvt_scalef32_pk_f16_fp4 %0, %1, %2 op_sel:[1,0,0]\n\ts_nop 1" : "=v"(r) : "v"(w), "v"(scale));
  else if constexpr (K == 2)
    asm volatile("v_cvt_scalef32_pk_f16_fp4 %0, %1, %2 op_sel:[0,1,0]\n\ts_nop 1" : "=v"(r) : "v"(w), "v"(scale));
  else
    asm volatile("v_cvt_scalef32_pk_f16_fp4 %0, %1, %2 op_sel:[1,1,0]\n\ts_nop 1" : "=v"(r) : "v"(w), "v"(scale));
  return r;
}

__global__ void k_cvt_fp4_f16_asm(const uint32_t* src, int n, float scale, uint32_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t w = src[i];
  out[4 * (int64_t)i + 0] = cvt_fp4_byte<0>(w, scale);
  out[4 * (int64_t)i + 1] = cvt_fp4_byte<1>(w, scale);
  out[4 * (int64_t)i + 2] = cvt_fp4_byte<2>(w, scale);
  out[4 * (int64_t)i + 3] = cvt_fp4_byte<3>(w, scale);
}

// E4M3 pairs -> binary16, issued directly: word i -> out[2i] (bytes 0, 1),
// out[2i + 1] (bytes 2, 3).
__global__ void k_cvt_fp8_f16_asm(const uint32_t* src, int n, uint32_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint32_t lo, hi;
  asm("s_nop 1\n\tv_cvt_scalef32_pk_f16_fp8 %0, %2, 1.0\n\t"
      "v_cvt_scalef32_pk_f16_fp8 %1, %2, 1.0 op_sel:[1,0,0]\n\ts_nop 1"
      : "=&v"(lo), "=&v"(hi) : "v"(src[i]));
  out[2 * (int64_t)i] = lo;
  out[2 * (int64_t)i + 1] = hi;
}

// One v_mfma_f32_16x16x32_f16 on operands given per lane: a and b hold 8
// binary16 values per lane (64 lanes), out gets the 4 results of each lane.
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
__global__ void k_mfma_f16(const half8_t* a, const half8_t* b, float4_t* out) {
  const int l = threadIdx.x;
  out[l] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[l], b[l], float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}

// E4M3 pairs -> binary16 with a scale operand, issued as the KVarN decode does:
// word i -> out[2i] (bytes 0, 1), out[2i + 1] (bytes 2, 3).
__global__ void k_cvt_fp8_f16_scaled(const uint32_t* src, int n, float scale, uint32_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint32_t lo, hi;
  asm("s_nop 1\n\tv_cvt_scalef32_pk_f16_fp8 %0, %2, %3\n\t"
      "v_cvt_scalef32_pk_f16_fp8 %1, %2, %3 op_sel:[1,0,0]\n\ts_nop 1"
      : "=&v"(lo), "=&v"(hi) : "v"(src[i]), "v"(scale));
  out[2 * (int64_t)i] = lo;
  out[2 * (int64_t)i + 1] = hi;
}

// Words of E2M1 codes -> binary32 with the scaled conversion at scale 1,
// one byte per instruction (byte-select operands 0..3), eight values per word.
typedef float float2_v __attribute__((ext_vector_type(2)));
__global__ void k_cvt_fp4_f32_bytes(const uint32_t* src, int n, float* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t w = src[i];
  const float2_v a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const float2_v b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const float2_v c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const float2_v d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  float* o = out + 8 * (int64_t)i;
  o[0] = a.x, o[1] = a.y, o[2] = b.x, o[3] = b.y, o[4] = c.x, o[5] = c.y, o[6] = d.x, o[7] = d.y;
}

extern "C" {
int probe_cvt_fp4_f32_bytes(const uint32_t* src, int n, float* out) {
  if (n <= 0) return 0;
  k_cvt_fp4_f32_bytes<<<(n + 255) / 256, 256>>>(src, n, out);
  return (int)hipGetLastError();
}
int probe_cvt_fp8_f16_scaled(const uint32_t* src, int n, float scale, uint32_t* out) {
  if (n <= 0) return 0;
  k_cvt_fp8_f16_scaled<<<(n + 255) / 256, 256>>>(src, n, scale, out);
  return (int)hipGetLastError();
}
int probe_mfma_f16(const void* a, const void* b, void* out) {
  k_mfma_f16<<<1, 64>>>(reinterpret_cast<const half8_t*>(a), reinterpret_cast<const half8_t*>(b),
                        reinterpret_cast<float4_t*>(out));
  return (int)hipGetLastError();
}
int probe_cvt_fp8_f16_asm(const uint32_t* src, int n, uint32_t* out) {
  if (n <= 0) return 0;
  k_cvt_fp8_f16_asm<<<(n + 255) / 256, 256>>>(src, n, out);
  return (int)hipGetLastError();
}
int probe_cvt_fp4_f16_asm(const uint32_t* src, int n, float scale, uint32_t* out) {
  if (n <= 0) return 0;
  k_cvt_fp4_f16_asm<<<(n + 255) / 256, 256>>>(src, n, scale, out);
  return (int)hipGetLastError();
}
int probe_cvt_f32_fp8(const float* x, int64_t n, uint8_t* out) {
  if (n <= 0) return 0;
  k_cvt_f32_fp8<<<(unsigned)((n + 255) / 256), 256>>>(x, n, out);
  return (int)hipGetLastError();
}
int probe_cvt_f32_fp8_pairs(const float* x, int64_t n4, uint32_t* out) {
  if (n4 <= 0) return 0;
  k_cvt_f32_fp8_pairs<<<(unsigned)((n4 + 255) / 256), 256>>>(x, n4, out);
  return (int)hipGetLastError();
}
int probe_cvt_f32_fp4_x8(const float* x, int64_t n8, uint32_t* out) {
  if (n8 <= 0) return 0;
  k_cvt_f32_fp4_x8<<<(unsigned)((n8 + 255) / 256), 256>>>(x, n8, out);
  return (int)hipGetLastError();
}
int probe_cvt_f32_fp4(const float* x, int64_t n, uint8_t* out) {
  if (n <= 0) return 0;
  k_cvt_f32_fp4<<<(unsigned)((n + 255) / 256), 256>>>(x, n, out);
  return (int)hipGetLastError();
}
}
