// kvq_internal.h -- launch interfaces between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// Byte offsets inside one (page, kv head) chunk; see the layout in kvq.h.
struct ChunkGeom {
  int64_t chunk_bytes;
  int64_t v_codes;   // start of the V codes
  int64_t k_scales;  // start of the K scales (per-token-head) / K block scales (NVFP4)
  int64_t v_scales;  // start of the V scales / V block scales
};

struct WriteArgs {
  const uint16_t* k;
  const uint16_t* v;
  const int64_t* slots;
  int64_t n_tok;
  uint8_t* cache;
  ChunkGeom geom;
  int H, D, P, num_pages;
  float k_scale, v_scale;
  int flags;
};

struct DecodeArgs {
  const uint8_t* cache;
  ChunkGeom geom;
  int H, D, P, num_pages;
  const uint16_t* q;
  int Hq, G;
  const int32_t* block_tables;
  int max_pages;
  const int32_t* ctx_lens;
  int B;
  float qk_scale;  // sm_scale * log2(e)
  float k_scale, v_scale;
  const uint16_t* tail;  // KVarN incomplete-tile tokens, or null
  uint16_t* out;
  uint8_t* workspace;
  int num_splits;
  int pages_per_split;
  int sp_shift;  // log2(P / 16)
  int waves;     // wavefronts per split workgroup: 4, or 8 for single-split plans
  // Append-and-decode: slot of each sequence's new token (or null).  The
  // split kernel then reads positions 0 .. ctx-2 of a sequence whose new
  // token is attended, and its split-0 workgroup quantises, stores and
  // attends the new token described by `wnew` (rows k_new / v_new
  // [batch][H][D]), folding it into its own partial.
  const int64_t* new_slots;
  WriteArgs wnew;
};

// Workspace: one partial record (m[8], l[8], o[8][D]) per (sequence, kv head,
// split); no workspace is needed when there is a single split, except for
// KVarN, whose merge kernel always runs (tail tokens, rotation back).
constexpr int kMaxGroup = 8;    // q heads per kv head served by one decode wave
constexpr int kMaxSplits = 256; // context splits per (sequence, kv head)

__host__ __device__ inline int64_t ws_record_floats(int D) { return 2 * kMaxGroup + (int64_t)kMaxGroup * D; }

// KVarN incremental append (tail rows and tile completion).
struct KvarnAppendArgs {
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* seq;
  const int32_t* pos;
  int64_t n_tok;
  uint16_t* tail;  // [batch][2][H][128][128] binary16
  int batch;
  const int32_t* block_tables;
  int max_pages;
  uint8_t* cache;
  int64_t chunk_bytes;
  int H, num_pages;
  int P;  // page size: 128 or 256 tokens, i.e. 1 or 2 tiles
};

hipError_t launch_quant_write(int fmt, const WriteArgs& a, hipStream_t s);
hipError_t launch_kvarn_append(const KvarnAppendArgs& a, hipStream_t s);
hipError_t launch_kvarn_write(const WriteArgs& a, hipStream_t s);
hipError_t launch_decode(int fmt, const DecodeArgs& a, hipStream_t s);
hipError_t launch_kvarn_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_dequant(int fmt, const WriteArgs& a, float* k_out, float* v_out, hipStream_t s);

// KVQ_DEVERR_* bits raised on the current device since the last call
// (read and cleared; synchronous).
hipError_t take_device_errors(uint32_t* flags);

// Device address of the current device's fixed decode workspace
// (KVQ_DECODE_SCRATCH_BYTES), looked up on the first call per device.
hipError_t decode_scratch(void** ptr);

// Resident workgroups per compute unit of the decode split kernel for a
// format, head size and GQA group on the current device (0 if unknown).
int decode_blocks_per_cu(int fmt, int D, int G);
int kvarn_decode_blocks_per_cu(int G);

}  // namespace kvq
