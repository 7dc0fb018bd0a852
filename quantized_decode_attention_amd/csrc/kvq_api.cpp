// kvq_api.cpp -- the C ABI of libkvq: argument validation, page geometry,
// split planning and kernel dispatch.  See include/kvq.h for the contract.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <atomic>
#include <cstdint>

#include "kvq.h"
#include "kvq_internal.h"

using namespace kvq;

namespace {

bool valid_scale(float s) { return isfinite(s) && s >= 0x1p-64f && s <= 0x1p64f; }

// Layout check shared by every entry point.
kvq_status check_layout(const kvq_layout* L) {
  if (!L) return KVQ_ERR_INVALID_ARG;
  if (L->num_kv_heads < 1 || L->num_pages < 1 || L->head_dim < 1 || L->page_size < 1)
    return KVQ_ERR_INVALID_ARG;
  switch (L->format) {
    case KVQ_FP8_PER_TENSOR:
    case KVQ_INT8_PTH:
    case KVQ_FP8_PTH:
    case KVQ_NVFP4:
    case KVQ_INT4_PTH:
    case KVQ_MXFP4:
      if (L->head_dim != 32 && L->head_dim != 64 && L->head_dim != 128) return KVQ_ERR_UNSUPPORTED;
      if (L->page_size < 16 || L->page_size > 256 || (L->page_size & (L->page_size - 1))) return KVQ_ERR_UNSUPPORTED;
      break;
    case KVQ_KVARN_K4V2_G128:
      if (L->head_dim != 128 || (L->page_size != 128 && L->page_size != 256)) return KVQ_ERR_UNSUPPORTED;
      break;
    default:
      return KVQ_ERR_UNSUPPORTED;
  }
  if (L->flags & ~KVQ_FLAG_NVFP4_4OVER6) return KVQ_ERR_INVALID_ARG;
  if ((L->flags & KVQ_FLAG_NVFP4_4OVER6) && L->format != KVQ_NVFP4) return KVQ_ERR_INVALID_ARG;
  if ((L->format == KVQ_FP8_PER_TENSOR || L->format == KVQ_NVFP4) &&
      !(valid_scale(L->k_scale) && valid_scale(L->v_scale)))
    return KVQ_ERR_INVALID_ARG;
  return KVQ_OK;
}

ChunkGeom geometry(const kvq_layout* L) {
  const int64_t D = L->head_dim, P = L->page_size;
  ChunkGeom g{};
  switch (L->format) {
    case KVQ_FP8_PER_TENSOR:
      g.v_codes = P * D;
      g.k_scales = g.v_scales = 2 * P * D;
      g.chunk_bytes = 2 * P * D;
      break;
    case KVQ_INT8_PTH:
    case KVQ_FP8_PTH:
      g.v_codes = P * D;
      g.k_scales = 2 * P * D;
      g.v_scales = 2 * P * D + 4 * P;
      g.chunk_bytes = 2 * P * D + 8 * P;
      break;
    case KVQ_INT4_PTH:
      g.v_codes = P * D / 2;
      g.k_scales = P * D;
      g.v_scales = P * D + 4 * P;
      g.chunk_bytes = P * D + 8 * P;
      break;
    case KVQ_NVFP4:
      g.v_codes = P * D / 2;
      g.k_scales = P * D;
      g.v_scales = P * D + P * D / 16;
      g.chunk_bytes = P * D + P * D / 8;
      break;
    case KVQ_MXFP4:
      g.v_codes = P * D / 2;
      g.k_scales = P * D;
      g.v_scales = P * D + P * D / 32;
      g.chunk_bytes = P * D + P * D / 16;
      break;
    case KVQ_KVARN_K4V2_G128: {
      // P / 128 tiles back to back; offsets inside one tile
      constexpr int64_t T = 128;
      g.v_codes = T * D / 2;
      g.k_scales = T * D / 2 + T * D / 4;  // start of the fp32 metadata
      g.v_scales = g.k_scales + 4 * (2 * D + T);
      g.chunk_bytes = (P / T) * (T * D / 2 + T * D / 4 + 4 * (3 * D + 3 * T));
      break;
    }
  }
  return g;
}

// Device capability, cached per device id (0 = unknown, 1 = gfx950, 2 = other).
std::atomic<int> g_dev_ok[64];

kvq_status device_ok(int dev) {
  if (dev < 0) return KVQ_ERR_DEVICE;
  if (dev < 64) {
    const int c = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (c) return c == 1 ? KVQ_OK : KVQ_ERR_DEVICE;
  }
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || dev >= count) return KVQ_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return KVQ_ERR_DEVICE;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_dev_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? KVQ_OK : KVQ_ERR_DEVICE;
}

kvq_status current_device_ok() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return KVQ_ERR_DEVICE;
  return device_ok(dev);
}

kvq_status from_hip(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

// The kernels move binary16 rows, cache bytes, split records and the KVarN
// tail with 16-byte vector accesses, and read the index arrays as naturally
// aligned words; a pointer off those alignments is rejected before launch.
bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

// The split kernel's unit of work along the context: a page, or for KVarN a
// 128-token tile (a page holds page_size / 128 of them).
int plan_units(const kvq_layout* L, int max_pages) {
  return L->format == KVQ_KVARN_K4V2_G128 ? max_pages * (L->page_size / 128) : max_pages;
}

// Context splits per (sequence, kv head): enough workgroups for one resident
// round of the split kernel, i.e. compute units x the kernel's resident
// workgroups per compute unit, while keeping at least 8 pages (two per
// wavefront) in a split.  Empty trailing splits are dropped.  The 4-bit
// formats' kernels are bound by instruction issue and latency, and a third
// resident workgroup per CU (their registers allow it) hides more of it
// (~10% on MI355X); the 8-bit formats are bound by HBM, where a third
// workgroup only adds contention, so they stay at 2.  Both figures come from
// the current device and are cached per device; without a usable device the
// plan assumes MI355X's 256 compute units and 2 workgroups per CU.
constexpr int kMaxDevices = 64;
constexpr int kFallbackCUs = 256;
constexpr int kFallbackBlocksPerCU = 2;
std::atomic<int> g_cu_count[kMaxDevices];
std::atomic<int> g_blocks_per_cu[kMaxDevices][8][3][4];  // [dev][format][D 32/64/128][G 1/2/4/8]

int index_of_d(int D) { return D == 32 ? 0 : (D == 64 ? 1 : 2); }
int index_of_g(int G) { return G == 1 ? 0 : (G == 2 ? 1 : (G == 4 ? 2 : 3)); }

struct Residency {
  int cus, per_cu;  // compute units; resident split workgroups (4 waves) per unit
};

Residency residency(const kvq_layout* L, int G) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices || device_ok(dev) != KVQ_OK ||
      L->format < 1 || L->format > 7 || (G != 1 && G != 2 && G != 4 && G != 8))
    return Residency{kFallbackCUs, kFallbackBlocksPerCU};
  int cus = g_cu_count[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = kFallbackCUs;
    g_cu_count[dev].store(cus, std::memory_order_relaxed);
  }
  std::atomic<int>& slot = g_blocks_per_cu[dev][L->format][index_of_d(L->head_dim)][index_of_g(G)];
  int per_cu = slot.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    per_cu = L->format == KVQ_KVARN_K4V2_G128 ? kvarn_decode_blocks_per_cu(G)
                                              : decode_blocks_per_cu(L->format, L->head_dim, G);
    if (per_cu < 1) per_cu = kFallbackBlocksPerCU;
    const bool eight_bit = L->format == KVQ_FP8_PER_TENSOR || L->format == KVQ_INT8_PTH || L->format == KVQ_FP8_PTH;
    if (eight_bit && per_cu > 2) per_cu = 2;
    slot.store(per_cu, std::memory_order_relaxed);
  }
  return Residency{cus, per_cu};
}

void plan_splits(int batch, int H, int max_pages, int hint, int64_t target, int* splits, int* pages_per_split,
                 int* waves) {
  const int64_t units = (int64_t)batch * H;
  int s = hint;
  if (s <= 0) {
    const int64_t want = units > 0 ? (target + units - 1) / units : 1;
    const int64_t cap = (max_pages + 7) / 8;
    s = (int)(want < cap ? want : cap);
  }
  if (s > kMaxSplits) s = kMaxSplits;
  if (s > max_pages) s = max_pages;
  if (s < 1) s = 1;
  int pps = (max_pages + s - 1) / s;
  if (pps < 1) pps = 1;
  *pages_per_split = pps;
  *splits = (max_pages + pps - 1) / pps;
  if (*splits < 1) *splits = 1;
  *waves = 4;
}

// The library's plan for a decode problem.  When the automatic plan asks for
// two splits of four-wave workgroups, two resident per compute unit, and
// every compute unit already gets a (sequence, kv head) of its own, one
// eight-wave workgroup per pair keeps the same waves resident with no split
// partials and no merge launch.
void plan(const kvq_layout* L, int batch, int G, int max_pages, int hint, int* splits, int* pps, int* waves) {
  const Residency r = residency(L, G);
  plan_splits(batch, L->num_kv_heads, plan_units(L, max_pages), hint, (int64_t)r.cus * r.per_cu, splits, pps,
              waves);
  if (hint == 0 && L->format != KVQ_KVARN_K4V2_G128 && r.per_cu == 2 && *splits == 2 &&
      (int64_t)batch * L->num_kv_heads >= r.cus) {
    *splits = 1;
    *pps = max_pages;
    *waves = 8;
  }
}

int64_t workspace_bytes_for(const kvq_layout* L, int batch, int splits) {
  if (splits <= 1 && L->format != KVQ_KVARN_K4V2_G128) return 0;
  return (int64_t)batch * L->num_kv_heads * splits * ws_record_floats(L->head_dim) * 4;
}

WriteArgs write_args(const kvq_layout* L, const void* k, const void* v, const int64_t* slots, int64_t n_tok,
                     void* cache) {
  WriteArgs a{};
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.slots = slots;
  a.n_tok = n_tok;
  a.cache = static_cast<uint8_t*>(cache);
  a.geom = geometry(L);
  a.H = L->num_kv_heads;
  a.D = L->head_dim;
  a.P = L->page_size;
  a.num_pages = L->num_pages;
  a.k_scale = L->k_scale;
  a.v_scale = L->v_scale;
  a.flags = L->flags;
  return a;
}

// Argument checks shared by the decode entry points, up to the workspace; on
// success the plan and the workspace bytes it needs.
kvq_status check_decode_plan(const kvq_layout* L, const void* cache, const void* q, int32_t num_q_heads,
                             const int32_t* block_tables, int32_t max_pages_per_seq, const int32_t* context_lens,
                             int32_t batch, float sm_scale, void* out, int32_t num_splits, int* splits, int* pps,
                             int* waves, int64_t* need) {
  kvq_status st = check_layout(L);
  if (st != KVQ_OK) return st;
  const int H = L->num_kv_heads;
  if (batch < 0 || num_q_heads < 1 || max_pages_per_seq < 1 || num_splits < 0 || !isfinite(sm_scale))
    return KVQ_ERR_INVALID_ARG;
  if (num_q_heads % H != 0) return KVQ_ERR_INVALID_ARG;
  const int G = num_q_heads / H;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVQ_ERR_UNSUPPORTED;
  if (batch > 0 && (!cache || !q || !block_tables || !context_lens || !out)) return KVQ_ERR_INVALID_ARG;
  if (!aligned(cache, 16) || !aligned(q, 16) || !aligned(out, 16) || !aligned(block_tables, 4) ||
      !aligned(context_lens, 4))
    return KVQ_ERR_INVALID_ARG;
  plan(L, batch, G, max_pages_per_seq, num_splits, splits, pps, waves);
  *need = workspace_bytes_for(L, batch, *splits);
  return KVQ_OK;
}

// The same, then the caller's workspace and the device.
kvq_status check_decode(const kvq_layout* L, const void* cache, const void* q, int32_t num_q_heads,
                        const int32_t* block_tables, int32_t max_pages_per_seq, const int32_t* context_lens,
                        int32_t batch, float sm_scale, void* out, void* workspace, int64_t workspace_bytes,
                        int32_t num_splits, int* splits, int* pps, int* waves) {
  int64_t need = 0;
  const kvq_status st = check_decode_plan(L, cache, q, num_q_heads, block_tables, max_pages_per_seq, context_lens,
                                          batch, sm_scale, out, num_splits, splits, pps, waves, &need);
  if (st != KVQ_OK) return st;
  if (workspace_bytes < need) return KVQ_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && (!workspace || !aligned(workspace, 16))) return KVQ_ERR_INVALID_ARG;
  return current_device_ok();
}

DecodeArgs decode_args(const kvq_layout* L, const void* cache, const void* q, int32_t num_q_heads,
                       const int32_t* block_tables, int32_t max_pages_per_seq, const int32_t* context_lens,
                       int32_t batch, float sm_scale, void* out, void* workspace, int splits, int pps, int waves) {
  DecodeArgs a{};
  a.cache = static_cast<const uint8_t*>(cache);
  a.geom = geometry(L);
  a.H = L->num_kv_heads;
  a.D = L->head_dim;
  a.P = L->page_size;
  a.num_pages = L->num_pages;
  a.q = static_cast<const uint16_t*>(q);
  a.Hq = num_q_heads;
  a.G = num_q_heads / a.H;
  a.block_tables = block_tables;
  a.max_pages = max_pages_per_seq;
  a.ctx_lens = context_lens;
  a.B = batch;
  a.qk_scale = sm_scale * 1.4426950408889634f;
  a.k_scale = L->k_scale;
  a.v_scale = L->v_scale;
  a.out = static_cast<uint16_t*>(out);
  a.workspace = static_cast<uint8_t*>(workspace);
  a.num_splits = splits;
  a.pages_per_split = pps;
  a.waves = waves;
  a.sp_shift = __builtin_ctz(L->page_size / 16);
  return a;
}

}  // namespace

extern "C" {

int64_t kvq_page_bytes(const kvq_layout* layout) {
  if (check_layout(layout) != KVQ_OK) return -1;
  return geometry(layout).chunk_bytes * layout->num_kv_heads;
}

kvq_status kvq_check_device(int hip_device) { return device_ok(hip_device); }

kvq_status kvq_quantize_write(const kvq_layout* layout, const void* k, const void* v,
                              const int64_t* slot_mapping, int64_t n_tok, void* cache, void* stream) {
  kvq_status st = check_layout(layout);
  if (st != KVQ_OK) return st;
  if (n_tok < 0) return KVQ_ERR_INVALID_ARG;
  if (layout->format == KVQ_KVARN_K4V2_G128 && n_tok % 128 != 0) return KVQ_ERR_INVALID_ARG;
  if (n_tok > 0 && (!k || !v || !slot_mapping || !cache)) return KVQ_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(cache, 16) || !aligned(slot_mapping, 8))
    return KVQ_ERR_INVALID_ARG;
  if ((st = current_device_ok()) != KVQ_OK) return st;
  if (n_tok == 0) return KVQ_OK;
  const WriteArgs a = write_args(layout, k, v, slot_mapping, n_tok, cache);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (layout->format == KVQ_KVARN_K4V2_G128) return from_hip(launch_kvarn_write(a, s));
  return from_hip(launch_quant_write(layout->format, a, s));
}

kvq_status kvq_kvarn_append(const kvq_layout* layout, const void* k, const void* v, const int32_t* seq,
                            const int32_t* pos, int64_t n_tok, void* tail, int32_t batch, const int32_t* block_tables,
                            int32_t max_pages_per_seq, void* cache, void* stream) {
  kvq_status st = check_layout(layout);
  if (st != KVQ_OK) return st;
  if (layout->format != KVQ_KVARN_K4V2_G128) return KVQ_ERR_INVALID_ARG;
  if (n_tok < 0 || batch < 0 || max_pages_per_seq < 1) return KVQ_ERR_INVALID_ARG;
  if (n_tok > 0 && (!k || !v || !seq || !pos || !tail || !block_tables || !cache)) return KVQ_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(tail, 16) || !aligned(cache, 16) || !aligned(seq, 4) ||
      !aligned(pos, 4) || !aligned(block_tables, 4))
    return KVQ_ERR_INVALID_ARG;
  if ((st = current_device_ok()) != KVQ_OK) return st;
  if (n_tok == 0 || batch == 0) return KVQ_OK;
  KvarnAppendArgs a{};
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.seq = seq;
  a.pos = pos;
  a.n_tok = n_tok;
  a.tail = static_cast<uint16_t*>(tail);
  a.batch = batch;
  a.block_tables = block_tables;
  a.max_pages = max_pages_per_seq;
  a.cache = static_cast<uint8_t*>(cache);
  a.chunk_bytes = geometry(layout).chunk_bytes;
  a.P = layout->page_size;
  a.H = layout->num_kv_heads;
  a.num_pages = layout->num_pages;
  return from_hip(launch_kvarn_append(a, static_cast<hipStream_t>(stream)));
}

int32_t kvq_decode_num_splits(const kvq_layout* layout, int32_t batch, int32_t num_q_heads,
                              int32_t max_pages_per_seq, int32_t num_splits) {
  if (check_layout(layout) != KVQ_OK || batch < 0 || max_pages_per_seq < 1 || num_splits < 0 ||
      num_q_heads < 1 || num_q_heads % layout->num_kv_heads != 0)
    return -1;
  int s, pps, waves;
  plan(layout, batch, num_q_heads / layout->num_kv_heads, max_pages_per_seq, num_splits, &s, &pps, &waves);
  return s;
}

int64_t kvq_decode_workspace_bytes(const kvq_layout* layout, int32_t batch, int32_t num_q_heads,
                                   int32_t max_pages_per_seq, int32_t num_splits) {
  if (check_layout(layout) != KVQ_OK || batch < 0 || max_pages_per_seq < 1 || num_splits < 0 ||
      num_q_heads < 1 || num_q_heads % layout->num_kv_heads != 0)
    return -1;
  int s, pps, waves;
  plan(layout, batch, num_q_heads / layout->num_kv_heads, max_pages_per_seq, num_splits, &s, &pps, &waves);
  return workspace_bytes_for(layout, batch, s);
}

kvq_status kvq_decode_attention(const kvq_layout* layout, const void* cache, const void* q,
                                int32_t num_q_heads, const int32_t* block_tables, int32_t max_pages_per_seq,
                                const int32_t* context_lens, int32_t batch, float sm_scale,
                                const void* kvarn_tail, void* out, void* workspace, int64_t workspace_bytes,
                                int32_t num_splits, void* stream) {
  if (kvarn_tail && layout && layout->format != KVQ_KVARN_K4V2_G128) return KVQ_ERR_INVALID_ARG;
  if (!aligned(kvarn_tail, 16)) return KVQ_ERR_INVALID_ARG;
  int splits, pps, waves;
  const kvq_status st = check_decode(layout, cache, q, num_q_heads, block_tables, max_pages_per_seq, context_lens,
                                     batch, sm_scale, out, workspace, workspace_bytes, num_splits, &splits, &pps,
                                     &waves);
  if (st != KVQ_OK || batch == 0) return st;
  DecodeArgs a = decode_args(layout, cache, q, num_q_heads, block_tables, max_pages_per_seq, context_lens, batch,
                             sm_scale, out, workspace, splits, pps, waves);
  a.tail = static_cast<const uint16_t*>(kvarn_tail);
  if (layout->format == KVQ_KVARN_K4V2_G128)
    return from_hip(launch_kvarn_decode(a, static_cast<hipStream_t>(stream)));
  return from_hip(launch_decode(layout->format, a, static_cast<hipStream_t>(stream)));
}

kvq_status kvq_decode_attention_noalloc(const kvq_layout* layout, const void* cache, const void* q,
                                        int32_t num_q_heads, const int32_t* block_tables, int32_t max_pages_per_seq,
                                        const int32_t* context_lens, int32_t batch, float sm_scale,
                                        const void* kvarn_tail, void* out, int32_t num_splits, void* stream) {
  if (kvarn_tail && layout && layout->format != KVQ_KVARN_K4V2_G128) return KVQ_ERR_INVALID_ARG;
  if (!aligned(kvarn_tail, 16)) return KVQ_ERR_INVALID_ARG;
  int splits, pps, waves;
  int64_t need = 0;
  kvq_status st = check_decode_plan(layout, cache, q, num_q_heads, block_tables, max_pages_per_seq, context_lens,
                                    batch, sm_scale, out, num_splits, &splits, &pps, &waves, &need);
  if (st != KVQ_OK) return st;
  if (need > (int64_t)KVQ_DECODE_SCRATCH_BYTES) return KVQ_ERR_SCRATCH_TOO_SMALL;
  if ((st = current_device_ok()) != KVQ_OK || batch == 0) return st;
  void* scratch = nullptr;
  if (need > 0) {
    const hipError_t e = decode_scratch(&scratch);
    if (e != hipSuccess) return from_hip(e);
  }
  DecodeArgs a = decode_args(layout, cache, q, num_q_heads, block_tables, max_pages_per_seq, context_lens, batch,
                             sm_scale, out, scratch, splits, pps, waves);
  a.tail = static_cast<const uint16_t*>(kvarn_tail);
  if (layout->format == KVQ_KVARN_K4V2_G128)
    return from_hip(launch_kvarn_decode(a, static_cast<hipStream_t>(stream)));
  return from_hip(launch_decode(layout->format, a, static_cast<hipStream_t>(stream)));
}

kvq_status kvq_decode_attention_append(const kvq_layout* layout, void* cache, const void* k_new,
                                       const void* v_new, const int64_t* slot_mapping, const void* q,
                                       int32_t num_q_heads, const int32_t* block_tables,
                                       int32_t max_pages_per_seq, const int32_t* context_lens, int32_t batch,
                                       float sm_scale, void* out, void* workspace, int64_t workspace_bytes,
                                       int32_t num_splits, void* stream) {
  if (layout && layout->format == KVQ_KVARN_K4V2_G128) return KVQ_ERR_INVALID_ARG;
  if (batch > 0 && (!k_new || !v_new || !slot_mapping)) return KVQ_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(slot_mapping, 8)) return KVQ_ERR_INVALID_ARG;
  int splits, pps, waves;
  const kvq_status st = check_decode(layout, cache, q, num_q_heads, block_tables, max_pages_per_seq, context_lens,
                                     batch, sm_scale, out, workspace, workspace_bytes, num_splits, &splits, &pps,
                                     &waves);
  if (st != KVQ_OK || batch == 0) return st;
  const WriteArgs w = write_args(layout, k_new, v_new, slot_mapping, batch, cache);
  DecodeArgs a = decode_args(layout, cache, q, num_q_heads, block_tables, max_pages_per_seq, context_lens, batch,
                             sm_scale, out, workspace, splits, pps, waves);
  hipStream_t s = static_cast<hipStream_t>(stream);
  a.new_slots = slot_mapping;
  a.wnew = w;
  return from_hip(launch_decode(layout->format, a, s));
}

kvq_status kvq_dequantize(const kvq_layout* layout, const void* cache, const int64_t* slot_mapping,
                          int64_t n_tok, float* k_out, float* v_out, void* stream) {
  kvq_status st = check_layout(layout);
  if (st != KVQ_OK) return st;
  if (n_tok < 0) return KVQ_ERR_INVALID_ARG;
  if (n_tok > 0 && (!cache || !slot_mapping || !k_out || !v_out)) return KVQ_ERR_INVALID_ARG;
  if (!aligned(cache, 16) || !aligned(slot_mapping, 8) || !aligned(k_out, 4) || !aligned(v_out, 4))
    return KVQ_ERR_INVALID_ARG;
  if ((st = current_device_ok()) != KVQ_OK) return st;
  if (n_tok == 0) return KVQ_OK;
  WriteArgs a{};
  a.slots = slot_mapping;
  a.n_tok = n_tok;
  a.cache = static_cast<uint8_t*>(const_cast<void*>(cache));
  a.geom = geometry(layout);
  a.H = layout->num_kv_heads;
  a.D = layout->head_dim;
  a.P = layout->page_size;
  a.num_pages = layout->num_pages;
  a.k_scale = layout->k_scale;
  a.v_scale = layout->v_scale;
  return from_hip(launch_dequant(layout->format, a, k_out, v_out, static_cast<hipStream_t>(stream)));
}

kvq_status kvq_take_device_errors(uint32_t* flags, void* stream) {
  if (!flags) return KVQ_ERR_INVALID_ARG;
  kvq_status st = current_device_ok();
  if (st != KVQ_OK) return st;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return KVQ_ERR_HIP;
  return from_hip(take_device_errors(flags));
}

const char* kvq_status_string(kvq_status status) {
  switch (status) {
    case KVQ_OK: return "success";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported layout or shape";
    case KVQ_ERR_WORKSPACE_TOO_SMALL: return "decode workspace too small";
    case KVQ_ERR_DEVICE: return "current device is not an MI355X (gfx950)";
    case KVQ_ERR_HIP: return "a HIP call failed (kernel launch or device query)";
    case KVQ_ERR_SCRATCH_TOO_SMALL:
      return "problem needs more split records than the fixed decode workspace (KVQ_DECODE_SCRATCH_BYTES) holds";
  }
  return "unknown status";
}

}  // extern "C"
