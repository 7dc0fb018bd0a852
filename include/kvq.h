/*
 * kvq.h -- C ABI of libkvq: KV-cache quantise-on-write and dequant-fused paged
 * GQA decode attention for AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (cited by page title and section):
 *   [P1] "KV Cache 量化深度解析：Per-Tensor、Per-Token-Head 与 NVFP4"
 *   [P2] "KVarN：华为推出的原生 vLLM KV-cache 量化后端"
 *   [P3] "KV Cache 量化 · LLM Glossary"
 *   [P4] "KV 量化" (vLLM / SGLang source walk-through)
 *   [P5] "NVFP4 KV Cache：Blackwell 上的 4-bit 缓存量化"
 *
 * Conventions for every entry point:
 *   - All pointers except `layout` are device pointers (HIP global memory) on the
 *     current HIP device, unless stated.  The caller owns every buffer; the
 *     library allocates no device memory and keeps no device state between
 *     calls (it only memoises, per device, the host-side answers of the HIP
 *     compute-unit and occupancy queries behind the split plan), apart from
 *     the fixed device array that kvq_decode_attention_noalloc uses as its
 *     workspace, which is part of the library's code object.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; the returned status covers argument validation and
 *     kernel-launch errors only.
 *   - Unsupported combinations are rejected with KVQ_ERR_UNSUPPORTED or
 *     KVQ_ERR_INVALID_ARG before anything is launched; the library never falls
 *     back to another format ([P5] §一条完整的上线验证路径 asks that a missing
 *     capability be explicit).
 *   - Tensors are dense and contiguous in the stated shapes; binary16 is IEEE
 *     half precision; inputs are finite.
 *   - Alignment: binary16 tensors, caches, workspaces and the KVarN tail start
 *     on 16-byte boundaries, int32 and int64 arrays and binary32 outputs on
 *     their own size (torch allocations satisfy all of them); other pointers
 *     are rejected with KVQ_ERR_INVALID_ARG before anything is launched.
 *
 * Cache layout (the storage contract; page_bytes = num_kv_heads * chunk_bytes):
 *   the chunk of (page p, kv head h) starts at byte (p * H + h) * chunk_bytes.
 *   Inside a chunk, with P = page_size, D = head_dim, t = token offset in the
 *   page and d = channel:
 *   8-bit formats (FP8 per-tensor, INT8 and FP8 per-token-head): K codes at
 *   0 and V codes at P*D, each 16*D bytes per group of 16 tokens (u = t/16,
 *   s = t%16, group at 16*D*u), B = min(16, D/4):
 *     K  d = (D/4)*g + B*h + e         ->  64*B*h + 16*B*g + B*s + e
 *     V  d = (D/16)*n + (B/4)*h + j    ->  64*B*h + 16*B*(s/4) + B*n + 4*j + s%4
 *     (so that each 16-byte decode load of a wavefront reads one contiguous
 *     run); per-token-head only: K scales fp32 [P] at 2*P*D, then V scales
 *   NVFP4 (low nibble = even channel):
 *     K codes  [P][D/2]     at 0         byte t*D/2 + d/2
 *     V codes  [P/4][D/2][4] at P*D/2    byte 2*D*(t/4) + 4*(d/2) + t%4
 *     K block scales E4M3 [P][D/16]  at P*D     byte t*D/16 + d/16
 *     V block scales E4M3 [D/16][P]  after them byte (d/16)*P + t
 *   MXFP4: the NVFP4 code layout, with E8M0 block scales per 32 channels
 *     K block scales E8M0 [P][D/32]  at P*D     byte t*D/32 + d/32
 *     V block scales E8M0 [D/32][P]  after them byte (d/32)*P + t
 *   INT4 per-token-head (two's-complement nibbles, low nibble = even channel):
 *     K codes  [P][D/2]     at 0         byte t*D/2 + d/2
 *     V codes  [P/4][D/2][4] at P*D/2    byte 2*D*(t/4) + 4*(d/2) + t%4
 *     K scales fp32 [P] at P*D, then V scales fp32 [P]
 *   KVarN k4v2 g128 (D = 128, P = 128 or 256): the chunk holds P/128 tiles
 *   of 128 tokens back to back, 15360 bytes each; tile k holds the page's
 *   tokens 128k .. 128k+127 and t below is a token's offset in its tile
 *   (T = 128):
 *     K codes 4-bit [T][D/2] at 0        byte t*D/2 + d/2, low nibble = even d
 *     V codes 2-bit [T/4][D] at T*D/2    byte D*(t/4) + d, bits 2(t%4)+1..2(t%4)
 *     fp32 K alpha[D], K beta[D], K rho[T], V alpha[T], V beta[T], V gamma[D]
 *     (rotated tile rebuilt as K = rho_t (alpha_d code + beta_d),
 *      V = gamma_d (alpha_t code + beta_t); see kvq_quantize_write)
 *   Codes: INT8 = two's-complement byte; FP8 = OCP E4M3 ("fn", max 448);
 *   NVFP4 = E2M1 nibble (sign bit 3) with E4M3 block scales; MXFP4 = E2M1
 *   nibble with E8M0 block scales (byte e is 2^(e-127)); INT4 =
 *   two's-complement nibble, -7..7.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage formats.  Values 1..4 follow the mode numbering of vLLM's
 * KVQuantMode listed in [P1] §二 (NONE = 0 is not a cache format here);
 * 5 is KVarN's k4v2 g128 preset ([P2] §配置与部署); 6 is vLLM's
 * int4_per_token_head mode ([P4] §scale 和数据放在一起); 7 is MXFP4, the
 * comparison point of [P5] §双层缩放怎样恢复动态范围. */
typedef enum {
  KVQ_FP8_PER_TENSOR = 1,  /* [P1] §2.1, [P4] §FP8 per-tensor */
  KVQ_INT8_PTH = 2,        /* per-token-head INT8, [P3] §它改变缓存表示 */
  KVQ_FP8_PTH = 3,         /* per-token-head FP8, [P1] §2.2 */
  KVQ_NVFP4 = 4,           /* [P5] §双层缩放怎样恢复动态范围 */
  KVQ_KVARN_K4V2_G128 = 5, /* [P2] §技术原理 */
  KVQ_INT4_PTH = 6,        /* per-token-head INT4, [P4] §scale 和数据放在一起 */
  KVQ_MXFP4 = 7            /* 32-value E2M1 blocks, E8M0 scale, [P5] §双层缩放怎样恢复动态范围 */
} kvq_format;

/* NVFP4 only: per block, keep the max/4 block scale instead of max/6 when its
 * squared reconstruction error is strictly smaller ([P5] §用一组数直观看缩放的作用). */
#define KVQ_FLAG_NVFP4_4OVER6 1u

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = 1,         /* NULL pointer, negative size, bad scale */
  KVQ_ERR_UNSUPPORTED = 2,         /* valid request the library does not serve */
  KVQ_ERR_WORKSPACE_TOO_SMALL = 3, /* decode workspace smaller than required */
  KVQ_ERR_DEVICE = 4,              /* current device is not gfx950 */
  KVQ_ERR_HIP = 5,                 /* a HIP call failed (launch error) */
  KVQ_ERR_SCRATCH_TOO_SMALL = 6    /* problem needs more than KVQ_DECODE_SCRATCH_BYTES of
                                      split records (kvq_decode_attention_noalloc) */
} kvq_status;

/* Size of the fixed per-device workspace of kvq_decode_attention_noalloc:
 * 16 MiB, i.e. 4032 split records at head size 128 (4160 bytes each). */
#define KVQ_DECODE_SCRATCH_BYTES (16u << 20)

/* One attention layer's cache description.
 *   format       kvq_format
 *   flags        KVQ_FLAG_* (only KVQ_FLAG_NVFP4_4OVER6, NVFP4 only)
 *   num_kv_heads H, >= 1
 *   head_dim     D: 32, 64 or 128 (KVarN: 128)
 *   page_size    P tokens per page: 16, 32, 64, 128 or 256 (KVarN: 128 or 256,
 *                i.e. one or two 128-token tiles)
 *   num_pages    pages in the pool, >= 1
 *   k_scale, v_scale  FP8 per-tensor: the layer's K and V scales (divide on
 *                write, multiply on read; [P4] §写和读).  NVFP4: the per-layer
 *                FP32 global scales s_t of K and V.  Finite, in
 *                [2^-64, 2^64].  Ignored by the other formats. */
typedef struct {
  int32_t format;
  int32_t flags;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t num_pages;
  float k_scale;
  float v_scale;
} kvq_layout;

/* Bytes of one page (all kv heads, K and V, codes and in-page scales): the real
 * page size the pool must be sized with ([P5] §“4 bit”为什么不是严格的 4
 * bits/value; [P4] §scale 和数据放在一起).  Host-only.  Returns -1 for an
 * invalid or unsupported layout. */
int64_t kvq_page_bytes(const kvq_layout* layout);

/* KVQ_OK if HIP device `hip_device` is a gfx950 (MI355X), else KVQ_ERR_DEVICE
 * (also when no device is present).  Host-only, no kernel launched.  The
 * load-time capability check of [P5] §需要记录的系统指标 (correctness list),
 * so that an unsupported device fails at initialisation rather than at the
 * first request (§Blackwell 支持不是一个单一布尔值: fail fast, never fall back
 * silently).  Every launching entry point makes the same check. */
kvq_status kvq_check_device(int hip_device);

/* Quantise-on-write ([P5] §KV 的写入与读取路径, write path; [P4] §写和读).
 *   k, v          binary16 [n_tok][H][D], freshly computed keys and values.
 *   slot_mapping  int64 [n_tok]: token i goes to slot page * P + offset.
 *                 Negative slots and slots >= num_pages * P are skipped.
 *   cache         uint8 [num_pages * page_bytes], written in place.
 * Per format (binary32 arithmetic, correctly rounded division, ties-to-even):
 *   FP8 per-tensor:   code = E4M3(x / k_scale) (v_scale for V), saturating at
 *                     448; no scale stored.
 *   INT8 per-token-head: s = max(max|x|, 1e-8) / 127, code = clip(rne(x / s),
 *                     -127, 127); s stored in-page ([P3] formula and script).
 *   FP8 per-token-head: s = max(max|x|, 1e-8) / 448, code = E4M3(x / s)
 *                     ([P1] §2.2 with FP8_MAX = 448).
 *   INT4 per-token-head: s = max(max|x|, 1e-8) / 7, code = clip(rne(x / s),
 *                     -7, 7), s stored in-page (the INT8 rule at 4 bits: the
 *                     page lists the mode and its half-width layout only).
 *   NVFP4:            per 16 channels, s_b = E4M3((max|x| / 6) / s_t),
 *                     code = E2M1(x / (s_t * s_b)) (ties to even, saturating
 *                     at 6); a block whose s_b decodes to 0 stores zero codes.
 *                     With KVQ_FLAG_NVFP4_4OVER6 the max/4 candidate is kept
 *                     when its binary32 squared error is strictly smaller.
 *   MXFP4:            per 32 channels, X = 2^(floor(log2 max|x|) - 2),
 *                     code = E2M1(x / X) (exact division; ties to even,
 *                     saturating at 6), scale byte floor(log2 max|x|) + 125;
 *                     an all-zero block stores byte 0.  The page names only
 *                     the block size and the E8M0 scale; the rule is the OCP
 *                     Microscaling block conversion.  No per-layer scale.
 *   KVarN k4v2 g128:  per 128-token tile and kv head ([P2] §技术原理):
 *                     normalised Sylvester Walsh-Hadamard rotation of every
 *                     token row, 4 sweeps of alternating token / channel
 *                     deviation normalisation, asymmetric RTN (K: 4-bit per
 *                     channel over the tile's tokens; V: 2-bit per token over
 *                     channels), scales folded into the metadata above.
 *                     Requires n_tok % 128 == 0; tokens 128i..128i+127 must
 *                     map to slots s0 + 0..127 of one tile of a page, s0 a
 *                     multiple of 128.  A run whose first slot is outside
 *                     the pool is skipped; a run that breaks the rule
 *                     otherwise is skipped and raises
 *                     KVQ_DEVERR_KVARN_TILE_SLOTS (kvq_take_device_errors).
 * Errors: KVQ_ERR_INVALID_ARG for NULL pointers, n_tok < 0, bad scales or a
 * KVarN n_tok not a multiple of 128; KVQ_ERR_UNSUPPORTED for layouts outside
 * the list above; KVQ_ERR_DEVICE off gfx950. */
kvq_status kvq_quantize_write(const kvq_layout* layout, const void* k, const void* v,
                              const int64_t* slot_mapping, int64_t n_tok, void* cache,
                              void* stream);

/* KVarN incremental write ([P2] §配置与部署: decode keeps the tokens of the
 * incomplete last tile unquantised in a small fixed buffer; a tile is
 * quantised once it is complete).  For decode steps and short appends.
 *   k, v          binary16 [n_tok][H][128], new tokens.
 *   seq           int32 [n_tok]: the sequence of each token, in [0, batch).
 *   pos           int32 [n_tok]: the token's position in its sequence (the
 *                 sequence's length before this token).
 *   tail          binary16 [batch][2][H][128][128], the same buffer
 *                 kvq_decode_attention reads: token i is copied to row
 *                 pos[i] % 128 of sequence seq[i] (keys, then values).
 *   block_tables  int32 [batch][max_pages_per_seq] as for decode.
 *   cache         the paged cache.
 * A token at position 127 mod 128 completes its tile: rows 0..127 of the
 * sequence's tail are then quantised into tile (pos / 128) % (P / 128) of
 * page block_tables[seq][pos / P], with exactly the bytes kvq_quantize_write
 * gives for those 128 tokens.  Within one call, the tokens of a sequence must
 * lie in one tile and have distinct positions (a token of the next tile would
 * overwrite a tail row before the tile is quantised): a call that breaks this
 * raises KVQ_DEVERR_KVARN_APPEND_SPAN (kvq_take_device_errors) and leaves
 * that sequence's tail and tile undefined.  Entries with a sequence outside
 * [0, batch), a negative position or a page outside the pool are skipped.  Two launches on `stream` (copy, then tile completion).
 * Errors: KVQ_ERR_INVALID_ARG for a non-KVarN layout, NULL pointers or
 * negative sizes; KVQ_ERR_DEVICE off gfx950. */
kvq_status kvq_kvarn_append(const kvq_layout* layout, const void* k, const void* v, const int32_t* seq,
                            const int32_t* pos, int64_t n_tok, void* tail, int32_t batch,
                            const int32_t* block_tables, int32_t max_pages_per_seq, void* cache,
                            void* stream);

/* Bytes of workspace kvq_decode_attention needs for this problem (-1 if
 * invalid, including num_q_heads not a multiple of H), the "workspace bytes"
 * [P5] §需要记录的系统指标 asks to record (its §KV 的写入与读取路径 notes that
 * a decode which first expands the cache into a temporary buffer changes the
 * bandwidth and workspace cost; this one keeps only the split records): one partial record of
 * binary32 (max, sum, output row) per (sequence, kv head, context split), 0
 * when a single split is used (KVarN: always at least one record).
 * num_splits: 0 = let the library choose, else the number of context splits
 * per (sequence, kv head) to use (clamped to [1, min(256, max_pages_per_seq)]).
 * The library's choice fills one resident round of the split kernel on the
 * current HIP device (its compute units times the kernel's resident
 * workgroups per unit for this format, D and GQA group), with at least 8 pages
 * per split; where that asks for two splits of a kernel with two resident
 * workgroups per unit and batch * H reaches the number of compute units, it
 * runs one split of eight-wave workgroups instead (no workspace, no merge).
 * The choice is fixed per device and process, so a workspace sized here fits
 * every later call with the same arguments.  Without a usable device the
 * plan assumes 256 compute units and 2 workgroups per unit.  Host-only (no
 * kernel launched). */
int64_t kvq_decode_workspace_bytes(const kvq_layout* layout, int32_t batch, int32_t num_q_heads,
                                   int32_t max_pages_per_seq, int32_t num_splits);

/* Number of context splits kvq_decode_attention will use (-1 if invalid).
 * Same arguments and rules as kvq_decode_workspace_bytes; the split count
 * fixes the workspace bytes above ([P5] §需要记录的系统指标). */
int32_t kvq_decode_num_splits(const kvq_layout* layout, int32_t batch, int32_t num_q_heads,
                              int32_t max_pages_per_seq, int32_t num_splits);

/* Dequant-fused paged GQA decode attention ([P5] §K 与 V 的量化误差进入 attention
 * 的位置不同: O = softmax(Q K^T / sqrt(d) + M) V with M = 0 for decode; the
 * cache is read through block tables and dequantised in registers, never
 * expanded to a full-precision copy in memory, [P5] §KV 的写入与读取路径).
 *   cache          as written by kvq_quantize_write.
 *   q              binary16 [batch][num_q_heads][D]; q head h reads kv head
 *                  h / (num_q_heads / H); num_q_heads / H must be 1, 2, 4 or 8.
 *   block_tables   int32 [batch][max_pages_per_seq]: page of each P-token
 *                  block of a sequence; entries outside [0, num_pages) are
 *                  treated as empty pages (their tokens get zero weight).
 *   context_lens   int32 [batch]: tokens per sequence, clamped to
 *                  [0, max_pages_per_seq * P]; 0 gives a zero output row.
 *   sm_scale       logit scale, normally 1/sqrt(D).
 *   kvarn_tail     KVarN only: binary16 [batch][2][H][128][D] (keys, then
 *                  values); row j holds token ctx - ctx%128 + j for
 *                  j < ctx % 128, i.e. the tokens of the incomplete last tile,
 *                  attended in full precision.  May be NULL when every
 *                  context is a multiple of 128.  Must be NULL for other
 *                  formats.
 *   out            binary16 [batch][num_q_heads][D].
 *   workspace      device buffer of at least kvq_decode_workspace_bytes(...)
 *                  bytes (may be NULL when that is 0); its contents need no
 *                  preparation.  Two calls that overlap in time must not share
 *                  a workspace.
 *   num_splits     as for kvq_decode_workspace_bytes.
 * Launches one kernel, plus a small merge kernel when the context is split
 * (KVarN: always; its merge also attends the tail and rotates back).
 * Accumulation is binary32 (scores and softmax) on MFMA with binary16
 * operands split into high and low halves, so before the final binary16
 * rounding results track a binary64 reference to about 1e-5 relative (the
 * tests hold them to 1e-4). */
kvq_status kvq_decode_attention(const kvq_layout* layout, const void* cache, const void* q,
                                int32_t num_q_heads, const int32_t* block_tables,
                                int32_t max_pages_per_seq, const int32_t* context_lens,
                                int32_t batch, float sm_scale, const void* kvarn_tail, void* out,
                                void* workspace, int64_t workspace_bytes, int32_t num_splits,
                                void* stream);

/* kvq_decode_attention without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The split records live in a fixed
 * device array of KVQ_DECODE_SCRATCH_BYTES that the library defines; every
 * GPU it runs on holds one copy until the process ends.  The call itself
 * allocates nothing (no hipMalloc or hipFree, no allocating library routine);
 * its first call on a device looks up that device's copy of the array.
 *   Arguments, plan, kernels and results are those of kvq_decode_attention
 *   (same outputs bit for bit); the records need no initialisation, so the
 *   array's contents left by an earlier call do not matter.
 *   All calls on one GPU share its array: two calls that overlap in time on
 *   one device (on different streams, or from different host threads) race
 *   and give undefined results.  Calls in one stream are ordered.
 * Errors: those of kvq_decode_attention (the workspace ones excepted), and
 * KVQ_ERR_SCRATCH_TOO_SMALL, before anything is launched, when the problem
 * needs more than KVQ_DECODE_SCRATCH_BYTES of records (kvq_decode_workspace_bytes
 * with the same arguments tells). */
kvq_status kvq_decode_attention_noalloc(const kvq_layout* layout, const void* cache, const void* q,
                                        int32_t num_q_heads, const int32_t* block_tables,
                                        int32_t max_pages_per_seq, const int32_t* context_lens,
                                        int32_t batch, float sm_scale, const void* kvarn_tail, void* out,
                                        int32_t num_splits, void* stream);

/* One decode step in one call: quantise-write each sequence's new token and
 * run decode attention over its context, the new token included ([P5]
 * §KV 的写入与读取路径: the step writes the new K/V into the page, then decode
 * reads the whole history).  Formats 1-4, 6 and 7 (not KVarN, whose steps go
 * through kvq_kvarn_append).
 *   cache          the paged cache (written).
 *   k_new, v_new   binary16 [batch][H][D]: the new token of each sequence.
 *   slot_mapping   int64 [batch]: its slot (page * P + offset), normally the
 *                  slot of position context_lens[b] - 1 in the block table.
 *   other arguments as for kvq_decode_attention (kvarn_tail excluded); the
 *   workspace is sized by kvq_decode_workspace_bytes with the same arguments.
 * The cache bytes written are exactly those of kvq_quantize_write(k_new,
 * v_new, slot_mapping, n_tok = batch).  Whatever the split plan, attention
 * covers positions 0 .. ctx-2 read from the cache plus the new token as
 * position ctx-1, so the output equals kvq_quantize_write followed by
 * kvq_decode_attention whenever each slot is that of position ctx-1; a slot
 * elsewhere receives the same bytes and the token is still attended as
 * position ctx-1.  A sequence whose slot is negative or outside the pool
 * stores nothing and attends its ctx cached tokens; ctx = 0 stores the token
 * and gives a zero row.  Two sequences must not share a slot, and no new slot
 * may lie among the positions 0 .. ctx-2 that any sequence reads (they are
 * read while the new tokens are stored).
 * The split kernel reads one token less; its first context split of each
 * (sequence, kv head) also quantises and stores the new token and attends it
 * as one more partial.  With a single split that is the whole step, one
 * launch; with a split context the merge kernel of kvq_decode_attention
 * follows.  No write launch precedes either.
 * Errors: as kvq_decode_attention; KVQ_ERR_INVALID_ARG for a KVarN layout or
 * NULL k_new, v_new or slot_mapping with batch > 0. */
kvq_status kvq_decode_attention_append(const kvq_layout* layout, void* cache, const void* k_new,
                                       const void* v_new, const int64_t* slot_mapping, const void* q,
                                       int32_t num_q_heads, const int32_t* block_tables,
                                       int32_t max_pages_per_seq, const int32_t* context_lens,
                                       int32_t batch, float sm_scale, void* out, void* workspace,
                                       int64_t workspace_bytes, int32_t num_splits, void* stream);

/* Expand cached tokens back to binary32 [n_tok][H][D] for inspection and tests
 * (x_hat = s q, [P3] §它改变缓存表示).  8-bit formats: code value times scale,
 * one rounding.  NVFP4: E2M1 value times the E4M3 block scale (exact), times
 * s_t (one rounding).  MXFP4: E2M1 value times 2^(e-127) (exact).  KVarN:
 * rebuilt in the rotated basis, then rotated back (binary32, a few ulps).
 * Skipped slots (as in kvq_quantize_write) leave their rows untouched. */
kvq_status kvq_dequantize(const kvq_layout* layout, const void* cache, const int64_t* slot_mapping,
                          int64_t n_tok, float* k_out, float* v_out, void* stream);

/* Static English description of a status code: the explicit, named failure
 * that [P5] §Blackwell 支持不是一个单一布尔值 asks for in place of a silent
 * fallback.  Never NULL; unknown codes give "unknown status". */
const char* kvq_status_string(kvq_status status);

/* Contract violations the kernels find in arguments that live in device
 * memory, where the host cannot check them before the launch ([P5]
 * §需要记录的系统指标 asks for failures to be recorded, not hidden): bits of
 * the word kvq_take_device_errors returns. */
#define KVQ_DEVERR_KVARN_TILE_SLOTS (1u << 0)  /* KVarN kvq_quantize_write: a 128-token run's slots are
                                                  not one tile of a page in order; that run was skipped */
#define KVQ_DEVERR_KVARN_APPEND_SPAN (1u << 1) /* kvq_kvarn_append: a sequence's tokens in one call span
                                                  two tiles or repeat a position */

/* Waits for `stream` (a hipStream_t, NULL = the default stream), then returns
 * in *flags the KVQ_DEVERR_* bits raised on the current HIP device since the
 * previous call, and clears them.  The word is per device and shared by all
 * streams: kernels still running on other streams may raise bits after the
 * read.  Synchronous (a device-to-host copy); not for use under graph
 * capture.
 * Errors: KVQ_ERR_INVALID_ARG for NULL flags; KVQ_ERR_DEVICE off gfx950;
 * KVQ_ERR_HIP when a HIP call fails. */
kvq_status kvq_take_device_errors(uint32_t* flags, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
