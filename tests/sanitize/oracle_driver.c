/*
 * oracle_driver.c -- drives every exported function of the CPU oracle
 * (oracle/kvq_oracle.c) over small random inputs and the edge cases of its
 * argument checks, so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py) sees every
 * buffer access and integer operation the oracle performs.  Test
 * infrastructure: it checks memory safety, not values (the pins do that).
 * Exits 0 when every call returned the expected status.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t format, flags;
  int32_t num_kv_heads, head_dim;
  int32_t page_size, num_pages;
  float k_scale, v_scale;
} layout_t;

float kvqo_half_to_float(uint16_t h);
double kvqo_e4m3_decode(uint8_t c);
uint8_t kvqo_e4m3_encode(float y);
double kvqo_e2m1_decode(uint8_t c);
uint8_t kvqo_e2m1_encode(float y);
int kvqo_quantize_row(int format, int flags, float scale, const uint16_t* x16, int D, uint8_t* codes,
                      uint8_t* scales);
void kvqo_kvarn_rotate_f32(float* y);
void kvqo_kvarn_tile(const uint16_t* x16, int64_t stride, int side, float* y_rot, float* y_norm, float* r_out,
                     float* c_out, uint8_t* codes, float* qs, float* qm, float* meta);
int64_t kvqo_chunk_bytes(const layout_t* L);
int64_t kvqo_page_bytes(const layout_t* L);
int kvqo_quantize_write(const layout_t* L, const uint16_t* k16, const uint16_t* v16, const int64_t* slots,
                        int64_t n_tok, uint8_t* cache);
int kvqo_dequantize(const layout_t* L, const uint8_t* cache, const int64_t* slots, int64_t n_tok, double* k_out,
                    double* v_out);
void kvqo_attention_dense(const double* q, const double* k, const double* v, int64_t T, int D, double scale,
                          double* out);
int kvqo_decode_attention(const layout_t* L, const uint8_t* cache, const uint16_t* q16, int32_t num_q_heads,
                          const int32_t* block_tables, int32_t max_pages, const int32_t* ctx_lens, int32_t batch,
                          float sm_scale, const uint16_t* tail16, const int32_t* pairs, int32_t n_pairs,
                          double* out);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(g_state >> 33);
}

/* A finite binary16 pattern with a biased exponent in [lo, hi]. */
static uint16_t rand_half(int lo, int hi) {
  const uint32_t r = next_u32();
  const int e = lo + (int)(r % (uint32_t)(hi - lo + 1));
  return (uint16_t)(((r >> 8) & 0x8000u) | ((uint32_t)e << 10) | ((r >> 12) & 0x3FFu));
}

static void fill_halves(uint16_t* x, int64_t n, int lo, int hi) {
  for (int64_t i = 0; i < n; i++) x[i] = rand_half(lo, hi);
}

static int g_fail = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      g_fail = 1;                                                      \
    }                                                                  \
  } while (0)

static void scalar_conversions(void) {
  double acc = 0.0;
  for (uint32_t b = 0; b < 65536; b++) acc += kvqo_half_to_float((uint16_t)b) == 0.0f;
  for (int c = 0; c < 256; c++) {
    const double v = kvqo_e4m3_decode((uint8_t)c); /* S.1111.111 decodes to NaN */
    acc += ((c & 0x7F) == 0x7F ? 0.0 : v) + kvqo_e4m3_encode((float)c - 128.0f);
  }
  for (int c = 0; c < 16; c++) acc += kvqo_e2m1_decode((uint8_t)c) + kvqo_e2m1_encode((float)c * 0.4f - 3.0f);
  EXPECT(acc == acc);
}

static void rows(void) {
  static const int fmts[] = {1, 2, 3, 4, 6, 7};
  for (int D = 32; D <= 4096; D *= 2) {
    uint16_t* x = malloc(sizeof(uint16_t) * D);
    uint8_t* codes = malloc(D);
    uint8_t* scales = malloc(D / 16 + 4);
    for (int rep = 0; rep < 3; rep++) {
      fill_halves(x, D, rep == 2 ? 0 : 1, rep == 1 ? 30 : 16);
      for (size_t f = 0; f < sizeof fmts / sizeof fmts[0]; f++)
        for (int flags = 0; flags < (fmts[f] == 4 ? 2 : 1); flags++)
          EXPECT(kvqo_quantize_row(fmts[f], flags, 0.37f, x, D, codes, scales) == 0);
    }
    free(x);
    free(codes);
    free(scales);
  }
  uint16_t x[64] = {0};
  uint8_t codes[64], scales[8];
  EXPECT(kvqo_quantize_row(2, 0, 1.0f, x, 48, codes, scales) != 0); /* not a multiple of 32 */
  EXPECT(kvqo_quantize_row(2, 0, 1.0f, x, 0, codes, scales) != 0);
  EXPECT(kvqo_quantize_row(2, 0, 1.0f, x, 8192, codes, scales) != 0); /* above the row limit */
  EXPECT(kvqo_quantize_row(5, 0, 1.0f, x, 32, codes, scales) != 0);    /* KVarN has no row form */
}

static void kvarn_tiles(void) {
  float y[128];
  for (int j = 0; j < 128; j++) y[j] = (float)j - 64.0f;
  kvqo_kvarn_rotate_f32(y);
  const int64_t stride = 3 * 128; /* a tile read out of a [tokens][3 heads][128] tensor */
  uint16_t* x = malloc(sizeof(uint16_t) * 128 * stride);
  float* yr = malloc(sizeof(float) * 128 * 128);
  float* yn = malloc(sizeof(float) * 128 * 128);
  uint8_t* codes = malloc(128 * 128);
  float r[128], c[128], qs[128], qm[128], meta[384];
  for (int side = 0; side < 2; side++) {
    fill_halves(x, 128 * stride, 1, 17);
    kvqo_kvarn_tile(x + 128, stride, side, yr, yn, r, c, codes, qs, qm, meta);
    kvqo_kvarn_tile(x, stride, side, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
    memset(x, 0, sizeof(uint16_t) * 128 * stride); /* all-zero tile */
    kvqo_kvarn_tile(x, stride, side, yr, yn, r, c, codes, qs, qm, meta);
  }
  free(x);
  free(yr);
  free(yn);
  free(codes);
}

/* Write, read back and attend one small pool of every format. */
static void paged(int format, int flags, int H, int D, int P, int num_pages) {
  layout_t L = {format, flags, H, D, P, num_pages, 0.05f, 0.07f};
  const int64_t pb = kvqo_page_bytes(&L);
  EXPECT(pb > 0 && kvqo_chunk_bytes(&L) * H == pb);
  uint8_t* cache = calloc((size_t)(pb * num_pages), 1);
  const int kvarn = format == 5;
  const int64_t n_tok = kvarn ? 2 * 128 : 3 * P + 5;
  uint16_t* k = malloc(sizeof(uint16_t) * n_tok * H * D);
  uint16_t* v = malloc(sizeof(uint16_t) * n_tok * H * D);
  fill_halves(k, n_tok * H * D, 1, 17);
  fill_halves(v, n_tok * H * D, 1, 17);
  int64_t* slots = malloc(sizeof(int64_t) * n_tok);
  const int64_t pool = (int64_t)num_pages * P;
  if (kvarn) {
    for (int64_t i = 0; i < n_tok; i++) slots[i] = (int64_t)(num_pages - 1) * P - (i / 128) * P + i % 128;
  } else {
    for (int64_t i = 0; i < n_tok; i++) slots[i] = (i * 7919) % pool;
    slots[1] = -1;        /* skipped */
    slots[2] = pool;      /* past the pool: skipped */
    slots[3] = pool + 99; /* skipped */
  }
  EXPECT(kvqo_quantize_write(&L, k, v, slots, n_tok, cache) == 0);
  double* kh = calloc((size_t)(n_tok * H * D), sizeof(double));
  double* vh = calloc((size_t)(n_tok * H * D), sizeof(double));
  EXPECT(kvqo_dequantize(&L, cache, slots, n_tok, kh, vh) == 0);

  const int B = 3, G = 2, Hq = G * H, maxp = num_pages;
  int32_t* bt = malloc(sizeof(int32_t) * B * maxp);
  for (int i = 0; i < B * maxp; i++) bt[i] = (i * 5 + 1) % num_pages;
  int32_t ctx[3] = {0, 1, maxp * P - (kvarn ? 37 : 3)};
  uint16_t* q = malloc(sizeof(uint16_t) * B * Hq * D);
  fill_halves(q, B * Hq * D, 10, 16);
  uint16_t* tail = NULL;
  if (kvarn) {
    tail = malloc(sizeof(uint16_t) * B * 2 * H * 128 * D);
    fill_halves(tail, (int64_t)B * 2 * H * 128 * D, 1, 16);
  }
  int32_t pairs[2 * 3 * 8];
  int np = 0;
  for (int b = 0; b < B; b++)
    for (int h = 0; h < Hq; h++) {
      pairs[2 * np] = b;
      pairs[2 * np + 1] = h;
      np++;
    }
  double* out = malloc(sizeof(double) * np * D);
  EXPECT(kvqo_decode_attention(&L, cache, q, Hq, bt, maxp, ctx, B, 0.125f, tail, pairs, np, out) == 0);
  /* argument checks: a pair outside the batch, a context past the table, a
   * page outside the pool, KVarN tail tokens without a tail */
  int32_t bad_pair[2] = {B, 0};
  EXPECT(kvqo_decode_attention(&L, cache, q, Hq, bt, maxp, ctx, B, 0.125f, tail, bad_pair, 1, out) != 0);
  int32_t ctx_long[3] = {0, 1, maxp * P + 1};
  int32_t last_pair[2] = {2, 0};
  EXPECT(kvqo_decode_attention(&L, cache, q, Hq, bt, maxp, ctx_long, B, 0.125f, tail, last_pair, 1, out) != 0);
  bt[2 * maxp] = num_pages;
  EXPECT(kvqo_decode_attention(&L, cache, q, Hq, bt, maxp, ctx, B, 0.125f, tail, last_pair, 1, out) != 0);
  bt[2 * maxp] = 0;
  if (kvarn) EXPECT(kvqo_decode_attention(&L, cache, q, Hq, bt, maxp, ctx, B, 0.125f, NULL, last_pair, 1, out) != 0);

  double* qd = malloc(sizeof(double) * D);
  for (int d = 0; d < D; d++) qd[d] = kvqo_half_to_float(q[d]);
  kvqo_attention_dense(qd, kh, vh, 4, D, 0.1, out);
  kvqo_attention_dense(qd, kh, vh, 0, D, 0.1, out);

  free(qd);
  free(out);
  free(tail);
  free(q);
  free(bt);
  free(kh);
  free(vh);
  free(slots);
  free(k);
  free(v);
  free(cache);
}

static void layouts_refused(void) {
  layout_t bad[] = {
      {2, 0, 2, 48, 16, 4, 1.0f, 1.0f},  /* head size */
      {2, 0, 2, 64, 24, 4, 1.0f, 1.0f},  /* page size */
      {5, 0, 2, 128, 64, 4, 1.0f, 1.0f}, /* KVarN page below one tile */
      {1, 0, 2, 64, 16, 4, 0.0f, 1.0f},  /* per-tensor scale 0 */
      {9, 0, 2, 64, 16, 4, 1.0f, 1.0f},  /* format */
  };
  uint16_t k[128 * 2 * 128] = {0};
  int64_t slots[128];
  for (int i = 0; i < 128; i++) slots[i] = i;
  uint8_t cache[64];
  for (size_t i = 0; i < sizeof bad / sizeof bad[0]; i++) {
    if (bad[i].format != 1) EXPECT(kvqo_page_bytes(&bad[i]) < 0);
    EXPECT(kvqo_quantize_write(&bad[i], k, k, slots, 1, cache) != 0);
  }
  /* KVarN: a token count off a multiple of 128, and a run that does not fill a tile */
  layout_t kv = {5, 0, 1, 128, 128, 2, 1.0f, 1.0f};
  uint8_t* kc = calloc((size_t)kvqo_page_bytes(&kv) * 2, 1);
  EXPECT(kvqo_quantize_write(&kv, k, k, slots, 100, kc) != 0);
  slots[5] = 77;
  EXPECT(kvqo_quantize_write(&kv, k, k, slots, 128, kc) != 0);
  free(kc);
}

int main(void) {
  scalar_conversions();
  rows();
  kvarn_tiles();
  static const int fmts[] = {1, 2, 3, 4, 6, 7};
  for (size_t f = 0; f < sizeof fmts / sizeof fmts[0]; f++)
    for (int D = 32; D <= 128; D *= 2)
      for (int P = 16; P <= 64; P *= 4) {
        paged(fmts[f], 0, 2, D, P, 5);
        if (fmts[f] == 4) paged(4, 1, 2, D, P, 5);
      }
  paged(5, 0, 2, 128, 128, 4);
  paged(5, 0, 1, 128, 256, 3);
  layouts_refused();
  if (g_fail) return 1;
  printf("oracle driver: all calls done\n");
  return 0;
}
