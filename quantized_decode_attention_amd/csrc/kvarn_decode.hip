// kvarn_decode.hip -- paged GQA decode attention over a KVarN k4v2 g128 cache
// (gfx950).
//
// [P2] "KVarN：华为推出的原生 vLLM KV-cache 量化后端", §技术原理: the cache holds
// each 128-token tile of a kv head in a rotated basis, k~ = H k and v~ = H v
// (H the normalised Walsh-Hadamard transform, orthogonal and its own
// inverse), as codes plus folded scales:
//   k~_tj = rho_t (alpha_j c_tj + beta_j),   v~_tj = gamma_j (alpha'_t c'_tj + beta'_t).
// Rotation leaves dot products unchanged, so with q~ = H q
//   q . k_t  = rho_t ( sum_j (q~_j alpha_j) c_tj + sum_j q~_j beta_j )
//   sum_t p_t v_t = H [ gamma (.) ( sum_t (p_t alpha'_t) c'_t + sum_t p_t beta'_t ) ]
// The first bracket is one MFMA product per 16 tokens with A = 4-bit codes
// (exact in binary16) and B = q~ (.) alpha (per page, split into binary16
// high and low halves in the MFMA's spare columns).  The second is the usual
// P V product with the per-token V scale folded into P; gamma changes from
// tile to tile, so the output is kept in the current page's gamma domain and
// rescaled once per page.  Tokens of the incomplete last tile are kept by the
// caller in binary16 and attended by the merge kernel, which also rotates the
// output back ([P2] §配置与部署: the decode path keeps a small fixed
// workspace for the unquantised tail).
//
// Decomposition as for the other formats: a workgroup of 4 wavefronts per
// (sequence, kv head, context split), wave w walks pages w, w+4, ... of the
// split; every page is one tile of 8 sub-pages of 16 tokens, kept 3 sub-pages
// ahead in a register ring.  Each wave stages the 3 KB metadata block of its
// current page in LDS (requested with the next page's first sub-page) and
// reads the per-token and per-channel scales from there.
#include "decode_common.h"

namespace kvq {
namespace {

constexpr int D = 128;
constexpr int P = 128;
constexpr int kUnits = P / 16;
constexpr int kRing = 4;  // sub-page buffers per wave (kRing - 1 in flight)
constexpr int kMergeWaves = 8;  // merge: wave w attends tail rows 16w .. 16w + 15 and finishes head w
constexpr int kVCodes = P * D / 2;          // V codes [32][128] 2-bit
constexpr int kMeta = kVCodes + P * D / 4;  // binary32 metadata
constexpr int kMetaFloats = 3 * D + 3 * P;
constexpr int kTileBytes = kMeta + 4 * kMetaFloats;  // 15360; a page of a.P tokens holds a.P / 128 tiles
static_assert(kTileBytes == 15360, "KVarN tile size");
// metadata vectors (float offsets)
constexpr int kKa = 0, kKb = 128, kKr = 256, kVa = 384, kVb = 512, kVg = 640;
constexpr float kInvSqrt128 = (float)0.088388347648318440550;  // RN(1/sqrt(128))

// Sixteen-token sub-page of one lane: K token row n, channels 32*gq .. +31
// (16 bytes); V channels 8*n .. 8*n+7 of tokens 4*gq .. +3 (8 bytes).
struct RawKv {
  uint32_t k[4];
  uint32_t v[2];
};

// The lane's byte offsets within a sub-page (fixed for the kernel); the
// tile's base and size sit in a buffer resource in scalar registers, and a
// sub-page's position in the tile is a scalar offset.
struct LaneOffs {
  uint32_t k, v;
};
__device__ __forceinline__ LaneOffs lane_offsets(int n, int gq) { return {(uint32_t)(64 * n + 16 * gq), (uint32_t)(128 * gq + 8 * n)}; }

__device__ __forceinline__ void load_kv(__amdgpu_buffer_rsrc_t rs, int u, const LaneOffs& lo, RawKv& r) {
  buf_dwords<4>(rs, lo.k, 1024 * u, r.k);
  buf_dwords<2>(rs, lo.v, kVCodes + 512 * u, r.v);
}
// the tile's 3 KB metadata block: 48 bytes per lane
__device__ __forceinline__ void load_meta(__amdgpu_buffer_rsrc_t rs, int l, uint32_t (&m)[12]) {
#pragma unroll
  for (int k = 0; k < 3; ++k) buf_dwords<4>(rs, 16 * l, kMeta + 1024 * k, m + 4 * k);
}

// K operand of QK MFMA kk: the 8 codes of dword kk as binary16.  The low
// nibbles (even channels) and high nibbles (odd channels) are separated into
// bytes.  A byte holding a code c in 0..15 is the E4M3 encoding of c * 2^-9
// (codes 0..7 are the subnormals m * 2^-9, codes 8..15 the first normal
// binade (8 + m) * 2^-9), so gfx950's scaled E4M3 -> binary16 conversion at
// scale 2^9 returns c exactly, two codes per instruction.  Slot i holds
// channel 8*kk + slot_channel(i): slots 0..3 = channels 0, 2, 4, 6 and slots
// 4..7 = channels 1, 3, 5, 7.
__device__ __forceinline__ half8_t k_operand(uint32_t w, float s512) {
  const uint32_t x = w & 0x0F0F0F0Fu, y = (w >> 4) & 0x0F0F0F0Fu;
  uint32_t a, b, c, d;
  e4m3x4_to_h_scaled(x, s512, a, b);
  e4m3x4_to_h_scaled(y, s512, c, d);
  return cat(as_h2(a), as_h2(b), as_h2(c), as_h2(d));
}
__host__ __device__ constexpr int slot_channel(int i) { return i < 4 ? 2 * i : 2 * (i - 4) + 1; }

// Beyond the binary16 bound on P * v_scale, the reference also keeps P itself
// below 2^64: a KVarN per-token V scale can be 0.
constexpr float kPMaxLog2 = 64.0f;

// V codes of one dword (byte m = channel m, bits 2k..2k+1 = token k) as
// binary16.  A nibble 00cc is the E2M1 encoding of c / 2, so masking the
// dword to 0x33333333 leaves tokens 0 and 2 of channel m in byte m's two
// nibbles, and the scaled E2M1 conversion at scale 2 returns both codes
// exactly; the dword shifted right by 2 gives tokens 1 and 3 the same way.
// The MFMA operand of channel m therefore lists its tokens in the order
// 0, 2, 1, 3, and P's operand is built in the same order.
struct VCodes {
  uint32_t t02[4], t13[4];  // per channel byte: binary16 pairs (token 0, 2) and (1, 3)
};
__device__ __forceinline__ void v_codes(uint32_t w, VCodes& c) {
  e2m1x8_to_h_scaled(w & 0x33333333u, 2.0f, c.t02);
  e2m1x8_to_h_scaled((w >> 2) & 0x33333333u, 2.0f, c.t13);
}
__device__ __forceinline__ half4_t v_operand(const VCodes& c, int m) { return cat4(as_h2(c.t02[m]), as_h2(c.t13[m])); }

// The output rows are kept in the gamma domain of the page being read
// (o = gamma (.) o'): moving to the next page rescales o' once by
// gamma_old / gamma_new, so a page's P V product accumulates straight into o'.
struct KvState {
  float4_t o[D / 16];  // output rows o', rotated basis, current page's gamma domain
  float pb;            // this lane's share of sum_t p_t beta'_t over the page
  float m_run, l_run;
};

// One sub-page of a valid page (invalid pages are skipped by the caller).
// q~ and the beta term carry the softmax scale (log2 domain): a score is
// rho_t times the MFMA column sum, whose accumulator starts at the beta term.
template <int G>
__device__ __forceinline__ void process_unit(const RawKv& r, const float* mt, int u, int n, int gq,
                                             const half8_t (&qB)[4], float qbc, KvState& st) {
  float4_t s = {qbc, qbc, qbc, qbc};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    s = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand(r.k[kk], 512.0f), qB[kk], s, 0, 0, 0);

  const float4 rho = *reinterpret_cast<const float4*>(mt + kKr + 16 * u + 4 * gq);
  const float4 va = *reinterpret_cast<const float4*>(mt + kVa + 16 * u + 4 * gq);
  const float4 vb = *reinterpret_cast<const float4*>(mt + kVb + 16 * u + 4 * gq);
  const float rh[4] = {rho.x, rho.y, rho.z, rho.w};
  const float vsc[4] = {va.x, va.y, va.z, va.w};
  const float vbe[4] = {vb.x, vb.y, vb.z, vb.w};

  // column n < G: high half of head n; column G + n: its low half
  float t[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = s[i] + __uint_as_float(row_shl<G>(__float_as_uint(s[i])));
  float p[4], arg[4];
  // P * v_scale as binary16 pairs in the V operand's token order (0, 2) and
  // (1, 3): high halves h and remainders lo
  uint32_t h02, h13, lo02, lo13;
  auto weights = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      arg[i] = __builtin_fmaf(rh[i], t[i], -st.m_run);
      p[i] = __builtin_amdgcn_exp2f(arg[i]);
    }
    split_products(p[0], vsc[0], p[2], vsc[2], h02, lo02);
    split_products(p[1], vsc[1], p[3], vsc[3], h13, lo13);
  };
  weights();
  // P * v_scale above 2^8 (read off the binary16 high halves) or P itself
  // above 2^64 (an exponent above 64; +inf, never NaN, while the reference is
  // still -inf).
  const float amax = fmaxf(fmaxf(arg[0], arg[1]), fmaxf(arg[2], arg[3]));
  const bool over = ((amax > kPMaxLog2) | pairs_exceed_tau(h02, h13)) & (n < G);  // no short-circuit branches

  // P (high/low halves) times V into the output rows.  Both sides of the
  // rare rescale branch below run their own copy, so the accumulators are
  // never merged between the branches (which costs a register copy of every
  // accumulator on the common path).
  auto accumulate = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st.l_run += p[i];
      st.pb += p[i] * vbe[i];
    }
    const half4_t pA = cat4(as_h2(hi_lo_rows<G>(h02, lo02)), as_h2(hi_lo_rows<G>(h13, lo13)));
    VCodes c0, c1;
    v_codes(r.v[0], c0);
    v_codes(r.v[1], c1);
#pragma unroll
    for (int nn = 0; nn < 4; ++nn)
      st.o[nn] = __builtin_amdgcn_mfma_f32_16x16x16f16(pA, v_operand(c0, nn), st.o[nn], 0, 0, 0);
#pragma unroll
    for (int nn = 0; nn < 4; ++nn)
      st.o[4 + nn] = __builtin_amdgcn_mfma_f32_16x16x16f16(pA, v_operand(c1, nn), st.o[4 + nn], 0, 0, 0);
  };

  if (__builtin_amdgcn_ballot_w64(over) != 0) {
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lg = rh[i] * t[i];
      mx = fmaxf(mx, fmaxf(lg + __log2f(vsc[i]), lg - kPMaxLog2));
    }
    mx = n < G ? mx : kNegInf;
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m_run, mx);
    const float alpha = (m_new > st.m_run) ? exp2f(st.m_run - m_new) : 1.0f;
    st.l_run *= alpha;
    st.pb *= alpha;
    float ar[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * gq + i;
      ar[i] = __shfl(alpha, row < G ? row : (row < 2 * G ? row - G : 0));
    }
#pragma unroll
    for (int nn = 0; nn < D / 16; ++nn)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.o[nn][i] *= ar[i];
    st.m_run = m_new;
    weights();
    accumulate();
  } else {
    accumulate();
  }
}

template <int G>
__global__ __launch_bounds__(256) void kvarn_decode_kernel(DecodeArgs a) {
  constexpr int NV = D / 16;
  __shared__ float lds_o[kWaves][2 * G][D];
  __shared__ float lds_m[kWaves][16];
  __shared__ float lds_l[kWaves][16];
  __shared__ int s_pages[kPageChunk];
  __shared__ __attribute__((aligned(16))) float s_meta[kWaves][kMetaFloats];
  __shared__ __attribute__((aligned(16))) float s_q[G + 1][D];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, l = tid & 63, n = l & 15, gq = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar register
  const int S = a.num_splits;
  const int64_t rec_floats = ws_record_floats(D);

  // the walk is over 128-token tiles; a page of a.P tokens holds a.P / 128
  const int tshift = a.P == 256 ? 1 : 0;
  // The first chunk's block-table entries are requested before the context
  // length arrives: tiles p_begin .. p_begin + 255 of the split lie inside the
  // table's row whatever the length is, so the two round trips overlap.
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_pages;
  const int t_first = split * a.pages_per_split;
  const int first_cap = min(kPageChunk, min(a.pages_per_split, (a.max_pages << tshift) - t_first));
  const int bt_first = tid < first_cap ? bt[(t_first + tid) >> tshift] : 0;

  int ctx = __builtin_amdgcn_readfirstlane(a.ctx_lens[b]);
  ctx = ctx < 0 ? 0 : (ctx > a.max_pages * a.P ? a.max_pages * a.P : ctx);
  const int n_pages = ctx / P;  // complete tiles; the rest is the caller's tail
  const int p_begin = split * a.pages_per_split;
  const int p_end = min(p_begin + a.pages_per_split, n_pages);

  // q~ = H q / sqrt(128), times the softmax scale, for the G heads, once per
  // workgroup into LDS: wave w rotates heads w, w+4; lane l holds channels
  // 2l and 2l+1, so the first butterfly stage is in-lane and the others pair
  // lanes l and l ^ (h/2).
  const bool lo_col = n >= G && n < 2 * G;
  const float qscale = kInvSqrt128 * a.qk_scale;
  const int q_row = n < G ? n : (n < 2 * G ? n - G : G);  // row G of s_q is zero
  for (int h2 = w; h2 < G; h2 += kWaves) {
    const uint16_t* qp = a.q + ((int64_t)b * a.Hq + kvh * G + h2) * D + 2 * l;
    const half2_t q2 = *reinterpret_cast<const half2_t*>(qp);
    float x0 = (float)q2[0], x1 = (float)q2[1];
    const float s0 = x0 + x1, d0 = x0 - x1;
    x0 = s0;
    x1 = d0;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float p0 = __shfl_xor(x0, m), p1 = __shfl_xor(x1, m);
      x0 = (l & m) ? p0 - x0 : x0 + p0;
      x1 = (l & m) ? p1 - x1 : x1 + p1;
    }
    s_q[h2][2 * l] = x0 * qscale;
    s_q[h2][2 * l + 1] = x1 * qscale;
  }
  if (tid < D) s_q[G][tid] = 0.0f;
  __syncthreads();

  KvState st;
#pragma unroll
  for (int nn = 0; nn < NV; ++nn) st.o[nn] = float4_t{0.f, 0.f, 0.f, 0.f};
  float gcur[NV];  // gamma of the output's current domain, channels 8n + nn
#pragma unroll
  for (int nn = 0; nn < NV; ++nn) gcur[nn] = 1.0f;
  bool have_gamma = false;
  st.pb = 0.0f;
  st.m_run = kNegInf;
  st.l_run = 0.0f;

  const uint8_t* head_base = a.cache + (int64_t)kvh * a.geom.chunk_bytes;
  const int64_t page_stride = (int64_t)a.H * a.geom.chunk_bytes;
  float* mt = s_meta[w];
  const LaneOffs lofs = lane_offsets(n, gq);

  for (int c0 = p_begin; c0 < p_end; c0 += kPageChunk) {
    const int nc = min(kPageChunk, p_end - c0);  // <= first_cap for the first chunk
    static_assert(kPageChunk <= 256, "one block-table entry per thread and chunk");
    __syncthreads();
    if (tid < nc) {
      if (c0 == p_begin)  // uniform
        s_pages[tid] = bt_first;
      else
        s_pages[tid] = bt[(c0 + tid) >> tshift];
    }
    __syncthreads();
    const int nj = w < nc ? (nc - w + kWaves - 1) / kWaves : 0;
    if (nj == 0) continue;
    auto page_ptr = [&](int j, bool& valid) {
      const int page = __builtin_amdgcn_readfirstlane(s_pages[w + kWaves * j]);
      const int sub = (c0 + w + kWaves * j) & ((1 << tshift) - 1);  // tile within the page
      valid = page >= 0 && page < a.num_pages;
      return head_base + (valid ? page : 0) * page_stride + (valid ? sub : 0) * kTileBytes;
    };
    // the current page's metadata travels with its first sub-page: both are
    // requested while the previous page's last sub-page is computed
    bool vcur;
    const uint8_t* pc = page_ptr(0, vcur);
    uint32_t mreg[12];
    load_meta(chunk_rsrc(pc, kTileBytes), l, mreg);
    // ring of kRing sub-page buffers, kRing-1 sub-pages in flight ahead of
    // the one being computed (the ring runs across page boundaries; 8 is a
    // multiple of kRing, so sub-page u of every page uses slot u % kRing)
    RawKv rr[kRing];
#pragma unroll
    for (int k = 0; k + 1 < kRing; ++k) load_kv(chunk_rsrc(pc, kTileBytes), k, lofs, rr[k]);

    for (int j = 0; j < nj; ++j) {
      // publish this page's metadata to the wave's LDS block (same-wave LDS
      // accesses complete in order, so the reads below see it)
#pragma unroll
      for (int k = 0; k < 3; ++k)
        *reinterpret_cast<uint4*>(mt + 256 * k + 4 * l) = uint4{mreg[4 * k], mreg[4 * k + 1], mreg[4 * k + 2],
                                                                  mreg[4 * k + 3]};
      const int jn = min(j + 1, nj - 1);
      bool vnext;
      const uint8_t* pn = page_ptr(jn, vnext);
      // sub-page u's loads: kRing-1 ahead, continuing into the next page (its
      // metadata goes first)
      auto issue = [&](int u) {
        const int ahead = u + kRing - 1;
        if (ahead < kUnits) {
          load_kv(chunk_rsrc(pc, kTileBytes), ahead, lofs, rr[ahead % kRing]);
        } else {
          if (ahead == kUnits) {
            load_meta(chunk_rsrc(pn, kTileBytes), l, mreg);
          }
          load_kv(chunk_rsrc(pn, kTileBytes), ahead - kUnits, lofs, rr[ahead % kRing]);
        }
        // keep the loads ahead of this sub-page's wait for its own data
        __builtin_amdgcn_sched_barrier(0);
      };
      if (vcur) {  // wave-uniform; an invalid page's tokens carry no weight
        // B operand q~ (.) alpha (high half in columns n < G, low half in
        // columns G + n, zero beyond) and the beta term sum_j q~_j beta_j
        half8_t qB[4];
        const float* qrow = s_q[q_row] + 32 * gq;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const float4 q0 = *reinterpret_cast<const float4*>(qrow + 8 * kk);
          const float4 q1 = *reinterpret_cast<const float4*>(qrow + 8 * kk + 4);
          const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
          const float4 a0 = *reinterpret_cast<const float4*>(mt + kKa + 32 * gq + 8 * kk);
          const float4 a1 = *reinterpret_cast<const float4*>(mt + kKa + 32 * gq + 8 * kk + 4);
          const float al[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
          uint32_t qw[4];
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            // both halves of a slot pair, then one select of the column's half
            const int c0 = slot_channel(i), c1 = slot_channel(i + 1);
            uint32_t h, r;
            split_products(qv[c0], al[c0], qv[c1], al[c1], h, r);
            qw[i / 2] = lo_col ? r : h;
          }
          qB[kk] = __builtin_bit_cast(half8_t, qw);
        }
        // beta term: a high column's lane sums channels 32 gq .. +15 of its
        // head, the matching low column's lane channels 32 gq + 16 .. +31
        float qb = 0.0f;
        {
          const int off = 32 * gq + (lo_col ? 16 : 0);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float4 qq = *reinterpret_cast<const float4*>(s_q[q_row] + off + 4 * j);
            const float4 bb = *reinterpret_cast<const float4*>(mt + kKb + off + 4 * j);
            qb += qq.x * bb.x + qq.y * bb.y + qq.z * bb.z + qq.w * bb.w;
          }
        }
        qb += __shfl_xor(qb, 16);
        qb += __shfl_xor(qb, 32);
        qb += __uint_as_float(row_shl<G>(__float_as_uint(qb)));
        const float qbc = n < G ? qb : 0.0f;  // score accumulators of the high columns start here
        // move the output into this page's gamma domain
        {
          const float4 g0 = *reinterpret_cast<const float4*>(mt + kVg + 8 * n);
          const float4 g1 = *reinterpret_cast<const float4*>(mt + kVg + 8 * n + 4);
          const float gn[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
          if (have_gamma) {
#pragma unroll
            for (int nn = 0; nn < NV; ++nn) {
              const float r = gcur[nn] * __builtin_amdgcn_rcpf(gn[nn]);
#pragma unroll
              for (int i = 0; i < 4; ++i) st.o[nn][i] *= r;
            }
          }
#pragma unroll
          for (int nn = 0; nn < NV; ++nn) gcur[nn] = gn[nn];
          have_gamma = true;
        }
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
          issue(u);
          process_unit<G>(rr[u % kRing], mt, u, n, gq, qB, qbc, st);
        }
        // end of page: o' += sum_t p_t beta'_t (every channel of the head)
        float pbh = st.pb + __shfl_xor(st.pb, 16);
        pbh += __shfl_xor(pbh, 32);
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 4 * gq + i;
          const float v = __shfl(pbh, row < G ? row : 0);
          pr[i] = row < G ? v : 0.0f;
        }
#pragma unroll
        for (int nn = 0; nn < NV; ++nn)
#pragma unroll
          for (int i = 0; i < 4; ++i) st.o[nn][i] += pr[i];
        st.pb = 0.0f;
      } else {
#pragma unroll
        for (int u = 0; u < kUnits; ++u) issue(u);
      }
      pc = pn;
      vcur = vnext;
    }
  }

  // ---- combine the four waves (and the high/low rows) in LDS
  float l_tot = st.l_run + __shfl_xor(st.l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (gq == 0) {
    lds_m[w][n] = st.m_run;
    lds_l[w][n] = l_tot;
  }
#pragma unroll
  for (int nn = 0; nn < NV; ++nn)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * gq + i;
      if (row < 2 * G) lds_o[w][row][8 * n + nn] = gcur[nn] * st.o[nn][i];
    }
  __syncthreads();

  float* rec = reinterpret_cast<float*>(a.workspace) + (((int64_t)b * a.H + kvh) * S + split) * rec_floats;
  for (int i = tid; i < G * D; i += 256) {
    const int g = i / D, d = i % D;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, lds_m[ww][g]);
    float L = 0.0f, O = 0.0f;
    if (M != kNegInf) {
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float f = exp2f(lds_m[ww][g] - M);
        L += f * lds_l[ww][g];
        O += f * (lds_o[ww][g][d] + lds_o[ww][g + G][d]);
      }
    }
    if (d == 0) {
      rec[g] = M;
      rec[kMaxGroup + g] = L;
    }
    rec[2 * kMaxGroup + g * D + d] = O;
  }
}

// Merge of one (sequence, kv head), all G of its query heads: the binary16
// tail tokens (original basis), the split partials (rotated basis) and the
// rotation back:
//   M = max(m_s, m_tail), L = sum 2^(m_s-M) l_s + 2^(m_tail-M) l_tail,
//   o = ( H sum 2^(m_s-M) o_s + 2^(m_tail-M) o_tail ) / L.
// Eight waves.  The tail is read once for the whole group: wave w attends
// tail rows 16w .. 16w+15 with the same two MFMA products as the split
// kernel's sub-pages (K as the A operand of S^T = K Q^T, P as the A operand
// of O = P V), K, V and q entering as the binary16 values they are and P as
// binary16 high halves plus remainders.  A wave first takes the maximum of
// its 16 scores per head, so every weight is at most 1 and no rescale is
// needed.  The waves' partials meet in LDS.  Then wave w finishes head w:
// lane l holds channels l and l+64, merges the split records for them,
// applies the inverse rotation (in-lane stage 64, shuffles for the others)
// and adds the tail.
template <int G>
__global__ __launch_bounds__(64 * kMergeWaves) void kvarn_merge_kernel(DecodeArgs a) {
  constexpr int MW = kMergeWaves;
  __shared__ float lds_o[MW][2 * G][D];
  __shared__ float lds_m[MW][16];
  __shared__ float lds_l[MW][16];
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, l = tid & 63, n = l & 15, gq = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.num_splits;
  const int64_t rf = ws_record_floats(D);
  int ctx = __builtin_amdgcn_readfirstlane(a.ctx_lens[b]);
  ctx = ctx < 0 ? 0 : (ctx > a.max_pages * a.P ? a.max_pages * a.P : ctx);
  const int n_tail = a.tail ? ctx % P : 0;

  // the first 8 split records of the wave's head, requested before the
  // tail is read so both round trips overlap
  const float* recs = reinterpret_cast<const float*>(a.workspace) + ((int64_t)b * a.H + kvh) * S * rf;
  RecGroup rg[1][2];  // [head w][channel l, l + 64]
#pragma unroll
  for (int j = 0; j < 1; ++j) {
    const int g = w + MW * j;
    if (g < G) {  // uniform per wave
      load_recs(recs, rf, S, 0, g, 2 * kMaxGroup + g * D + l, rg[j][0]);
      load_recs(recs, rf, S, 0, g, 2 * kMaxGroup + g * D + l + 64, rg[j][1]);
    }
  }

  if (n_tail > 0) {  // uniform across the block
    const uint16_t* kt = a.tail + (((int64_t)b * 2 + 0) * a.H + kvh) * P * D;
    const uint16_t* vt = a.tail + (((int64_t)b * 2 + 1) * a.H + kvh) * P * D;
    // B operand Q^T: column n = head n (zero beyond G), rows = channels
    // 32 gq + 8 kk .. +7, as the K operand below
    half8_t qB[4];
    {
      const half8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
      const uint16_t* qp = a.q + ((int64_t)b * a.Hq + kvh * G + (n < G ? n : 0)) * D + 32 * gq;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const half8_t v = *reinterpret_cast<const half8_t*>(qp + 8 * kk);
        qB[kk] = n < G ? v : z;
      }
    }
    // rows 16w + n (K: channels 32 gq .. +31) and 16w + 4 gq + i (V:
    // channels 8n .. 8n+7) of the wave's sub-page; every row below 128 is
    // inside the tail buffer, rows at or past the tail length get weight 0
    half8_t kr[1][4], vr[1][4];
#pragma unroll
    for (int h = 0; h < 1; ++h) {
      const int u = w + MW * h;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        kr[h][kk] = *reinterpret_cast<const half8_t*>(kt + (int64_t)(16 * u + n) * D + 32 * gq + 8 * kk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vr[h][i] = *reinterpret_cast<const half8_t*>(vt + (int64_t)(16 * u + 4 * gq + i) * D + 8 * n);
    }
    float lg[1][4];
    float mx = kNegInf;
#pragma unroll
    for (int h = 0; h < 1; ++h) {
      float4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) s = __builtin_amdgcn_mfma_f32_16x16x32_f16(kr[h][kk], qB[kk], s, 0, 0, 0);
      const int row0 = 16 * (w + MW * h) + 4 * gq;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lg[h][i] = row0 + i < n_tail ? s[i] * a.qk_scale : kNegInf;
        mx = fmaxf(mx, lg[h][i]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mref = mx == kNegInf ? 0.0f : mx;  // a wave with no tail row: every weight 0
    float4_t acc[D / 16];
#pragma unroll
    for (int nn = 0; nn < D / 16; ++nn) acc[nn] = float4_t{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.0f;
#pragma unroll
    for (int h = 0; h < 1; ++h) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(lg[h][i] - mref);
        lsum += p[i];
      }
      uint32_t h01, h23, lo01, lo23;
      split_products(p[0], 1.0f, p[1], 1.0f, h01, lo01);
      split_products(p[2], 1.0f, p[3], 1.0f, h23, lo23);
      const half4_t pA = cat4(as_h2(hi_lo_rows<G>(h01, lo01)), as_h2(hi_lo_rows<G>(h23, lo23)));
#pragma unroll
      for (int nn = 0; nn < D / 16; ++nn) {
        const half4_t vB = {vr[h][0][nn], vr[h][1][nn], vr[h][2][nn], vr[h][3][nn]};
        acc[nn] = __builtin_amdgcn_mfma_f32_16x16x16f16(pA, vB, acc[nn], 0, 0, 0);
      }
    }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (gq == 0) {
      lds_m[w][n] = mx;
      lds_l[w][n] = lsum;
    }
#pragma unroll
    for (int nn = 0; nn < D / 16; ++nn)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * gq + i;
        if (row < 2 * G) lds_o[w][row][8 * n + nn] = acc[nn][i];
      }
  }
  __syncthreads();

#pragma unroll
  for (int j = 0; j < 1; ++j) {
    const int g = w + MW * j;
    if (g >= G) continue;  // uniform per wave
    float M = kNegInf, L = 0.0f, O0 = 0.0f, O1 = 0.0f;
    float M1 = kNegInf, L1 = 0.0f;
    merge_recs(rg[j][0], M, L, O0);
    merge_recs(rg[j][1], M1, L1, O1);
    for (int s0 = 8; s0 < S; s0 += 8) {
      RecGroup r0, r1;
      load_recs(recs, rf, S, s0, g, 2 * kMaxGroup + g * D + l, r0);
      load_recs(recs, rf, S, s0, g, 2 * kMaxGroup + g * D + l + 64, r1);
      merge_recs(r0, M, L, O0);
      merge_recs(r1, M1, L1, O1);
    }
    // the tail partial of head g over the eight waves
    float Mt = kNegInf, Lt = 0.0f, T0 = 0.0f, T1 = 0.0f;
    if (n_tail > 0) {
#pragma unroll
      for (int ww = 0; ww < MW; ++ww) Mt = fmaxf(Mt, lds_m[ww][g]);
      if (Mt != kNegInf) {
#pragma unroll
        for (int ww = 0; ww < MW; ++ww) {
          const float f = exp2f(lds_m[ww][g] - Mt);
          Lt += f * lds_l[ww][g];
          T0 += f * (lds_o[ww][g][l] + lds_o[ww][g + G][l]);
          T1 += f * (lds_o[ww][g][l + 64] + lds_o[ww][g + G][l + 64]);
        }
      }
    }
    const float mx = fmaxf(M, Mt);
    uint16_t* orow = a.out + ((int64_t)b * a.Hq + kvh * G + g) * D;
    if (mx == kNegInf) {  // empty context (uniform)
      orow[l] = 0;
      orow[l + 64] = 0;
      continue;
    }
    const float sp = exp2f(M - mx), st = exp2f(Mt - mx);
    L = L * sp + Lt * st;
    O0 *= sp;
    O1 *= sp;
    // inverse rotation of the split part across the 128 channels: stages
    // 1 .. 32 pair lanes l and l ^ h, stage 64 pairs the lane's two channels
#pragma unroll
    for (int hb = 1; hb < 64; hb <<= 1) {
      const float p0 = __shfl_xor(O0, hb), p1 = __shfl_xor(O1, hb);
      O0 = (l & hb) ? p0 - O0 : O0 + p0;
      O1 = (l & hb) ? p1 - O1 : O1 + p1;
    }
    const float r0 = O0 + O1, r1 = O0 - O1;
    orow[l] = __builtin_bit_cast(uint16_t, (half_t)((r0 * kInvSqrt128 + T0 * st) / L));
    orow[l + 64] = __builtin_bit_cast(uint16_t, (half_t)((r1 * kInvSqrt128 + T1 * st) / L));
  }
}

}  // namespace

namespace {
template <int G>
int kvarn_occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&kvarn_decode_kernel<G>), 256,
                                                   0) != hipSuccess)
    return 0;
  return n;
}
}  // namespace

int kvarn_decode_blocks_per_cu(int G) {
  switch (G) {
    case 1: return kvarn_occupancy<1>();
    case 2: return kvarn_occupancy<2>();
    case 4: return kvarn_occupancy<4>();
    case 8: return kvarn_occupancy<8>();
  }
  return 0;
}

hipError_t launch_kvarn_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const dim3 grid((unsigned)a.num_splits, (unsigned)a.H, (unsigned)a.B);
  switch (a.G) {
    case 1: kvarn_decode_kernel<1><<<grid, 256, 0, s>>>(a); break;
    case 2: kvarn_decode_kernel<2><<<grid, 256, 0, s>>>(a); break;
    case 4: kvarn_decode_kernel<4><<<grid, 256, 0, s>>>(a); break;
    case 8: kvarn_decode_kernel<8><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 mgrid((unsigned)a.H, (unsigned)a.B);
  switch (a.G) {
    case 1: kvarn_merge_kernel<1><<<mgrid, 64 * kMergeWaves, 0, s>>>(a); break;
    case 2: kvarn_merge_kernel<2><<<mgrid, 64 * kMergeWaves, 0, s>>>(a); break;
    case 4: kvarn_merge_kernel<4><<<mgrid, 64 * kMergeWaves, 0, s>>>(a); break;
    case 8: kvarn_merge_kernel<8><<<mgrid, 64 * kMergeWaves, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace kvq
