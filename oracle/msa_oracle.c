/*
 * msa_oracle.c -- plain, slow CPU oracle for the MiniMax Sparse Attention (MSA)
 * decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this library.  It shares no
 * code, header, table or constant generator with the HIP library; the byte
 * formats are implemented here a second time, from their definitions.
 *
 * Sources (cited by page title and section):
 *  [P2] "vLLM 对 MiniMax-M3.1-Flash 的 Day-0 支持：NVFP4 MSA 内核、MegaMoE 与
 *       Agentic 基准测试" (agentlenshq.com), sections "MiniMax 稀疏注意力的工作原理"
 *       (how MSA works), "MiniMax-M3.1 架构的变化" (NVFP4 KV cache bytes),
 *       "NVIDIA Blackwell MSA 内核优化" (NVFP4 keys, FP8 queries),
 *       "通过查表实现的 NVFP4 MSA 内核" (E4M3 scales x E2M1 magnitudes).
 *  [P1] spke.com article on vLLM's MiniMax-M3.1-Flash support, section "MSA入門".
 *  [P3] "MiniMax goes sparse" (atlascloud.ai), section 1, Step 1 (index branch:
 *       one shared index-key head, block max pool, TopK per layer and GQA
 *       group) and Step 2 (sparse branch: heads of a group share the set).
 *  [OCP] OCP Microscaling Formats (MX) v1.0: the E4M3 and E2M1 element encodings.
 *
 * Arithmetic: every score, probability and output is computed in double.
 * Dequantised cache values are exact in double (at most 30 significant bits).
 * Readings of points the pages leave open are listed next to the code that
 * takes them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define REF_PAGE 128        /* tokens per page = tokens per selection block [P2 how MSA works] */
#define REF_DIM 128         /* head dim of K, V, index keys and queries */
#define REF_NVFP4_GROUP 16  /* elements per E4M3 scale (from 34,560/61,440 B, [P2 M3.1 changes]) */
#define REF_NVFP4_SLAB 9216 /* 128 tokens x (64 B codes + 8 B scales) */
#define REF_F32_SLAB (REF_PAGE * REF_DIM * 4)
#define REF_FP8_SLAB (REF_PAGE * REF_DIM) /* one byte per element: 128 B per token per head, the pages'
                                            FP8 index-key cost [P2 how MSA works] */

enum { REF_F32 = 0, REF_FP8_E4M3 = 1, REF_NVFP4 = 2 };
enum { REF_TOKEN_MAJOR = 0, REF_DIM_MAJOR = 1, REF_HALF_ROWS = 2 };

/* ------------------------------------------------------------------------- */
/* E4M3 [OCP]: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent 0
 * is subnormal (m/8 * 2^-6).  S.1111.111 is NaN; there is no infinity.      */
double ref_e4m3_value(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* E2M1 [OCP]: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit. */
double ref_e2m1_value(uint8_t code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* Round |x| to the nearest of the non-negative finite values of a format,
 * listed in increasing order with their codes.  An exact tie goes to the even
 * code (the one whose mantissa LSB, i.e. code LSB, is 0): round-to-nearest-even.
 * Magnitudes at or beyond the largest value saturate to it (satfinite).     */
static uint8_t nearest_code(double ax, const double* vals, const uint8_t* codes, int n) {
  if (ax >= vals[n - 1]) return codes[n - 1];
  for (int i = 0; i + 1 < n; ++i) {
    if (ax < vals[i + 1]) {
      double mid = 0.5 * (vals[i] + vals[i + 1]); /* exact: few significant bits */
      if (ax < mid) return codes[i];
      if (ax > mid) return codes[i + 1];
      return (codes[i] & 1) ? codes[i + 1] : codes[i];
    }
  }
  return codes[n - 1];
}

static double g_e4m3_vals[127];
static uint8_t g_e4m3_codes[127];
static double g_e2m1_vals[8];
static uint8_t g_e2m1_codes[8];
static int g_tables_ready = 0;

__attribute__((constructor)) static void build_tables(void) {
  if (g_tables_ready) return;
  for (int c = 0; c < 127; ++c) { /* codes 0x00..0x7E are the non-negative finite values, increasing */
    g_e4m3_codes[c] = (uint8_t)c;
    g_e4m3_vals[c] = ref_e4m3_value((uint8_t)c);
  }
  for (int c = 0; c < 8; ++c) {
    g_e2m1_codes[c] = (uint8_t)c;
    g_e2m1_vals[c] = ref_e2m1_value((uint8_t)c);
  }
  g_tables_ready = 1;
}

/* FP32 -> E4M3, round to nearest even, saturating.  NaN -> 0x7F (sign kept). */
uint8_t ref_e4m3_encode(float x) {
  build_tables();
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return (uint8_t)(sign | 0x7F);
  return (uint8_t)(sign | nearest_code(fabs((double)x), g_e4m3_vals, g_e4m3_codes, 127));
}

/* FP32 -> E2M1 nibble, round to nearest even, saturating at 6. */
uint8_t ref_e2m1_encode(float x) {
  build_tables();
  uint8_t sign = signbit(x) ? 0x8 : 0x0;
  return (uint8_t)(sign | nearest_code(fabs((double)x), g_e2m1_vals, g_e2m1_codes, 8));
}

/* ------------------------------------------------------------------------- */
/* NVFP4 group quantiser.  The pages say the cache is NVFP4 with E4M3 scales
 * and E2M1 magnitudes [P2 table-lookup kernel section] and that the model is
 * trained for it [P2 M3.1 changes]; they do not give the rounding recipe.
 * Reading taken (amax recipe, all steps in FP32 round-to-nearest-even):
 *   s32   = (amax / 6) / tensor_scale         two FP32 divisions
 *   scale = E4M3(s32)                          RNE, saturating
 *   scale == 0  ->  all sixteen codes +0
 *   else   y_i = x_i / (scale * tensor_scale)  FP32 multiply, then FP32 divide
 *          code_i = sign(x_i) | E2M1(|y_i|)    RNE, saturating at 6
 * Element 2i sits in the low nibble of byte i, element 2i+1 in the high one.  */
void ref_nvfp4_quantize_group(const float* x, float tensor_scale, uint8_t* codes8, uint8_t* scale_out) {
  float amax = 0.0f;
  for (int i = 0; i < REF_NVFP4_GROUP; ++i) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  volatile float t1 = amax / 6.0f; /* volatile: keep each FP32 rounding step */
  volatile float s32 = t1 / tensor_scale;
  uint8_t sc = ref_e4m3_encode(s32);
  *scale_out = sc;
  memset(codes8, 0, REF_NVFP4_GROUP / 2);
  double sv = ref_e4m3_value(sc);
  if (sv == 0.0) return;
  volatile float denom = (float)sv * tensor_scale;
  for (int i = 0; i < REF_NVFP4_GROUP; ++i) {
    volatile float y = x[i] / denom;
    uint8_t c = ref_e2m1_encode(y);
    codes8[i / 2] |= (uint8_t)((i & 1) ? (c << 4) : c);
  }
}

/* Value of one NVFP4 element: (e2m1 * e4m3_scale) * tensor_scale, exact in
 * double.  Its FP32 rounding is the single rounding of this exact product.  */
double ref_nvfp4_value(uint8_t code, uint8_t scale, float tensor_scale) {
  return ref_e2m1_value(code) * ref_e4m3_value(scale) * (double)tensor_scale;
}

/* ------------------------------------------------------------------------- */
/* FP8 cache element.  The pages name an FP8 cache beside NVFP4 and give its
 * cost -- 128 B of index keys and 1,024 B of K/V (4 heads x 128 dims) per
 * token and layer [P2 how MSA works], 61,440 B per token over the model
 * [P2 M3.1 changes] -- i.e. one byte per element; they give no scale
 * granularity.  Reading taken: E4M3 elements with one FP32 scale per cache
 * tensor, as for the NVFP4 tensor scale:
 *   code  = E4M3(x / tensor_scale)   FP32 division, RNE, saturating (NaN -> 0x7F)
 *   value = e4m3 * tensor_scale      exact in double                         */
uint8_t ref_fp8_quantize(float x, float tensor_scale) {
  volatile float y = x / tensor_scale;
  return ref_e4m3_encode(y);
}

double ref_fp8_value(uint8_t code, float tensor_scale) { return ref_e4m3_value(code) * (double)tensor_scale; }

/* ------------------------------------------------------------------------- */
/* Paged cache.  One slab per (page, head); page p, head h starts at byte
 * (p * num_heads + h) * slab_bytes.  Slab layouts:
 *   F32 token-major : float [128 tokens][128 dims]
 *   NVFP4 token-major (K and index keys):
 *       codes  [128 tokens][64 B]  (byte i of token t: dims 2i lo nibble, 2i+1 hi)
 *       scales [128 tokens][8 B]   (byte j: scale of dims 16j..16j+15)
 *   NVFP4 dim-major (V):
 *       codes  [128 dims][64 B]    (byte i of dim d: tokens 2i lo nibble, 2i+1 hi)
 *       scales [8 groups][128 tokens] (byte (j, t): scale of token t, dims 16j..)
 *   FP8 token-major (K): [128 tokens][128 dims], one E4M3 byte each
 *   FP8 dim-major (V): [128 dims][128 tokens]
 *   FP8 half rows (index keys): [8 chunks of 16 tokens][2 halves of 64 dims]
 *       [16 tokens][64 dims] -- a byte placement, the values are unchanged
 * The NVFP4 quantisation group is always 16 consecutive dims of one token;
 * only the placement of the bytes differs between the two layouts.          */
typedef struct {
  int32_t dtype;
  int32_t layout;
  int32_t num_heads;
  int32_t num_pages;
  float tensor_scale;
  uint8_t* pages;
} ref_cache;

/* Byte of token t, dim d in an FP8 slab. */
static int64_t fp8_byte(int layout, int t, int d) {
  if (layout == REF_DIM_MAJOR) return (int64_t)d * REF_PAGE + t;
  if (layout == REF_HALF_ROWS) return (int64_t)(t / 16) * 2048 + (d / 64) * 1024 + (t % 16) * 64 + d % 64;
  return (int64_t)t * REF_DIM + d;
}

static int64_t slab_bytes(const ref_cache* c) {
  return c->dtype == REF_F32 ? REF_F32_SLAB : (c->dtype == REF_FP8_E4M3 ? REF_FP8_SLAB : REF_NVFP4_SLAB);
}

static uint8_t* slab(const ref_cache* c, int64_t page, int head) {
  return c->pages + (page * c->num_heads + head) * slab_bytes(c);
}

/* Write one token's vector (128 values) for one head into page slot `slot`
 * (page = slot / 128, offset = slot % 128). Returns 0, or -1 on a bad slot. */
int ref_cache_write(const ref_cache* c, int64_t slot, int head, const float* x) {
  if (slot < 0 || slot >= (int64_t)c->num_pages * REF_PAGE || head < 0 || head >= c->num_heads) return -1;
  int64_t page = slot / REF_PAGE;
  int t = (int)(slot % REF_PAGE);
  uint8_t* s = slab(c, page, head);
  if (c->dtype == REF_F32) {
    memcpy(s + (int64_t)t * REF_DIM * 4, x, REF_DIM * 4);
    return 0;
  }
  if (c->dtype == REF_FP8_E4M3) {
    for (int d = 0; d < REF_DIM; ++d) {
      s[fp8_byte(c->layout, t, d)] = ref_fp8_quantize(x[d], c->tensor_scale);
    }
    return 0;
  }
  for (int j = 0; j < REF_DIM / REF_NVFP4_GROUP; ++j) {
    uint8_t codes[8], sc;
    ref_nvfp4_quantize_group(x + 16 * j, c->tensor_scale, codes, &sc);
    if (c->layout == REF_TOKEN_MAJOR) {
      memcpy(s + t * 64 + 8 * j, codes, 8);
      s[8192 + t * 8 + j] = sc;
    } else {
      for (int i = 0; i < 16; ++i) {
        int d = 16 * j + i;
        uint8_t nib = (uint8_t)((codes[i / 2] >> ((i & 1) * 4)) & 0xF);
        uint8_t* byte = s + d * 64 + t / 2;
        if (t & 1)
          *byte = (uint8_t)((*byte & 0x0F) | (nib << 4));
        else
          *byte = (uint8_t)((*byte & 0xF0) | nib);
      }
      s[8192 + j * 128 + t] = sc;
    }
  }
  return 0;
}

/* Write n tokens: x is [n][num_heads][128], slots[i] the slot of token i.
 * Slots must be distinct.  Parallel over tokens in two passes (even, then odd
 * in-page offsets) so that no two threads touch the same byte of a
 * dim-major page.  Returns the number of rejected slots.                   */
int64_t ref_cache_write_many(const ref_cache* c, const int64_t* slots, int64_t n, const float* x) {
  int64_t bad = 0;
  for (int parity = 0; parity < 2; ++parity) {
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t i = 0; i < n; ++i) {
      if (slots[i] < 0 || (slots[i] % REF_PAGE) % 2 != parity) {
        if (parity == 0 && slots[i] < 0) bad += 1;
        continue;
      }
      for (int h = 0; h < c->num_heads; ++h)
        if (ref_cache_write(c, slots[i], h, x + (i * c->num_heads + h) * REF_DIM) != 0) bad += (h == 0);
    }
  }
  return bad;
}

/* Dequantised value of dim d of token t (0..127 within the page) of a head. */
double ref_cache_value(const ref_cache* c, int64_t page, int head, int t, int d) {
  const uint8_t* s = slab(c, page, head);
  if (c->dtype == REF_F32) {
    float v;
    memcpy(&v, s + ((int64_t)t * REF_DIM + d) * 4, 4);
    return (double)v;
  }
  if (c->dtype == REF_FP8_E4M3)
    return ref_fp8_value(s[fp8_byte(c->layout, t, d)], c->tensor_scale);
  uint8_t code, sc;
  if (c->layout == REF_TOKEN_MAJOR) {
    uint8_t b = s[t * 64 + d / 2];
    code = (d & 1) ? (b >> 4) : (b & 0xF);
    sc = s[8192 + t * 8 + d / 16];
  } else {
    uint8_t b = s[d * 64 + t / 2];
    code = (t & 1) ? (b >> 4) : (b & 0xF);
    sc = s[8192 + (d / 16) * 128 + t];
  }
  return ref_nvfp4_value(code, sc, c->tensor_scale);
}

/* Dequantise whole pages: out[n][heads][128 tokens][128 dims] as FP32, each
 * element the single FP32 rounding of its exact value.                      */
void ref_cache_dequant_pages(const ref_cache* c, const int32_t* pages, int32_t n, float* out) {
  for (int32_t i = 0; i < n; ++i)
    for (int h = 0; h < c->num_heads; ++h)
      for (int t = 0; t < REF_PAGE; ++t)
        for (int d = 0; d < REF_DIM; ++d)
          out[(((int64_t)i * c->num_heads + h) * REF_PAGE + t) * REF_DIM + d] =
              (float)ref_cache_value(c, pages[i], h, t, d);
}

/* Queries: FP8 E4M3 bytes times a per-tensor FP32 scale [P2 Blackwell section:
 * queries stay FP8], or plain FP32.  Output in double.                      */
void ref_decode_queries(const void* q, int32_t dtype, float q_scale, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) {
    if (dtype == REF_F32)
      out[i] = (double)((const float*)q)[i];
    else
      out[i] = ref_e4m3_value(((const uint8_t*)q)[i]) * (double)q_scale;
  }
}

/* FP32 -> E4M3 query bytes: code = E4M3(x / q_scale), FP32 division. */
void ref_quantize_queries(const float* x, int64_t n, float q_scale, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    volatile float y = x[i] / q_scale;
    out[i] = ref_e4m3_encode(y);
  }
}

/* ------------------------------------------------------------------------- */
/* Batch of one decode step.  Request b has ctx_lens[b] = L_b cached tokens,
 * its R new rows included; row r sits at position p = L_b - R + r and sees
 * tokens 0..p (rows are independent causal queries).  Logical block j of
 * request b is physical page block_table[b * max_pages + j].                */
typedef struct {
  int32_t B, R, max_pages;
  const int32_t* block_table;
  const int32_t* ctx_lens;
} ref_batch;

static int64_t row_pos(const ref_batch* bt, int b, int r) { return (int64_t)bt->ctx_lens[b] - bt->R + r; }

/* Step 1, indexer [P2 how MSA works; P3 step 1]: one index query per GQA
 * group, dotted with the single shared index-key head, for every cached
 * token the row can see.  No scaling or activation is applied (the pages print
 * none; a positive scale could not change the selection).
 * q_idx: [B][R][G][128] (double); token_scores: [B][R][G][max_pages*128],
 * -inf where the token is outside 0..p.  abs_scores (optional, same shape)
 * receives sum_k |q_k * K_k|, the scale of the rounding error of any
 * finite-precision evaluation.                                              */
void ref_index_scores(const ref_batch* bt, int G, const double* q_idx, const ref_cache* idx,
                      double* token_scores, double* abs_scores) {
  int64_t T = (int64_t)bt->max_pages * REF_PAGE;
#pragma omp parallel for collapse(3) schedule(dynamic)
  for (int b = 0; b < bt->B; ++b)
    for (int r = 0; r < bt->R; ++r)
      for (int g = 0; g < G; ++g) {
        const double* q = q_idx + (((int64_t)b * bt->R + r) * G + g) * REF_DIM;
        double* out = token_scores + (((int64_t)b * bt->R + r) * G + g) * T;
        double* aout = abs_scores ? abs_scores + (((int64_t)b * bt->R + r) * G + g) * T : NULL;
        int64_t p = row_pos(bt, b, r);
        for (int64_t t = 0; t < T; ++t) {
          if (t > p) {
            out[t] = -INFINITY;
            if (aout) aout[t] = 0.0;
            continue;
          }
          int64_t page = bt->block_table[(int64_t)b * bt->max_pages + t / REF_PAGE];
          double s = 0.0, a = 0.0;
          for (int d = 0; d < REF_DIM; ++d) {
            double kv = ref_cache_value(idx, page, 0, (int)(t % REF_PAGE), d);
            s += q[d] * kv;
            a += fabs(q[d] * kv);
          }
          out[t] = s;
          if (aout) aout[t] = a;
        }
      }
}

/* Step 2, block max-pool [P2 how MSA works; P3 step 1]: one score per
 * 128-token block, the max over the block's tokens the row can see.
 * Blocks with no visible token get -inf.                                    */
void ref_block_maxpool(const ref_batch* bt, int G, const double* token_scores, double* block_scores) {
  int64_t T = (int64_t)bt->max_pages * REF_PAGE;
  for (int64_t row = 0; row < (int64_t)bt->B * bt->R * G; ++row)
    for (int j = 0; j < bt->max_pages; ++j) {
      double m = -INFINITY;
      for (int t = 0; t < REF_PAGE; ++t) {
        double s = token_scores[row * T + (int64_t)j * REF_PAGE + t];
        if (s > m) m = s;
      }
      block_scores[row * bt->max_pages + j] = m;
    }
}

/* Step 3, selection [P2 how MSA works; P1 MSA入門; P3 step 1].
 * Readings: the latest block counts inside the budget (latest + topk-1 best
 * others, so at most topk*128 keys, the pages' 2,048-key cap for topk=16);
 * the latest block is the one holding the row's own position; a tie in score
 * goes to the lower block index; a NaN score ranks below every number; with
 * n <= topk visible blocks all are taken.  Output is ascending, -1 padded.  */
typedef struct {
  double s;
  int32_t j;
} cand;

static int cand_cmp(const void* a, const void* b) {
  const cand* x = (const cand*)a;
  const cand* y = (const cand*)b;
  int xn = isnan(x->s), yn = isnan(y->s);
  if (xn != yn) return xn ? 1 : -1;
  if (!xn && x->s != y->s) return x->s > y->s ? -1 : 1;
  return (x->j > y->j) - (x->j < y->j);
}

static int int_cmp(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

void ref_select(const ref_batch* bt, int G, const double* block_scores, int topk, int32_t* sel, int32_t* cnt) {
  cand* c = (cand*)malloc(sizeof(cand) * (size_t)(bt->max_pages > 0 ? bt->max_pages : 1));
  for (int b = 0; b < bt->B; ++b)
    for (int r = 0; r < bt->R; ++r)
      for (int g = 0; g < G; ++g) {
        int64_t row = ((int64_t)b * bt->R + r) * G + g;
        int32_t* out = sel + row * topk;
        for (int i = 0; i < topk; ++i) out[i] = -1;
        int64_t p = row_pos(bt, b, r);
        int n = p < 0 ? 0 : (int)(p / REF_PAGE) + 1;
        if (n > bt->max_pages) n = bt->max_pages;
        if (n <= topk) {
          for (int i = 0; i < n; ++i) out[i] = i;
          cnt[row] = n;
          continue;
        }
        int latest = n - 1;
        for (int j = 0; j < latest; ++j) {
          c[j].s = block_scores[row * bt->max_pages + j];
          c[j].j = j;
        }
        qsort(c, (size_t)latest, sizeof(cand), cand_cmp);
        for (int i = 0; i < topk - 1; ++i) out[i] = c[i].j;
        out[topk - 1] = latest;
        qsort(out, (size_t)topk, sizeof(int32_t), int_cmp);
        cnt[row] = topk;
      }
  free(c);
}

/* Step 4, exact GQA softmax attention over the selected blocks only
 * [P2 how MSA works; P1 MSA入門 Fig. 1 caption; P3 step 2]: every query
 * head h of group g = h / (H/G) uses group g's set; over the tokens t <= p of
 * the selected blocks, out = sum_t softmax_t(sm_scale * q_h . K_t) V_t.
 * Rows with no selected block get zeros.  q: [B][R][H][128] double,
 * out: [B][R][H][128] double.                                              */
void ref_attention(const ref_batch* bt, int H, int G, const double* q, double sm_scale, const ref_cache* kc,
                   const ref_cache* vc, const int32_t* sel, const int32_t* cnt, int topk, double* out) {
  int hpg = H / G;
#pragma omp parallel for collapse(3) schedule(dynamic)
  for (int b = 0; b < bt->B; ++b)
    for (int r = 0; r < bt->R; ++r)
      for (int h = 0; h < H; ++h) {
        int g = h / hpg;
        int64_t row = ((int64_t)b * bt->R + r) * G + g;
        const double* qh = q + (((int64_t)b * bt->R + r) * H + h) * REF_DIM;
        double* o = out + (((int64_t)b * bt->R + r) * H + h) * REF_DIM;
        for (int d = 0; d < REF_DIM; ++d) o[d] = 0.0;
        int n = cnt[row];
        if (n <= 0) continue;
        int64_t p = row_pos(bt, b, r);
        int64_t ntok = (int64_t)n * REF_PAGE;
        double* z = (double*)malloc(sizeof(double) * (size_t)ntok);
        int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)ntok);
        int64_t m_tok = 0;
        double zmax = -INFINITY;
        for (int i = 0; i < n; ++i) {
          int j = sel[row * topk + i];
          for (int t = 0; t < REF_PAGE; ++t) {
            int64_t pos = (int64_t)j * REF_PAGE + t;
            if (pos > p) break;
            int64_t page = bt->block_table[(int64_t)b * bt->max_pages + j];
            double s = 0.0;
            for (int d = 0; d < REF_DIM; ++d) s += qh[d] * ref_cache_value(kc, page, g, t, d);
            z[m_tok] = sm_scale * s;
            tok[m_tok] = pos;
            if (z[m_tok] > zmax) zmax = z[m_tok];
            ++m_tok;
          }
        }
        double denom = 0.0;
        for (int64_t i = 0; i < m_tok; ++i) {
          double w = exp(z[i] - zmax);
          denom += w;
          int64_t pos = tok[i];
          int64_t page = bt->block_table[(int64_t)b * bt->max_pages + pos / REF_PAGE];
          for (int d = 0; d < REF_DIM; ++d) o[d] += w * ref_cache_value(vc, page, g, (int)(pos % REF_PAGE), d);
        }
        for (int d = 0; d < REF_DIM; ++d) o[d] /= denom;
        free(z);
        free(tok);
      }
}

/* Whole decode step (steps 1 to 4) on caches that already hold the tokens.
 * token_scores / abs_scores / block_scores may be passed as scratch.        */
void ref_decode_step(const ref_batch* bt, int H, int G, const double* q_idx, const double* q, double sm_scale,
                     const ref_cache* idx, const ref_cache* kc, const ref_cache* vc, int topk,
                     double* token_scores, double* block_scores, int32_t* sel, int32_t* cnt, double* out) {
  ref_index_scores(bt, G, q_idx, idx, token_scores, NULL);
  ref_block_maxpool(bt, G, token_scores, block_scores);
  ref_select(bt, G, block_scores, topk, sel, cnt);
  ref_attention(bt, H, G, q, sm_scale, kc, vc, sel, cnt, topk, out);
}

/* ------------------------------------------------------------------------- */
/* The projection that produces a step's new rows and the norm and rotary
 * embedding applied to them before they are quantised ([P2] section
 * "QKV GEMM + norm + RoPE + KV 插入融合": the projection's output is taken
 * head by head; queries and index queries get norm and RoPE; K, V and the
 * index key are quantised into the caches).  The pages state neither the
 * norm nor the rotary detail.  Readings taken: a per-head RMS norm with one
 * learned weight vector per head kind, then rotate-half rotary embedding of
 * dims (i, i + 64) from a caller-supplied cos/sin table, applied to every
 * head except the values (keys need the same rotation as the queries for the
 * scores to depend on relative position).
 *
 * Output columns: 45 heads of 128 -- query heads 0..31, key heads 32..35,
 * value heads 36..39, index queries 40..43, index key 44.  Head kinds for the
 * norm weight: 0 queries, 1 keys, 2 index queries, 3 index key. */
#define REF_QKV_HEADS 45

/* BF16: the upper 16 bits of an IEEE binary32. */
double ref_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* x: [n][hidden] BF16, w: [45*128][hidden] BF16 (row c produces column c),
 * norm_weight: [4][128], rope: [rope_rows][128] (cos of the 64 frequencies,
 * then their sin), pos: [n].  out: [n][45][128] FP32, each value rounded once
 * from double; a token whose position is outside [0, rope_rows) gets NaN. */
void ref_qkv_project(const uint16_t* x, const uint16_t* w, int32_t n, int32_t hidden, const float* norm_weight,
                     float eps, const float* rope, int32_t rope_rows, const int32_t* pos, float* out) {
  double h[REF_DIM], y[REF_DIM];
  for (int32_t t = 0; t < n; ++t) {
    const int p = pos[t];
    for (int hd = 0; hd < REF_QKV_HEADS; ++hd) {
      float* o = out + ((int64_t)t * REF_QKV_HEADS + hd) * REF_DIM;
      if (p < 0 || p >= rope_rows) {
        for (int d = 0; d < REF_DIM; ++d) o[d] = NAN;
        continue;
      }
      /* the projection: h_d = sum_k x[t][k] w[hd*128 + d][k] */
      for (int d = 0; d < REF_DIM; ++d) {
        const uint16_t* wr = w + ((int64_t)hd * REF_DIM + d) * hidden;
        const uint16_t* xr = x + (int64_t)t * hidden;
        double acc = 0.0;
        for (int k = 0; k < hidden; ++k) acc += ref_bf16_value(xr[k]) * ref_bf16_value(wr[k]);
        h[d] = acc;
      }
      const int is_value = hd >= 36 && hd < 40;
      if (is_value) {
        for (int d = 0; d < REF_DIM; ++d) o[d] = (float)h[d];
        continue;
      }
      const int kind = hd < 32 ? 0 : hd < 36 ? 1 : hd < 44 ? 2 : 3;
      /* RMS norm over the head's 128 values, times the kind's weight */
      double ms = 0.0;
      for (int d = 0; d < REF_DIM; ++d) ms += h[d] * h[d];
      ms /= REF_DIM;
      const double inv = 1.0 / sqrt(ms + (double)eps);
      for (int d = 0; d < REF_DIM; ++d) y[d] = h[d] * inv * (double)norm_weight[kind * REF_DIM + d];
      /* rotate-half: the pair (i, i + 64) turns by the angle whose cos and sin
       * are the table's entries i and 64 + i at the token's position */
      const float* cs = rope + (int64_t)p * REF_DIM;
      for (int i = 0; i < REF_DIM / 2; ++i) {
        const double c = cs[i], s = cs[REF_DIM / 2 + i];
        o[i] = (float)(y[i] * c - y[i + REF_DIM / 2] * s);
        o[i + REF_DIM / 2] = (float)(y[i + REF_DIM / 2] * c + y[i] * s);
      }
    }
  }
}
