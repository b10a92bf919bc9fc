/*
 * Sanitizer run of the CPU oracle (test infrastructure, built by
 * tests/test_sanitizers.py with gcc -fsanitize=address,undefined).  Every
 * oracle entry point runs on small ragged inputs in every cache format and
 * layout, with the edge cases the tests use: empty and one-token requests,
 * contexts ending on a page boundary, slots outside the pool, NaN and
 * infinite inputs, selections smaller than the context.  The values are
 * checked by the pytest pins; this run only has to finish without a
 * sanitizer report.
 */
#include "../../oracle/msa_oracle.c"

#include <stdio.h>
#include <stdlib.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) { /* splitmix64 */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static float uniform_pm(float a) { return (float)((double)(next_u64() >> 11) / 9007199254740992.0 * 2.0 - 1.0) * a; }

enum { B = 4, R = 3, G = 4, H = 32, MAXP = 5, NPAGES = 12 };

static void fill_rows(float* x, int64_t n) {
  for (int64_t i = 0; i < n; ++i) x[i] = uniform_pm(3.0f);
  if (n > 40) {
    x[3] = NAN, x[7] = INFINITY, x[11] = -INFINITY, x[13] = 1e-40f, x[17] = -0.0f, x[19] = 1e30f;
    for (int i = 20; i < 36; ++i) x[i] = 0.0f; /* an all-zero 16-element group */
  }
}

int main(void) {
  /* ---- codecs over special values */
  const float specials[] = {0.0f, -0.0f, 1e-45f, 1e-40f, 0.25f, 0.75f, 5.0f, 6.0f, 448.0f, 464.0f, 1e30f,
                            INFINITY, -INFINITY, NAN, -NAN};
  double acc = 0.0;
  for (unsigned i = 0; i < sizeof(specials) / sizeof(specials[0]); ++i) {
    acc += ref_e4m3_encode(specials[i]) + ref_e2m1_encode(specials[i]) + ref_fp8_quantize(specials[i], 0.01f);
  }
  for (int c = 0; c < 256; ++c) acc += isnan(ref_e4m3_value((uint8_t)c)) ? 1.0 : 0.0;
  for (int c = 0; c < 16; ++c) acc += ref_e2m1_value((uint8_t)c);
  for (int s = 0; s < 256; s += 5)
    for (int c = 0; c < 16; ++c) {
      double v = ref_nvfp4_value((uint8_t)c, (uint8_t)s, 0.5f);
      acc += isnan(v) ? 0.0 : v;
    }

  /* ---- caches in every format and layout */
  const int32_t lens[B] = {0, 1, 129, MAXP * REF_PAGE};
  int32_t table[B * MAXP];
  for (int i = 0; i < B * MAXP; ++i) table[i] = (int32_t)(next_u64() % NPAGES);
  const int combos[][3] = {{REF_F32, REF_TOKEN_MAJOR, 1},      {REF_F32, REF_TOKEN_MAJOR, G},
                           {REF_NVFP4, REF_TOKEN_MAJOR, 1},    {REF_NVFP4, REF_TOKEN_MAJOR, G},
                           {REF_NVFP4, REF_DIM_MAJOR, G},      {REF_FP8_E4M3, REF_TOKEN_MAJOR, G},
                           {REF_FP8_E4M3, REF_DIM_MAJOR, G},   {REF_FP8_E4M3, REF_HALF_ROWS, 1}};
  const int n_tok = 300;
  int64_t* slots = malloc(sizeof(int64_t) * n_tok);
  for (int i = 0; i < n_tok; ++i) slots[i] = i * 5 % (NPAGES * REF_PAGE); /* distinct */
  slots[0] = -1;                                                        /* rejected */
  slots[1] = (int64_t)NPAGES * REF_PAGE;                                /* rejected */
  float* rows = malloc(sizeof(float) * n_tok * G * REF_DIM);
  fill_rows(rows, (int64_t)n_tok * G * REF_DIM);
  ref_cache caches[8];
  for (int k = 0; k < 8; ++k) {
    ref_cache* c = &caches[k];
    c->dtype = combos[k][0];
    c->layout = combos[k][1];
    c->num_heads = combos[k][2];
    c->num_pages = NPAGES;
    c->tensor_scale = c->dtype == REF_F32 ? 1.0f : 0.0078125f;
    c->pages = calloc((size_t)slab_bytes(c) * NPAGES * c->num_heads, 1);
    int64_t bad = ref_cache_write_many(c, slots, n_tok, rows);
    if (bad != 2) {
      fprintf(stderr, "combo %d: %lld rejected slots, expected 2\n", k, (long long)bad);
      return 1;
    }
    float* pages_out = malloc(sizeof(float) * NPAGES * c->num_heads * REF_PAGE * REF_DIM);
    int32_t all[NPAGES];
    for (int p = 0; p < NPAGES; ++p) all[p] = p;
    ref_cache_dequant_pages(c, all, NPAGES, pages_out);
    acc += isnan(pages_out[5]) ? 0.0 : pages_out[5];
    free(pages_out);
  }

  /* ---- queries */
  const int64_t nqi = (int64_t)B * R * G * REF_DIM, nq = (int64_t)B * R * H * REF_DIM;
  float* qf = malloc(sizeof(float) * nq);
  fill_rows(qf, nq);
  uint8_t* qb = malloc(nq);
  ref_quantize_queries(qf, nq, 1.0f, qb);
  double* q = malloc(sizeof(double) * nq);
  double* qi = malloc(sizeof(double) * nqi);
  ref_decode_queries(qb, REF_FP8_E4M3, 1.0f, nq, q);
  ref_decode_queries(qb, REF_FP8_E4M3, 1.0f, nqi, qi);
  ref_decode_queries(qf, REF_F32, 1.0f, nqi, qi);

  /* ---- the step, per cache format: index, pool, select (topk below and above the
     context), attention, and the whole step */
  ref_batch bt = {B, R, MAXP, table, lens};
  const int64_t T = (int64_t)MAXP * REF_PAGE;
  double* ts = malloc(sizeof(double) * B * R * G * T);
  double* as = malloc(sizeof(double) * B * R * G * T);
  double* bs = malloc(sizeof(double) * B * R * G * MAXP);
  int32_t* sel = malloc(sizeof(int32_t) * B * R * G * 64);
  int32_t* cnt = malloc(sizeof(int32_t) * B * R * G);
  double* out = malloc(sizeof(double) * nq);
  const int sets[][3] = {{0, 1, 1}, {2, 3, 4}, {2, 3, 4}, {7, 5, 6}}; /* index, key, value cache */
  const int topks[] = {1, 2, 4, 16, 64};
  for (int s = 0; s < 4; ++s) {
    const ref_cache* ic = &caches[sets[s][0]];
    const ref_cache* kc = &caches[sets[s][1]];
    const ref_cache* vc = &caches[sets[s][2]];
    ref_index_scores(&bt, G, qi, ic, ts, as);
    ref_block_maxpool(&bt, G, ts, bs);
    bs[3] = NAN;
    for (unsigned t = 0; t < sizeof(topks) / sizeof(topks[0]); ++t) {
      ref_select(&bt, G, bs, topks[t], sel, cnt);
      ref_attention(&bt, H, G, q, 0.08838834764831845, kc, vc, sel, cnt, topks[t], out);
    }
    ref_decode_step(&bt, H, G, qi, q, 0.08838834764831845, ic, kc, vc, 16, ts, bs, sel, cnt, out);
    acc += isnan(out[0]) ? 0.0 : out[0];
  }

  /* ---- the projection, with positions outside the rotary table */
  enum { NT = 3, HID = 256, ROWS = 8 };
  uint16_t* xw = malloc(sizeof(uint16_t) * (NT + REF_QKV_HEADS * REF_DIM) * HID);
  for (int i = 0; i < (NT + REF_QKV_HEADS * REF_DIM) * HID; ++i) xw[i] = (uint16_t)(next_u64() & 0x7F7F);
  float norm_w[4 * REF_DIM], rope[ROWS * REF_DIM], proj[NT * REF_QKV_HEADS * REF_DIM];
  for (int i = 0; i < 4 * REF_DIM; ++i) norm_w[i] = 1.0f;
  for (int i = 0; i < ROWS * REF_DIM; ++i) rope[i] = uniform_pm(1.0f);
  const int32_t pos[NT] = {0, ROWS - 1, ROWS};
  ref_qkv_project(xw, xw + NT * HID, NT, HID, norm_w, 1e-6f, rope, ROWS, pos, proj);
  acc += isnan(proj[0]) ? 0.0 : proj[0];

  for (int k = 0; k < 8; ++k) free(caches[k].pages);
  free(slots), free(rows), free(qf), free(qb), free(q), free(qi), free(ts), free(as), free(bs), free(sel);
  free(cnt), free(out), free(xw);
  printf("oracle sanitizer run ok (checksum %g)\n", acc);
  return 0;
}
