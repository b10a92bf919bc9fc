// msa_scan.h -- the per-request NVFP4 index scan (steps 1 and 2: indexer
// scores fused with the 128-token block max-pool; vLLM M3.1 post, "MiniMax
// 稀疏注意力的工作原理"; "MiniMax goes sparse", section 1 Step 1), as device
// code shared by the scan kernel (msa_index.hip) and the shared-prefix kernel
// that runs scan chunks inside its own workgroups (msa_prefix.hip).
//
// NVFP4 path.  Each step streams the whole index cache (72 B per token), so
// the kernel is an HBM-bound scan; the dot products run on the matrix cores
// so that the vector ALUs are left with a handful of operations per token.
// The E2M1 codes are fed to v_mfma_scale_f32_16x16x128_f8f6f4 as they sit in
// memory (B operand, FP4) against the FP8 index queries (A operand), with
// the per-16 E4M3 scales applied after the product, once per partial result
// -- the "scale once per MMA result" idea of the post's Rubin section, which
// keeps the scores exact in the operands (no FP8 re-rounding of the keys).
// To keep the sixteen-element groups apart, A row (g, j) holds query g only
// on group j's sixteen dims and zeros elsewhere; two MFMAs per 16 tokens then
// give all 8 group partials of 4 queries.  The operand pairing of this
// instruction (measured on gfx950): the fp4 operand lane group c (lanes
// 16c..16c+15) carries dims 32c..32c+31 of its column (nibble e = dim
// 32c + e); the fp8 operand lane group c, byte e pairs with dim
// 64*(e/16) + 16c + e%16, so each 16-byte half of an A lane is one scale group
// (j = c for bytes 0..15, j = 4 + c for bytes 16..31).
// Output lane l holds rows 4*(l/16)+q: with row (g, q) -> group g = l/16 and
// j = q (first MFMA) or 4 + q (second), and column l%16 = token.  So lane l
// ends with the complete score of (group l/16, token l%16) after 8 FMAs, and
// the block max is a 16-lane row reduction.
#pragma once

#include "msa.h"
#include "msa_device.h"

namespace msa {

// One page of the index cache as one wave holds it: lane l keeps, for each
// 16-token chunk c, the 16 code bytes of token 16c + l%16, dims
// 32*(l/16)..+31 (the fp4 operand), and the 8 scale bytes of that token.  The
// 1 KB of scales arrives as one 16-byte load per lane (tokens 2l, 2l+1) and
// is redistributed through a 1 KB LDS slot of the wave (stage_scales),
// instead of eight 8-byte loads per lane.  Every load carries the streaming
// (non-temporal) hint: the index is read once per step.
struct PageRegs {
  uint4 cw[8];
  uint2 sw[8];
  uint4 sraw;
};

__device__ __forceinline__ void load_page(PageRegs& pr, const uint8_t* __restrict__ slab, int col, int grp, int lane) {
#pragma unroll
  for (int c = 0; c < 8; ++c) pr.cw[c] = nt_load4(slab + (16 * c + col) * 64 + 16 * grp);
  pr.sraw = nt_load4(slab + kScaleOff + 16 * lane);
}

// Every lane's 8 scale bytes per chunk from the wave's LDS slot.
__device__ __forceinline__ void stage_scales(PageRegs& pr, uint4* slot, int lane, int col) {
  slot[lane] = pr.sraw;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint2* s2 = reinterpret_cast<const uint2*>(slot);
#pragma unroll
  for (int c = 0; c < 8; ++c) pr.sw[c] = s2[16 * c + col];
  // the slot is rewritten by this wave's next page: keep those stores behind these reads
  __builtin_amdgcn_wave_barrier();
}

// Inclusive prefix sum over the wave's 64 lanes: within each 16-lane row by
// row shifts (a lane shifted in from outside the row reads 0), then the
// totals of the rows before, read as scalars.
__device__ __forceinline__ int wave_incl_sum(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  const int t0 = __builtin_amdgcn_readlane(v, 15), t1 = __builtin_amdgcn_readlane(v, 31);
  const int t2 = __builtin_amdgcn_readlane(v, 47);
  const int r = lane >> 4;
  return v + (r > 0 ? t0 : 0) + (r > 1 ? t1 : 0) + (r > 2 ? t2 : 0);
}

// The chunk of workgroup id (pages p0 + 4*chunk ..) and its request b,
// with b's clamped length L and newest chunk.  Workgroups 0..B-1 take each
// request's newest chunk.  Unpacked, workgroup B + b*(C-1) + i takes chunk i
// of request b, skipping the newest (C chunks per table row; the chunks past
// a context are empty).  Packed (COMPACT, B <= 64), workgroups B.. take only
// the chunks below each newest one, request after request, from a prefix sum
// of the B lengths held one per lane; false for the leftovers at the end.
// PRE: lane_len holds lens[lane] (lanes below B), loaded by the caller.
template <bool COMPACT, bool PRE = false>
__device__ __forceinline__ bool chunk_of(int id, int B, const int32_t* __restrict__ lens, int max_pages, int p0,
                                         int lane, int& b, int& L, int& latest, int& chunk, int lane_len = 0) {
  if (COMPACT && id >= B) {
    int Ll = 0, nl = 0;
    if (lane < B) {
      Ll = clamp_len(PRE ? lane_len : lens[lane], max_pages);
      const int np = (Ll + kPage - 1) / kPage;
      nl = np > p0 ? (np - 1 - p0) / 4 : 0;
    }
    const int incl = wave_incl_sum(nl, lane);
    const int k = id - B;
    if (k >= __builtin_amdgcn_readlane(incl, 63)) return false;
    b = (int)__popcll(__ballot(incl <= k));  // requests whose chunks all lie before k
    if (b >= B) return false;                // (never, with k below the total: keeps b in range)
    chunk = k - __builtin_amdgcn_readlane(incl - nl, b);
    L = __builtin_amdgcn_readlane(Ll, b);
    latest = __builtin_amdgcn_readlane(nl, b);
    return chunk >= 0 && chunk < latest;
  }
  const int C = (max_pages - p0 + 3) / 4;
  b = id < B ? id : (id - B) / max(C - 1, 1);
  const int i_rest = id < B ? 0 : (id - B) % max(C - 1, 1);
  L = clamp_len(lens[b], max_pages);  // id < B: a scalar load, first in the newest chunk's chain
  const int np = (L + kPage - 1) / kPage;
  latest = np > p0 ? (np - 1 - p0) / 4 : 0;
  chunk = id < B ? latest : (i_rest < latest ? i_rest : i_rest + 1);
  return true;
}

// Packed grid: the pages past request b's newest chunk (from page jf on) have
// no workgroup; the newest chunk's waves write their -inf block scores, each
// wave its share of every row, after its own pages.
template <int R>
__device__ __forceinline__ void fill_past_chunks(float* __restrict__ block_scores, int b, int jf, int max_pages) {
  for (int rg = 0; rg < R * kGroups; ++rg) {
    float* row = block_scores + ((int64_t)b * R * kGroups + rg) * max_pages;
    for (int j = jf + (int)threadIdx.x; j < max_pages; j += 256) row[j] = -__builtin_inff();
  }
}

// Scores of one resident page for all R rows; returns per-row maxima (unscaled).
template <int R, bool kTok>
__device__ __forceinline__ void score_page(const PageRegs& pr, const v8i (&A)[R][2], const int (&pos_lim)[R], int j,
                                           int b, int grp, int col, float out_scale, int64_t T,
                                           float* __restrict__ token_scores, float (&m)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) m[r] = -__builtin_inff();
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const v8i Bop = v8i{(int)pr.cw[c].x, (int)pr.cw[c].y, (int)pr.cw[c].z, (int)pr.cw[c].w, 0, 0, 0, 0};
    float s[8];
    {
      auto s01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)pr.sw[c].x, false);
      auto s23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)pr.sw[c].x, true);
      auto s45 = __builtin_amdgcn_cvt_pk_f32_fp8((int)pr.sw[c].y, false);
      auto s67 = __builtin_amdgcn_cvt_pk_f32_fp8((int)pr.sw[c].y, true);
      s[0] = s01[0]; s[1] = s01[1]; s[2] = s23[0]; s[3] = s23[1];
      s[4] = s45[0]; s[5] = s45[1]; s[6] = s67[0]; s[7] = s67[1];
    }
    const int t = j * kPage + 16 * c + col;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const v4f z = {0.f, 0.f, 0.f, 0.f};
      const v4f d0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[r][0], Bop, z, 0, 4, 0, 127, 0, 127);
      const v4f d1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[r][1], Bop, z, 0, 4, 0, 127, 0, 127);
      float sc = s[0] * d0[0];
      sc = fmaf(s[1], d0[1], sc);
      sc = fmaf(s[2], d0[2], sc);
      sc = fmaf(s[3], d0[3], sc);
      sc = fmaf(s[4], d1[0], sc);
      sc = fmaf(s[5], d1[1], sc);
      sc = fmaf(s[6], d1[2], sc);
      sc = fmaf(s[7], d1[3], sc);
      const bool vis = t <= pos_lim[r];
      if (kTok)
        token_scores[(((int64_t)b * R + r) * kGroups + grp) * T + t] = vis ? sc * out_scale : -__builtin_inff();
      if (vis) m[r] = pool_max(m[r], sc);
    }
  }
}

// FP16 form for several rows (R >= 3): the page's keys are converted exactly
// to FP16 (E2M1 code x E4M3 group scale has at most 6 significant bits) and
// S^T = K Q^T runs on v_mfma_f32_16x16x32_f16 with 16 index queries per tile
// (query 4r + g = column of the tile), instead of two masked FP4 products per
// row.  The contraction dims are taken in the order the page registers hold
// them: in k-step ks, lane group a carries dims 32a + 8ks .. 32a + 8ks + 7 of
// both operands.  Output lane (n, a) holds tokens 4a .. 4a+3 of the chunk for
// query n; the block max is a running max over the chunks, then a reduction
// over the four lane groups.  Writes the block scores (and token scores) of
// page j itself.
template <int R>
constexpr int f16_tiles() { return (R * kGroups + 15) / 16; }

template <int R>
__device__ __forceinline__ void load_queries_f16(const uint8_t* __restrict__ q_idx, int b, int lane,
                                                 h8 (&Q)[f16_tiles<R>()][4]) {
  const int n = lane & 15, a = lane >> 4;
#pragma unroll
  for (int qt = 0; qt < f16_tiles<R>(); ++qt) {
    const int qi = 16 * qt + n;  // (row qi / 4, group qi % 4)
    const bool ok = qi < R * kGroups;
    const uint8_t* q = q_idx + ((int64_t)b * R * kGroups + (ok ? qi : 0)) * kDim;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint2 w = *reinterpret_cast<const uint2*>(q + 32 * a + 8 * ks);
      w = ok ? w : make_uint2(0, 0);
      const h2 x0 = e4m3x2_to_h2<false>(w.x), x1 = e4m3x2_to_h2<true>(w.x);
      const h2 x2 = e4m3x2_to_h2<false>(w.y), x3 = e4m3x2_to_h2<true>(w.y);
      Q[qt][ks] = h8{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
    }
  }
}

template <int R, bool kTok>
__device__ __forceinline__ void score_page_f16(const PageRegs& pr, const h8 (&Q)[f16_tiles<R>()][4], int L, int j,
                                               int b, int lane, int max_pages, float out_scale, int64_t T,
                                               float* __restrict__ block_scores, float* __restrict__ token_scores,
                                               bool keep = true) {
  constexpr int QT = f16_tiles<R>();
  const int n = lane & 15, a = lane >> 4;
  float mx[QT];
  int plim[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mx[qt] = -__builtin_inff();
    plim[qt] = L - R + (16 * qt + n) / kGroups;  // last visible position of this column's row
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    // this lane's dims 32a .. 32a+31 are scale groups 2a and 2a+1 of its token
    const h2 sc = e4m3x2_to_h2<false>(a < 2 ? pr.sw[c].x >> (16 * a) : pr.sw[c].y >> (16 * (a - 2)));
    const uint32_t w[4] = {pr.cw[c].x, pr.cw[c].y, pr.cw[c].z, pr.cw[c].w};
    h8 kv[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const _Float16 s1 = ks < 2 ? sc[0] : sc[1];
      kv[ks] = e2m1x8_to_h8(w[ks]) * h8{s1, s1, s1, s1, s1, s1, s1, s1};
    }
    const int t0 = j * kPage + 16 * c + 4 * a;  // token of this lane's first output row
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv[ks], Q[qt][ks], acc, 0, 0, 0);
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool vis = t0 + i <= plim[qt];
        v[i] = vis ? acc[i] : -__builtin_inff();
        if (vis) mx[qt] = pool_max(mx[qt], acc[i]);
      }
      const int qi = 16 * qt + n;
      if (kTok && qi < R * kGroups)
        *reinterpret_cast<float4*>(&token_scores[((int64_t)b * R * kGroups + qi) * T + t0]) =
            make_float4(v[0] * out_scale, v[1] * out_scale, v[2] * out_scale, v[3] * out_scale);
    }
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float m = mx[qt];
    m = rows_max4(m);
    const int qi = 16 * qt + n;
    if (keep && a == 0 && qi < R * kGroups) block_scores[((int64_t)b * R * kGroups + qi) * max_pages + j] = m * out_scale;
  }
}

// The step's new tokens, for the insert fused into the index launch: rows of
// positions L_b - R .. L_b - 1 of every request ([B][R][4][128] keys and
// values, [B][R][128] index keys, FP32), written into the NVFP4 caches (keys
// and index keys token-major, values dim-major) at the slots the block table
// gives them.
struct NewRows {
  const float* k;
  const float* v;
  const float* idx;
  uint8_t* kpages;
  uint8_t* vpages;
  uint8_t* ipages;
  int32_t kv_num_pages;
  float ts_k, ts_v, ts_i;
};

// The step's new tokens of request b that fall in [t0, t1) (t0 < t1, within
// [L - R, L)), written into the three caches by a whole workgroup of 256
// threads (one 16-lane row per 16-element group, as the insert kernel does).
// The caller makes them visible to its waves (workgroup release, barrier,
// acquire) before reading the pages.
// Which caches insert_new_rows writes: all three, the index keys only, or the
// keys and values only.
enum InsertPart { kInsertAll = 0, kInsertIndex = 1, kInsertKV = 2 };

template <int R, int PART = kInsertAll>
__device__ __forceinline__ void insert_new_rows(const int32_t* __restrict__ table, int32_t max_pages, int32_t num_pages,
                                                int b, int L, int t0, int t1, const NewRows& NR) {
  // 16-dim groups per token: 32 keys, 32 values, 8 index keys (or a part of them)
  constexpr int G = PART == kInsertIndex ? 8 : (PART == kInsertKV ? 64 : 72);
  const int i = threadIdx.x & 15;
  const int nrow = (t1 - t0) * G;
  // row rr: token t0 + rr / G, then its key, value and index-key groups
  auto locate = [&](int rr, int& tok, int& c, int& head, int& grp) {
    tok = t0 + rr / G;
    int u = rr % G + (PART == kInsertIndex ? 64 : 0);
    c = u < 32 ? 0 : (u < 64 ? 1 : 2);
    u -= 32 * c;
    head = u >> 3;
    grp = u & 7;
  };
  // a batch of rows per 16-lane row of threads: every source load issues
  // before the first store (which could alias them), so a batch is one
  // memory round -- sized for all of a chunk's rows (one round) up to four
  // new rows, two rounds beyond.  The new tokens lie on at most two pages
  // (R <= 128), whose table entries load with the sources.
  constexpr int kBatch = (G * R + 15) / 16 < 18 ? (G * R + 15) / 16 : 18;
  const int pa = t0 / kPage;
  const int ph_a = table[(int64_t)b * max_pages + pa], ph_b = table[(int64_t)b * max_pages + (t1 - 1) / kPage];
  for (int rb = threadIdx.x >> 4; rb < nrow; rb += 16 * kBatch) {
    float x[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      int tok, c, head, grp;
      locate(min(rb + 16 * k, nrow - 1), tok, c, head, grp);
      const float* src = c == 0 ? NR.k : (c == 1 ? NR.v : NR.idx);
      x[k] = src[(((int64_t)b * R + tok - (L - R)) * (c == 2 ? 1 : kGroups) + head) * kDim + grp * 16 + i];
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (rb + 16 * k >= nrow) break;  // uniform over the 16-lane row
      int tok, c, head, grp;
      locate(rb + 16 * k, tok, c, head, grp);
      const int heads = c == 2 ? 1 : kGroups;
      const int ph = tok / kPage == pa ? ph_a : ph_b;
      const bool valid = ph >= 0 && ph < (c == 2 ? num_pages : NR.kv_num_pages);
      uint8_t* base = c == 0 ? NR.kpages : (c == 1 ? NR.vpages : NR.ipages);
      uint32_t code;
      const uint32_t sc = nvfp4_row_quantize(x[k], c == 0 ? NR.ts_k : (c == 1 ? NR.ts_v : NR.ts_i), code);
      nvfp4_row_store(base + ((int64_t)(valid ? ph : 0) * heads + head) * kNvSlab, tok & (kPage - 1), grp, i, code, sc,
                      c == 1, valid);
    }
  }
}

// Index queries of request b in the scan's operand form: the FP4 form's A
// operands (the query of row r masked to one scale group per MFMA row) or the
// FP16 form's tiles of 16 index queries.
template <int R, bool F16>
struct ScanQueries {
  v8i A[F16 ? 1 : R][2];
  h8 Qh[F16 ? f16_tiles<R>() : 1][4];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ q_idx, int b, int lane) {
    if constexpr (F16) {
      load_queries_f16<R>(q_idx, b, lane, Qh);
    } else {
      const int grp = lane >> 4, i = lane & 15;
      const int gq = i >> 2, jj = i & 3;
      const bool on = (jj == grp);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint8_t* q = q_idx + (((int64_t)b * R + r) * kGroups + gq) * kDim;
        uint4 lo = on ? *reinterpret_cast<const uint4*>(q + 16 * grp) : make_uint4(0, 0, 0, 0);
        uint4 hi = on ? *reinterpret_cast<const uint4*>(q + 64 + 16 * grp) : make_uint4(0, 0, 0, 0);
        A[r][0] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
        A[r][1] = v8i{0, 0, 0, 0, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    }
  }
};

// Page j of request b, resident in pr: its scale bytes go through the wave's
// LDS slot, then the scores of all R rows (positions past L - R + r masked),
// their block maxima and the block-score stores (token scores too with kTok);
// keep = false scores the page but stores nothing.
template <int R, bool kTok, bool F16>
__device__ __forceinline__ void score_resident_page(PageRegs& pr, const ScanQueries<R, F16>& q, uint4* slot, int L,
                                                    int j, int b, int lane, int max_pages, float out_scale, int64_t T,
                                                    float* __restrict__ block_scores,
                                                    float* __restrict__ token_scores, bool keep = true) {
  const int grp = lane >> 4, col = lane & 15;
  stage_scales(pr, slot, lane, col);
  if constexpr (F16) {
    score_page_f16<R, kTok>(pr, q.Qh, L, j, b, lane, max_pages, out_scale, T, block_scores, token_scores, keep);
  } else {
    int pos_lim[R];
#pragma unroll
    for (int r = 0; r < R; ++r) pos_lim[r] = L - R + r;
    float m[R];
    score_page<R, kTok>(pr, q.A, pos_lim, j, b, grp, col, out_scale, T, token_scores, m);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float mm = wave_max16(m[r]);
      if (keep && col == 0) block_scores[(((int64_t)b * R + r) * kGroups + grp) * max_pages + j] = mm * out_scale;
    }
  }
}

// Block j of request b holds no visible token (past the context, or its page
// is outside the pool): -inf block scores for all R rows (token scores too).
template <int R, bool kTok>
__device__ __forceinline__ void empty_block(int j, int b, int lane, int max_pages, int64_t T,
                                            float* __restrict__ block_scores, float* __restrict__ token_scores) {
  const int grp = lane >> 4, col = lane & 15;
  if (kTok)
#pragma unroll
    for (int r = 0; r < R; ++r)
      for (int c = 0; c < 8; ++c)
        token_scores[(((int64_t)b * R + r) * kGroups + grp) * T + j * kPage + 16 * c + col] = -__builtin_inff();
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (col == 0) block_scores[(((int64_t)b * R + r) * kGroups + grp) * max_pages + j] = -__builtin_inff();
}

// One chunk of the scan, run by a whole workgroup of 4 waves: page
// p0 + 4*chunk + wave of request b per wave (one page per wave).  The scan
// covers pages p0 .. max_pages-1 of every request (p0 > 0: the leading pages
// are shared by all requests and scored once, by the prefix product).
// Chunk ids 0 .. B*C-1 (C = page chunks per request row of the table past
// p0) map to chunks by chunk_of.  Ids 0..B-1 take the chunk holding each
// request's newest tokens, so the chunks that insert the step's tokens start
// first.  Each request's other chunks are consecutive ids, which the
// dispatcher deals round-robin to the 8 XCDs.  Unpacked, the chunks past a
// context (nothing to score) close its run; packed (COMPACT: B <= 64, block
// scores only) they get no id, so a ragged batch no longer spends workgroup
// slots on them between the real chunks.  With INSERT the workgroup first
// writes the new tokens that fall in its chunk into the caches (one 16-lane
// row per 16-element group, as the insert kernel does) and makes them visible
// to its own waves before any page is read.  Control flow is uniform over the
// workgroup up to the insert's barrier; a return ends the chunk, not the
// caller.  PRE, lane_len: see chunk_of.
template <int R, bool kTok, bool INSERT = false, bool F16 = false, bool COMPACT = false, bool PRE = false>
__device__ __forceinline__ void nvfp4_scan_chunk(
    int id, const int32_t* __restrict__ table, const int32_t* __restrict__ lens, int32_t max_pages,
    const uint8_t* __restrict__ q_idx, float out_scale, const uint8_t* __restrict__ pages, int32_t num_pages,
    float* __restrict__ block_scores, float* __restrict__ token_scores, int32_t B, int32_t p0, const NewRows& NR,
    int lane_len = 0) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int b, L, latest, chunk;
  if (!chunk_of<COMPACT, PRE>(id, B, lens, max_pages, p0, lane, b, L, latest, chunk, lane_len)) return;
  const int npb = (L + kPage - 1) / kPage;
  if (INSERT) {
    // new tokens [max(L - R, 0), L) that lie in this chunk's token range
    const int lo = (p0 + chunk * 4) * kPage;
    const int t0 = max(max(L - R, 0), lo), t1 = min(L, lo + 4 * kPage);
    if (t0 < t1) {
      insert_new_rows<R>(table, max_pages, num_pages, b, L, t0, t1, NR);
      // the index keys just written are read back by this workgroup's waves
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __syncthreads();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
  }
  auto fill_past = [&] {
    if (COMPACT && id < B) fill_past_chunks<R>(block_scores, b, min(p0 + (latest + 1) * 4, max_pages), max_pages);
  };
  const int j = p0 + chunk * 4 + wave;
  if (j >= max_pages) {
    fill_past();
    return;
  }
  const int grp = lane >> 4;  // this lane's query group (output) and fp4 lane group
  const int col = lane & 15;  // token within a 16-token chunk
  const int64_t T = (int64_t)max_pages * kPage;

  // this wave's physical page (-1: past the context or outside the pool)
  int phys = j < npb ? table[(int64_t)b * max_pages + j] : -1;
  if (phys >= num_pages) phys = -1;

  ScanQueries<R, F16> q;
  q.load(q_idx, b, lane);
  __shared__ uint4 s_scales[4][64];
  if (phys >= 0) {
    PageRegs pr;
    load_page(pr, pages + (int64_t)phys * kNvSlab, col, grp, lane);
    score_resident_page<R, kTok, F16>(pr, q, &s_scales[wave][0], L, j, b, lane, max_pages, out_scale, T,
                                      block_scores, token_scores);
  } else {
    empty_block<R, kTok>(j, b, lane, max_pages, T, block_scores, token_scores);
  }
  fill_past();
}

// Shared-prefix decode with the scan fused into the prefix product's launch
// (msa_prefix.hip): 1 when the fused form does not apply, else 0 or -1.
int launch_prefix_scan(const msa_batch* bt, const uint8_t* q, float q_scale, const msa_cache* ic, float* bs,
                       float* ts, const NewRows& nr, bool insert, hipStream_t s);

}  // namespace msa
