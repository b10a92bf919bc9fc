// msa_prefix.hip -- steps 1 and 2 over the leading pages that every request
// of the batch shares (a common system prompt or document: the shared-prefix
// workload).  The indexer scores each context token against one index query
// per (request, row, group) (vLLM M3.1 post, "MiniMax 稀疏注意力的工作原理";
// "MiniMax goes sparse", section 1 Step 1); when the tokens are the same
// physical pages for every request, one read of a page serves all B x R x 4
// queries, and the scores of that page form a dense product
//     S[t, c] = K_idx[t, :] . q_idx[c, :]     (128 tokens x B*R*4 columns)
// -- a contraction, so it runs on the matrix cores.
//
// Exactness: an NVFP4 key element is e2m1 x e4m3 (at most 6 significant
// bits), exact in FP16; the E4M3 queries are exact in FP16 too.  So the keys
// are dequantised to FP16 (hardware E2M1 -> FP16 conversion, then one packed
// FP16 multiply by the E4M3 group scale) and multiplied on
// v_mfma_f32_16x16x32_f16 with FP32 accumulation; the tensor scale and the
// query scale multiply the FP32 result.  (The FP8 x FP4 instruction of the
// per-request scan would need one masked query row per 16-dim scale group --
// eight times the matrix work of this dense product.)
//
// Work split: a workgroup of 4 waves walks PPW consecutive prefix pages for
// 64*NTILE query columns, 16*NTILE per wave (held in registers as FP16 for
// the whole walk).  Each page is read and dequantised once per workgroup,
// into an LDS image laid out exactly as the matrix operand is consumed:
// block (m, ks) holds, for lane (n, a) = (lane % 16, lane / 16), the 8 FP16
// keys of token 16m + n at dims 32a + 8ks .. +7 (the queries use the same dim
// order, so the product is unchanged).  Wave w dequantises M-tiles w and
// w + 4 of a page -- its lanes load exactly the 16 code bytes they write
// back, so both the LDS writes and the operand reads are 1 KB contiguous per
// instruction.  Pages are double-buffered in LDS, and their codes are loaded
// two pages ahead into registers, with one workgroup barrier per page.  Output lane (n, a) holds tokens 16m + 4a + 0..3 of
// column n: the block max is kept per lane over the eight M-tiles and
// finished across the four lane groups.
#include <climits>
#include <type_traits>

#include "msa_device.h"
#include "msa_kernels.h"
#include "msa_scan.h"

namespace msa {

namespace {

// E4M3 index queries of 16 columns -> FP16, in the k-step order above.
template <int NTILE>
__device__ __forceinline__ void load_prefix_queries(const uint8_t* __restrict__ q_idx, int col0, int ncols, int n,
                                                    int a, h8 (&Q)[NTILE][4]) {
#pragma unroll
  for (int nt = 0; nt < NTILE; ++nt) {
    const int c = col0 + 16 * nt + n;
    const bool ok = c < ncols;
    const uint8_t* q = q_idx + (int64_t)(ok ? c : 0) * kDim;
    // the lane's 32 bytes in two 16-byte loads (every workgroup reads the same
    // queries at its start: fewer, wider requests)
    uint4 w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      w[h] = *reinterpret_cast<const uint4*>(q + 32 * a + 16 * h);
      w[h] = ok ? w[h] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint32_t lo = (ks & 1) ? w[ks >> 1].z : w[ks >> 1].x, hi = (ks & 1) ? w[ks >> 1].w : w[ks >> 1].y;
      const h2 x0 = e4m3x2_to_h2<false>(lo), x1 = e4m3x2_to_h2<true>(lo);
      const h2 x2 = e4m3x2_to_h2<false>(hi), x3 = e4m3x2_to_h2<true>(hi);
      Q[nt][ks] = h8{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
    }
  }
}

constexpr int kPfxImgH8 = 8 * 4 * 64;  // one dequantised page in LDS: [m][ks][lane] x 8 FP16 = 32 KB

// The part of a page wave w dequantises: M-tiles w and w + 4, token 16m + n,
// dims 32a .. 32a+31 (16 code bytes) and the E4M3 scales of groups 2a, 2a+1.
struct PrefixPart {
  uint4 kc[2];
  uint32_t ks[2];
};

__device__ __forceinline__ void load_prefix_part(const uint8_t* __restrict__ slab, int wave, int n, int a,
                                                 PrefixPart& p) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int m = wave + 4 * h;
    p.kc[h] = nt_load4(slab + (16 * m + n) * 64 + 16 * a);
    p.ks[h] = *reinterpret_cast<const uint16_t*>(slab + kScaleOff + (16 * m + n) * 8 + 2 * a);
  }
}

// Piece `piece` (0..3) of the part into the LDS image: M-tile wave + 4*(piece/2),
// k-steps 2*(piece%2) and 2*(piece%2) + 1 (one E4M3 scale group).
__device__ __forceinline__ void store_prefix_piece(const PrefixPart& p, int wave, int lane, h8* __restrict__ img,
                                                   int piece) {
  const int h = piece >> 1, m = wave + 4 * h;
  const uint32_t sw = p.ks[h];
  const _Float16 s = e4m3x2_to_h2<false>(sw)[piece & 1];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ks = 2 * (piece & 1) + i;
    const uint32_t w = ks == 0 ? p.kc[h].x : ks == 1 ? p.kc[h].y : ks == 2 ? p.kc[h].z : p.kc[h].w;
    img[(m * 4 + ks) * 64 + lane] = e2m1x8_to_h8(w) * h8{s, s, s, s, s, s, s, s};
  }
}

// FP8 index cache (E4M3 per element, half-rows slab: [t/16][d/64][t%16][d%64]):
// the same part of a page, token 16m + n, dims 32a .. 32a+31 -- 32 bytes at
// one place of the slab; E4M3 is exact in FP16 and the tensor scale is
// applied to the FP32 result, as for NVFP4.
struct PrefixPart8 {
  uint4 kc[2][2];
};

__device__ __forceinline__ void load_prefix_part(const uint8_t* __restrict__ slab, int wave, int n, int a,
                                                 PrefixPart8& p) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int m = wave + 4 * h;
    const uint8_t* src = slab + m * 2048 + (a >> 1) * 1024 + n * 64 + (a & 1) * 32;
    p.kc[h][0] = nt_load4(src);
    p.kc[h][1] = nt_load4(src + 16);
  }
}

__device__ __forceinline__ void store_prefix_piece(const PrefixPart8& p, int wave, int lane, h8* __restrict__ img,
                                                   int piece) {
  const int h = piece >> 1, m = wave + 4 * h;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ks = 2 * (piece & 1) + i;
    const uint4& q = p.kc[h][ks >> 1];
    const uint32_t lo = (ks & 1) ? q.z : q.x, hi = (ks & 1) ? q.w : q.y;
    const h2 x0 = e4m3x2_to_h2<false>(lo), x1 = e4m3x2_to_h2<true>(lo);
    const h2 x2 = e4m3x2_to_h2<false>(hi), x3 = e4m3x2_to_h2<true>(hi);
    img[(m * 4 + ks) * 64 + lane] = h8{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
  }
}

template <typename Part>
__device__ __forceinline__ void store_prefix_part(const Part& p, int wave, int lane, h8* __restrict__ img) {
#pragma unroll
  for (int piece = 0; piece < 4; ++piece) store_prefix_piece(p, wave, lane, img, piece);
}

// Scores of one page (its LDS image) for this wave's columns; mx = per-lane
// maxima over the lane's tokens (unscaled).  Two M-tiles at a time (2*NTILE
// independent accumulators).  The vector ALUs may only read an MFMA result
// once the instruction has completed, so reading each pair's accumulators
// right after its last MFMA would drain the matrix pipe eight times a page:
// instead the accumulators are double-buffered and pair p is max-pooled after
// the MFMAs of pair p+1 have been issued.  side(p) runs right after the
// MFMAs of pair p are issued: vector work of the caller's (the next page's
// dequantisation) that then overlaps them.  MASK: some column does not see
// the whole page (token t counts for column c only when t <= pos[c]).
template <int NTILE, bool MASK, bool kTok, typename Side>
__device__ __forceinline__ void score_prefix_page(const h8* __restrict__ img, const h8 (&Q)[NTILE][4],
                                                  const int (&pos)[NTILE], int j, int lane, int col0, int ncols,
                                                  float out_scale, int64_t T, float* __restrict__ token_scores,
                                                  float (&mx)[NTILE], Side&& side) {
  const int n = lane & 15, a = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NTILE; ++nt) mx[nt] = -__builtin_inff();
  v4f acc[2][2][NTILE];  // [buffer][M-tile of the pair][column tile]
  auto multiply = [&](int m2, v4f (&ac)[2][NTILE]) {
    h8 kv[2][4];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kv[mm][ks] = img[((m2 + mm) * 4 + ks) * 64 + lane];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int nt = 0; nt < NTILE; ++nt) ac[mm][nt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int nt = 0; nt < NTILE; ++nt)
          ac[mm][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv[mm][ks], Q[nt][ks], ac[mm][nt], 0, 0, 0);
  };
  auto pool = [&](int m2, const v4f (&ac)[2][NTILE]) {
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int t0 = j * kPage + 16 * (m2 + mm) + 4 * a;  // token of ac[mm][.][0]
#pragma unroll
      for (int nt = 0; nt < NTILE; ++nt) {
        const v4f& x = ac[mm][nt];
        if (!MASK) {
          mx[nt] = pool_max(pool_max(pool_max(pool_max(mx[nt], x[0]), x[1]), x[2]), x[3]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) mx[nt] = pool_max(mx[nt], t0 + i <= pos[nt] ? x[i] : -__builtin_inff());
        }
        if (kTok) {
          const int c = col0 + 16 * nt + n;
          if (c < ncols) {
            float4 o;
            o.x = t0 + 0 <= pos[nt] ? x[0] * out_scale : -__builtin_inff();
            o.y = t0 + 1 <= pos[nt] ? x[1] * out_scale : -__builtin_inff();
            o.z = t0 + 2 <= pos[nt] ? x[2] * out_scale : -__builtin_inff();
            o.w = t0 + 3 <= pos[nt] ? x[3] * out_scale : -__builtin_inff();
            *reinterpret_cast<float4*>(token_scores + (int64_t)c * T + t0) = o;
          }
        }
      }
    }
  };
  multiply(0, acc[0]);
  side(0);
#pragma unroll
  for (int p = 1; p < 4; ++p) {
    multiply(2 * p, acc[p & 1]);
    side(p);
    pool(2 * (p - 1), acc[(p - 1) & 1]);
  }
  pool(6, acc[1]);
}

}  // namespace

// One workgroup's work: pages pg*PPW .. +PPW-1 of table row `trow` (those
// below n_valid have a table entry; the rest score -inf), for query columns
// col_lo + 64*NTILE*yt .. (below col_hi).  Column c = (b*R + r)*4 + g is
// index query (b, r, g); its last visible token is pos = L_b - R + r.
// between() runs once, workgroup-uniformly, while the first two pages are in
// flight (or at once when the workgroup has no page).
template <int NTILE, int PPW, bool kTok, bool FP8 = false, typename Between>
__device__ __forceinline__ void dense_index_body(const int32_t* __restrict__ trow, const int32_t* __restrict__ lens,
                                                 int32_t max_pages, int32_t R, int32_t n_pages, int32_t n_valid,
                                                 int32_t col_lo, int32_t col_hi, int pg, int yt,
                                                 const uint8_t* __restrict__ q_idx, float out_scale,
                                                 const uint8_t* __restrict__ pages, int32_t num_pages,
                                                 float* __restrict__ block_scores, float* __restrict__ token_scores,
                                                 h8 (&s_img)[2][kPfxImgH8], Between&& between) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, a = lane >> 4;
  const int j0 = pg * PPW;
  if (j0 >= n_pages) {  // the whole workgroup
    between();
    return;
  }
  const int jn = min(PPW, n_pages - j0);
  const int ncols = col_hi;
  const int col0 = col_lo + yt * 64 * NTILE + wave * 16 * NTILE;
  const bool has_cols = col0 < ncols;  // wave-uniform; a wave without columns still dequantises
  const int64_t T = (int64_t)max_pages * kPage;

  // Order of the start-up loads: the page table, then (once it has arrived)
  // the first two pages, and only then the queries and context lengths, whose
  // conversion waits on them -- so the page loads do not queue behind it.
  int my_phys = -1;
  if (lane < jn && j0 + lane < n_valid) {
    my_phys = trow[j0 + lane];
    if (my_phys < 0 || my_phys >= num_pages) my_phys = -1;
  }
  auto phys_of = [&](int k) { return __builtin_amdgcn_readfirstlane(__shfl(my_phys, k)); };

  // Register ring of page parts: the load of page k+2 is issued before page k
  // is multiplied, and page k+1 is dequantised into the other LDS image after
  // it, so every load has two pages of matrix work to land.  Loads and
  // dequantisation are unconditional (page 0 of the pool stands in for a
  // missing page, whose image is then never read), so that each wait covers
  // exactly the loads it needs.
  constexpr int kSlab = FP8 ? kFp8Slab : kNvSlab;
  std::conditional_t<FP8, PrefixPart8, PrefixPart> part[2];
  int phys[PPW];
#pragma unroll
  for (int k = 0; k < PPW; ++k) phys[k] = k < jn ? phys_of(k) : -1;
  auto slab_of = [&](int k) { return pages + (int64_t)max(phys[k], 0) * kSlab; };
#pragma unroll
  for (int k = 0; k < 2 && k < PPW; ++k) load_prefix_part(slab_of(k), wave, n, a, part[k]);
  between();

  h8 Q[NTILE][4];
  load_prefix_queries<NTILE>(q_idx, col0, ncols, n, a, Q);
  // context lengths of the columns' requests: all loads first (unconditional,
  // clamped), then one wait
  int lb[NTILE];
#pragma unroll
  for (int nt = 0; nt < NTILE; ++nt) lb[nt] = lens[min(col0 + 16 * nt + n, ncols - 1) / (R * kGroups)];
  // (keeps the compiler from sinking a load into the page loop, where its wait
  // would also wait for the page loads issued there)
#pragma unroll
  for (int nt = 0; nt < NTILE; ++nt) asm volatile("" : : "v"(lb[nt]));
  int pos[NTILE];
  uint32_t pkey = 0;  // max of (INT_MAX - pos) over valid columns: the wave's smallest pos
#pragma unroll
  for (int nt = 0; nt < NTILE; ++nt) {
    const int c = col0 + 16 * nt + n;
    if (c < ncols) {
      const int r = (c / kGroups) % R;
      pos[nt] = clamp_len(lb[nt], max_pages) - R + r;
      pkey = max(pkey, (uint32_t)(INT_MAX - pos[nt]));
    } else {
      pos[nt] = -1;
    }
  }
  const int pmin = INT_MAX - (int)wave_umax(pkey);

  store_prefix_part(part[0], wave, lane, s_img[0]);
  __syncthreads();
#pragma unroll
  for (int k = 0; k < PPW; ++k) {
    if (k >= jn) break;
    const int j = j0 + k;
    if (k + 2 < PPW)  // slot k%2 held page k, already in LDS
      load_prefix_part(slab_of(k + 2), wave, n, a, part[k & 1]);
    // page k+1 -> the other image (last read before the previous barrier), a
    // piece at a time between this page's matrix products
    auto next_piece = [&](int piece) {
      if (k + 1 < PPW) store_prefix_piece(part[(k + 1) & 1], wave, lane, s_img[(k + 1) & 1], piece);
    };
    bool pieces_done = false;
    if (has_cols) {
      float mx[NTILE];
      if (phys[k] >= 0) {
        const h8* img = s_img[k & 1];
        if (pmin >= j * kPage + kPage - 1)  // every column sees the whole page
          score_prefix_page<NTILE, false, kTok>(img, Q, pos, j, lane, col0, ncols, out_scale, T, token_scores, mx,
                                                next_piece);
        else
          score_prefix_page<NTILE, true, kTok>(img, Q, pos, j, lane, col0, ncols, out_scale, T, token_scores, mx,
                                               next_piece);
        pieces_done = true;
      } else {
        // a page id outside the pool: no visible token
#pragma unroll
        for (int nt = 0; nt < NTILE; ++nt) mx[nt] = -__builtin_inff();
        if (kTok)
#pragma unroll
          for (int nt = 0; nt < NTILE; ++nt) {
            const int c = col0 + 16 * nt + n;
            if (c < ncols)
#pragma unroll
              for (int m = 0; m < 8; ++m) {
                const float ninf = -__builtin_inff();
                *reinterpret_cast<float4*>(token_scores + (int64_t)c * T + j * kPage + 16 * m + 4 * a) =
                    make_float4(ninf, ninf, ninf, ninf);
              }
          }
      }
      // block max: across the four lane groups holding the same column
#pragma unroll
      for (int nt = 0; nt < NTILE; ++nt) {
        const float v = rows_max4(mx[nt]);
        const int c = col0 + 16 * nt + n;
        if (a == 0 && c < ncols) block_scores[(int64_t)c * max_pages + j] = v * out_scale;
      }
    }
    if (!pieces_done)
#pragma unroll
      for (int piece = 0; piece < 4; ++piece) next_piece(piece);
    __syncthreads();
  }
}


// Shared prefix: pages 0 .. P-1 of table row 0, every request's columns.
// grid: one workgroup per (PPW pages, column tile of 64*NTILE), numbered so
// that the column tiles of one page group fall on the same XCD (workgroups
// are dealt round-robin to the 8 XCDs): id = 8*ny*(pg/8) + 8*yt + pg%8.
template <int NTILE, int PPW, bool kTok>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefix_index_kernel(
    const int32_t* __restrict__ table, const int32_t* __restrict__ lens, int32_t max_pages, int32_t B, int32_t R,
    int32_t prefix_pages, const uint8_t* __restrict__ q_idx, float out_scale, const uint8_t* __restrict__ pages,
    int32_t num_pages, float* __restrict__ block_scores, float* __restrict__ token_scores, int32_t ny) {
  __shared__ h8 s_img[2][kPfxImgH8];
  const int id = (int)blockIdx.x;
  dense_index_body<NTILE, PPW, kTok>(table, lens, max_pages, R, prefix_pages, prefix_pages, 0, B * R * kGroups,
                                     (id / (8 * ny)) * 8 + (id & 7), (id >> 3) % ny, q_idx, out_scale, pages,
                                     num_pages, block_scores, token_scores, s_img, [] {});
}

// Prefill (many query rows per request): request b = blockIdx.y, all its
// pages (those past its context score -inf) against its R*4 index queries;
// the rows' causal limits mask the chunk's own pages per column.
template <int NTILE, int PPW, bool kTok, bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_index_kernel(
    const int32_t* __restrict__ table, const int32_t* __restrict__ lens, int32_t max_pages, int32_t R,
    const uint8_t* __restrict__ q_idx, float out_scale, const uint8_t* __restrict__ pages, int32_t num_pages,
    float* __restrict__ block_scores, float* __restrict__ token_scores, int32_t ny) {
  __shared__ h8 s_img[2][kPfxImgH8];
  const int id = (int)blockIdx.x, b = (int)blockIdx.y;
  const int L = clamp_len(lens[b], max_pages);
  const int ncols = R * kGroups;
  dense_index_body<NTILE, PPW, kTok, FP8>(table + (int64_t)b * max_pages, lens, max_pages, R, max_pages,
                                     (L + kPage - 1) / kPage, b * ncols, (b + 1) * ncols,
                                     (id / (8 * ny)) * 8 + (id & 7), (id >> 3) % ny, q_idx, out_scale, pages,
                                     num_pages, block_scores, token_scores, s_img, [] {});
}

// Decode with a shared prefix, the per-request scan fused in (one row per
// request): each workgroup of the prefix product (NTILE = PPW = 4) also runs
// up to two scan chunk ids (nvfp4_scan_chunk, with its insert and -inf
// fill), between issuing its first two prefix pages and consuming them.  The
// scan's dependent load round trips then run while those pages are in
// flight, and the two passes share one launch instead of running one after
// the other.
template <bool INSERT, bool COMPACT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefix_scan_kernel(
    const int32_t* __restrict__ table, const int32_t* __restrict__ lens, int32_t max_pages, int32_t B,
    int32_t prefix_pages, const uint8_t* __restrict__ q_idx, float out_scale, const uint8_t* __restrict__ pages,
    int32_t num_pages, float* __restrict__ block_scores, int32_t ny, int32_t n_chunk_ids, NewRows NR) {
  __shared__ h8 s_img[2][kPfxImgH8];
  const int id = (int)blockIdx.x;
  // chunk ids id and 2 * gridDim.x - 1 - id, those below n_chunk_ids (the
  // launcher keeps the count within twice the grid; an id past it would map
  // to a request past the batch in the unpacked chunk map): the second ones,
  // numbered from the end, fall on the last workgroups rather than on the
  // first ones, which also insert
  // (packed ids: the context lengths the chunk map needs are loaded first,
  // alongside the prefix's table entries, instead of inside the scan's chain)
  const int lane = threadIdx.x & 63;
  const int lane_len = COMPACT && lane < B ? lens[lane] : 0;
  auto scan = [&] {
    const int G = (int)gridDim.x;
    if (id < n_chunk_ids)
      nvfp4_scan_chunk<1, false, INSERT, false, COMPACT, COMPACT>(id, table, lens, max_pages, q_idx, out_scale, pages,
                                                                  num_pages, block_scores, nullptr, B, prefix_pages,
                                                                  NR, lane_len);
    if (2 * G - 1 - id < n_chunk_ids)
      nvfp4_scan_chunk<1, false, INSERT, false, COMPACT, COMPACT>(2 * G - 1 - id, table, lens, max_pages, q_idx,
                                                                  out_scale, pages, num_pages, block_scores, nullptr, B,
                                                                  prefix_pages, NR, lane_len);
  };
  dense_index_body<4, 4, false>(table, lens, max_pages, 1, prefix_pages, prefix_pages, 0, B * kGroups,
                                (id / (8 * ny)) * 8 + (id & 7), (id >> 3) % ny, q_idx, out_scale, pages, num_pages,
                                block_scores, nullptr, s_img, scan);
}

template <int NTILE, int PPW>
static int launch_prefix_cfg(const msa_batch* bt, const uint8_t* q, float out_scale, const msa_cache* ic, float* bs,
                             float* ts, hipStream_t s) {
  const int ncols = bt->num_reqs * bt->rows_per_req * kGroups;
  const int ny = (ncols + 64 * NTILE - 1) / (64 * NTILE);
  const int npg = (bt->shared_prefix_pages + PPW - 1) / PPW;
  const int npg8 = (npg + 7) / 8 * 8;
  const dim3 grid((unsigned)(npg8 * ny));
  if (ts)
    hipLaunchKernelGGL((prefix_index_kernel<NTILE, PPW, true>), grid, dim3(256), 0, s, bt->block_table, bt->ctx_lens,
                       bt->max_pages_per_req, bt->num_reqs, bt->rows_per_req, bt->shared_prefix_pages, q, out_scale,
                       (const uint8_t*)ic->pages, ic->num_pages, bs, ts, ny);
  else
    hipLaunchKernelGGL((prefix_index_kernel<NTILE, PPW, false>), grid, dim3(256), 0, s, bt->block_table,
                       bt->ctx_lens, bt->max_pages_per_req, bt->num_reqs, bt->rows_per_req, bt->shared_prefix_pages, q,
                       out_scale, (const uint8_t*)ic->pages, ic->num_pages, bs, ts, ny);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int NTILE, int PPW>
static int launch_prefill_cfg(const msa_batch* bt, const uint8_t* q, float out_scale, const msa_cache* ic, float* bs,
                              float* ts, hipStream_t s) {
  const int ncols = bt->rows_per_req * kGroups;
  const int ny = (ncols + 64 * NTILE - 1) / (64 * NTILE);
  const int npg = (bt->max_pages_per_req + PPW - 1) / PPW;
  const int npg8 = (npg + 7) / 8 * 8;
  const dim3 grid((unsigned)(npg8 * ny), (unsigned)bt->num_reqs);
#define MSA_PREFILL_INDEX(TOK, FP8)                                                                             \
  hipLaunchKernelGGL((prefill_index_kernel<NTILE, PPW, TOK, FP8>), grid, dim3(256), 0, s, bt->block_table,      \
                     bt->ctx_lens, bt->max_pages_per_req, bt->rows_per_req, q, out_scale, (const uint8_t*)ic->pages, \
                     ic->num_pages, bs, ts, ny)
  const bool fp8 = ic->dtype == MSA_FP8_E4M3;
  if (ts) {
    if (fp8) MSA_PREFILL_INDEX(true, true); else MSA_PREFILL_INDEX(true, false);
  } else {
    if (fp8) MSA_PREFILL_INDEX(false, true); else MSA_PREFILL_INDEX(false, false);
  }
#undef MSA_PREFILL_INDEX
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// The fused form when it applies: NVFP4, one row per request, block scores
// only, and at most two scan chunk ids per workgroup (a suffix past the
// prefix that is short next to it).  Returns 1 when it does not apply (the
// caller launches the two passes), else 0, or -1 when the launch failed.
int launch_prefix_scan(const msa_batch* bt, const uint8_t* q, float q_scale, const msa_cache* ic, float* bs,
                       float* ts, const NewRows& nr, bool insert, hipStream_t s) {
  const int p0 = bt->shared_prefix_pages;
  if (p0 <= 0 || ts || bt->rows_per_req != 1 || ic->dtype != MSA_NVFP4) return 1;
  const int chunks = (bt->max_pages_per_req - p0 + 3) / 4;
  if (chunks <= 0) return 1;
  const int B = bt->num_reqs;
  const int ncols = B * kGroups;
  const int ny = (ncols + 255) / 256;
  const int npg8 = ((p0 + 3) / 4 + 7) / 8 * 8;
  const int64_t grid = (int64_t)npg8 * ny, n_ids = (int64_t)chunks * B;
  if (n_ids > 2 * grid) return 1;
  const float out_scale = ic->tensor_scale * q_scale;
#define MSA_PREFIX_SCAN(INS, CMP)                                                                                \
  hipLaunchKernelGGL((prefix_scan_kernel<INS, CMP>), dim3((unsigned)grid), dim3(256), 0, s, bt->block_table,      \
                     bt->ctx_lens, bt->max_pages_per_req, B, p0, q, out_scale, (const uint8_t*)ic->pages,          \
                     ic->num_pages, bs, ny, (int32_t)n_ids, nr)
  const bool compact = B <= 64;
  if (insert) {
    if (compact) MSA_PREFIX_SCAN(true, true); else MSA_PREFIX_SCAN(true, false);
  } else {
    if (compact) MSA_PREFIX_SCAN(false, true); else MSA_PREFIX_SCAN(false, false);
  }
#undef MSA_PREFIX_SCAN
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace msa

using namespace msa;

// Many query rows per request (a prefill chunk): every page of every request
// scored for the request's R*4 index queries as a dense matrix-core product.
// Eight pages per workgroup (measured at 4 x 2,048 rows of 64K contexts: 420
// us, against 453 us with four and 614 us with sixteen): the workgroup's
// start-up load round is spread over more pages, and the column tiles still
// give thousands of workgroups.
extern "C" int msa_launch_prefill_index(const msa_batch* bt, const void* q_idx, float q_scale, const msa_cache* ic,
                                        float* block_scores, float* token_scores, hipStream_t s) {
  const float out_scale = ic->tensor_scale * q_scale;
  return launch_prefill_cfg<4, 8>(bt, (const uint8_t*)q_idx, out_scale, ic, block_scores, token_scores, s);
}

// Scores and block maxima of pages [0, shared_prefix_pages) for every
// (request, row, group); the per-request scan covers the pages after them.
extern "C" int msa_launch_prefix_index(const msa_batch* bt, const void* q_idx, float q_scale, const msa_cache* ic,
                                       float* block_scores, float* token_scores, hipStream_t s) {
  if (bt->shared_prefix_pages <= 0) return 0;
  const float out_scale = ic->tensor_scale * q_scale;
  return launch_prefix_cfg<4, 4>(bt, (const uint8_t*)q_idx, out_scale, ic, block_scores, token_scores, s);
}
