// msa_index.hip -- steps 1 and 2: indexer scores fused with the 128-token
// block max-pool (vLLM M3.1 post, "MiniMax 稀疏注意力的工作原理"; "MiniMax
// goes sparse", section 1 Step 1).
//
// NVFP4 pages are scanned by nvfp4_scan_chunk (msa_scan.h); this file holds
// its launch, the FP8 and FP32 scans and the exported launchers.
#include "msa_device.h"
#include "msa_kernels.h"
#include "msa_scan.h"

namespace msa {

// The scan launch: one workgroup per chunk id (nvfp4_scan_chunk).
// Occupancy target: 4 waves per SIMD (4-6 measured equal, 8 thrash).
template <int R, bool kTok, bool INSERT = false, bool F16 = false, bool COMPACT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void index_nvfp4_kernel(
    const int32_t* __restrict__ table, const int32_t* __restrict__ lens, int32_t max_pages,
    const uint8_t* __restrict__ q_idx, float out_scale, const uint8_t* __restrict__ pages, int32_t num_pages,
    float* __restrict__ block_scores, float* __restrict__ token_scores, int32_t B, int32_t p0, NewRows NR) {
  nvfp4_scan_chunk<R, kTok, INSERT, F16, COMPACT>((int)blockIdx.x, table, lens, max_pages, q_idx, out_scale, pages,
                                                  num_pages, block_scores, token_scores, B, p0, NR);
}

// The scan in physical page order, for a batch that carries page_owner (the
// block table's inverse: entry p = b * max_pages + j where table[b][j] == p).
// Workgroup b < B belongs to request b: it writes the index keys of the
// request's new rows (INSERT), scores the one or two pages that hold rows
// L_b - R .. L_b - 1 through the block table, records those pages in
// page_owner and writes the -inf scores of the blocks past the context.  With
// INSERT, workgroup B + b writes request b's new keys and values (nothing in
// this launch reads them, so they stay off the index keys' path to the
// scoring).  The next workgroups, from B (2B with INSERT) on, take pool pages
// 4i .. 4i+3, one per wave.  A wave reads its page's owner entry and
// issues the page's loads before anything else; the page counts only if the
// entry names a block of some request that lies before that request's
// new-row pages and whose table entry names the page back (free pages and
// stale entries are dropped after their loads).  So no lookup chain (lengths,
// chunk, table) stands before the page loads, as one does in the
// chunk-mapped scan; the price is that every pool page is read, in use or not.
template <int R, bool INSERT, bool F16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void index_nvfp4_owned_kernel(
    const int32_t* __restrict__ table, const int32_t* __restrict__ lens, int32_t max_pages, int32_t* owner,
    const uint8_t* __restrict__ q_idx, float out_scale, const uint8_t* __restrict__ pages, int32_t num_pages,
    float* __restrict__ block_scores, int32_t B, NewRows NR) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, col = lane & 15;
  __shared__ uint4 s_scales[4][64];
  if ((int)blockIdx.x < B) {
    const int b = (int)blockIdx.x;
    const int L = clamp_len(lens[b], max_pages);
    const int t0 = max(L - R, 0);
    if (INSERT && t0 < L) {
      insert_new_rows<R, kInsertIndex>(table, max_pages, num_pages, b, L, t0, L, NR);
      // the index keys just written are read back by this workgroup's waves
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __syncthreads();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    const int npb = (L + kPage - 1) / kPage;
    const int j = t0 / kPage + wave;  // R <= 128: the new rows lie on at most two pages
    if (wave < 2 && j < npb) {
      int phys = table[(int64_t)b * max_pages + j];
      if (phys >= num_pages) phys = -1;
      ScanQueries<R, F16> q;
      q.load(q_idx, b, lane);
      if (phys >= 0) {
        if (lane == 0) owner[phys] = b * max_pages + j;
        PageRegs pr;
        load_page(pr, pages + (int64_t)phys * kNvSlab, col, grp, lane);
        score_resident_page<R, false, F16>(pr, q, &s_scales[wave][0], L, j, b, lane, max_pages, out_scale, 0,
                                           block_scores, nullptr);
      } else {
        empty_block<R, false>(j, b, lane, max_pages, 0, block_scores, nullptr);
      }
    }
    fill_past_chunks<R>(block_scores, b, npb, max_pages);
    return;
  }
  if (INSERT && (int)blockIdx.x < 2 * B) {  // request b's new keys and values
    const int b = (int)blockIdx.x - B;
    const int L = clamp_len(lens[b], max_pages);
    if (max(L - R, 0) < L) insert_new_rows<R, kInsertKV>(table, max_pages, num_pages, b, L, max(L - R, 0), L, NR);
    return;
  }
  const int p = ((int)blockIdx.x - (INSERT ? 2 * B : B)) * 4 + wave;
  if (p >= num_pages) return;
  const int own = owner[p];
  PageRegs pr;
  load_page(pr, pages + (int64_t)p * kNvSlab, col, grp, lane);
  // (the scheduler would otherwise start on the page's first words between its loads)
  __builtin_amdgcn_sched_barrier(0);
  // the owner's length, table entry and queries load together, in one round
  // behind the page (request 0's stand in for an entry that names no
  // request); a page that is not the owner's is scored all the same, its
  // stores dropped, so that no branch waits on one load before issuing the next
  const bool named = (own >= 0) & (own / max_pages < B);
  const int b = named ? own / max_pages : 0, j = named ? own - b * max_pages : 0;
  const int Lraw = lens[b], back = table[(int64_t)b * max_pages + j];
  ScanQueries<R, F16> q;
  q.load(q_idx, b, lane);
  __builtin_amdgcn_sched_barrier(0);
  const int L = clamp_len(Lraw, max_pages);
  const bool mine = named & (back == p) & (j < max(L - R, 0) / kPage);
  score_resident_page<R, false, F16>(pr, q, &s_scales[wave][0], L, j, b, lane, max_pages, out_scale, 0, block_scores,
                                     nullptr, mine);
}

// page_owner from the block table: every entry -1, then entry table[b][j] =
// b * max_pages + j for the blocks j < ceil(L_b / 128) of every request whose
// page lies in the pool (a page named twice keeps one of the two).
__global__ __launch_bounds__(256) void page_owner_clear_kernel(int32_t* __restrict__ owner, int32_t num_pages) {
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < num_pages; p += (int64_t)gridDim.x * 256)
    owner[p] = -1;
}

__global__ __launch_bounds__(256) void page_owner_scatter_kernel(const int32_t* __restrict__ table,
                                                                 const int32_t* __restrict__ lens, int32_t max_pages,
                                                                 int32_t num_pages, int32_t* __restrict__ owner) {
  const int b = (int)blockIdx.y;
  const int npb = (clamp_len(lens[b], max_pages) + kPage - 1) / kPage;
  for (int j = (int)blockIdx.x * 256 + (int)threadIdx.x; j < npb; j += (int)gridDim.x * 256) {
    const int p = table[(int64_t)b * max_pages + j];
    if (p >= 0 && p < num_pages) owner[p] = b * max_pages + j;
  }
}

// FP8 caches (one E4M3 byte per element, FP32 tensor scale): the same scan
// over 128 B per token.  Keys and index queries are both FP8, so one
// v_mfma_scale_f32_16x16x128_f8f6f4 (unit block scales) multiplies 16 tokens'
// full 128-dim rows against 16 query rows with exact products: A row 4g + i
// holds index query (group g, row 4*rp + i), B column n token n of a 16-token
// chunk.  Lane group c of either operand carries dims 16c..16c+15 and
// 64+16c..64+16c+15 of its row (the instruction's FP8 operand layout, the
// same for A and B, so every product pairs equal dims).  The index keys are
// stored in half rows (16 tokens x dims 0..63, then x dims 64..127, 1 KB
// each), so each of a chunk's two loads reads one whole, contiguous 1 KB.  Output
// lane (n, c) holds the scores of group c, rows 4*rp .. 4*rp+3, token n; the
// block max is a 16-lane row reduction.  Grid, chunk order and the fused
// insert follow index_nvfp4_kernel (one page per wave, 4 per workgroup).
// The step's new tokens of request b in [t0, t1) (t0 < t1, within [L - R,
// L)) written into the three FP8 caches by a whole workgroup of 256 threads,
// one thread per element (4 x 128 keys, 4 x 128 values, 128 index keys per
// token).  The caller makes them visible to its waves before reading pages.
template <int R, int PART = kInsertAll>
__device__ __forceinline__ void fp8_insert_rows(const int32_t* __restrict__ table, int32_t max_pages, int32_t num_pages,
                                                int b, int L, int t0, int t1, NewRows NR) {
  // elements per token: 4 x 128 keys, 4 x 128 values, 128 index keys (or a part of them)
  constexpr int kPerTok = PART == kInsertIndex ? kDim : (PART == kInsertKV ? 8 * kDim : 9 * kDim);
  // element e: token t0 + e / kPerTok, then its keys, values, index key.
  // A batch of elements per thread: every source load issues before the
  // first store (which could alias them), so a batch is one memory round
  // -- sized for all of a chunk's elements up to four new rows.  The new
  // tokens lie on at most two pages, whose table entries load with them.
  const int ne = (t1 - t0) * kPerTok;
  constexpr int kBatch = (kPerTok * R + 255) / 256 < 18 ? (kPerTok * R + 255) / 256 : 18;
  const int pa = t0 / kPage;
  const int ph_a = table[(int64_t)b * max_pages + pa], ph_b = table[(int64_t)b * max_pages + (t1 - 1) / kPage];
  auto locate = [&](int e, int& tok, int& c, int& head, int& d) {
    tok = t0 + e / kPerTok;
    int u = e % kPerTok + (PART == kInsertIndex ? 8 * kDim : 0);
    c = u < 4 * kDim ? 0 : (u < 8 * kDim ? 1 : 2);
    u -= c * 4 * kDim;
    head = u / kDim;
    d = u % kDim;
  };
  for (int e0 = threadIdx.x; e0 < ne; e0 += 256 * kBatch) {
    float x[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      int tok, c, head, d;
      locate(min(e0 + 256 * k, ne - 1), tok, c, head, d);
      const float* src = c == 0 ? NR.k : (c == 1 ? NR.v : NR.idx);
      x[k] = src[(((int64_t)b * R + tok - (L - R)) * (c == 2 ? 1 : kGroups) + head) * kDim + d];
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int e = e0 + 256 * k;
      if (e >= ne) break;
      int tok, c, head, d;
      locate(e, tok, c, head, d);
      const int heads = c == 2 ? 1 : kGroups;
      const int ph = tok / kPage == pa ? ph_a : ph_b;
      const bool valid = ph >= 0 && ph < (c == 2 ? num_pages : NR.kv_num_pages);
      uint8_t* slab = (c == 0 ? NR.kpages : (c == 1 ? NR.vpages : NR.ipages)) +
                      ((int64_t)(valid ? ph : 0) * heads + head) * kFp8Slab;
      const float ts = c == 0 ? NR.ts_k : (c == 1 ? NR.ts_v : NR.ts_i);
      const int layout = c == 0 ? MSA_TOKEN_MAJOR : (c == 1 ? MSA_DIM_MAJOR : MSA_HALF_ROWS);
      if (valid) slab[fp8_offset(layout, tok & (kPage - 1), d)] = (uint8_t)e4m3_encode(x[k] / ts);
    }
  }
}

// A operands of the FP8 product: row m = lane % 16 -> (group m / 4, row 4 rp + m % 4).
// Lanes of rows r >= R load row R - 1 and zero it: no branch, so nothing
// waits on these loads before the loads that follow them issue.
template <int R>
__device__ __forceinline__ void fp8_load_queries(const uint8_t* __restrict__ q_idx, int b, int lane,
                                                 v8i (&A)[(R + 3) / 4]) {
  const int n = lane & 15, c = lane >> 4;
#pragma unroll
  for (int rp = 0; rp < (R + 3) / 4; ++rp) {
    const int r = 4 * rp + (n & 3), g = n >> 2;
    const uint8_t* q = q_idx + (((int64_t)b * R + min(r, R - 1)) * kGroups + g) * kDim;
    const uint4 lo = *reinterpret_cast<const uint4*>(q + 16 * c);
    const uint4 hi = *reinterpret_cast<const uint4*>(q + 64 + 16 * c);
    const bool on = r < R;
    A[rp] = v8i{on ? (int)lo.x : 0, on ? (int)lo.y : 0, on ? (int)lo.z : 0, on ? (int)lo.w : 0,
                on ? (int)hi.x : 0, on ? (int)hi.y : 0, on ? (int)hi.z : 0, on ? (int)hi.w : 0};
  }
}

// A page's 16 KB: lane (n, c) takes dims 16c.. and 64 + 16c.. of token 16 ch + n, per chunk ch.
__device__ __forceinline__ void fp8_load_page(uint4 (&kw)[8][2], const uint8_t* __restrict__ slab, int lane) {
  const int n = lane & 15, c = lane >> 4;
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) {
    kw[ch][0] = nt_load4(slab + ch * 2048 + n * 64 + 16 * c);
    kw[ch][1] = nt_load4(slab + ch * 2048 + 1024 + n * 64 + 16 * c);
  }
}

// Scores of page j of request b (resident in kw) for all R rows, positions
// past pos_lim[r] masked; m[r] gets the block maxima (token scores too with kTok).
template <int R, bool kTok>
__device__ __forceinline__ void fp8_score_page(const uint4 (&kw)[8][2], const v8i (&A)[(R + 3) / 4],
                                               const int (&pos_lim)[R], int j, int b, int lane, float out_scale,
                                               int64_t T, float* __restrict__ token_scores, float (&m)[R]) {
  constexpr int RP = (R + 3) / 4;
  const int n = lane & 15, c = lane >> 4;
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) {
    const v8i Bop = v8i{(int)kw[ch][0].x, (int)kw[ch][0].y, (int)kw[ch][0].z, (int)kw[ch][0].w,
                        (int)kw[ch][1].x, (int)kw[ch][1].y, (int)kw[ch][1].z, (int)kw[ch][1].w};
    const int t = j * kPage + 16 * ch + n;
#pragma unroll
    for (int rp = 0; rp < RP; ++rp) {
      const v4f z = {0.f, 0.f, 0.f, 0.f};
      const v4f d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[rp], Bop, z, 0, 0, 0, 127, 0, 127);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * rp + i;
        if (r >= R) break;
        const bool vis = t <= pos_lim[r];
        if (kTok)
          token_scores[(((int64_t)b * R + r) * kGroups + c) * T + t] = vis ? d[i] * out_scale : -__builtin_inff();
        if (vis) m[r] = pool_max(m[r], d[i]);
      }
    }
  }
}

// The block maxima of page j (16-lane row reductions), stored when keep.
template <int R>
__device__ __forceinline__ void fp8_finish(const float (&m)[R], int j, int b, int lane, int max_pages,
                                           float out_scale, float* __restrict__ block_scores, bool keep = true) {
  const int n = lane & 15, c = lane >> 4;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float mm = wave_max16(m[r]);
    if (keep && n == 0) block_scores[(((int64_t)b * R + r) * kGroups + c) * max_pages + j] = mm * out_scale;
  }
}

template <int R, bool kTok, bool INSERT, int WPE = 4, bool COMPACT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE))) void index_fp8_kernel(
    const int32_t* __restrict__ table, const int32_t* __restrict__ lens, int32_t max_pages,
    const uint8_t* __restrict__ q_idx, float out_scale, const uint8_t* __restrict__ pages, int32_t num_pages,
    float* __restrict__ block_scores, float* __restrict__ token_scores, int32_t B, NewRows NR) {
  constexpr int RP = (R + 3) / 4;  // MFMAs per 16-token chunk (4 rows each)
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int id = (int)blockIdx.x;
  int b, L, latest, chunk;
  if (!chunk_of<COMPACT>(id, B, lens, max_pages, 0, lane, b, L, latest, chunk)) return;
  const int npb = (L + kPage - 1) / kPage;
  if (INSERT) {
    // new tokens [max(L - R, 0), L) in this chunk: one thread per element
    // (4 x 128 keys, 4 x 128 values, 128 index keys per token)
    const int lo = chunk * 4 * kPage;
    const int t0 = max(max(L - R, 0), lo), t1 = min(L, lo + 4 * kPage);
    if (t0 < t1) {  // uniform over the workgroup
      fp8_insert_rows<R>(table, max_pages, num_pages, b, L, t0, t1, NR);
      // the index keys just written are read back by this workgroup's waves
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __syncthreads();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
  }
  const bool fill = COMPACT && id < B;
  const int j = chunk * 4 + wave;
  if (j >= max_pages) {
    if (fill) fill_past_chunks<R>(block_scores, b, min((latest + 1) * 4, max_pages), max_pages);
    return;
  }
  const int n = lane & 15, c = lane >> 4;
  const int64_t T = (int64_t)max_pages * kPage;

  v8i A[RP];
  fp8_load_queries<R>(q_idx, b, lane, A);
  int pos_lim[R];
#pragma unroll
  for (int r = 0; r < R; ++r) pos_lim[r] = L - R + r;

  int phys = j < npb ? table[(int64_t)b * max_pages + j] : -1;
  if (phys >= num_pages) phys = -1;
  float m[R];
#pragma unroll
  for (int r = 0; r < R; ++r) m[r] = -__builtin_inff();
  if (phys >= 0) {
    uint4 kw[8][2];
    fp8_load_page(kw, pages + (int64_t)phys * kFp8Slab, lane);
    // the whole page's loads go out before the first product waits on one
    // (left alone, the scheduler interleaves them with the products to save
    // registers and the page arrives in several serial round trips)
    __builtin_amdgcn_sched_barrier(0);
    fp8_score_page<R, kTok>(kw, A, pos_lim, j, b, lane, out_scale, T, token_scores, m);
  } else if (kTok) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      for (int ch = 0; ch < 8; ++ch)
        token_scores[(((int64_t)b * R + r) * kGroups + c) * T + j * kPage + 16 * ch + n] = -__builtin_inff();
  }
  fp8_finish<R>(m, j, b, lane, max_pages, out_scale, block_scores);
  if (fill) fill_past_chunks<R>(block_scores, b, min((latest + 1) * 4, max_pages), max_pages);
}

// The FP8 scan in physical page order (batches with page_owner), split as in
// index_nvfp4_owned_kernel: workgroup b < B writes the index keys of request
// b's new rows (INSERT), scores the one or two pages that hold rows L_b - R ..
// L_b - 1 through the block table, records them in page_owner and writes the
// -inf scores past the context; with INSERT, workgroup B + b writes the new
// keys and values; the next workgroups take pool pages 4i .. 4i+3, one per
// wave, loading the page before its owner's length, table entry and
// queries.  A page that counts holds only blocks below the page of the first
// new row, whose tokens every row sees, so that path applies no position mask.
template <int R, bool INSERT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void index_fp8_owned_kernel(
    const int32_t* __restrict__ table, const int32_t* __restrict__ lens, int32_t max_pages, int32_t* owner,
    const uint8_t* __restrict__ q_idx, float out_scale, const uint8_t* __restrict__ pages, int32_t num_pages,
    float* __restrict__ block_scores, int32_t B, NewRows NR) {
  constexpr int RP = (R + 3) / 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float m[R];
#pragma unroll
  for (int r = 0; r < R; ++r) m[r] = -__builtin_inff();
  if ((int)blockIdx.x < B) {
    const int b = (int)blockIdx.x;
    const int L = clamp_len(lens[b], max_pages);
    const int t0 = max(L - R, 0);
    if (INSERT && t0 < L) {
      fp8_insert_rows<R, kInsertIndex>(table, max_pages, num_pages, b, L, t0, L, NR);
      // the index keys just written are read back by this workgroup's waves
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __syncthreads();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    const int npb = (L + kPage - 1) / kPage;
    const int j = t0 / kPage + wave;  // R <= 128: the new rows lie on at most two pages
    if (wave < 2 && j < npb) {
      int phys = table[(int64_t)b * max_pages + j];
      if (phys >= num_pages) phys = -1;
      v8i A[RP];
      fp8_load_queries<R>(q_idx, b, lane, A);
      int pos_lim[R];
#pragma unroll
      for (int r = 0; r < R; ++r) pos_lim[r] = L - R + r;
      if (phys >= 0) {
        if (lane == 0) owner[phys] = b * max_pages + j;
        uint4 kw[8][2];
        fp8_load_page(kw, pages + (int64_t)phys * kFp8Slab, lane);
        __builtin_amdgcn_sched_barrier(0);
        fp8_score_page<R, false>(kw, A, pos_lim, j, b, lane, out_scale, 0, nullptr, m);
      }
      fp8_finish<R>(m, j, b, lane, max_pages, out_scale, block_scores);
    }
    fill_past_chunks<R>(block_scores, b, npb, max_pages);
    return;
  }
  if (INSERT && (int)blockIdx.x < 2 * B) {  // request b's new keys and values
    const int b = (int)blockIdx.x - B;
    const int L = clamp_len(lens[b], max_pages);
    if (max(L - R, 0) < L) fp8_insert_rows<R, kInsertKV>(table, max_pages, num_pages, b, L, max(L - R, 0), L, NR);
    return;
  }
  const int p = ((int)blockIdx.x - (INSERT ? 2 * B : B)) * 4 + wave;
  if (p >= num_pages) return;
  const int own = owner[p];
  uint4 kw[8][2];
  fp8_load_page(kw, pages + (int64_t)p * kFp8Slab, lane);
  __builtin_amdgcn_sched_barrier(0);
  // the owner's length, table entry and queries in one round behind the page
  // (request 0's stand in for an entry that names no request); a page that
  // is not the owner's is scored all the same and its stores dropped
  const bool named = (own >= 0) & (own / max_pages < B);
  const int b = named ? own / max_pages : 0, j = named ? own - b * max_pages : 0;
  const int Lraw = lens[b], back = table[(int64_t)b * max_pages + j];
  v8i A[RP];
  fp8_load_queries<R>(q_idx, b, lane, A);
  __builtin_amdgcn_sched_barrier(0);
  const int L = clamp_len(Lraw, max_pages);
  const bool mine = named & (back == p) & (j < max(L - R, 0) / kPage);
  int pos_lim[R];
#pragma unroll
  for (int r = 0; r < R; ++r) pos_lim[r] = 0x7fffffff;
  fp8_score_page<R, false>(kw, A, pos_lim, j, b, lane, out_scale, 0, nullptr, m);
  fp8_finish<R>(m, j, b, lane, max_pages, out_scale, block_scores, mine);
}

template <int R, bool INSERT>
static void launch_fp8(const msa_batch* bt, const uint8_t* q, float out_scale, const msa_cache* ic, float* bs,
                       float* ts, const NewRows& nr, hipStream_t s) {
  const dim3 grid((unsigned)(((bt->max_pages_per_req + 3) / 4) * bt->num_reqs));
  if (ts)
    hipLaunchKernelGGL((index_fp8_kernel<R, true, INSERT>), grid, dim3(256), 0, s, bt->block_table, bt->ctx_lens,
                       bt->max_pages_per_req, q, out_scale, (const uint8_t*)ic->pages, ic->num_pages, bs, ts,
                       bt->num_reqs, nr);
  else if (bt->num_reqs <= 64)
    hipLaunchKernelGGL((index_fp8_kernel<R, false, INSERT, 4, true>), grid, dim3(256), 0, s, bt->block_table,
                       bt->ctx_lens, bt->max_pages_per_req, q, out_scale, (const uint8_t*)ic->pages, ic->num_pages, bs,
                       ts, bt->num_reqs, nr);
  else
    hipLaunchKernelGGL((index_fp8_kernel<R, false, INSERT>), grid, dim3(256), 0, s, bt->block_table, bt->ctx_lens,
                       bt->max_pages_per_req, q, out_scale, (const uint8_t*)ic->pages, ic->num_pages, bs, ts,
                       bt->num_reqs, nr);
}

template <bool INSERT>
static int launch_fp8_rows(const msa_batch* bt, const uint8_t* q, float out_scale, const msa_cache* ic, float* bs,
                           float* ts, const NewRows& nr, hipStream_t s) {
  switch (bt->rows_per_req) {
    case 1: launch_fp8<1, INSERT>(bt, q, out_scale, ic, bs, ts, nr, s); break;
    case 2: launch_fp8<2, INSERT>(bt, q, out_scale, ic, bs, ts, nr, s); break;
    case 3: launch_fp8<3, INSERT>(bt, q, out_scale, ic, bs, ts, nr, s); break;
    case 4: launch_fp8<4, INSERT>(bt, q, out_scale, ic, bs, ts, nr, s); break;
    case 5: launch_fp8<5, INSERT>(bt, q, out_scale, ic, bs, ts, nr, s); break;
    case 6: launch_fp8<6, INSERT>(bt, q, out_scale, ic, bs, ts, nr, s); break;
    case 7: launch_fp8<7, INSERT>(bt, q, out_scale, ic, bs, ts, nr, s); break;
    case 8: launch_fp8<8, INSERT>(bt, q, out_scale, ic, bs, ts, nr, s); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// F32 cache, F32 queries: one workgroup per (page, request), one thread per token.
template <bool kTok>
__global__ __launch_bounds__(128) void index_f32_kernel(const int32_t* __restrict__ table,
                                                        const int32_t* __restrict__ lens, int32_t max_pages,
                                                        int32_t R, const float* __restrict__ q_idx,
                                                        const uint8_t* __restrict__ pages, int32_t num_pages,
                                                        float* __restrict__ block_scores,
                                                        float* __restrict__ token_scores) {
  __shared__ float qs[MSA_MAX_ROWS * kGroups * kDim];
  __shared__ float red[2][MSA_MAX_ROWS * kGroups];
  const int j = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int L = clamp_len(lens[b], max_pages);
  const int npb = (L + kPage - 1) / kPage;
  for (int i = t; i < R * kGroups * kDim; i += 128) qs[i] = q_idx[(int64_t)b * R * kGroups * kDim + i];
  __syncthreads();
  const int phys = j < npb ? table[(int64_t)b * max_pages + j] : -1;
  const bool ok = phys >= 0 && phys < num_pages;
  const float* krow = ok ? reinterpret_cast<const float*>(pages + (int64_t)phys * kF32Slab) + t * kDim : nullptr;
  const int64_t T = (int64_t)max_pages * kPage;
  const int pos = j * kPage + t;
  for (int rg = 0; rg < R * kGroups; ++rg) {
    const int r = rg / kGroups;
    float s = -__builtin_inff();
    if (ok && pos <= L - R + r) {
      s = 0.f;
      const float* q = qs + rg * kDim;
      for (int d = 0; d < kDim; ++d) s = fmaf(q[d], krow[d], s);
    }
    if (kTok) token_scores[((int64_t)b * R * kGroups + rg) * T + pos] = s;
    float m = s;
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((t & 63) == 0) red[t >> 6][rg] = m;
  }
  __syncthreads();
  for (int rg = t; rg < R * kGroups; rg += 128)
    block_scores[((int64_t)b * R * kGroups + rg) * max_pages + j] = fmaxf(red[0][rg], red[1][rg]);
}

// Three rows or more: the FP16 form (the masked FP4 products grow with R and
// bound the scan from R = 3 on).
template <int R, bool INSERT>
static void launch_nvfp4(const msa_batch* bt, const uint8_t* q, float out_scale, const msa_cache* ic, float* bs,
                         float* ts, const NewRows& nr, hipStream_t s) {
  constexpr bool F16 = R >= 3;
  const int p0 = ic->dtype == MSA_NVFP4 ? bt->shared_prefix_pages : 0;
  const int chunks = (bt->max_pages_per_req - p0 + 3) / 4;
  if (chunks <= 0) return;  // every page is shared: the prefix kernel scored them all
  const dim3 grid((unsigned)(chunks * bt->num_reqs));
  if (ts)
    hipLaunchKernelGGL((index_nvfp4_kernel<R, true, INSERT, F16>), grid, dim3(256), 0, s, bt->block_table,
                       bt->ctx_lens, bt->max_pages_per_req, q, out_scale, (const uint8_t*)ic->pages, ic->num_pages, bs,
                       ts, bt->num_reqs, p0, nr);
  else if (bt->num_reqs <= 64)
    hipLaunchKernelGGL((index_nvfp4_kernel<R, false, INSERT, F16, true>), grid, dim3(256), 0, s, bt->block_table,
                       bt->ctx_lens, bt->max_pages_per_req, q, out_scale, (const uint8_t*)ic->pages, ic->num_pages, bs,
                       ts, bt->num_reqs, p0, nr);
  else
    hipLaunchKernelGGL((index_nvfp4_kernel<R, false, INSERT, F16>), grid, dim3(256), 0, s, bt->block_table,
                       bt->ctx_lens, bt->max_pages_per_req, q, out_scale, (const uint8_t*)ic->pages, ic->num_pages, bs,
                       ts, bt->num_reqs, p0, nr);
}

template <int R, bool INSERT>
static void launch_owned(const msa_batch* bt, const uint8_t* q, float out_scale, const msa_cache* ic, float* bs,
                         const NewRows& nr, hipStream_t s) {
  // request workgroups, their key / value writers (with INSERT), then the pool's pages
  const int kv = INSERT ? bt->num_reqs : 0;
  const dim3 grid((unsigned)(bt->num_reqs + kv + (ic->num_pages + 3) / 4));
  if (ic->dtype == MSA_FP8_E4M3)
    hipLaunchKernelGGL((index_fp8_owned_kernel<R, INSERT>), grid, dim3(256), 0, s, bt->block_table, bt->ctx_lens,
                       bt->max_pages_per_req, bt->page_owner, q, out_scale, (const uint8_t*)ic->pages, ic->num_pages,
                       bs, bt->num_reqs, nr);
  else
    hipLaunchKernelGGL((index_nvfp4_owned_kernel<R, INSERT, (R >= 3)>), grid, dim3(256), 0, s, bt->block_table,
                       bt->ctx_lens, bt->max_pages_per_req, bt->page_owner, q, out_scale, (const uint8_t*)ic->pages,
                       ic->num_pages, bs, bt->num_reqs, nr);
}

template <bool INSERT>
static int launch_owned_rows(const msa_batch* bt, const uint8_t* q, float out_scale, const msa_cache* ic, float* bs,
                             const NewRows& nr, hipStream_t s) {
  switch (bt->rows_per_req) {
    case 1: launch_owned<1, INSERT>(bt, q, out_scale, ic, bs, nr, s); break;
    case 2: launch_owned<2, INSERT>(bt, q, out_scale, ic, bs, nr, s); break;
    case 3: launch_owned<3, INSERT>(bt, q, out_scale, ic, bs, nr, s); break;
    case 4: launch_owned<4, INSERT>(bt, q, out_scale, ic, bs, nr, s); break;
    case 5: launch_owned<5, INSERT>(bt, q, out_scale, ic, bs, nr, s); break;
    case 6: launch_owned<6, INSERT>(bt, q, out_scale, ic, bs, nr, s); break;
    case 7: launch_owned<7, INSERT>(bt, q, out_scale, ic, bs, nr, s); break;
    case 8: launch_owned<8, INSERT>(bt, q, out_scale, ic, bs, nr, s); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// The physical-order scan takes decode batches with an owner map, no shared
// prefix and no token scores (NVFP4 or FP8 index cache).
static bool owned_scan(const msa_batch* bt, const msa_cache* ic, const float* ts) {
  return bt->page_owner && !ts && bt->shared_prefix_pages == 0 && bt->rows_per_req <= MSA_MAX_ROWS &&
         (ic->dtype == MSA_NVFP4 || ic->dtype == MSA_FP8_E4M3);
}

template <bool INSERT>
static int launch_nvfp4_rows(const msa_batch* bt, const uint8_t* q, float out_scale, const msa_cache* ic, float* bs,
                             float* ts, const NewRows& nr, hipStream_t s) {
  switch (bt->rows_per_req) {
    case 1: launch_nvfp4<1, INSERT>(bt, q, out_scale, ic, bs, ts, nr, s); break;
    case 2: launch_nvfp4<2, INSERT>(bt, q, out_scale, ic, bs, ts, nr, s); break;
    case 3: launch_nvfp4<3, INSERT>(bt, q, out_scale, ic, bs, ts, nr, s); break;
    case 4: launch_nvfp4<4, INSERT>(bt, q, out_scale, ic, bs, ts, nr, s); break;
    case 5: launch_nvfp4<5, INSERT>(bt, q, out_scale, ic, bs, ts, nr, s); break;
    case 6: launch_nvfp4<6, INSERT>(bt, q, out_scale, ic, bs, ts, nr, s); break;
    case 7: launch_nvfp4<7, INSERT>(bt, q, out_scale, ic, bs, ts, nr, s); break;
    case 8: launch_nvfp4<8, INSERT>(bt, q, out_scale, ic, bs, ts, nr, s); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace msa

using namespace msa;

extern "C" int msa_launch_index_score(const msa_batch* bt, const void* q_idx, int32_t q_dtype, float q_scale,
                                      const msa_cache* ic, float* block_scores, float* token_scores,
                                      hipStream_t s) {
  if (ic->dtype == MSA_F32) {
    dim3 grid(bt->max_pages_per_req, bt->num_reqs);
    if (token_scores)
      hipLaunchKernelGGL(index_f32_kernel<true>, grid, dim3(128), 0, s, bt->block_table, bt->ctx_lens,
                         bt->max_pages_per_req, bt->rows_per_req, (const float*)q_idx, (const uint8_t*)ic->pages,
                         ic->num_pages, block_scores, token_scores);
    else
      hipLaunchKernelGGL(index_f32_kernel<false>, grid, dim3(128), 0, s, bt->block_table, bt->ctx_lens,
                         bt->max_pages_per_req, bt->rows_per_req, (const float*)q_idx, (const uint8_t*)ic->pages,
                         ic->num_pages, block_scores, token_scores);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  if (bt->rows_per_req > MSA_MAX_ROWS)  // a prefill chunk (NVFP4): the dense matrix-core scorer
    return msa_launch_prefill_index(bt, q_idx, q_scale, ic, block_scores, token_scores, s);
  const float out_scale = ic->tensor_scale * q_scale;
  if (owned_scan(bt, ic, token_scores))
    return launch_owned_rows<false>(bt, (const uint8_t*)q_idx, out_scale, ic, block_scores, NewRows{}, s);
  if (ic->dtype == MSA_FP8_E4M3)  // the shared-prefix declaration is not used with FP8 caches
    return launch_fp8_rows<false>(bt, (const uint8_t*)q_idx, out_scale, ic, block_scores, token_scores, NewRows{}, s);
  const int fused = launch_prefix_scan(bt, (const uint8_t*)q_idx, q_scale, ic, block_scores, token_scores, NewRows{},
                                       false, s);
  if (fused <= 0) return fused;
  if (msa_launch_prefix_index(bt, q_idx, q_scale, ic, block_scores, token_scores, s) != 0) return -1;
  return launch_nvfp4_rows<false>(bt, (const uint8_t*)q_idx, out_scale, ic, block_scores, token_scores, NewRows{}, s);
}

extern "C" int msa_launch_insert_index_score(const msa_batch* bt, const float* k_new, const float* v_new,
                                             const float* idx_new, const void* q_idx, float q_scale,
                                             const msa_cache* kc, const msa_cache* vc, const msa_cache* ic,
                                             float* block_scores, float* token_scores, hipStream_t s) {
  NewRows nr{k_new, v_new, idx_new, (uint8_t*)kc->pages, (uint8_t*)vc->pages, (uint8_t*)ic->pages,
             kc->num_pages, kc->tensor_scale, vc->tensor_scale, ic->tensor_scale};
  const float out_scale = ic->tensor_scale * q_scale;
  if (owned_scan(bt, ic, token_scores))
    return launch_owned_rows<true>(bt, (const uint8_t*)q_idx, out_scale, ic, block_scores, nr, s);
  if (ic->dtype == MSA_FP8_E4M3)
    return launch_fp8_rows<true>(bt, (const uint8_t*)q_idx, out_scale, ic, block_scores, token_scores, nr, s);
  const int fused = launch_prefix_scan(bt, (const uint8_t*)q_idx, q_scale, ic, block_scores, token_scores, nr, true, s);
  if (fused <= 0) return fused;
  if (msa_launch_prefix_index(bt, q_idx, q_scale, ic, block_scores, token_scores, s) != 0) return -1;
  return launch_nvfp4_rows<true>(bt, (const uint8_t*)q_idx, out_scale, ic, block_scores, token_scores, nr, s);
}

extern "C" int msa_launch_page_owner(const msa_batch* bt, int32_t num_pages, int32_t* owner, hipStream_t s) {
  const int64_t need = ((int64_t)num_pages + 255) / 256;
  const unsigned clear_wgs = (unsigned)(need < 4096 ? need : 4096);
  hipLaunchKernelGGL(page_owner_clear_kernel, dim3(clear_wgs), dim3(256), 0, s, owner, num_pages);
  const int cols = (bt->max_pages_per_req + 255) / 256;
  const unsigned per_req = (unsigned)(cols < 64 ? cols : 64);
  hipLaunchKernelGGL(page_owner_scatter_kernel, dim3(per_req, (unsigned)bt->num_reqs), dim3(256), 0, s,
                     bt->block_table, bt->ctx_lens, bt->max_pages_per_req, num_pages, owner);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
