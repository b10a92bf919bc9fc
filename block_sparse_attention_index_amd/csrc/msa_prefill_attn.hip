// msa_prefill_attn.hip -- step 4 for prompt chunks, block by block (vLLM M3.1
// post, "MiniMax 稀疏注意力的工作原理": each row attends to its own top-k
// blocks; spke.com post, "パフォーマンス最適化": a sparse-attention prefill
// kernel).
//
// The rows of a chunk select their blocks independently, but a whole chunk
// (thousands of rows) selects each block of its request many times over.  So
// this route takes the attention block-major: one workgroup per (request,
// group, block, up to kPfRows of the rows that selected the block).  It reads
// and dequantises the block once into FP16 images in LDS and runs every one of
// those rows against it, writing each (row, rank) pair's softmax partial --
// the block's max and denominator of the scaled scores, and its output
// normalised by that denominator, in FP16 -- to the caller's workspace.  A
// merge launch then combines each row's partials in rank order (bitwise
// reproducible; the result does not depend on which rows shared a workgroup,
// since every query column's products are its own).
//
//  1. pf_bucket_kernel, one workgroup per (request, group): counts each
//     block's selections in LDS, lays the (row, rank) entries out block by
//     block and cuts each block's run into work items of at most kPfRows rows.
//  2. pf_block_attend_kernel, one workgroup per work item: FP16 K and V
//     images in LDS, stored in the order the matrix instructions take them
//     (each operand load of a wave is one contiguous 1 KB, and each lane
//     dequantises exactly the 16-byte pieces it will load, so neither side
//     has bank conflicts); per wave, 4 rows at a time (two 16-column query
//     tiles of 2 rows x 8 heads): S^T = K Q^T and O^T = V^T P on
//     v_mfma_f32_16x16x32_f16, with the token order of the decode form (row i
//     of M-tile m is token 32(i/4) + 8(m/2) + 4(m%2) + i%4), so that the
//     softmax registers are the P operand as they stand.
//  3. pf_combine_kernel, one workgroup per two (request, row, group): with M the
//     largest partial max and w_k = exp2(m_k - M), out = v_scale *
//     sum_k w_k l_k O_k / sum_k w_k l_k, summed over ranks k in order.
#include <algorithm>

#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {

constexpr int kPfRows = 64;          // rows per work item
constexpr int kPfMaxPages = 8192;    // widest block table the bucketing counts in LDS

// Workspace layout (byte offsets from the caller's workspace).
struct PfLayout {
  size_t o, ml, list, items, total;
  int max_items;
};

static PfLayout pf_layout(const msa_batch* bt, int topk) {
  const size_t B = (size_t)bt->num_reqs, R = (size_t)bt->rows_per_req, P = (size_t)bt->max_pages_per_req;
  const size_t slots = B * R * kGroups * (size_t)topk;
  const size_t N = R * (size_t)topk;  // entries of one (request, group)
  // sum over blocks of ceil(count / kPfRows) <= N / kPfRows + (blocks with a count)
  const size_t max_items = std::min(P, N) + (N + kPfRows - 1) / kPfRows;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  PfLayout l;
  l.o = 0;
  l.ml = up(l.o + slots * kHpg * kDim * sizeof(_Float16));
  l.list = up(l.ml + slots * kHpg * 2 * sizeof(float));
  l.items = up(l.list + B * kGroups * N * sizeof(int32_t));
  l.total = up(l.items + B * kGroups * max_items * sizeof(int4));
  l.max_items = (int)max_items;
  return l;
}

// ---------------------------------------------------------------- 1. bucketing
// Entry i of (b, g) is row i / topk, rank i % topk; it counts when the rank is
// below the row's count and the block id lies in [0, max_pages).  list gets
// the entries block by block (r * 64 + k; within a block in no fixed order),
// items the work items {block, first entry, rows, physical page or -1 when the
// table entry lies outside the pool}, then {0, 0, 0, -1} up to max_items, so
// that a workgroup of the attention launch reads its item with no count first.
// The entries are read kEB per thread at a time, every load of a batch before
// its first LDS atomic, so that a batch is one memory round.
__global__ __launch_bounds__(1024) void pf_bucket_kernel(const int32_t* __restrict__ sel,
                                                         const int32_t* __restrict__ cnt, int32_t R,
                                                         int32_t max_pages, int32_t topk, int32_t max_items,
                                                         const int32_t* __restrict__ table, int32_t num_pages,
                                                         int32_t* __restrict__ list, int4* __restrict__ items) {
  constexpr int NT = 1024, PER = kPfMaxPages / NT, kEB = 16;
  __shared__ int s_cnt[kPfMaxPages];  // counts, then each block's next free entry
  __shared__ int s_wave[2][NT / 64];
  const int bg = (int)blockIdx.x, b = bg / kGroups, g = bg % kGroups;
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = R * topk;
  for (int j = tid; j < kPfMaxPages; j += NT) s_cnt[j] = 0;
  // entries i0 + e NT + tid, e < kEB: their block ids, and whether each counts
  auto load_batch = [&](int i0, int (&v)[kEB], bool (&ok)[kEB]) {
#pragma unroll
    for (int e = 0; e < kEB; ++e) {
      const int i = i0 + e * NT + tid, ic = min(i, N - 1);
      const int r = ic / topk, k = ic % topk;
      const int64_t row = ((int64_t)b * R + r) * kGroups + g;
      const int c = cnt[row];
      v[e] = sel[row * topk + k];
      ok[e] = i < N && k < c && v[e] >= 0 && v[e] < max_pages;
    }
  };
  __syncthreads();
  for (int i0 = 0; i0 < N; i0 += kEB * NT) {
    int v[kEB];
    bool ok[kEB];
    load_batch(i0, v, ok);
#pragma unroll
    for (int e = 0; e < kEB; ++e)
      if (ok[e]) atomicAdd(&s_cnt[v[e]], 1);
  }
  __syncthreads();
  // exclusive scans over the blocks of entries and of items: PER blocks per thread
  int c[PER], se = 0, si = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    c[e] = s_cnt[tid * PER + e];
    se += c[e];
    si += (c[e] + kPfRows - 1) / kPfRows;
  }
  int xe = se, xi = si;  // inclusive scans within the wave
#pragma unroll
  for (int d = 1; d < 64; d *= 2) {
    const int ye = __shfl_up(xe, d), yi = __shfl_up(xi, d);
    if (lane >= d) xe += ye, xi += yi;
  }
  if (lane == 63) s_wave[0][wave] = xe, s_wave[1][wave] = xi;
  __syncthreads();
  int be = xe - se, bi = xi - si;
  for (int w = 0; w < wave; ++w) be += s_wave[0][w], bi += s_wave[1][w];
  int total = 0;  // items of (b, g)
  for (int w = 0; w < NT / 64; ++w) total += s_wave[1][w];
  __syncthreads();  // every count is read: the array becomes the cursors
  int4* it = items + (int64_t)bg * max_items;
  // the table entries of this thread's blocks, loaded together (a clamped
  // index for blocks past the table: only blocks with a count use them)
  int phv[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) phv[e] = table[(int64_t)b * max_pages + min(tid * PER + e, max_pages - 1)];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int j = tid * PER + e;
    if (c[e] > 0) {
      const int ph = phv[e] >= 0 && phv[e] < num_pages ? phv[e] : -1;
      for (int t = 0; t * kPfRows < c[e]; ++t)
        it[bi++] = make_int4(j, be + t * kPfRows, min(kPfRows, c[e] - t * kPfRows), ph);
    }
    s_cnt[j] = be;
    be += c[e];
  }
  for (int i = total + tid; i < max_items; i += NT) it[i] = make_int4(0, 0, 0, -1);
  __syncthreads();
  int32_t* out = list + (int64_t)bg * N;
  for (int i0 = 0; i0 < N; i0 += kEB * NT) {
    int v[kEB];
    bool ok[kEB];
    load_batch(i0, v, ok);
#pragma unroll
    for (int e = 0; e < kEB; ++e) {
      const int i = i0 + e * NT + tid;
      if (ok[e]) out[atomicAdd(&s_cnt[v[e]], 1)] = (i / topk) * 64 + i % topk;
    }
  }
}

// ---------------------------------------------------------------- 2. block-major attention
// token held in row i of M-tile m (the decode form's order)
__device__ __forceinline__ constexpr int pf_tile_token(int m, int i) {
  return 32 * (i >> 2) + 8 * (m >> 1) + 4 * (m & 1) + (i & 3);
}

// One work item: rows list[first .. first + rows) of (b, g) against block j.
// Partial of (row r, rank k) of (b, g): slot ((b R + r) 4 + g) topk + k;
// part_o [slot][8 heads][128] FP16 (output / denominator), part_ml [slot][8][2]
// FP32 (max of the scaled scores in base 2, or -inf when no token of the block
// is visible to the row; denominator).
// FP8: FP8 caches (one E4M3 byte per element, exact in FP16; the tensor scales
// sit in qk2 and in the merge's v_scale), else NVFP4.
template <bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void pf_block_attend_kernel(
    const int32_t* __restrict__ lens, int32_t R, int32_t max_pages, const uint8_t* __restrict__ q, float qk2,
    const uint8_t* __restrict__ kpages, const uint8_t* __restrict__ vpages, int32_t topk, int32_t max_items,
    const int32_t* __restrict__ list, const int4* __restrict__ items, _Float16* __restrict__ part_o,
    float* __restrict__ part_ml) {
  // operand images: piece (m, s, lane) of K holds token tok(m, lane % 16), dims
  // 32 (lane / 16) + 8s .. + 7; piece (nt, kk, lane) of V holds dim 16 nt + lane % 16,
  // tokens 32 (lane / 16) + 8 kk .. + 7
  __shared__ h8 s_k[8 * 4 * 64];
  __shared__ h8 s_v[8 * 4 * 64];
  const int bg = (int)blockIdx.y, b = bg / kGroups, g = bg % kGroups;
  const int4 item = items[(int64_t)bg * max_items + blockIdx.x];
  const int j = item.x, first = item.y, rows = item.z, ph = item.w;
  if (rows == 0) return;  // past the last item of (b, g)
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, a = lane >> 4;
  const int L = clamp_len(lens[b], max_pages);
  const bool valid = ph >= 0;  // uniform: a page outside the pool adds nothing
  const int32_t* ent = list + (int64_t)bg * R * topk + first;
  // this wave's passes: rows 4 quad .. 4 quad + 3 for quad = wave + 4i; the entry
  // (r * 64 + k, or -1) of this lane's query column n of tile qt, row 4 quad + 2 qt + n / 8
  constexpr int kPasses = kPfRows / 16;
  int ents[kPasses][2];
#pragma unroll
  for (int i = 0; i < kPasses; ++i)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int li = 4 * (wave + 4 * i) + 2 * qt + (n >> 3);
      const int e = ent[min(li, rows - 1)];
      ents[i][qt] = li < rows ? e : -1;
    }
  auto slot_of = [&](int e) {  // partial row of entry e: (slot, head n % 8)
    return ((((int64_t)b * R + (e >> 6)) * kGroups + g) * topk + (e & 63)) * kHpg + (n & 7);
  };

  if (!valid) {  // a page outside the pool: nothing visible (max -inf, denominator 0)
#pragma unroll
    for (int i = 0; i < kPasses; ++i)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        if (ents[i][qt] < 0) continue;
        const int64_t sl = slot_of(ents[i][qt]);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
          *reinterpret_cast<uint2*>(part_o + sl * kDim + 16 * nt + 4 * a) = make_uint2(0, 0);
        if (a == 0) *reinterpret_cast<float2*>(part_ml + sl * 2) = make_float2(-__builtin_inff(), 0.f);
      }
    return;
  }
  // query bytes of one pass (this lane's column of both tiles: dims 32a + 8s .. + 7), raw,
  // then as FP16 operands; a column with no row loads row 0 and is zeroed when converted
  auto fetch_q = [&](const int (&e2)[2], uint2 (&w)[2][4]) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int e = max(e2[qt], 0);
      const uint8_t* qrow = q + ((((int64_t)b * R + (e >> 6)) * kGroups + g) * kHpg + (n & 7)) * kDim;
#pragma unroll
      for (int s = 0; s < 4; ++s) w[qt][s] = *reinterpret_cast<const uint2*>(qrow + 32 * a + 8 * s);
    }
  };
  auto convert_q = [&](const int (&e2)[2], const uint2 (&w)[2][4], h8 (&Qd)[2][4]) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint2 x = e2[qt] >= 0 ? w[qt][s] : make_uint2(0, 0);
        const h2 x0 = e4m3x2_to_h2<false>(x.x), x1 = e4m3x2_to_h2<true>(x.x);
        const h2 x2 = e4m3x2_to_h2<false>(x.y), x3 = e4m3x2_to_h2<true>(x.y);
        Qd[qt][s] = h8{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
      }
  };

  {
    // ---- dequantise: wave w writes K M-tiles and V dim tiles 2w, 2w + 1, each
    // lane the pieces it will read (its 32 elements of one token / dim per tile)
    constexpr int kSlab = FP8 ? kFp8Slab : kNvSlab;
    const uint8_t* ks = kpages + ((int64_t)ph * kGroups + g) * kSlab;
    const uint8_t* vs = vpages + ((int64_t)ph * kGroups + g) * kSlab;
    uint2 qn[2][4];
    if constexpr (FP8) {
      // keys [token][dim], values [dim][token]: 32 bytes per tile and lane
      uint4 kc[2][2], vc[2][2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int t = pf_tile_token(2 * wave + i, n), d = 16 * (2 * wave + i) + n;
        kc[i][0] = *reinterpret_cast<const uint4*>(ks + t * kDim + 32 * a);
        kc[i][1] = *reinterpret_cast<const uint4*>(ks + t * kDim + 32 * a + 16);
        vc[i][0] = *reinterpret_cast<const uint4*>(vs + d * kPage + 32 * a);
        vc[i][1] = *reinterpret_cast<const uint4*>(vs + d * kPage + 32 * a + 16);
      }
      fetch_q(ents[0], qn);
      auto to_h8 = [](uint32_t lo, uint32_t hi) {
        const h2 x0 = e4m3x2_to_h2<false>(lo), x1 = e4m3x2_to_h2<true>(lo);
        const h2 x2 = e4m3x2_to_h2<false>(hi), x3 = e4m3x2_to_h2<true>(hi);
        return h8{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
      };
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int tile = 2 * wave + i;
#pragma unroll
        for (int st = 0; st < 4; ++st) {  // elements 32a + 8st .. + 7: bytes 8 (st % 2) .. of word st / 2
          const uint4 kq = kc[i][st >> 1], vq = vc[i][st >> 1];
          s_k[(tile * 4 + st) * 64 + lane] = to_h8((st & 1) ? kq.z : kq.x, (st & 1) ? kq.w : kq.y);
          s_v[(tile * 4 + st) * 64 + lane] = to_h8((st & 1) ? vq.z : vq.x, (st & 1) ? vq.w : vq.y);
        }
      }
    } else {
      uint4 kc[2], vc[2], vsc[2][2];
      uint32_t ksc[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int t = pf_tile_token(2 * wave + i, n), d = 16 * (2 * wave + i) + n;
        kc[i] = *reinterpret_cast<const uint4*>(ks + t * 64 + 16 * a);
        ksc[i] = *reinterpret_cast<const uint16_t*>(ks + kScaleOff + t * 8 + 2 * a);  // groups 2a, 2a + 1
        vc[i] = *reinterpret_cast<const uint4*>(vs + d * 64 + 16 * a);
        // value scales of dim group 2w + i ([group][token]), tokens 32a .. 32a + 31
        vsc[i][0] = *reinterpret_cast<const uint4*>(vs + kScaleOff + (2 * wave + i) * kPage + 32 * a);
        vsc[i][1] = *reinterpret_cast<const uint4*>(vs + kScaleOff + (2 * wave + i) * kPage + 32 * a + 16);
      }
      fetch_q(ents[0], qn);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int tile = 2 * wave + i;
        const h2 sk = e4m3x2_to_h2<false>(ksc[i]);
        const uint32_t kw[4] = {kc[i].x, kc[i].y, kc[i].z, kc[i].w};
        const uint32_t vw[4] = {vc[i].x, vc[i].y, vc[i].z, vc[i].w};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const _Float16 sc = st < 2 ? sk[0] : sk[1];  // dims 32a + 8st ..: group 2a + st / 2
          s_k[(tile * 4 + st) * 64 + lane] = e2m1x8_to_h8(kw[st]) * h8{sc, sc, sc, sc, sc, sc, sc, sc};
          const uint4 sq = vsc[i][st >> 1];  // tokens 32a + 8st .. + 7: bytes 8 (st % 2) .. of word st / 2
          const uint32_t lo = (st & 1) ? sq.z : sq.x, hi = (st & 1) ? sq.w : sq.y;
          const h2 s0 = e4m3x2_to_h2<false>(lo), s1 = e4m3x2_to_h2<true>(lo);
          const h2 s2 = e4m3x2_to_h2<false>(hi), s3 = e4m3x2_to_h2<true>(hi);
          s_v[(tile * 4 + st) * 64 + lane] =
              e2m1x8_to_h8(vw[st]) * h8{s0[0], s0[1], s1[0], s1[1], s2[0], s2[1], s3[0], s3[1]};
        }
      }
    }
    // the first pass's queries: converted before the barrier, so that their loads
    // run beside the block's instead of after it
    h8 Q[2][4];
    convert_q(ents[0], qn, Q);
    __syncthreads();

    // ---- 4 rows per pass: column n of tile qt is row 2qt + n / 8 of the four, head n % 8;
    // the next pass's query bytes load while this pass computes
    const h8 ones = h8{1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
    for (int pi = 0; pi < kPasses; ++pi) {
      const int quad = wave + 4 * pi;
      if (4 * quad >= rows) break;
      const bool more = pi + 1 < kPasses && 4 * (quad + 4) < rows;
      if (more) fetch_q(ents[pi + 1 < kPasses ? pi + 1 : pi], qn);
      int lim[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int e = ents[pi][qt];
        // last visible token of the block for this row (padding columns: all, never stored)
        lim[qt] = e >= 0 ? min(kPage - 1, L - R + (e >> 6) - j * kPage) : kPage - 1;
      }
      // ---- S^T = K Q^T
      v4f S[2][8];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int m = 0; m < 8; ++m) S[qt][m] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const h8 kv = s_k[(m * 4 + s) * 64 + lane];
#pragma unroll
          for (int qt = 0; qt < 2; ++qt)
            S[qt][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, Q[qt][s], S[qt][m], 0, 0, 0);
        }
      // ---- block-local softmax in base 2 (token of S[qt][m][i] = 32a + 8(m/2) + 4(m%2) + i):
      // the max is taken on the raw scores (qk2 > 0 keeps the order), and the scale
      // and the max's subtraction are one fused multiply-add
      const bool partial = __any(lim[0] < kPage - 1 || lim[1] < kPage - 1) != 0;
      h8 P[2][4];
      float mx[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        if (partial) {
          const int lr = lim[qt] - 32 * a;
#pragma unroll
          for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              S[qt][m][i] = 8 * (m >> 1) + 4 * (m & 1) + i <= lr ? S[qt][m][i] : -__builtin_inff();
        }
        float v = -__builtin_inff();
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) v = fmaxf(v, S[qt][m][i]);
        mx[qt] = rows_max4(v) * qk2;
        const float nbase = mx[qt] == -__builtin_inff() ? 0.f : -mx[qt];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          h8 pk;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pk[e] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(S[qt][2 * kk + (e >> 2)][e & 3], qk2, nbase));
          P[qt][kk] = pk;
        }
      }
      // ---- denominators (column sums of the FP16 P) and O^T = V^T P
      v4f l[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) l[qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, P[qt][kk], l[qt], 0, 0, 0);
      v4f O[2][8];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) O[qt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const h8 vv = s_v[(nt * 4 + kk) * 64 + lane];
#pragma unroll
          for (int qt = 0; qt < 2; ++qt)
            O[qt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vv, P[qt][kk], O[qt][nt], 0, 0, 0);
        }
      // ---- partials: lane (n, a) holds dims 16nt + 4a .. + 3 of column n
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        if (ents[pi][qt] < 0) continue;
        const int64_t sl = slot_of(ents[pi][qt]);
        const float den = l[qt][0];
        const float inv = den > 0.f ? 1.f / den : 0.f;
        _Float16* po = part_o + sl * kDim;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const h2 lo = h2{(_Float16)(O[qt][nt][0] * inv), (_Float16)(O[qt][nt][1] * inv)};
          const h2 hi = h2{(_Float16)(O[qt][nt][2] * inv), (_Float16)(O[qt][nt][3] * inv)};
          *reinterpret_cast<uint2*>(po + 16 * nt + 4 * a) =
              make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
        }
        if (a == 0) *reinterpret_cast<float2*>(part_ml + sl * 2) = make_float2(mx[qt], den);
      }
      if (more) convert_q(ents[pi + 1 < kPasses ? pi + 1 : pi], qn, Q);
    }
  }
}

// ---------------------------------------------------------------- 3. merge
// One workgroup per two (request, row, group) rows; thread t: row 2 blockIdx + t / 128,
// head (t % 128) / 16, dims 8 (t % 16) .. + 7 (one 16-byte load per rank).  The
// partials load 16 ranks at a time, all at once: the slots of ranks 0..15 load
// together with the row's count and selection, so no load waits on another, and
// an absent rank's values (its slot was not written) are replaced by an empty
// partial (max -inf, denominator 0, output 0) before use; later groups of 16 load
// only while the count reaches them.  Each group then joins the running result
// (max, weighted denominator and sum), in rank order.
__global__ __launch_bounds__(256) void pf_combine_kernel(const int32_t* __restrict__ sel,
                                                         const int32_t* __restrict__ cnt, int64_t rows,
                                                         int32_t topk, int32_t max_pages,
                                                         const _Float16* __restrict__ part_o,
                                                         const float* __restrict__ part_ml, float v_scale,
                                                         float* __restrict__ out) {
  constexpr int KC = 16;
  const int64_t row = 2 * (int64_t)blockIdx.x + ((int)threadIdx.x >> 7);
  if (row >= rows) return;  // (uniform per wave: a wave lies within one row)
  const int hh = ((int)threadIdx.x >> 4) & 7, d = 8 * ((int)threadIdx.x & 15);
  const int32_t* srow = sel + row * topk;
  const int c = cnt[row];
  float M = -__builtin_inff(), den = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < topk; k0 += KC) {
    if (k0 > 0 && k0 >= c) break;
    float mk[KC], lk[KC];
    uint4 ok[KC];
    // lanes 0..15 of each wave load ranks k0 .. k0 + 15 at once; each rank is read from its lane
    const int vl = srow[min(k0 + ((int)threadIdx.x & (KC - 1)), topk - 1)];
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int64_t s = (row * topk + min(k0 + i, topk - 1)) * kHpg + hh;
      const float2 ml = *reinterpret_cast<const float2*>(part_ml + s * 2);
      ok[i] = *reinterpret_cast<const uint4*>(part_o + s * kDim + d);
      mk[i] = ml.x;
      lk[i] = ml.y;
    }
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int k = k0 + i;
      const int v = __builtin_amdgcn_readlane(vl, i);
      const bool present = k < topk && k < c && v >= 0 && v < max_pages;
      mk[i] = present ? mk[i] : -__builtin_inff();
      lk[i] = present ? lk[i] : 0.f;
      // a mask rather than a select, so that no load is moved under a branch
      const uint32_t keep = present ? ~0u : 0u;
      ok[i].x &= keep, ok[i].y &= keep, ok[i].z &= keep, ok[i].w &= keep;
    }
    float Mc = M;
#pragma unroll
    for (int i = 0; i < KC; ++i) Mc = fmaxf(Mc, mk[i]);
    // (a group with nothing visible leaves M at -inf and adds weights of 0)
    const float r = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(M - Mc);
    den *= r;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= r;
    M = Mc;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const float wl = mk[i] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mk[i] - M) * lk[i];
      const uint32_t w4[4] = {ok[i].x, ok[i].y, ok[i].z, ok[i].w};
      den += wl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const h2 x = __builtin_bit_cast(h2, w4[e]);
        acc[2 * e] += wl * (float)x[0];
        acc[2 * e + 1] += wl * (float)x[1];
      }
    }
  }
  const float inv = den > 0.f ? v_scale / den : 0.f;
  float* o = out + (row * kHpg + hh) * kDim + d;
  *reinterpret_cast<float4*>(o) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
}

}  // namespace msa

using namespace msa;

extern "C" size_t msa_prefill_block_bytes(const msa_batch* bt, int32_t topk) {
  if (bt->rows_per_req <= MSA_MAX_ROWS || bt->max_pages_per_req > kPfMaxPages) return 0;
  return pf_layout(bt, topk).total;
}

extern "C" int msa_launch_prefill_block_attend(const msa_batch* bt, const uint8_t* q, float q_scale, float sm_scale,
                                               const msa_cache* kc, const msa_cache* vc, const int32_t* sel,
                                               const int32_t* cnt, int32_t topk, float* out, void* workspace,
                                               hipStream_t s) {
  const PfLayout ly = pf_layout(bt, topk);
  uint8_t* ws = (uint8_t*)workspace;
  _Float16* part_o = (_Float16*)(ws + ly.o);
  float* part_ml = (float*)(ws + ly.ml);
  int32_t* list = (int32_t*)(ws + ly.list);
  int4* items = (int4*)(ws + ly.items);
  const int B = bt->num_reqs, R = bt->rows_per_req, P = bt->max_pages_per_req;
  hipLaunchKernelGGL(pf_bucket_kernel, dim3((unsigned)(B * kGroups)), dim3(1024), 0, s, sel, cnt, R, P, topk,
                     ly.max_items, bt->block_table, kc->num_pages, list, items);
  if (hipGetLastError() != hipSuccess) return -1;
  // scores enter the softmax in base 2
  const float qk2 = sm_scale * kc->tensor_scale * q_scale * 1.4426950408889634f;
  const dim3 grid((unsigned)ly.max_items, (unsigned)(B * kGroups));
  if (kc->dtype == MSA_FP8_E4M3)
    hipLaunchKernelGGL(pf_block_attend_kernel<true>, grid, dim3(256), 0, s, bt->ctx_lens, R, P, q, qk2,
                       (const uint8_t*)kc->pages, (const uint8_t*)vc->pages, topk, ly.max_items, list, items, part_o,
                       part_ml);
  else
    hipLaunchKernelGGL(pf_block_attend_kernel<false>, grid, dim3(256), 0, s, bt->ctx_lens, R, P, q, qk2,
                       (const uint8_t*)kc->pages, (const uint8_t*)vc->pages, topk, ly.max_items, list, items, part_o,
                       part_ml);
  if (hipGetLastError() != hipSuccess) return -1;
  const int64_t rows = (int64_t)B * R * kGroups;
  hipLaunchKernelGGL(pf_combine_kernel, dim3((unsigned)((rows + 1) / 2)), dim3(256), 0, s, sel, cnt, rows, topk, P,
                     part_o, part_ml, vc->tensor_scale, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
