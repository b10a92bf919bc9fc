// msa_attn.hip -- step 4: exact GQA softmax attention over the selected
// blocks (vLLM M3.1 post, "MiniMax 稀疏注意力的工作原理"; spke.com "MSA入門"
// Fig. 1 caption; "MiniMax goes sparse", section 1 Step 2: every query head
// of a group attends to the group's selected blocks), alone or fused with
// step 3 (the selection) in one launch.
//
// Work split (NVFP4 and FP8): one workgroup of 8 waves per (request, group,
// row) while the batch's rows x groups fit the CUs; beyond that, one per
// (request, group, group of up to 4 rows), the waves walking the union of the
// rows' selected blocks (4 waves with two query tiles when R > 2).  The waves
// take the blocks two at a time with both blocks' loads in flight, each
// keeping an online softmax (running max, denominator, unnormalised output);
// they then merge through LDS and the workgroup writes the normalised output
// -- no partial results leave the chip and no second launch merges them.
// With the selection fused in, waves 0..nr-1 first run the top-k of one row
// each (msa_select.h) from the block scores, while the block-table row and
// the queries load.  The 8 heads of a group share each dequantised K/V
// element (GQA); 4 rows' 32 query vectors fill two 16-column query tiles.
// Prefill chunks (more than 8 rows) take one row per workgroup of 4 waves,
// one block per wave at a time, three workgroups per CU: their rows select
// independently, so a row group's union would only multiply the work.
//
// Per block and wave:
//  * S^T = K Q^T on v_mfma_f32_16x16x32_f16.  K codes go through the exact
//    E2M1->FP16 conversion and one packed FP16 multiply by their E4M3 scale
//    (E2M1 x E4M3 has at most 6 significant bits, so the product is exact);
//    the K tensor scale, the query scale, sm_scale and log2(e) are applied to
//    the FP32 accumulators.  Queries (E4M3) are exact in FP16 as well.
//  * Row i of M-tile m is token 32*(i/4) + 8*(m/2) + 4*(m%2) + i%4: a lane
//    (column n, quad a) then holds, for the 32-token step kk of the P.V
//    product, tokens 32a + 8kk + 0..7 -- already the P operand, with no
//    shuffle -- and the value codes of those tokens for one dim are 4
//    consecutive bytes, so a lane loads the codes of all four steps of a
//    16-dim tile as one 16-byte word of the dim-major value slab.
//  * P is rounded to FP16 (FP32 accumulation); its row sums come from one
//    more MFMA against a ones operand, so the denominator adds exactly the P
//    that the numerator uses.  V codes are scaled per token by their E4M3
//    group scale in FP16 (converted once per block into LDS).
//  * K and V are read with 16-byte loads, non-temporal in decode (each
//    selected block is read once per step), cacheable in prefill (the other
//    rows of the chunk read the same blocks).
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "msa_device.h"
#include "msa_kernels.h"
#include "msa_select.h"

namespace msa {


// Sorted union of the sets already in s_rowsel (nr rows of topk ids, -1 padded).
// One row: the ids are already sorted; the valid ones are compacted by a
// ballot of the first wave.
__device__ int union_of_rows(const int* s_rowsel, int nr, int topk, int* s_first, int* s_union, int* s_nu) {
  const int tid = threadIdx.x;
  const int N = nr * topk;
  if (nr == 1) {
    if (tid < 64) {
      const int v = tid < topk ? s_rowsel[tid] : -1;
      const uint64_t m = __ballot(v >= 0);
      const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      if (v >= 0) s_union[before] = v;
      if (tid == 0) *s_nu = __popcll(m);
    }
    __syncthreads();
    return *s_nu;
  }
  if (tid == 0) *s_nu = 0;
  for (int i = tid; i < N; i += blockDim.x) {
    const int v = s_rowsel[i];
    bool first = v >= 0;
    for (int e = 0; e < i && first; ++e) first = s_rowsel[e] != v;
    s_first[i] = first ? 1 : 0;
  }
  __syncthreads();
  for (int i = tid; i < N; i += blockDim.x) {
    if (!s_first[i]) continue;
    const int v = s_rowsel[i];
    int rank = 0;
    for (int e = 0; e < N; ++e) rank += (s_first[e] && s_rowsel[e] < v) ? 1 : 0;
    s_union[rank] = v;
    atomicAdd(s_nu, 1);
  }
  __syncthreads();
  return *s_nu;
}

// Rows [r0, r0 + nr) of (b, g): load their selected sets into s_rowsel and
// form the sorted union in LDS.  Returns the union size.  Entries past a
// row's count, or naming a block beyond the table, read as absent (-1).
__device__ int build_union(const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt, int b, int g, int R,
                           int r0, int nr, int topk, int max_pages, int* s_rowsel, int* s_first, int* s_union,
                           int* s_nu) {
  const int N = nr * topk;
  for (int i = threadIdx.x; i < N; i += blockDim.x) {
    const int r = r0 + i / topk, k = i % topk;
    const int64_t row = ((int64_t)b * R + r) * kGroups + g;
    const int c = cnt[row];
    const int v = sel[row * topk + k];
    s_rowsel[i] = (k < c && v < max_pages) ? v : -1;
  }
  __syncthreads();
  return union_of_rows(s_rowsel, nr, topk, s_first, s_union, s_nu);
}

__device__ __forceinline__ bool row_has_block(const int* s_rowsel, int rl, int topk, int j) {
  for (int k = 0; k < topk; ++k)
    if (s_rowsel[rl * topk + k] == j) return true;
  return false;
}

// Running softmax state of one wave over QT query tiles of 16 columns, in the
// base-2 domain (scores pre-multiplied by log2 e).
template <int QT>
struct AttnState {
  float m[QT];   // running max of query column n = lane%16 (same in its 4 lanes)
  v4f L[QT];     // running denominator of queries 4*(lane/16)+q (every column holds it)
  v4f O[QT][8];  // unnormalised output: rows 4*(lane/16)+q (queries), dims 16*nt + lane%16
};

// Query operands: column n of tile qt = query qi = 16qt + n -> (row qi/8, head qi%8 of group g),
// dims 32a + 8ks + 0..7 for k-step ks (the K operand uses the same dim order).
template <int QT>
__device__ __forceinline__ void load_q(const uint8_t* __restrict__ q, int b, int R, int r0, int nr, int g, int lane,
                                       h8 (&Q)[QT][4]) {
  const int n = lane & 15, a = lane >> 4;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qi = qt * 16 + n;
    const int rl = qi / kHpg, hh = qi % kHpg;
    const bool ok = rl < nr;
    const uint8_t* qrow = q + ((((int64_t)b * R + r0 + (ok ? rl : 0)) * kGroups + g) * kHpg + hh) * kDim;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint2 w = *reinterpret_cast<const uint2*>(qrow + 32 * a + 8 * ks);
      w = ok ? w : make_uint2(0, 0);
      const h2 x0 = e4m3x2_to_h2<false>(w.x), x1 = e4m3x2_to_h2<true>(w.x);
      const h2 x2 = e4m3x2_to_h2<false>(w.y), x3 = e4m3x2_to_h2<true>(w.y);
      Q[qt][ks] = h8{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
    }
  }
}

// What one wave reads of one 128-token block: the key part, then the value
// part.  Every load is 16 bytes per lane.
struct KRegs {
  uint4 kc[8];  // K codes of token tok(m): dims 32a .. 32a+31
  uint4 ksc;    // K scales of tokens 2 lane, 2 lane + 1 (8 bytes each)
};
struct VRegs {
  uint4 vw[8];  // V codes of dim 16nt + n: tokens 32a .. 32a+31 (dword kk = tokens 32a + 8kk ..)
  uint4 vsc;    // V scales, bytes 16 lane .. 16 lane + 15 of the block's 1 KB ([group][token])
};

// token held in row i of M-tile m (see the file comment)
__device__ __forceinline__ constexpr int tile_token(int m, int i) {
  return 32 * (i >> 2) + 8 * (m >> 1) + 4 * (m & 1) + (i & 3);
}

// K/V loads: with the streaming hint where each selected block is read once
// (decode); NT = false where other rows read the same block again soon
// (prefill chunks), so that the caches may keep it.
template <bool NT>
__device__ __forceinline__ uint4 kv_load4(const uint8_t* p) {
  if constexpr (NT) return nt_load4(p);
  return *reinterpret_cast<const uint4*>(p);
}

template <bool NT = true>
__device__ __forceinline__ void load_k(const uint8_t* __restrict__ ks_, int lane, KRegs& r) {
  const int n = lane & 15, a = lane >> 4;
#pragma unroll
  for (int m = 0; m < 8; ++m) r.kc[m] = kv_load4<NT>(ks_ + tile_token(m, n) * 64 + 16 * a);
  r.ksc = kv_load4<NT>(ks_ + kScaleOff + 16 * lane);
}

template <bool NT = true>
__device__ __forceinline__ void load_v(const uint8_t* __restrict__ vs_, int lane, VRegs& r) {
  const int n = lane & 15, a = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) r.vw[nt] = kv_load4<NT>(vs_ + (16 * nt + n) * 64 + 16 * a);
  r.vsc = kv_load4<NT>(vs_ + kScaleOff + 16 * lane);
}

// FP8 caches: a lane's 32 bytes per M-tile (keys) or per 16-dim tile
// (values), one E4M3 byte per element, no per-element scales (the tensor
// scales are folded into the softmax and output scales).
struct KRegs8 {
  uint4 kc[8][2];  // K bytes of token tok(m): dims 32a .. 32a+15, 32a+16 .. 32a+31
};
struct VRegs8 {
  uint4 vw[8][2];  // V bytes of dim 16nt + n: tokens 32a .. 32a+15, 32a+16 .. 32a+31
};

template <bool NT = true>
__device__ __forceinline__ void load_k(const uint8_t* __restrict__ ks_, int lane, KRegs8& r) {
  const int n = lane & 15, a = lane >> 4;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    r.kc[m][0] = kv_load4<NT>(ks_ + tile_token(m, n) * kDim + 32 * a);
    r.kc[m][1] = kv_load4<NT>(ks_ + tile_token(m, n) * kDim + 32 * a + 16);
  }
}

template <bool NT = true>
__device__ __forceinline__ void load_v(const uint8_t* __restrict__ vs_, int lane, VRegs8& r) {
  const int n = lane & 15, a = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    r.vw[nt][0] = kv_load4<NT>(vs_ + (16 * nt + n) * kPage + 32 * a);
    r.vw[nt][1] = kv_load4<NT>(vs_ + (16 * nt + n) * kPage + 32 * a + 16);
  }
}

// 8 E4M3 bytes (step s of a 32-byte lane tile: bytes 8s .. 8s+7) -> exact FP16.
__device__ __forceinline__ h8 e4m3x8_step(const uint4 (&w)[2], int s) {
  const uint4& q = w[s >> 1];
  const uint32_t lo = (s & 1) ? q.z : q.x, hi = (s & 1) ? q.w : q.y;
  const h2 x0 = e4m3x2_to_h2<false>(lo), x1 = e4m3x2_to_h2<true>(lo);
  const h2 x2 = e4m3x2_to_h2<false>(hi), x3 = e4m3x2_to_h2<true>(hi);
  return h8{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
}

// Per-wave LDS slots of one block's scales.
struct ScaleSlot {
  uint4 k[64];  // raw K scale bytes, [token][group]
  h8 v[128];    // V scales in FP16, [group][token]
};

// NVFP4 value scales of one block to FP16 in the wave's LDS slot ([group][token]).
__device__ __forceinline__ void stage_vscales(const VRegs& vr, ScaleSlot* slot, int lane) {
  const uint32_t w[4] = {vr.vsc.x, vr.vsc.y, vr.vsc.z, vr.vsc.w};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const h2 s0 = e4m3x2_to_h2<false>(w[2 * i]), s1 = e4m3x2_to_h2<true>(w[2 * i]);
    const h2 s2 = e4m3x2_to_h2<false>(w[2 * i + 1]), s3 = e4m3x2_to_h2<true>(w[2 * i + 1]);
    slot->v[2 * lane + i] = h8{s0[0], s0[1], s1[0], s1[1], s2[0], s2[1], s3[0], s3[1]};
  }
}
__device__ __forceinline__ void stage_vscales(const VRegs8&, ScaleSlot*, int) {}

// One 128-token block: S^T = K Q^T, online-softmax update of `st`, O += P V.
// lim[qt]: last visible token of the block for this lane's query column (-1:
// none); `partial` (wave-uniform) says whether any lim is below 127; `first`
// (wave-uniform) says the state is still empty, so nothing needs rescaling.
// after_qk() runs once the key registers are consumed (the caller issues the
// next block's loads there); before_pv() once the scores are consumed too.
struct NoOp {
  __device__ void operator()() const {}
};

template <int QT, bool LATE_VSC = false, typename KR, typename VR, typename AfterQK, typename BeforePV = NoOp>
__device__ __forceinline__ void attend_block(const KR& kr, const VR& vr, const h8 (&Q)[QT][4],
                                             const int (&lim)[QT], bool partial, bool first, float qk2, int lane,
                                             ScaleSlot* slot, AttnState<QT>& st, AfterQK after_qk,
                                             BeforePV before_pv = {}) {
  constexpr bool FP8 = __is_same(KR, KRegs8);
  const int n = lane & 15, a = lane >> 4;
  // ---- NVFP4 scales through LDS: each lane needs scales that other lanes of
  // this wave loaded.  Value scales go with the key scales, or with LATE_VSC
  // after the softmax (the caller issues the value loads in after_qk)
  if constexpr (!FP8) {
    slot->k[lane] = kr.ksc;
    if constexpr (!LATE_VSC) stage_vscales(vr, slot, lane);
    wave_lds_sync();
  }
  const uint8_t* kraw = reinterpret_cast<const uint8_t*>(slot->k);

  // ---- S^T = K Q^T (k-steps outermost: the 8 accumulators are independent)
  h2 ksc[8];
  if constexpr (!FP8)
#pragma unroll
    for (int m = 0; m < 8; ++m)
      ksc[m] = e4m3x2_to_h2<false>(*reinterpret_cast<const uint16_t*>(kraw + tile_token(m, n) * 8 + 2 * a));
  v4f Sacc[QT][8];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int m = 0; m < 8; ++m) Sacc[qt][m] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      h8 kv;
      if constexpr (FP8) {
        kv = e4m3x8_step(kr.kc[m], ks);
      } else {
        const uint32_t word = ks == 0 ? kr.kc[m].x : ks == 1 ? kr.kc[m].y : ks == 2 ? kr.kc[m].z : kr.kc[m].w;
        const _Float16 s = ks < 2 ? ksc[m][0] : ksc[m][1];
        kv = e2m1x8_to_h8(word) * h8{s, s, s, s, s, s, s, s};
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        Sacc[qt][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, Q[qt][ks], Sacc[qt][m], 0, 0, 0);
    }
  }
  // with LATE_VSC the value loads issue here: keep them behind the key registers' last use
  if constexpr (LATE_VSC) __builtin_amdgcn_sched_barrier(0);
  after_qk();

  // ---- online softmax, base 2 (token of Sacc[qt][m][q] = 32a + 8(m/2) + 4(m%2) + q)
  h8 P[QT][4];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int m = 0; m < 8; ++m) Sacc[qt][m] *= qk2;
    if (partial) {
      const int lr = lim[qt] - 32 * a;  // visible iff 8(m/2) + 4(m%2) + q <= lr
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          Sacc[qt][m][qq] = 8 * (m >> 1) + 4 * (m & 1) + qq <= lr ? Sacc[qt][m][qq] : -__builtin_inff();
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) mx = fmaxf(mx, Sacc[qt][m][qq]);
    mx = rows_max4(mx);
    const float m_new = fmaxf(st.m[qt], mx);
    // exponent base: a column with nothing visible yet keeps m = -inf and uses 0,
    // so exp2(-inf - base) = 0 throughout
    const float base = m_new == -__builtin_inff() ? 0.f : m_new;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      h8 pk;
#pragma unroll
      for (int e = 0; e < 8; ++e) pk[e] = (_Float16)__builtin_amdgcn_exp2f(Sacc[qt][2 * kk + (e >> 2)][e & 3] - base);
      P[qt][kk] = pk;
    }
    if (!first) {
      // rescale the rows this lane holds (query 4a + q is column 4a + q of lane 4a + q)
      const float alpha = __builtin_amdgcn_exp2f(st.m[qt] - base);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const float aq = __shfl(alpha, 4 * a + qq);
        st.L[qt][qq] *= aq;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) st.O[qt][nt][qq] *= aq;
      }
    }
    st.m[qt] = m_new;
  }

  if constexpr (LATE_VSC) __builtin_amdgcn_sched_barrier(0);
  before_pv();
  if constexpr (!FP8 && LATE_VSC) {
    stage_vscales(vr, slot, lane);
    wave_lds_sync();
  }

  // ---- denominators: L += P . 1 (row sums of the FP16 P that the numerator uses)
  const h8 ones = h8{1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) st.L[qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P[qt][kk], ones, st.L[qt], 0, 0, 0);

  // ---- O += P V (dims d = 16 nt + n; step kk: tokens 32a + 8kk .. of dim d; k-steps outermost)
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      h8 vv;
      if constexpr (FP8) {
        vv = e4m3x8_step(vr.vw[nt], kk);
      } else {
        const uint32_t word = kk == 0 ? vr.vw[nt].x : kk == 1 ? vr.vw[nt].y : kk == 2 ? vr.vw[nt].z : vr.vw[nt].w;
        vv = e2m1x8_to_h8(word) * slot->v[nt * 16 + 4 * a + kk];
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        st.O[qt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P[qt][kk], vv, st.O[qt][nt], 0, 0, 0);
    }
  }
  // the slot is rewritten for this wave's next block: keep those stores behind these reads
  __builtin_amdgcn_wave_barrier();
}

constexpr int kTabLds = 2048;  // block-table rows up to this width are staged in LDS
constexpr int kSplitPart = 2 * kHpg + kHpg * kDim;  // floats of one split's partial: M[8], l[8], O[8][128]
constexpr int kMaxSplit = 4;

// Merge of the SPLIT partials of each (request, row, group): with M = max_s
// M_s and w_s = exp2(M_s - M), out = v_scale * sum_s w_s O_s / sum_s w_s l_s,
// summed in split order (bitwise reproducible).  One workgroup per (request,
// row, group); thread t handles head t / 32, dims 4 (t % 32) .. + 3.
template <int SPLIT>
__global__ __launch_bounds__(256) void split_combine_kernel(const float* __restrict__ part, float v_scale,
                                                            float* __restrict__ out) {
  const int64_t row = blockIdx.x;
  const int hh = threadIdx.x >> 5, d = 4 * (threadIdx.x & 31);
  const float* p = part + row * SPLIT * kSplitPart;
  float ms[SPLIT], ls[SPLIT];
  float4 os[SPLIT];
#pragma unroll
  for (int s = 0; s < SPLIT; ++s) {
    ms[s] = p[s * kSplitPart + hh];
    ls[s] = p[s * kSplitPart + kHpg + hh];
    os[s] = *reinterpret_cast<const float4*>(p + s * kSplitPart + 2 * kHpg + hh * kDim + d);
  }
  float M = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < SPLIT; ++s) M = fmaxf(M, ms[s]);
  float den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s = 0; s < SPLIT; ++s) {
    const float w = ms[s] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(ms[s] - M);
    den += ls[s] * w;
    acc.x += os[s].x * w, acc.y += os[s].y * w, acc.z += os[s].z * w, acc.w += os[s].w * w;
  }
  const float inv = den > 0.f ? v_scale / den : 0.f;
  *reinterpret_cast<float4*>(out + (row * kHpg + hh) * kDim + d) =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

// Steps 3 (when SELECT) and 4 for one (request, group, row group); grid (groups x row groups, requests).
// WAVES per workgroup: 8 with one query tile; 4 with two, so that each wave can
// hold the doubled accumulators in registers (one wave per SIMD).
// FP8: FP8 caches (one E4M3 byte per element), else NVFP4.
// PREFILL (one query tile, 4 waves): one row per workgroup and one
// block per wave at a time (keys, then values once S = K Q^T is done), within
// 128 registers, so that four workgroups share a CU and hide each other's
// load latency -- the throughput form for chunks of thousands of rows, whose
// rows select independently (no union to share).
// RPW: rows per workgroup, 4 (the union of a row group) or 1 (each row on
// its own, more workgroups: used while the batch leaves CUs idle).
// SPLIT > 1 (one row per workgroup, while SPLIT workgroups per row still fit
// the CUs): workgroup s of a row takes union blocks s, s + SPLIT, ... and
// writes its softmax partial -- running max M, denominator l and unnormalised
// output O of each query row -- to part ([row][SPLIT][16 + 8 x 128] floats: M
// of the 8 heads, l of the 8 heads, O); split_combine_kernel merges them.
template <int QT, bool SELECT, int KMAX, int WAVES, bool FP8, int RPW, bool PREFILL = false, int SPLIT = 1>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(PREFILL ? 3 : 1))) void attend_kernel(
    const int32_t* __restrict__ table, const int32_t* __restrict__ lens, int32_t R, int32_t max_pages,
    const uint8_t* __restrict__ q, float qk2, float v_scale, const uint8_t* __restrict__ kpages,
    const uint8_t* __restrict__ vpages, int32_t num_pages, const float* __restrict__ block_scores,
    int32_t* __restrict__ sel, int32_t* __restrict__ cnt, int32_t topk, float* __restrict__ out,
    float* __restrict__ part) {
  static_assert(!PREFILL || (QT == 1 && WAVES == 4 && RPW == 1), "the prefill form: one tile, 4 waves, one row");
  static_assert(RPW == 1 || RPW == 4, "rows per workgroup: 1 or 4");
  static_assert(SPLIT == 1 || (RPW == 1 && QT == 1 && !PREFILL), "split rows: one row per workgroup");
  constexpr int NT = WAVES * 64;
  constexpr int NQ = QT * 16;  // query columns of the workgroup (rows nq.. are padding)
  __shared__ int s_tab[PREFILL ? 1 : kTabLds];
  __shared__ int s_rowsel[4 * MSA_MAX_TOPK];
  __shared__ int s_first[4 * MSA_MAX_TOPK];
  __shared__ int s_union[4 * MSA_MAX_TOPK];
  __shared__ int s_phys[4 * MSA_MAX_TOPK];
  __shared__ int s_nu;
  __shared__ float s_m[WAVES][NQ];
  __shared__ float s_l[WAVES][NQ];
  __shared__ float s_fac[WAVES][NQ];  // each wave's factor exp2(m_w - M) per query row
  __shared__ float s_inv[NQ];         // v_scale / denominator per query row
  __shared__ ScaleSlot s_slot[FP8 ? 1 : WAVES];  // NVFP4: scales of each wave's current block
  __shared__ SelectScratch s_sel[SELECT ? RPW : 1];  // selection scratch of waves 0..nr-1
  // each wave's rescaled output rows (half the rows at a time); rows padded by 4 floats so that
  // the 4-row stride of a wave's stores spreads over the banks instead of hitting the same 16
  __shared__ __align__(16) float s_o[WAVES][NQ / 2][kDim + 4];

  const int RG = (R + RPW - 1) / RPW;
  const int split = SPLIT > 1 ? (int)(blockIdx.x % SPLIT) : 0;
  const int g = (blockIdx.x / SPLIT) / RG, rg = (blockIdx.x / SPLIT) % RG;
  const int b = blockIdx.y;
  const int r0 = rg * RPW, nr = min(RPW, R - r0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, a = lane >> 4;

  // ---- loads that need no context length go first: this wave's selection
  // scores, the queries, the block-table row (staged in LDS when it fits)
  float sc[KMAX > 0 ? KMAX : 1];
  const int64_t row_id = ((int64_t)b * R + r0 + min(wave, nr - 1)) * kGroups + g;
  if (SELECT && wave < nr) load_row_scores<KMAX>(block_scores + row_id * max_pages, max_pages, lane, sc);
  h8 Q[QT][4];
  load_q<QT>(q, b, R, r0, nr, g, lane, Q);
  const int32_t* trow = table + (int64_t)b * max_pages;
  const bool tab_lds = !PREFILL && max_pages <= kTabLds;
  if (tab_lds) {
    constexpr int PER = kTabLds / NT;
    int tv[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) tv[i] = trow[min(tid + i * NT, max_pages - 1)];
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (tid + i * NT < max_pages) s_tab[tid + i * NT] = tv[i];
  }
  const int L = clamp_len(lens[b], max_pages);

  int nu;
  if (SELECT) {
    // ---- step 3: wave w selects for row r0 + w; the sets go to LDS and to the outputs
    if (wave < nr) {
      const int r = r0 + wave;
      const int p = L - R + r;
      const int nb = p < 0 ? 0 : p / kPage + 1;
      const float* srow_scores = block_scores + row_id * max_pages;
      int32_t* o = sel + row_id * topk;
      int* srow = s_rowsel + wave * topk;
      // the selection's outputs are written once per row, by split 0
      const int c = select_fast<KMAX>(sc, [&](int j) { return srow_scores[j]; }, nb, topk, lane, &s_sel[SELECT ? wave : 0],
                                      [&](int rank, int id) {
                                        srow[rank] = id;
                                        if (split == 0) o[rank] = id;
                                      });
      if (lane >= c && lane < topk) {
        srow[lane] = -1;
        if (split == 0) o[lane] = -1;
      }
      if (lane == 0 && split == 0) cnt[row_id] = c;
    }
    __syncthreads();
    nu = union_of_rows(s_rowsel, nr, topk, s_first, s_union, &s_nu);
  } else {
    nu = build_union(sel, cnt, b, g, R, r0, nr, topk, max_pages, s_rowsel, s_first, s_union, &s_nu);
  }
  // physical pages of the union blocks; -1 when the table entry is out of range
  for (int ui = tid; ui < nu; ui += NT) {
    const int j = s_union[ui];
    const int ph = (j >= 0 && j < max_pages) ? (tab_lds ? s_tab[j] : trow[j]) : -1;
    s_phys[ui] = (ph >= 0 && ph < num_pages) ? ph : -1;
  }
  __syncthreads();

  // this workgroup's share of the union: blocks split, split + SPLIT, ...
  const int nus = SPLIT > 1 ? (nu > split ? (nu - split + SPLIT - 1) / SPLIT : 0) : nu;
  auto U = [&](int i) { return SPLIT > 1 ? split + SPLIT * i : i; };

  AttnState<QT> st;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    st.m[qt] = -__builtin_inff();
    st.L[qt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) st.O[qt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  // visibility of block j to this lane's query columns
  auto block_lim = [&](int j, int (&lim)[QT]) {
    bool any_partial = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int rl = (qt * 16 + n) / kHpg;  // row within the row group
      int v = kPage - 1;                    // padding columns: never stored, left unmasked
      if (rl < nr)
        v = (nr == 1 || row_has_block(s_rowsel, rl, topk, j)) ? min(kPage - 1, L - R + r0 + rl - j * kPage) : -1;
      lim[qt] = v;
      any_partial |= v < kPage - 1;
    }
    return __any(any_partial) != 0;
  };
  constexpr int kSlab = FP8 ? kFp8Slab : kNvSlab;
  auto kslab = [&](int ph) { return kpages + ((int64_t)max(ph, 0) * kGroups + g) * kSlab; };
  auto vslab = [&](int ph) { return vpages + ((int64_t)max(ph, 0) * kGroups + g) * kSlab; };
  bool first = true;
  if constexpr (PREFILL) {
    // one block at a time: its keys, then its values once the keys are consumed
    for (int u = wave; u < nu; u += WAVES) {
      const int ph = s_phys[u];
      if (ph < 0) continue;
      std::conditional_t<FP8, KRegs8, KRegs> K;
      std::conditional_t<FP8, VRegs8, VRegs> V;
      load_k<false>(kslab(ph), lane, K);
      int lim[QT];
      const bool partial = block_lim(s_union[u], lim);
      // NVFP4 values load during the softmax; FP8 values (twice the
      // registers) once the scores are consumed
      auto ld_v = [&] { load_v<false>(vslab(ph), lane, V); };
      if constexpr (FP8)
        attend_block<QT, true>(K, V, Q, lim, partial, first, qk2, lane, &s_slot[0], st, NoOp{}, ld_v);
      else
        attend_block<QT, true>(K, V, Q, lim, partial, first, qk2, lane, &s_slot[wave], st, ld_v);
      first = false;
    }
  } else if constexpr (FP8) {
    // FP8 blocks are twice the register bytes of NVFP4 ones, so one block's
    // keys and values are held at a time, rolling: the next block's keys load
    // once this block's keys are consumed (after S = K Q^T), its values once
    // this block's P V is done
    KRegs8 K;
    VRegs8 V;
    if (wave < nus) {
      load_k(kslab(s_phys[U(wave)]), lane, K);
      load_v(vslab(s_phys[U(wave)]), lane, V);
    }
    for (int i = wave; i < nus; i += WAVES) {
      const int u = U(i);
      const int ph = s_phys[u];
      const int in = i + WAVES;
      auto next_k = [&]() {
        if (in < nus) load_k(kslab(s_phys[U(in)]), lane, K);
      };
      if (ph >= 0) {
        int lim[QT];
        const bool partial = block_lim(s_union[u], lim);
        attend_block<QT>(K, V, Q, lim, partial, first, qk2, lane, &s_slot[0], st, next_k);
        first = false;
      } else {
        next_k();
      }
      if (in < nus) load_v(vslab(s_phys[U(in)]), lane, V);
    }
  } else if (nus <= WAVES) {
    // at most one block per wave (a split row): its keys and values load
    // together, and no wave issues loads for a second block it does not have
    if (wave < nus && s_phys[U(wave)] >= 0) {
      const int u = U(wave);
      KRegs K;
      VRegs V;
      load_k(kslab(s_phys[u]), lane, K);
      load_v(vslab(s_phys[u]), lane, V);
      int lim[QT];
      const bool partial = block_lim(s_union[u], lim);
      attend_block<QT>(K, V, Q, lim, partial, first, qk2, lane, &s_slot[wave], st, [] {});
      first = false;
    }
  } else
  // blocks wave, wave + WAVES, ... of the union, two at a time: the second
  // block's keys load with the first block's, its values once the first
  // block's keys are consumed (register budget of two waves per SIMD)
  for (int i0 = wave; i0 < nus; i0 += 2 * WAVES) {
    const bool has1 = i0 + WAVES < nus;
    const int u0 = U(i0), u1 = U(i0 + WAVES);
    const int ph0 = s_phys[u0], ph1 = has1 ? s_phys[u1] : -1;
    KRegs K0, K1;
    VRegs V0, V1;
    load_k(kslab(ph0), lane, K0);
    load_v(vslab(ph0), lane, V0);
    load_k(kslab(ph1), lane, K1);  // page 0 stands in when there is no second block
    auto load_v1 = [&]() { load_v(vslab(ph1), lane, V1); };
    if (ph0 >= 0) {
      int lim[QT];
      const bool partial = block_lim(s_union[u0], lim);
      attend_block<QT>(K0, V0, Q, lim, partial, first, qk2, lane, &s_slot[wave], st, load_v1);
      first = false;
    } else {
      load_v1();
    }
    if (ph1 >= 0) {
      int lim[QT];
      const bool partial = block_lim(s_union[u1], lim);
      attend_block<QT>(K1, V1, Q, lim, partial, first, qk2, lane, &s_slot[wave], st, [] {});
      first = false;
    }
  }

  // ---- merge the waves: per query row, the common max, each wave's factor
  // and the reciprocal denominator once; then each wave stores its rows
  // scaled by its factor and every thread sums its outputs over the waves in a
  // fixed order (bitwise reproducible)
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    if (a == 0) s_m[wave][qt * 16 + n] = st.m[qt];
    if (n == 0)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) s_l[wave][qt * 16 + 4 * a + qq] = st.L[qt][qq];
  }
  __syncthreads();
  const int nq = nr * kHpg;
  if (tid < nq) {
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, s_m[w][tid]);
    float den = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float mw = s_m[w][tid];
      const float f = mw == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      s_fac[w][tid] = f;
      den += s_l[w][tid] * f;
    }
    s_inv[tid] = SPLIT > 1 ? 1.f : (den > 0.f ? v_scale / den : 0.f);
    if (SPLIT > 1) {  // this split's max and denominator of query row tid (row r0, head tid)
      float* pr = part + ((((int64_t)b * R + r0) * kGroups + g) * SPLIT + split) * kSplitPart;
      pr[tid] = M;
      pr[kHpg + tid] = den;
    }
  }
  __syncthreads();
  // the output rows go through LDS in two halves of NQ/2 rows (LDS budget)
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int q_lo = half * (NQ / 2);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int qi = qt * 16 + 4 * a + qq;
        if (qi >= q_lo && qi < q_lo + NQ / 2 && qi < nq) {
          const float f = s_fac[wave][qi];
#pragma unroll
          for (int nt = 0; nt < 8; ++nt) s_o[wave][qi - q_lo][16 * nt + n] = st.O[qt][nt][qq] * f;
        }
      }
    __syncthreads();
    const int rows = min(NQ / 2, nq - q_lo);
    for (int i = tid; i < rows * (kDim / 4); i += NT) {
      const int ql = i / (kDim / 4), d4 = i % (kDim / 4);
      const int qi = q_lo + ql;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float4 o4 = *reinterpret_cast<const float4*>(&s_o[w][ql][4 * d4]);
        acc.x += o4.x, acc.y += o4.y, acc.z += o4.z, acc.w += o4.w;
      }
      const float inv = s_inv[qi];
      const int r = r0 + qi / kHpg, hh = qi % kHpg;
      float* dst = SPLIT > 1 ? part + ((((int64_t)b * R + r) * kGroups + g) * SPLIT + split) * kSplitPart + 2 * kHpg +
                                   hh * kDim
                             : out + ((((int64_t)b * R + r) * kGroups + g) * kHpg + hh) * kDim;
      *reinterpret_cast<float4*>(dst + 4 * d4) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
    if (half == 0 && nq > NQ / 2) __syncthreads();  // s_o is rewritten for the second half
  }
}

// F32 caches (the tiny correctness configuration): one wave per union block.
__global__ __launch_bounds__(64) void decode_f32_kernel(
    const int32_t* __restrict__ table, const int32_t* __restrict__ lens, int32_t R, int32_t max_pages,
    const float* __restrict__ q, float sm_scale, const uint8_t* __restrict__ kpages,
    const uint8_t* __restrict__ vpages, int32_t num_pages, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ cnt, int32_t topk, float* __restrict__ part_o, float* __restrict__ part_ml,
    int32_t S) {
  __shared__ int s_rowsel[MSA_MAX_ROWS * MSA_MAX_TOPK];
  __shared__ int s_first[MSA_MAX_ROWS * MSA_MAX_TOPK];
  __shared__ int s_union[MSA_MAX_ROWS * MSA_MAX_TOPK];
  __shared__ int s_nu;
  __shared__ float s_p[MSA_MAX_ROWS * kHpg][kPage];
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int L = clamp_len(lens[b], max_pages);
  const int nu = build_union(sel, cnt, b, g, R, 0, R, topk, max_pages, s_rowsel, s_first, s_union, &s_nu);
  const int nq = R * kHpg;
  const int j = split < nu ? s_union[split] : -1;
  int phys = j >= 0 ? table[(int64_t)b * max_pages + j] : -1;
  if (phys >= num_pages) phys = -1;
  const int64_t base = (((int64_t)b * kGroups + g) * S + split) * (int64_t)nq;
  const float* K = phys >= 0 ? reinterpret_cast<const float*>(kpages + ((int64_t)phys * kGroups + g) * kF32Slab) : nullptr;
  const float* V = phys >= 0 ? reinterpret_cast<const float*>(vpages + ((int64_t)phys * kGroups + g) * kF32Slab) : nullptr;
  for (int qi = 0; qi < nq; ++qi) {
    const int r = qi / kHpg, hh = qi % kHpg;
    int lim = -1;
    if (phys >= 0 && row_has_block(s_rowsel, r, topk, j)) lim = min(kPage - 1, L - R + r - j * kPage);
    const float* qv = q + ((((int64_t)b * R + r) * kGroups + g) * kHpg + hh) * kDim;
    float mx = -__builtin_inff();
    for (int t = lane; t < kPage; t += 64) {
      float z = -__builtin_inff();
      if (t <= lim) {
        float s = 0.f;
        for (int d = 0; d < kDim; ++d) s = fmaf(qv[d], K[t * kDim + d], s);
        z = s * sm_scale;
      }
      s_p[qi][t] = z;
      mx = fmaxf(mx, z);
    }
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float sum = 0.f;
    for (int t = lane; t < kPage; t += 64) {
      const float z = s_p[qi][t];
      const float pz = (z == -__builtin_inff()) ? 0.f : __expf(z - mx);
      s_p[qi][t] = pz;
      sum += pz;
    }
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    __syncthreads();
    for (int d = lane; d < kDim; d += 64) {
      float acc = 0.f;
      if (phys >= 0)
        for (int t = 0; t <= lim; ++t) acc = fmaf(s_p[qi][t], V[t * kDim + d], acc);
      part_o[(base + qi) * kDim + d] = acc;
    }
    if (lane == 0) {
      part_ml[(base + qi) * 2] = mx;
      part_ml[(base + qi) * 2 + 1] = sum;
    }
    __syncthreads();
  }
}

// Merge the splits of each (request, group): out = sum_s e^(M_s - M) O_s / sum_s e^(M_s - M) L_s.
// One thread per output element; its split loads are independent of each other.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml, int32_t B, int32_t R,
                                                      int32_t S, float* __restrict__ out) {
  const int nq = R * kHpg;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)B * kGroups * nq * kDim) return;
  const int d = (int)(i % kDim);
  const int qi = (int)((i / kDim) % nq);
  const int g = (int)((i / ((int64_t)kDim * nq)) % kGroups);
  const int b = (int)(i / ((int64_t)kDim * nq * kGroups));
  const int64_t base = ((int64_t)b * kGroups + g) * S;
  float M = -__builtin_inff();
  for (int s = 0; s < S; ++s) M = fmaxf(M, part_ml[((base + s) * nq + qi) * 2]);
  float num = 0.f, den = 0.f;
  if (M != -__builtin_inff()) {
    for (int s = 0; s < S; ++s) {
      const float ms = part_ml[((base + s) * nq + qi) * 2];
      const float f = ms == -__builtin_inff() ? 0.f : __expf(ms - M);
      num = fmaf(f, part_o[((base + s) * nq + qi) * kDim + d], num);
      den = fmaf(f, part_ml[((base + s) * nq + qi) * 2 + 1], den);
    }
  }
  const int r = qi / kHpg, hh = qi % kHpg;
  out[((((int64_t)b * R + r) * kGroups + g) * kHpg + hh) * kDim + d] = den > 0.f ? num / den : 0.f;
}

}  // namespace msa

using namespace msa;

static size_t f32_splits(const msa_batch* bt, int32_t topk) {
  return (size_t)std::min(bt->rows_per_req * topk, bt->max_pages_per_req);
}

extern "C" size_t msa_decode_partials_bytes(const msa_batch* bt, int32_t topk) {
  const size_t S = f32_splits(bt, topk);
  const size_t q = (size_t)bt->num_reqs * kGroups * S * bt->rows_per_req * kHpg;
  return q * (kDim + 2) * sizeof(float);
}

// Compute units of the current device (the runtime answers from its cached
// device properties; 256, the MI355X's count, if it cannot).
static int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

// Workgroups per (request, row, group) of the NVFP4 / FP8 decode route: the
// attention is bound by the vector ALUs' dequantisation of the selected
// blocks, so a batch that leaves CUs idle with one workgroup per row spreads
// each row's blocks over 2 or 4 workgroups (the largest that still fits the
// CUs), whose partial results split_combine_kernel merges.
static int attend_splits(const msa_batch* bt) {
  const int R = bt->rows_per_req;
  if (R > MSA_MAX_ROWS) return 1;  // prefill chunks: thousands of rows already
  const int64_t rows = (int64_t)bt->num_reqs * R * kGroups;
  const int cus = cu_count();
  for (int S = kMaxSplit; S > 1; S /= 2)
    if (rows * S <= cus) return S;
  return 1;
}

extern "C" size_t msa_split_partials_bytes(const msa_batch* bt) {
  const int S = attend_splits(bt);
  if (S == 1) return 0;
  return (size_t)bt->num_reqs * bt->rows_per_req * kGroups * S * kSplitPart * sizeof(float);
}

// NVFP4 and FP8 route: one launch, selection fused in when block_scores != NULL,
// plus the merge of split rows when part != NULL and the batch splits.
template <bool SELECT, bool FP8>
static int launch_attend(const msa_batch* bt, const uint8_t* q, float q_scale, float sm_scale,
                         const msa_cache* kc, const msa_cache* vc, const float* block_scores, int32_t* sel,
                         int32_t* cnt, int32_t topk, float* out, float* part, size_t part_bytes, hipStream_t s) {
  const int R = bt->rows_per_req, P = bt->max_pages_per_req;
  // scores enter the kernel's softmax in base 2
  const float qk2 = sm_scale * kc->tensor_scale * q_scale * 1.4426950408889634f;
  const int km = SELECT ? select_kmax(P) : 8;
  const size_t block_bytes = msa_prefill_block_bytes(bt, topk);
  if (R > MSA_MAX_ROWS && part && block_bytes > 0 && part_bytes >= block_bytes) {
    // prefill chunk with room for the block-major partials: the selection first
    // (when fused), then each selected block once for all the rows that chose it
    if (SELECT && msa_launch_topk(bt, block_scores, 0, topk, sel, cnt, s) != 0) return -1;
    return msa_launch_prefill_block_attend(bt, q, q_scale, sm_scale, kc, vc, sel, cnt, topk, out, part, s);
  }
  if (R > MSA_MAX_ROWS) {  // prefill chunk: one row per workgroup
    const dim3 pgrid(kGroups * R, bt->num_reqs);
#define MSA_PREFILL(K)                                                                                          \
  hipLaunchKernelGGL((attend_kernel<1, SELECT, K, 4, FP8, 1, true>), pgrid, dim3(256), 0, s, bt->block_table,     \
                     bt->ctx_lens, R, P, q, qk2, vc->tensor_scale, (const uint8_t*)kc->pages,                     \
                     (const uint8_t*)vc->pages, kc->num_pages, block_scores, sel, cnt, topk, out, nullptr)
    switch (km) {  // 48 candidates per lane do not fit the prefill form's registers: read them on demand
      case 8: MSA_PREFILL(8); break;
      case 24: MSA_PREFILL(24); break;
      default: MSA_PREFILL(0); break;
    }
#undef MSA_PREFILL
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  // Several rows per request: one workgroup per row while that grid does not
  // exceed the CU count (a small batch, latency-bound: rows that select
  // independently share few blocks, so a row group's union is nearly R times
  // one row's work on one CU); beyond it, one workgroup per group of up to 4
  // rows walking the union of their sets (rows that select alike share the
  // reads and the dequantisation).
  const bool per_row = R == 1 || (int64_t)bt->num_reqs * R * kGroups <= cu_count();
  const int S = part ? attend_splits(bt) : 1;
#define MSA_ATTEND(QT, K, RPW, SPLIT)                                                                           \
  hipLaunchKernelGGL((attend_kernel<QT, SELECT, K, (QT == 1 ? 8 : 4), FP8, RPW, false, SPLIT>),                  \
                     dim3(kGroups * ((R + RPW - 1) / RPW) * SPLIT, bt->num_reqs), dim3((QT == 1 ? 8 : 4) * 64), 0, \
                     s, bt->block_table, bt->ctx_lens, R, P, q, qk2, vc->tensor_scale, (const uint8_t*)kc->pages,  \
                     (const uint8_t*)vc->pages, kc->num_pages, block_scores, sel, cnt, topk, out, part)
#define MSA_ATTEND_K(QT, RPW, SPLIT)           \
  switch (km) {                                \
    case 8: MSA_ATTEND(QT, 8, RPW, SPLIT); break;   \
    case 24: MSA_ATTEND(QT, 24, RPW, SPLIT); break; \
    case 48: MSA_ATTEND(QT, 48, RPW, SPLIT); break; \
    default: MSA_ATTEND(QT, 0, RPW, SPLIT); break;  \
  }
  if (per_row && S == 4) {
    MSA_ATTEND_K(1, 1, 4)
  } else if (per_row && S == 2) {
    MSA_ATTEND_K(1, 1, 2)
  } else if (per_row) {
    MSA_ATTEND_K(1, 1, 1)
  } else if (R <= 2) {
    MSA_ATTEND_K(1, 4, 1)
  } else {
    MSA_ATTEND_K(2, 4, 1)
  }
#undef MSA_ATTEND_K
#undef MSA_ATTEND
  if (hipGetLastError() != hipSuccess) return -1;
  if (S > 1) {
    const dim3 cgrid((unsigned)((int64_t)bt->num_reqs * R * kGroups));
    if (S == 4)
      hipLaunchKernelGGL(split_combine_kernel<4>, cgrid, dim3(256), 0, s, part, vc->tensor_scale, out);
    else
      hipLaunchKernelGGL(split_combine_kernel<2>, cgrid, dim3(256), 0, s, part, vc->tensor_scale, out);
    if (hipGetLastError() != hipSuccess) return -1;
  }
  return 0;
}

extern "C" int msa_launch_sparse_decode(const msa_batch* bt, const void* q, int32_t q_dtype, float q_scale,
                                        float sm_scale, const msa_cache* kc, const msa_cache* vc,
                                        const int32_t* sel, const int32_t* cnt, int32_t topk, float* out,
                                        void* workspace, size_t workspace_bytes, hipStream_t s) {
  const int B = bt->num_reqs, R = bt->rows_per_req, P = bt->max_pages_per_req;
  if (kc->dtype == MSA_NVFP4)
    return launch_attend<false, false>(bt, (const uint8_t*)q, q_scale, sm_scale, kc, vc, nullptr, (int32_t*)sel,
                                       (int32_t*)cnt, topk, out, (float*)workspace, workspace_bytes, s);
  if (kc->dtype == MSA_FP8_E4M3)
    return launch_attend<false, true>(bt, (const uint8_t*)q, q_scale, sm_scale, kc, vc, nullptr, (int32_t*)sel,
                                      (int32_t*)cnt, topk, out, (float*)workspace, workspace_bytes, s);
  const int S = (int)f32_splits(bt, topk);
  float* part_o = (float*)workspace;
  float* part_ml = part_o + (size_t)B * kGroups * S * R * kHpg * kDim;
  hipLaunchKernelGGL(decode_f32_kernel, dim3(S, kGroups, B), dim3(64), 0, s, bt->block_table, bt->ctx_lens, R, P,
                     (const float*)q, sm_scale, (const uint8_t*)kc->pages, (const uint8_t*)vc->pages, kc->num_pages,
                     sel, cnt, topk, part_o, part_ml, S);
  if (hipGetLastError() != hipSuccess) return -1;
  const int64_t total = (int64_t)B * kGroups * R * kHpg * kDim;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part_o, part_ml, B, R, S,
                     out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---------------------------------------------------------------- allocation-free variant
// msa_sparse_decode_noalloc keeps the F32 route's per-block partial results in
// this file-scope array instead of a caller workspace.  Each GPU the library
// runs on holds its own copy until the process ends.  In host code `scratch`
// is only a stand-in name; the array's device address on each device comes
// from hipGetSymbolAddress, taken once per device (on the first call with that
// device current) and used for every kernel argument.
static __device__ __align__(256) unsigned char scratch[MSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_addr[kMaxDevices];

extern "C" int msa_launch_sparse_decode_noalloc(const msa_batch* bt, const void* q, int32_t q_dtype, float q_scale,
                                                float sm_scale, const msa_cache* kc, const msa_cache* vc,
                                                const int32_t* sel, const int32_t* cnt, int32_t topk, float* out,
                                                hipStream_t s) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  void* ptr = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return -1;
    g_scratch_addr[dev].store(ptr, std::memory_order_release);
  }
  return msa_launch_sparse_decode(bt, q, q_dtype, q_scale, sm_scale, kc, vc, sel, cnt, topk, out, ptr,
                                  MSA_NOALLOC_SCRATCH_BYTES, s);
}

extern "C" int msa_launch_select_decode(const msa_batch* bt, const float* block_scores, int32_t topk,
                                        const void* q, float q_scale, float sm_scale, const msa_cache* kc,
                                        const msa_cache* vc, int32_t* sel, int32_t* cnt, float* out,
                                        void* workspace, size_t workspace_bytes, hipStream_t s) {
  if (kc->dtype == MSA_FP8_E4M3)
    return launch_attend<true, true>(bt, (const uint8_t*)q, q_scale, sm_scale, kc, vc, block_scores, sel, cnt, topk,
                                     out, (float*)workspace, workspace_bytes, s);
  return launch_attend<true, false>(bt, (const uint8_t*)q, q_scale, sm_scale, kc, vc, block_scores, sel, cnt, topk,
                                    out, (float*)workspace, workspace_bytes, s);
}
