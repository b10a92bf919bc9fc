// msa_attn.hip -- step 4: exact GQA softmax attention over the selected
// blocks (vLLM M3.1 post, "MiniMax 稀疏注意力的工作原理"; spke.com "MSA入門"
// Fig. 1 caption; "MiniMax goes sparse", section 1 Step 2: every query head
// of a group attends to the group's selected blocks), alone or fused with
// step 3 (the selection) in one launch.
//
// Work split (NVFP4): one workgroup of 8 waves (4 with two query tiles) per
// (request, group, group of up to 4 rows).  The waves walk the union of the rows' selected blocks,
// one 128-token block at a time, each keeping an online softmax (running
// max, denominator, unnormalised output); the waves merge through LDS and the
// workgroup writes the normalised output -- no partial results leave the
// chip and no second launch merges them.  With the selection fused in, waves
// 0..nr-1 first run the top-k of one row each (msa_select.h) from the block
// scores.  With one row per request, the 8 heads of a group share each
// dequantised K/V element (GQA); with 4 speculative rows the 32 query vectors
// of a group fill two 16-column query tiles.
//
// Per block and wave:
//  * S^T = K Q^T on v_mfma_f32_16x16x32_f16.  K codes go through the exact
//    E2M1->FP16 conversion and one packed FP16 multiply by their E4M3 scale
//    (E2M1 x E4M3 has at most 6 significant bits, so the product is exact);
//    the K tensor scale, the query scale and sm_scale are applied to the FP32
//    accumulators.  Queries (E4M3) are exact in FP16 as well.
//  * The 16 rows of M-tile m are tokens 32*(m/2) + 8*(i/4) + 4*(m%2) + i%4,
//    so that the accumulator rows a lane holds are 8 consecutive tokens per
//    32-token step: they are then already the P operand of the P.V product,
//    with no shuffle through LDS.
//  * P is rounded to FP16 (FP32 accumulation); V comes from the dim-major
//    value slab, where the 8 tokens of one dim that a P.V operand lane needs
//    are one dword, scaled per token by the E4M3 group scale in FP16.
//  * K and V are read with non-temporal loads (each selected block is read
//    once per step).
#include <algorithm>

#include "msa_device.h"
#include "msa_kernels.h"
#include "msa_select.h"

namespace msa {


// Sorted union of the sets already in s_rowsel (nr rows of topk ids, -1 padded).
__device__ int union_of_rows(const int* s_rowsel, int nr, int topk, int* s_first, int* s_union, int* s_nu) {
  const int tid = threadIdx.x;
  const int N = nr * topk;
  if (nr == 1) {
    if (tid == 0) {
      int n = 0;
      while (n < topk && s_rowsel[n] >= 0) ++n;
      *s_nu = n;
    }
    for (int i = tid; i < topk; i += blockDim.x) s_union[i] = s_rowsel[i];
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
// form the sorted union in LDS.  Returns the union size.
__device__ int build_union(const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt, int b, int g, int R,
                           int r0, int nr, int topk, int max_pages, int* s_rowsel, int* s_first, int* s_union,
                           int* s_nu) {
  const int N = nr * topk;
  for (int i = threadIdx.x; i < N; i += blockDim.x) {
    const int r = r0 + i / topk, k = i % topk;
    const int64_t row = ((int64_t)b * R + r) * kGroups + g;
    int v = k < cnt[row] ? sel[row * topk + k] : -1;
    if (v >= max_pages) v = -1;
    s_rowsel[i] = v;
  }
  __syncthreads();
  return union_of_rows(s_rowsel, nr, topk, s_first, s_union, s_nu);
}

__device__ __forceinline__ bool row_has_block(const int* s_rowsel, int rl, int topk, int j) {
  for (int k = 0; k < topk; ++k)
    if (s_rowsel[rl * topk + k] == j) return true;
  return false;
}

// Running softmax state of one wave over QT query tiles of 16 columns.
template <int QT>
struct AttnState {
  float m[QT];   // running max of query column n = lane%16 (same in its 4 lanes)
  float l[QT];   // running denominator, same layout
  v4f O[QT][8];  // unnormalised output: rows 4*(lane/16)+q (queries), dims 16*nt + lane%16
};

typedef unsigned int u4v __attribute__((ext_vector_type(4)));
typedef unsigned int u2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 nt_load4(const uint8_t* p) {
  const u4v v = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t nt_load1(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const unsigned int*>(p));
}

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
      const uint2 w = ok ? *reinterpret_cast<const uint2*>(qrow + 32 * a + 8 * ks) : make_uint2(0, 0);
      const h2 x0 = e4m3x2_to_h2<false>(w.x), x1 = e4m3x2_to_h2<true>(w.x);
      const h2 x2 = e4m3x2_to_h2<false>(w.y), x3 = e4m3x2_to_h2<true>(w.y);
      Q[qt][ks] = h8{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
    }
  }
}

// One 128-token block: S^T = K Q^T, online-softmax update of `st`, O += P V.
// lim[qt]: last visible token of the block for this lane's query column (-1: none).
template <int QT>
__device__ __forceinline__ void attend_block(const uint8_t* __restrict__ ks_, const uint8_t* __restrict__ vs_,
                                             const h8 (&Q)[QT][4], const int (&lim)[QT], float qk_scale, int lane,
                                             uint4* vsc_slot, AttnState<QT>& st) {
  const int n = lane & 15, a = lane >> 4;
  // ---- every load of the block up front: K codes + scales, V codes, V scales
  uint4 kc[8];
  uint32_t ksc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int tok = 32 * (m >> 1) + 8 * (n >> 2) + 4 * (m & 1) + (n & 3);
    kc[m] = nt_load4(ks_ + tok * 64 + 16 * a);
    ksc[m] = *reinterpret_cast<const uint16_t*>(ks_ + kScaleOff + tok * 8 + 2 * a);
  }
  uint32_t vw[8][4];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) vw[nt][kk] = nt_load1(vs_ + (16 * nt + n) * 64 + 16 * kk + 4 * a);
  const uint4 vsc_regs = nt_load4(vs_ + kScaleOff + 16 * lane);

  // ---- S^T = K Q^T
  v4f Sacc[QT][8];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int m = 0; m < 8; ++m) Sacc[qt][m] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const h2 sc = e4m3x2_to_h2<false>(ksc[m]);
    const uint32_t words[4] = {kc[m].x, kc[m].y, kc[m].z, kc[m].w};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const _Float16 s = ks < 2 ? sc[0] : sc[1];
      h8 kv = e2m1x8_to_h8(words[ks]);
      const h8 sv = h8{s, s, s, s, s, s, s, s};
      kv = kv * sv;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        Sacc[qt][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, Q[qt][ks], Sacc[qt][m], 0, 0, 0);
    }
  }

  // ---- online softmax (token of Sacc[qt][m][q] = 32(m/2) + 8a + 4(m%2) + q)
  h8 P[QT][4];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float mx = -__builtin_inff();
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int tok = 32 * (m >> 1) + 8 * a + 4 * (m & 1) + qq;
        float z = Sacc[qt][m][qq] * qk_scale;
        z = tok <= lim[qt] ? z : -__builtin_inff();
        Sacc[qt][m][qq] = z;
        mx = fmaxf(mx, z);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m[qt], mx);
    const float alpha = st.m[qt] == -__builtin_inff() ? 0.f : __expf(st.m[qt] - m_new);
    float sum = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      h8 pk;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int m = 2 * kk + (e >> 2), qq = e & 3;
        const float z = Sacc[qt][m][qq];
        const float pz = z == -__builtin_inff() ? 0.f : __expf(z - m_new);
        sum += pz;
        pk[e] = (_Float16)pz;
      }
      P[qt][kk] = pk;
    }
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    st.l[qt] = alpha * st.l[qt] + sum;
    st.m[qt] = m_new;
    // rescale the output rows this lane holds (queries 4a + q live in lanes 4a + q as columns)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const float aq = __shfl(alpha, 4 * a + qq);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) st.O[qt][nt][qq] *= aq;
    }
  }

  // ---- O += P V (dims d = 16 nt + n; V operand: 8 tokens 32kk + 8a.. of dim d).
  // The block's 1 KB of value scales goes through this wave's LDS slot: each
  // lane needs 8 scale bytes loaded by another lane of the same wave.
  vsc_slot[lane] = vsc_regs;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint8_t* vsc = reinterpret_cast<const uint8_t*>(vsc_slot);
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      h8 vv = e2m1x8_to_h8(vw[nt][kk]);
      const uint2 sw = *reinterpret_cast<const uint2*>(vsc + nt * kPage + 32 * kk + 8 * a);
      const h2 s0 = e4m3x2_to_h2<false>(sw.x), s1 = e4m3x2_to_h2<true>(sw.x);
      const h2 s2 = e4m3x2_to_h2<false>(sw.y), s3 = e4m3x2_to_h2<true>(sw.y);
      const h8 sv = h8{s0[0], s0[1], s1[0], s1[1], s2[0], s2[1], s3[0], s3[1]};
      vv = vv * sv;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        st.O[qt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P[qt][kk], vv, st.O[qt][nt], 0, 0, 0);
    }
  }
  // the slot is rewritten by this wave's next block: keep those stores behind these reads
  __builtin_amdgcn_wave_barrier();
}

// Steps 3 (when SELECT) and 4 for one (request, group, row group); grid (groups x row groups, requests).
// WAVES per workgroup: 8 with one query tile; 4 with two, so that each wave can
// hold the doubled accumulators in registers (one wave per SIMD).
template <int QT, bool SELECT, int KMAX, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void attend_nvfp4_kernel(
    const int32_t* __restrict__ table, const int32_t* __restrict__ lens, int32_t R, int32_t max_pages,
    const uint8_t* __restrict__ q, float qk_scale, float v_scale, const uint8_t* __restrict__ kpages,
    const uint8_t* __restrict__ vpages, int32_t num_pages, const float* __restrict__ block_scores,
    int32_t* __restrict__ sel, int32_t* __restrict__ cnt, int32_t topk, float* __restrict__ out) {
  __shared__ int s_rowsel[4 * MSA_MAX_TOPK];
  __shared__ int s_first[4 * MSA_MAX_TOPK];
  __shared__ int s_union[4 * MSA_MAX_TOPK];
  __shared__ int s_nu;
  __shared__ float s_m[WAVES][QT * 16];
  __shared__ float s_l[WAVES][QT * 16];
  __shared__ float s_o[QT * 16][kDim];
  __shared__ uint4 s_vsc[WAVES][64];  // value scales of each wave's current block

  const int RG = (R + 3) / 4;
  const int g = blockIdx.x / RG, rg = blockIdx.x % RG;
  const int b = blockIdx.y;
  const int r0 = rg * 4, nr = min(4, R - r0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, a = lane >> 4;
  const int L = clamp_len(lens[b], max_pages);

  int nu;
  if (SELECT) {
    // ---- step 3: wave w selects for row r0 + w; the sets go to LDS and to the outputs
    if (wave < nr) {
      const int r = r0 + wave;
      const int p = L - R + r;
      const int nb = p < 0 ? 0 : p / kPage + 1;
      const int64_t row_id = ((int64_t)b * R + r) * kGroups + g;
      int32_t* o = sel + row_id * topk;
      int* srow = s_rowsel + wave * topk;
      const int c = select_row<false, KMAX>(block_scores + row_id * max_pages, nb, p, topk, lane,
                                            [&](int rank, int id) {
                                              srow[rank] = id;
                                              o[rank] = id;
                                            });
      if (lane >= c && lane < topk) {
        srow[lane] = -1;
        o[lane] = -1;
      }
      if (lane == 0) cnt[row_id] = c;
    }
    __syncthreads();
    nu = union_of_rows(s_rowsel, nr, topk, s_first, s_union, &s_nu);
  } else {
    nu = build_union(sel, cnt, b, g, R, r0, nr, topk, max_pages, s_rowsel, s_first, s_union, &s_nu);
  }

  AttnState<QT> st;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    st.m[qt] = -__builtin_inff();
    st.l[qt] = 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) st.O[qt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  if (wave < nu) {
    h8 Q[QT][4];
    load_q<QT>(q, b, R, r0, nr, g, lane, Q);
    for (int ui = wave; ui < nu; ui += WAVES) {
      const int j = s_union[ui];
      int phys = table[(int64_t)b * max_pages + j];
      if (phys < 0 || phys >= num_pages) continue;
      int lim[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int rl = (qt * 16 + n) / kHpg;  // row within the row group
        int v = -1;
        if (rl < nr && (nr == 1 || row_has_block(s_rowsel, rl, topk, j))) v = min(kPage - 1, L - R + r0 + rl - j * kPage);
        lim[qt] = v;
      }
      attend_block<QT>(kpages + ((int64_t)phys * kGroups + g) * kNvSlab,
                       vpages + ((int64_t)phys * kGroups + g) * kNvSlab, Q, lim, qk_scale, lane, &s_vsc[wave][0], st);
    }
  }

  // ---- merge the waves through LDS, one wave after the other (fixed order:
  // bitwise reproducible), then normalise and store
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
    if (a == 0) {
      s_m[wave][qt * 16 + n] = st.m[qt];
      s_l[wave][qt * 16 + n] = st.l[qt];
    }
  __syncthreads();
  float fac[QT][4];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int qi = qt * 16 + 4 * a + qq;  // O row held by this lane
      float M = -__builtin_inff();
#pragma unroll
      for (int w = 0; w < WAVES; ++w) M = fmaxf(M, s_m[w][qi]);
      const float mine = s_m[wave][qi];
      fac[qt][qq] = mine == -__builtin_inff() ? 0.f : __expf(mine - M);
    }
  for (int w = 0; w < WAVES; ++w) {
    if (wave == w) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
          for (int nt = 0; nt < 8; ++nt) {
            float* dst = &s_o[qt * 16 + 4 * a + qq][16 * nt + n];
            const float val = st.O[qt][nt][qq] * fac[qt][qq];
            *dst = (w == 0) ? val : *dst + val;
          }
    }
    __syncthreads();
  }
  const int nq = nr * kHpg;
  for (int i = tid; i < nq * (kDim / 4); i += WAVES * 64) {
    const int qi = i / (kDim / 4), d4 = i % (kDim / 4);
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, s_m[w][qi]);
    float den = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w)
      if (s_m[w][qi] != -__builtin_inff()) den += s_l[w][qi] * __expf(s_m[w][qi] - M);
    const float inv = den > 0.f ? v_scale / den : 0.f;
    const float4 o4 = *reinterpret_cast<const float4*>(&s_o[qi][4 * d4]);
    const int r = r0 + qi / kHpg, hh = qi % kHpg;
    *reinterpret_cast<float4*>(&out[((((int64_t)b * R + r) * kGroups + g) * kHpg + hh) * kDim + 4 * d4]) =
        make_float4(o4.x * inv, o4.y * inv, o4.z * inv, o4.w * inv);
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

// NVFP4 route: one launch, selection fused in when block_scores != NULL.
template <bool SELECT>
static int launch_attend_nvfp4(const msa_batch* bt, const uint8_t* q, float q_scale, float sm_scale,
                               const msa_cache* kc, const msa_cache* vc, const float* block_scores, int32_t* sel,
                               int32_t* cnt, int32_t topk, float* out, hipStream_t s) {
  const int R = bt->rows_per_req, P = bt->max_pages_per_req;
  const int RG = (R + 3) / 4;
  const float qk_scale = sm_scale * kc->tensor_scale * q_scale;
  const dim3 grid(kGroups * RG, bt->num_reqs);
#define MSA_ATTEND(QT, K)                                                                                      \
  hipLaunchKernelGGL((attend_nvfp4_kernel<QT, SELECT, K, (QT == 1 ? 8 : 4)>), grid, dim3((QT == 1 ? 8 : 4) * 64), \
                     0, s, bt->block_table, bt->ctx_lens, R, P, q, qk_scale, vc->tensor_scale,                   \
                     (const uint8_t*)kc->pages, (const uint8_t*)vc->pages, kc->num_pages, block_scores, sel, cnt,  \
                     topk, out)
  const int km = SELECT ? select_kmax(P) : 8;
  if (R <= 2) {
    switch (km) {
      case 8: MSA_ATTEND(1, 8); break;
      case 24: MSA_ATTEND(1, 24); break;
      case 48: MSA_ATTEND(1, 48); break;
      default: MSA_ATTEND(1, 0); break;
    }
  } else {
    switch (km) {
      case 8: MSA_ATTEND(2, 8); break;
      case 24: MSA_ATTEND(2, 24); break;
      case 48: MSA_ATTEND(2, 48); break;
      default: MSA_ATTEND(2, 0); break;
    }
  }
#undef MSA_ATTEND
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int msa_launch_sparse_decode(const msa_batch* bt, const void* q, int32_t q_dtype, float q_scale,
                                        float sm_scale, const msa_cache* kc, const msa_cache* vc,
                                        const int32_t* sel, const int32_t* cnt, int32_t topk, float* out,
                                        void* workspace, hipStream_t s) {
  const int B = bt->num_reqs, R = bt->rows_per_req, P = bt->max_pages_per_req;
  if (kc->dtype == MSA_NVFP4)
    return launch_attend_nvfp4<false>(bt, (const uint8_t*)q, q_scale, sm_scale, kc, vc, nullptr, (int32_t*)sel,
                                      (int32_t*)cnt, topk, out, s);
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

extern "C" int msa_launch_select_decode(const msa_batch* bt, const float* block_scores, int32_t topk,
                                        const void* q, float q_scale, float sm_scale, const msa_cache* kc,
                                        const msa_cache* vc, int32_t* sel, int32_t* cnt, float* out,
                                        hipStream_t s) {
  return launch_attend_nvfp4<true>(bt, (const uint8_t*)q, q_scale, sm_scale, kc, vc, block_scores, sel, cnt, topk,
                                   out, s);
}
