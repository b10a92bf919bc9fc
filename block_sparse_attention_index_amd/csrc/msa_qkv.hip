// msa_qkv.hip -- the projection that produces a step's new rows, fused with
// their norm, rotary embedding and quantisation into the caches (vLLM M3.1
// post, "QKV GEMM + norm + RoPE + KV insert fusion": the epilogue takes the
// FP32 accumulators head by head, normalises and rotates the queries and
// index queries, quantises K, V and the index key to NVFP4 and writes them
// into their pages, so the projected rows never go to HBM).
//
// The pages give neither the model width nor the norm and rotary details;
// this kernel takes the plain reading: per-head RMS norm with a learned
// weight per dim (one weight vector per head kind), then rotate-half rotary
// embedding of dims (i, i + 64) by the caller's cos/sin table row at the
// token's position -- applied to queries, keys, index queries and the index
// key; values are stored as projected.
//
// Output columns: 45 heads of 128 -- 32 query heads, 4 key heads, 4 value
// heads, 4 index queries (one per group), 1 index key.  One workgroup of 16
// waves computes one head for 64 tokens (16 for a call of at most 64 rows):
//  * GEMM on v_mfma_f32_16x16x32_bf16.  Each lane's operand is 8 consecutive
//    k of one row: one 16-byte load.  x [n][hidden] is row-major; the weights
//    come in 32-k blocks, w[head][k/32][row][k%32], so a wave's operand for 16
//    rows is one contiguous 1 KB and a head's weights one contiguous range (in
//    the plain [column][hidden] layout a wave touches 16 rows a hidden row
//    apart, and the stream ran at about 1 TB/s).  Wave w takes 32 columns
//    (w % 4) over a quarter of the hidden dimension (w / 4); the quarters are
//    summed through one LDS tile in four rounds.
//  * Epilogue: each wave takes 1/16 of the tokens; lane l holds dims l and
//    l + 64, which is both a rotary pair and, per 16-lane row, two NVFP4
//    groups (the insert's row quantiser and store).
#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf8 load_bf8(const uint16_t* p) {
  return __builtin_bit_cast(bf8, *reinterpret_cast<const uint4*>(p));
}

// U k-steps of loads, then their products (all loads issue before the first product waits).
template <int MT, int U>
__device__ __forceinline__ void qkv_ksteps(const uint16_t* const (&wp)[2], const uint16_t* const (&xp)[MT], int k,
                                           int mts, v4f (&acc)[MT][2]) {
  bf8 bw[U][2], bx[U][MT];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) bw[u][nt] = load_bf8(wp[nt] + (int64_t)(k + 32 * u) * kDim);
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      if (mt < mts) bx[u][mt] = load_bf8(xp[mt] + k + 32 * u);
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      if (mt < mts)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bx[u][mt], bw[u][nt], acc[mt][nt], 0, 0, 0);
}

// MT: 16-token tiles per workgroup -- 4 (64 tokens) for a prompt chunk, 1
// for a decode step's few rows: a workgroup per (head, 16 rows) puts more CUs
// on the weight stream (each CU sustains only part of it) and leaves each
// wave one token of the epilogue; the extra weight reads of the other token
// tiles hit the caches.
template <int MT>
__global__ __launch_bounds__(1024) void qkv_insert_kernel(QkvArgs A) {
  constexpr int kTok = 16 * MT;
  __shared__ float tile[kTok][kDim + 4];
  const int head = blockIdx.x;  // heads fastest: the workgroups in flight share a few token tiles
  const int t0 = blockIdx.y * kTok;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, a = lane >> 4;
  const int cg = wave & 3, kq = wave >> 2;
  const int mts = min(MT, (A.n - t0 + 15) / 16);  // token tiles of 16 holding real tokens (uniform)

  // ---- GEMM: acc[mt][nt][i] = out[t0 + 16 mt + 4a + i][32 cg + 16 nt + n] over this wave's k quarter
  v4f acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
  const int kl = A.hidden / 4;  // a multiple of 64 (hidden: of 256)
  const int kb = kq * kl + 8 * a;
  // weights in 32-k blocks: w[head][k / 32][row][k % 32], so that a k-step of 16 rows is one 1 KB run
  const uint16_t* wp[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
    wp[nt] = A.w + ((int64_t)head * A.hidden + (kb - 8 * a)) * kDim + (32 * cg + 16 * nt + n) * 32 + 8 * a;
  const uint16_t* xp[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xp[mt] = A.x + (int64_t)min(t0 + 16 * mt + n, A.n - 1) * A.hidden + kb;
  constexpr int U = MT == 1 ? 8 : 2;
  int k = 0;
  for (; k + 32 * U <= kl; k += 32 * U) qkv_ksteps<MT, U>(wp, xp, k, mts, acc);
  for (; k < kl; k += 64) qkv_ksteps<MT, 2>(wp, xp, k, mts, acc);
  // ---- sum the four k quarters into the tile
  for (int q = 0; q < 4; ++q) {
    if (kq == q)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (mt < mts)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float& c = tile[16 * mt + 4 * a + i][32 * cg + 16 * nt + n];
              c = q == 0 ? acc[mt][nt][i] : c + acc[mt][nt][i];
            }
    __syncthreads();
  }
  // ---- epilogue, one token per wave at a time
  // head kinds: 0 query, 1 key, 2 value, 3 index query, 4 index key
  const int kind = head < 32 ? 0 : head < 36 ? 1 : head < 40 ? 2 : head < 44 ? 3 : 4;
  const int sub = kind == 0 ? head : kind == 1 ? head - 32 : kind == 2 ? head - 36 : kind == 3 ? head - 40 : 0;
  const int gsel = kind == 0 ? 0 : kind == 1 ? 1 : kind == 3 ? 2 : 3;  // norm weight row
  float g_lo = 0.f, g_hi = 0.f;
  if (kind != 2) {
    g_lo = A.norm_weight[gsel * kDim + lane];
    g_hi = A.norm_weight[gsel * kDim + 64 + lane];
  }
  for (int r = 0; r < MT; ++r) {
    const int tl = wave * MT + r;
    const int tok = t0 + tl;
    if (tok >= A.n) break;
    const int p = A.pos[tok];
    if (p < 0 || p >= A.rope_rows) continue;  // no rotation for this token: nothing of it is written
    float lo = tile[tl][lane], hi = tile[tl][64 + lane];
    if (kind != 2) {
      // RMS norm: sum of squares over the head's 128 values (every lane gets it)
      float ss = lo * lo + hi * hi;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
      const float inv = 1.0f / sqrtf(ss / (float)kDim + A.eps);
      const float ylo = lo * inv * g_lo, yhi = hi * inv * g_hi;
      const float c = A.rope[(int64_t)p * kDim + lane], s = A.rope[(int64_t)p * kDim + 64 + lane];
      lo = ylo * c - yhi * s;
      hi = yhi * c + ylo * s;
    }
    if (A.pre) {
      float* pr = A.pre + ((int64_t)tok * MSA_QKV_HEADS + head) * kDim;
      pr[lane] = lo;
      pr[64 + lane] = hi;
    }
    if (kind == 0 || kind == 3) {
      uint8_t* q = kind == 0 ? A.q_out + ((int64_t)tok * 32 + sub) * kDim : A.qidx_out + ((int64_t)tok * 4 + sub) * kDim;
      q[lane] = (uint8_t)e4m3_encode(lo / A.q_scale);
      q[64 + lane] = (uint8_t)e4m3_encode(hi / A.q_scale);
      continue;
    }
    uint8_t* pages = kind == 1 ? A.kpages : kind == 2 ? A.vpages : A.ipages;
    const int np = kind == 1 ? A.knp : kind == 2 ? A.vnp : A.inp;
    const int heads = kind == 4 ? 1 : kGroups;
    const float ts = kind == 1 ? A.kts : kind == 2 ? A.vts : A.its;
    const int64_t slot = A.slots[tok];
    const bool valid = slot >= 0 && slot < (int64_t)np * kPage;
    uint8_t* slab = pages + ((valid ? slot >> 7 : 0) * heads + sub) * (int64_t)kNvSlab;
    const int off = (int)(slot & (kPage - 1));
    uint32_t code;
    uint32_t sc = nvfp4_row_quantize(lo, ts, code);
    nvfp4_row_store(slab, off, a, n, code, sc, kind == 2, valid);
    sc = nvfp4_row_quantize(hi, ts, code);
    nvfp4_row_store(slab, off, 4 + a, n, code, sc, kind == 2, valid);
  }
}

}  // namespace msa

using namespace msa;

extern "C" int msa_launch_qkv_insert(const QkvArgs* args, hipStream_t stream) {
  if (args->n == 0) return 0;
  if (args->n <= 64)
    hipLaunchKernelGGL(qkv_insert_kernel<1>, dim3(MSA_QKV_HEADS, (unsigned)((args->n + 15) / 16)), dim3(1024), 0,
                       stream, *args);
  else
    hipLaunchKernelGGL(qkv_insert_kernel<4>, dim3(MSA_QKV_HEADS, (unsigned)((args->n + 63) / 64)), dim3(1024), 0,
                       stream, *args);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
