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
// heads, 4 index queries (one per group), 1 index key.  A call of at most 64
// rows runs qkv_insert_kernel, one workgroup of 16 waves per (head, 8 or 16
// rows); a prompt chunk runs qkv_insert_tiled_kernel (LDS-staged, below).  In
// the first:
//  * GEMM on v_mfma_f32_16x16x32_bf16.  Each lane's operand is 8 consecutive
//    k of one row: one 16-byte load.  x [n][hidden] is row-major; the weights
//    come in 32-k blocks, w[head][k/32][row][k%32], so a wave's operand for 16
//    rows is one contiguous 1 KB and a head's weights one contiguous range (in
//    the plain [column][hidden] layout a wave touches 16 rows a hidden row
//    apart, and the stream ran at about 1 TB/s).  Wave w takes 32 columns
//    (w % 4) over a quarter of the hidden dimension (w / 4); the quarters are
//    summed through one LDS tile in four rounds.
//  * Epilogue (both kernels): a wave takes one token of the head at a time;
//    lane l holds dims l and l + 64, which is both a rotary pair and, per
//    16-lane row, two NVFP4 groups (the insert's row quantiser and store).
#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf8 load_bf8(const uint16_t* p) {
  return __builtin_bit_cast(bf8, *reinterpret_cast<const uint4*>(p));
}

// The epilogue's view of one head: its kind (0 query, 1 key, 2 value,
// 3 index query, 4 index key), index within the kind, and this lane's two
// norm weights (dims lane and lane + 64).
struct QkvHead {
  int head, kind, sub;
  float g_lo, g_hi;
};

__device__ __forceinline__ QkvHead qkv_head(const QkvArgs& A, int head, int lane) {
  QkvHead h;
  h.head = head;
  h.kind = head < 32 ? 0 : head < 36 ? 1 : head < 40 ? 2 : head < 44 ? 3 : 4;
  h.sub = h.kind == 0 ? head : h.kind == 1 ? head - 32 : h.kind == 2 ? head - 36 : h.kind == 3 ? head - 40 : 0;
  const int gsel = h.kind == 0 ? 0 : h.kind == 1 ? 1 : h.kind == 3 ? 2 : 3;  // norm weight row
  h.g_lo = h.g_hi = 0.f;
  if (h.kind != 2) {
    h.g_lo = A.norm_weight[gsel * kDim + lane];
    h.g_hi = A.norm_weight[gsel * kDim + 64 + lane];
  }
  return h;
}

// One token of one head, on one wave: lo / hi are the projected values of
// dims lane and lane + 64.  Norm, rotation, then the head's destination.
__device__ __forceinline__ void qkv_epilogue_token(const QkvArgs& A, const QkvHead& hd, int tok, float lo, float hi,
                                                   int lane) {
  const int n = lane & 15, a = lane >> 4;
  const int p = A.pos[tok];
  if (p < 0 || p >= A.rope_rows) return;  // no rotation for this token: nothing of it is written
  if (hd.kind != 2) {
    // RMS norm: sum of squares over the head's 128 values (every lane gets it)
    float ss = lo * lo + hi * hi;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    const float inv = 1.0f / sqrtf(ss / (float)kDim + A.eps);
    const float ylo = lo * inv * hd.g_lo, yhi = hi * inv * hd.g_hi;
    const float c = A.rope[(int64_t)p * kDim + lane], s = A.rope[(int64_t)p * kDim + 64 + lane];
    lo = ylo * c - yhi * s;
    hi = yhi * c + ylo * s;
  }
  if (A.pre) {
    float* pr = A.pre + ((int64_t)tok * MSA_QKV_HEADS + hd.head) * kDim;
    pr[lane] = lo;
    pr[64 + lane] = hi;
  }
  if (hd.kind == 0 || hd.kind == 3) {
    uint8_t* q = hd.kind == 0 ? A.q_out + ((int64_t)tok * 32 + hd.sub) * kDim
                              : A.qidx_out + ((int64_t)tok * 4 + hd.sub) * kDim;
    q[lane] = (uint8_t)e4m3_encode(lo / A.q_scale);
    q[64 + lane] = (uint8_t)e4m3_encode(hi / A.q_scale);
    return;
  }
  uint8_t* pages = hd.kind == 1 ? A.kpages : hd.kind == 2 ? A.vpages : A.ipages;
  const int np = hd.kind == 1 ? A.knp : hd.kind == 2 ? A.vnp : A.inp;
  const int heads = hd.kind == 4 ? 1 : kGroups;
  const float ts = hd.kind == 1 ? A.kts : hd.kind == 2 ? A.vts : A.its;
  const int64_t slot = A.slots[tok];
  const bool valid = slot >= 0 && slot < (int64_t)np * kPage;
  uint8_t* slab = pages + ((valid ? slot >> 7 : 0) * heads + hd.sub) * (int64_t)kNvSlab;
  const int off = (int)(slot & (kPage - 1));
  uint32_t code;
  uint32_t sc = nvfp4_row_quantize(lo, ts, code);
  nvfp4_row_store(slab, off, a, n, code, sc, hd.kind == 2, valid);
  sc = nvfp4_row_quantize(hi, ts, code);
  nvfp4_row_store(slab, off, 4 + a, n, code, sc, hd.kind == 2, valid);
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

// Calls of at most 64 rows (a decode step's new rows): a workgroup per
// (head, ROWS rows), ROWS = 8 or 16 of the 16-row matrix tile (the padding
// rows repeat a real row and are not stored).  Small workgroups put more CUs
// on the weight stream, which each CU sustains only in part; the other
// workgroups' reads of the same weights hit the caches.  A 32-row call: 64
// rows per workgroup 44.1 us, 16 rows 29.5 us, 8 rows 25.7 us.  Larger calls
// go to qkv_insert_tiled_kernel.
template <int ROWS>
__global__ __launch_bounds__(1024) void qkv_insert_kernel(QkvArgs A) {
  constexpr int MT = 1;  // one 16-row matrix tile
  __shared__ float tile[16][kDim + 4];
  const int head = blockIdx.x;  // heads fastest: the workgroups in flight share a few token tiles
  const int t0 = blockIdx.y * ROWS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, a = lane >> 4;
  const int cg = wave & 3, kq = wave >> 2;
  const int mts = 1;

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
  for (int mt = 0; mt < MT; ++mt) xp[mt] = A.x + (int64_t)min(t0 + min(n, ROWS - 1), A.n - 1) * A.hidden + kb;
  constexpr int U = 8;
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
  const QkvHead hd = qkv_head(A, head, lane);
  if (wave < ROWS && t0 + wave < A.n) qkv_epilogue_token(A, hd, t0 + wave, tile[wave][lane], tile[wave][64 + lane], lane);
}

// Prompt chunks (more than 64 rows): one workgroup per (head, TT tokens), TT
// = 128 (4 waves) or 256 (8 waves), a GEMM from LDS-staged operand blocks of
// 64 k, double-buffered.  Per block each thread moves 16-byte chunks of the
// hidden-state and weight rows with coalesced loads (a weight block pair is
// one contiguous 16 KB in the packed layout); each wave then multiplies a 64
// x 64 part from LDS, 16 MFMAs per 32 k.  Operands are read from HBM or the
// caches once per workgroup instead of once per wave.  The FP32 result tile
// reuses the staging memory.  Launched with 128: 256 tokens (each staged
// weight block serving twice the rows, one workgroup per CU) measured slower
// for an 8,192-row chunk (599 against 557 us).
constexpr int kBK = 64;           // k per staged block
constexpr int kLdsRow = kBK + 16;  // bf16 per staged row: 32 bytes of padding against bank conflicts
                                   // (16 bytes: 1.6% slower; 48: two workgroups no longer fit a CU's LDS)

template <int TT>
__global__ __launch_bounds__(TT * 2) void qkv_insert_tiled_kernel(QkvArgs A) {
  constexpr int NT = TT * 2;                  // threads: TT / 32 waves
  constexpr int kStageA = TT * kLdsRow * 2;   // bytes of one hidden-state stage
  constexpr int kStageB = kDim * kLdsRow * 2; // bytes of one weight stage
  constexpr int kStages = 2 * (kStageA + kStageB);
  constexpr int kTile = TT * (kDim + 4) * 4;  // the FP32 result tile
  constexpr int AX = TT * 8 / NT;             // 16-byte hidden-state chunks per thread per block: 4
  constexpr int BX = kDim * 8 / NT;           // weight chunks per thread per block: 4 or 2
  __shared__ __align__(16) uint8_t lds[kStages > kTile ? kStages : kTile];
  typedef uint16_t RowA[TT][kLdsRow];
  typedef uint16_t RowB[kDim][kLdsRow];
  RowA* sA = reinterpret_cast<RowA*>(lds);                // [2 stages] hidden states
  RowB* sB = reinterpret_cast<RowB*>(lds + 2 * kStageA);  // [2 stages] weights
  float(*tile)[kDim + 4] = reinterpret_cast<float(*)[kDim + 4]>(lds);
  const int head = blockIdx.x, t0 = blockIdx.y * TT;  // heads fastest: in-flight workgroups share token tiles
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, a = lane >> 4;
  constexpr int WM = TT / 64;                  // waves along the tokens
  const int wm = wave % WM, wn = wave / WM;    // this wave's part: tokens 64 wm.., columns 64 wn..
  const int lr = tid >> 3, lc = tid & 7;       // staging: rows lr + (NT / 8) i, 16-byte chunk lc
  static_assert(AX == 4, "four hidden-state chunks per thread");
  const uint16_t* xg[AX];
  const uint16_t* wg[BX];
#pragma unroll
  for (int i = 0; i < AX; ++i)
    xg[i] = A.x + (int64_t)min(t0 + lr + (NT / 8) * i, A.n - 1) * A.hidden + 8 * lc;
#pragma unroll
  for (int i = 0; i < BX; ++i)
    wg[i] = A.w + (((int64_t)head * (A.hidden / 32) + (lc >> 2)) * kDim + lr + (NT / 8) * i) * 32 + 8 * (lc & 3);
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 rx[AX], rw[BX];
  v4f acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
  const int nkb = A.hidden / kBK;
#pragma unroll
  for (int i = 0; i < AX; ++i) rx[i] = *reinterpret_cast<const u32x4*>(xg[i]);
#pragma unroll
  for (int i = 0; i < BX; ++i) rw[i] = *reinterpret_cast<const u32x4*>(wg[i]);
#pragma unroll
  for (int i = 0; i < AX; ++i) *reinterpret_cast<u32x4*>(&sA[0][lr + (NT / 8) * i][8 * lc]) = rx[i];
#pragma unroll
  for (int i = 0; i < BX; ++i) *reinterpret_cast<u32x4*>(&sB[0][lr + (NT / 8) * i][8 * lc]) = rw[i];
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nkb) {  // the next block lands in registers while this one is multiplied
#pragma unroll
      for (int i = 0; i < AX; ++i) rx[i] = *reinterpret_cast<const u32x4*>(xg[i] + (kb + 1) * kBK);
#pragma unroll
      for (int i = 0; i < BX; ++i)
        rw[i] = *reinterpret_cast<const u32x4*>(wg[i] + (int64_t)(kb + 1) * 2 * kDim * 32);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf8 fa[4], fb[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        fa[mt] = __builtin_bit_cast(bf8, *reinterpret_cast<const u32x4*>(&sA[cur][64 * wm + 16 * mt + n][32 * ks + 8 * a]));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        fb[nt] = __builtin_bit_cast(bf8, *reinterpret_cast<const u32x4*>(&sB[cur][64 * wn + 16 * nt + n][32 * ks + 8 * a]));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[mt], fb[nt], acc[mt][nt], 0, 0, 0);
    }
    // the other stage was last read before the previous barrier
    if (kb + 1 < nkb) {
#pragma unroll
      for (int i = 0; i < AX; ++i) *reinterpret_cast<u32x4*>(&sA[cur ^ 1][lr + (NT / 8) * i][8 * lc]) = rx[i];
#pragma unroll
      for (int i = 0; i < BX; ++i) *reinterpret_cast<u32x4*>(&sB[cur ^ 1][lr + (NT / 8) * i][8 * lc]) = rw[i];
    }
    __syncthreads();
  }
  // every wave is past its last staging read: the result tile may overwrite the stages
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) tile[64 * wm + 16 * mt + 4 * a + i][64 * wn + 16 * nt + n] = acc[mt][nt][i];
  __syncthreads();
  const QkvHead hd = qkv_head(A, head, lane);
  for (int r = 0; r < 32; ++r) {  // TT / 32 waves x 32 tokens
    const int tl = wave * 32 + r;
    if (t0 + tl >= A.n) break;
    qkv_epilogue_token(A, hd, t0 + tl, tile[tl][lane], tile[tl][64 + lane], lane);
  }
}

}  // namespace msa

using namespace msa;

extern "C" int msa_launch_qkv_insert(const QkvArgs* args, hipStream_t stream) {
  if (args->n == 0) return 0;
  if (args->n <= 32)
    hipLaunchKernelGGL(qkv_insert_kernel<8>, dim3(MSA_QKV_HEADS, (unsigned)((args->n + 7) / 8)), dim3(1024), 0,
                       stream, *args);
  else if (args->n <= 64)
    hipLaunchKernelGGL(qkv_insert_kernel<16>, dim3(MSA_QKV_HEADS, (unsigned)((args->n + 15) / 16)), dim3(1024), 0,
                       stream, *args);
  else
    hipLaunchKernelGGL(qkv_insert_tiled_kernel<128>, dim3(MSA_QKV_HEADS, (unsigned)((args->n + 127) / 128)),
                       dim3(256), 0, stream, *args);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
