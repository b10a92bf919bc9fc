// msa_topk.hip -- step 3 as a kernel of its own: top-k block selection with
// the latest block kept (vLLM M3.1 post, "MiniMax 稀疏注意力的工作原理";
// "MiniMax goes sparse", section 1 Step 1).  One wave per (request, row,
// group) runs select_fast (block scores) or select_row (token scores)
// (msa_select.h); the ids are stored ascending, -1 padded, with their count.
#include "msa_kernels.h"
#include "msa_select.h"

namespace msa {

template <bool kTok, int KMAX>
__global__ __launch_bounds__(256) void topk_kernel(const int32_t* __restrict__ lens, int32_t B, int32_t R,
                                                   int32_t max_pages, const float* __restrict__ scores,
                                                   int32_t topk, int32_t* __restrict__ sel,
                                                   int32_t* __restrict__ cnt) {
  __shared__ SelectScratch scratch[4];
  const int lane = threadIdx.x & 63;
  const int row_id = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row_id >= B * R * kGroups) return;
  const int b = row_id / (R * kGroups);
  const int r = (row_id / kGroups) % R;
  const int64_t stride = kTok ? (int64_t)max_pages * kPage : max_pages;
  const float* row = scores + (int64_t)row_id * stride;
  // block scores are loaded before the row length arrives (masked by the selection)
  float sc[KMAX > 0 ? KMAX : 1];
  if (!kTok) load_row_scores<KMAX>(row, max_pages, lane, sc);
  const int L = clamp_len(lens[b], max_pages);
  const int p = L - R + r;
  const int n = p < 0 ? 0 : p / kPage + 1;
  int32_t* out = sel + (int64_t)row_id * topk;
  auto emit = [&](int rank, int id) { out[rank] = id; };
  const int c = kTok ? select_row<true, KMAX>(row, n, p, topk, lane, emit)
                     : select_fast<KMAX>(sc, [&](int j) { return row[j]; }, n, topk, lane, &scratch[threadIdx.x >> 6],
                                         emit);
  if (lane >= c && lane < topk) out[lane] = -1;
  if (lane == 0) cnt[row_id] = c;
}

template <bool kTok>
static void launch_topk(const msa_batch* bt, const float* scores, int32_t topk, int32_t* sel, int32_t* cnt,
                        hipStream_t s) {
  const int rows = bt->num_reqs * bt->rows_per_req * kGroups;
  const dim3 grid((rows + 3) / 4);
  const int P = bt->max_pages_per_req;
#define MSA_TOPK_LAUNCH(K)                                                                                      \
  hipLaunchKernelGGL((topk_kernel<kTok, K>), grid, dim3(256), 0, s, bt->ctx_lens, bt->num_reqs, bt->rows_per_req, \
                     P, scores, topk, sel, cnt)
  switch (select_kmax(P)) {
    case 8: MSA_TOPK_LAUNCH(8); break;
    case 24: MSA_TOPK_LAUNCH(24); break;
    case 48: MSA_TOPK_LAUNCH(48); break;
    default: MSA_TOPK_LAUNCH(0); break;
  }
#undef MSA_TOPK_LAUNCH
}

}  // namespace msa

using namespace msa;

extern "C" int msa_launch_topk(const msa_batch* bt, const float* scores, int32_t token_level, int32_t topk,
                               int32_t* sel, int32_t* cnt, hipStream_t s) {
  if (token_level)
    launch_topk<true>(bt, scores, topk, sel, cnt, s);
  else
    launch_topk<false>(bt, scores, topk, sel, cnt, s);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
