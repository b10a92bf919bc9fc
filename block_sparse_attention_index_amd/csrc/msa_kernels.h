// msa_kernels.h -- launchers of the gfx950 MSA kernels, called by the C ABI
// layer (msa_api.hip) after it has validated every host-side argument.
// Each returns 0, or -1 when the launch failed.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "msa.h"

// Arguments of msa_qkv_project_insert after validation (caches unpacked).
struct QkvArgs {
  const uint16_t* x;
  const uint16_t* w;
  int32_t n, hidden;
  const float* norm_weight;  // [4][128]
  float eps;
  const float* rope;  // [rope_rows][128]: cos, then sin
  int32_t rope_rows;
  const int32_t* pos;
  const int64_t* slots;
  float q_scale;
  uint8_t* q_out;
  uint8_t* qidx_out;
  uint8_t *kpages, *vpages, *ipages;
  int32_t knp, vnp, inp;
  float kts, vts, its;
  float* pre;
};

extern "C" {
int msa_launch_qkv_insert(const QkvArgs* args, hipStream_t stream);
int msa_launch_kv_insert(const float* k, const float* v, const float* idx_k, const int64_t* slots, int32_t n,
                         const msa_cache* kc, const msa_cache* vc, const msa_cache* ic, hipStream_t stream);
int msa_launch_quantize_e4m3(const float* x, int64_t n, float scale, uint8_t* out, hipStream_t stream);
int msa_launch_debug_dequant(const msa_cache* c, const int32_t* pages, int32_t n_pages, int32_t mode, float* out,
                             hipStream_t stream);
int msa_launch_index_score(const msa_batch* b, const void* q_idx, int32_t q_dtype, float q_scale,
                           const msa_cache* ic, float* block_scores, float* token_scores, hipStream_t stream);
int msa_launch_insert_index_score(const msa_batch* b, const float* k_new, const float* v_new, const float* idx_new,
                                  const void* q_idx, float q_scale, const msa_cache* kc, const msa_cache* vc,
                                  const msa_cache* ic, float* block_scores, float* token_scores, hipStream_t stream);
int msa_launch_page_owner(const msa_batch* b, int32_t num_pages, int32_t* owner, hipStream_t stream);
int msa_launch_prefix_index(const msa_batch* b, const void* q_idx, float q_scale, const msa_cache* ic,
                            float* block_scores, float* token_scores, hipStream_t stream);
int msa_launch_prefill_index(const msa_batch* b, const void* q_idx, float q_scale, const msa_cache* ic,
                             float* block_scores, float* token_scores, hipStream_t stream);
int msa_launch_topk(const msa_batch* b, const float* scores, int32_t token_level, int32_t topk, int32_t* sel,
                    int32_t* cnt, hipStream_t stream);
size_t msa_decode_partials_bytes(const msa_batch* b, int32_t topk);
size_t msa_split_partials_bytes(const msa_batch* b);
int msa_launch_select_decode(const msa_batch* b, const float* block_scores, int32_t topk, const void* q,
                             float q_scale, float sm_scale, const msa_cache* kc, const msa_cache* vc, int32_t* sel,
                             int32_t* cnt, float* out, void* workspace, size_t workspace_bytes, hipStream_t stream);
size_t msa_prefill_block_bytes(const msa_batch* b, int32_t topk);
int msa_launch_prefill_block_attend(const msa_batch* b, const uint8_t* q, float q_scale, float sm_scale,
                                    const msa_cache* kc, const msa_cache* vc, const int32_t* sel, const int32_t* cnt,
                                    int32_t topk, float* out, void* workspace, hipStream_t stream);
int msa_launch_sparse_decode_noalloc(const msa_batch* b, const void* q, int32_t q_dtype, float q_scale,
                                     float sm_scale, const msa_cache* kc, const msa_cache* vc, const int32_t* sel,
                                     const int32_t* cnt, int32_t topk, float* out, hipStream_t stream);
int msa_launch_stream_read(const void* src, int64_t bytes, int32_t workgroups, uint32_t* sink, hipStream_t stream);
int msa_launch_sparse_decode(const msa_batch* b, const void* q, int32_t q_dtype, float q_scale, float sm_scale,
                             const msa_cache* kc, const msa_cache* vc, const int32_t* sel, const int32_t* cnt,
                             int32_t topk, float* out, void* workspace, size_t workspace_bytes, hipStream_t stream);
}
