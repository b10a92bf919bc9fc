// msa_api.hip -- the C ABI declared in include/msa.h: host-side validation of
// every argument the host can see, then one launcher call per step.  No call
// allocates, frees, synchronises or keeps state.
#include <math.h>

#include "msa.h"
#include "msa_kernels.h"

namespace {

bool finite_pos(float x) { return isfinite(x) && x > 0.0f; }

enum Role { KEYS, VALUES, INDEX };

// The one slab layout each (dtype, role) uses.
int required_layout(int32_t dtype, Role role) {
  if (dtype == MSA_F32) return MSA_TOKEN_MAJOR;
  if (role == VALUES) return MSA_DIM_MAJOR;
  if (role == INDEX && dtype == MSA_FP8_E4M3) return MSA_HALF_ROWS;
  return MSA_TOKEN_MAJOR;
}

int check_cache(const msa_cache* c, Role role) {
  const int want_heads = role == INDEX ? 1 : 4;
  if (!c || !c->pages || c->num_pages < 1 || c->num_heads != want_heads) return MSA_ERR_INVALID_ARG;
  if (c->dtype != MSA_NVFP4 && c->dtype != MSA_FP8_E4M3 && c->dtype != MSA_F32) return MSA_ERR_UNSUPPORTED;
  if (c->layout != MSA_TOKEN_MAJOR && c->layout != MSA_DIM_MAJOR && c->layout != MSA_HALF_ROWS)
    return MSA_ERR_INVALID_ARG;
  if (c->layout != required_layout(c->dtype, role)) return MSA_ERR_UNSUPPORTED;
  if (!finite_pos(c->tensor_scale)) return MSA_ERR_INVALID_ARG;
  return MSA_OK;
}

// max_rows: MSA_MAX_ROWS for decode-only calls, MSA_MAX_PREFILL_ROWS where a
// prefill chunk is accepted.
int check_batch(const msa_batch* b, int max_rows = MSA_MAX_ROWS) {
  if (!b || !b->block_table || !b->ctx_lens) return MSA_ERR_INVALID_ARG;
  if (b->num_reqs < 1 || b->rows_per_req < 1 || b->rows_per_req > max_rows || b->max_pages_per_req < 1)
    return MSA_ERR_INVALID_ARG;
  // (request, row, group) rows are counted in 32-bit integers
  if ((int64_t)b->num_reqs * b->rows_per_req * 4 > (int64_t)1 << 30) return MSA_ERR_INVALID_ARG;
  if (b->shared_prefix_pages < 0 || b->shared_prefix_pages > b->max_pages_per_req) return MSA_ERR_INVALID_ARG;
  // grid dimensions: y and z are 16-bit on this hardware
  if (b->num_reqs > 65535) return MSA_ERR_INVALID_ARG;
  // owner entries b * max_pages + j are 32-bit
  if (b->page_owner && (int64_t)b->num_reqs * b->max_pages_per_req >= (int64_t)1 << 31) return MSA_ERR_INVALID_ARG;
  return MSA_OK;
}

int query_dtype_ok(int32_t q_dtype, const msa_cache* c) {
  if (c->dtype != MSA_F32) return q_dtype == MSA_FP8_E4M3 ? MSA_OK : MSA_ERR_UNSUPPORTED;
  return q_dtype == MSA_F32 ? MSA_OK : MSA_ERR_UNSUPPORTED;
}

int insert_impl(const float* k, const float* v, const float* idx_k, const int64_t* slots, int32_t n,
                const msa_cache* kc, const msa_cache* vc, const msa_cache* ic, hipStream_t stream, bool nvfp4_only) {
  if (n < 0 || (n > 0 && !slots)) return MSA_ERR_INVALID_ARG;
  if (!k && !v && !idx_k) return MSA_ERR_INVALID_ARG;
  if ((k != nullptr) != (kc != nullptr) || (v != nullptr) != (vc != nullptr) || (idx_k != nullptr) != (ic != nullptr))
    return MSA_ERR_INVALID_ARG;
  int st;
  if (kc && (st = check_cache(kc, KEYS)) != MSA_OK) return st;
  if (vc && (st = check_cache(vc, VALUES)) != MSA_OK) return st;
  if (ic && (st = check_cache(ic, INDEX)) != MSA_OK) return st;
  if (nvfp4_only)
    for (const msa_cache* c : {kc, vc, ic})
      if (c && c->dtype != MSA_NVFP4) return MSA_ERR_UNSUPPORTED;
  if (n == 0) return MSA_OK;
  return msa_launch_kv_insert(k, v, idx_k, slots, n, kc, vc, ic, stream) == 0 ? MSA_OK : MSA_ERR_HIP;
}

}  // namespace

extern "C" {

int msa_kv_insert(const float* k, const float* v, const float* idx_k, const int64_t* slot_mapping, int32_t n,
                  const msa_cache* k_cache, const msa_cache* v_cache, const msa_cache* idx_cache,
                  hipStream_t stream) {
  return insert_impl(k, v, idx_k, slot_mapping, n, k_cache, v_cache, idx_cache, stream, false);
}

int msa_kv_insert_nvfp4(const float* k, const float* v, const float* idx_k, const int64_t* slot_mapping,
                        int32_t n, const msa_cache* k_cache, const msa_cache* v_cache,
                        const msa_cache* idx_cache, hipStream_t stream) {
  return insert_impl(k, v, idx_k, slot_mapping, n, k_cache, v_cache, idx_cache, stream, true);
}

int msa_qkv_project_insert(const uint16_t* x, const uint16_t* w, int32_t n, int32_t hidden,
                           const float* norm_weight, float eps, const float* rope_cos_sin, int32_t rope_rows,
                           const int32_t* positions, const int64_t* slot_mapping, float q_scale, uint8_t* q_out,
                           uint8_t* q_idx_out, const msa_cache* k_cache, const msa_cache* v_cache,
                           const msa_cache* idx_cache, float* pre_quant, hipStream_t stream) {
  if (n < 0 || hidden < 256 || hidden % 256 != 0 || hidden > (1 << 16)) return MSA_ERR_INVALID_ARG;
  if (!isfinite(eps) || eps < 0.0f || !finite_pos(q_scale) || rope_rows < 1) return MSA_ERR_INVALID_ARG;
  int st;
  if ((st = check_cache(k_cache, KEYS)) != MSA_OK) return st;
  if ((st = check_cache(v_cache, VALUES)) != MSA_OK) return st;
  if ((st = check_cache(idx_cache, INDEX)) != MSA_OK) return st;
  for (const msa_cache* c : {k_cache, v_cache, idx_cache})
    if (c->dtype != MSA_NVFP4) return MSA_ERR_UNSUPPORTED;
  if (n == 0) return MSA_OK;
  if (!x || !w || !norm_weight || !rope_cos_sin || !positions || !slot_mapping || !q_out || !q_idx_out)
    return MSA_ERR_INVALID_ARG;
  if ((n + 63) / 64 > 65535) return MSA_ERR_INVALID_ARG;  // grid y: 64 tokens per workgroup past 64 rows
  QkvArgs A{x, w, n, hidden, norm_weight, eps, rope_cos_sin, rope_rows, positions, slot_mapping, q_scale, q_out,
            q_idx_out, (uint8_t*)k_cache->pages, (uint8_t*)v_cache->pages, (uint8_t*)idx_cache->pages,
            k_cache->num_pages, v_cache->num_pages, idx_cache->num_pages, k_cache->tensor_scale,
            v_cache->tensor_scale, idx_cache->tensor_scale, pre_quant};
  return msa_launch_qkv_insert(&A, stream) == 0 ? MSA_OK : MSA_ERR_HIP;
}

int msa_quantize_e4m3(const float* x, int64_t n, float scale, uint8_t* out, hipStream_t stream) {
  if (n < 0 || (n > 0 && (!x || !out)) || !finite_pos(scale)) return MSA_ERR_INVALID_ARG;
  if (n == 0) return MSA_OK;
  return msa_launch_quantize_e4m3(x, n, scale, out, stream) == 0 ? MSA_OK : MSA_ERR_HIP;
}

int msa_index_score(const msa_batch* batch, const void* q_idx, int32_t q_dtype, float q_scale,
                    const msa_cache* idx_cache, float* block_scores, float* token_scores, hipStream_t stream) {
  int st;
  if ((st = check_batch(batch, MSA_MAX_PREFILL_ROWS)) != MSA_OK) return st;
  if ((st = check_cache(idx_cache, INDEX)) != MSA_OK) return st;
  if (batch->rows_per_req > MSA_MAX_ROWS && idx_cache->dtype == MSA_F32) return MSA_ERR_UNSUPPORTED;
  if (!q_idx || !block_scores) return MSA_ERR_INVALID_ARG;
  if ((st = query_dtype_ok(q_dtype, idx_cache)) != MSA_OK) return st;
  if (q_dtype == MSA_FP8_E4M3 && !finite_pos(q_scale)) return MSA_ERR_INVALID_ARG;
  return msa_launch_index_score(batch, q_idx, q_dtype, q_scale, idx_cache, block_scores, token_scores, stream) == 0
             ? MSA_OK
             : MSA_ERR_HIP;
}

int msa_block_maxpool_topk(const msa_batch* batch, const float* scores, int32_t scores_are_token_level,
                           int32_t topk, int32_t* sel_blocks, int32_t* sel_count, hipStream_t stream) {
  int st;
  if ((st = check_batch(batch, MSA_MAX_PREFILL_ROWS)) != MSA_OK) return st;
  if (!scores || !sel_blocks || !sel_count) return MSA_ERR_INVALID_ARG;
  if (topk < 1 || topk > MSA_MAX_TOPK) return MSA_ERR_INVALID_ARG;
  if (scores_are_token_level != 0 && scores_are_token_level != 1) return MSA_ERR_INVALID_ARG;
  return msa_launch_topk(batch, scores, scores_are_token_level, topk, sel_blocks, sel_count, stream) == 0
             ? MSA_OK
             : MSA_ERR_HIP;
}

size_t msa_workspace_bytes(const msa_batch* batch, int32_t topk) {
  if (check_batch(batch, MSA_MAX_PREFILL_ROWS) != MSA_OK || topk < 1 || topk > MSA_MAX_TOPK) return 0;
  // prefill chunks (NVFP4 / FP8 only): the block-major route's partials, 0 where it does not apply
  if (batch->rows_per_req > MSA_MAX_ROWS) return msa_prefill_block_bytes(batch, topk);
  // F32 caches: per-block partial results; NVFP4 / FP8: the partials of rows split over several workgroups
  const size_t f32 = msa_decode_partials_bytes(batch, topk), split = msa_split_partials_bytes(batch);
  return f32 > split ? f32 : split;
}

int msa_sparse_decode(const msa_batch* batch, const void* q, int32_t q_dtype, float q_scale, float sm_scale,
                      const msa_cache* k_cache, const msa_cache* v_cache, const int32_t* sel_blocks,
                      const int32_t* sel_count, int32_t topk, float* out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  int st;
  if ((st = check_batch(batch, MSA_MAX_PREFILL_ROWS)) != MSA_OK) return st;
  if ((st = check_cache(k_cache, KEYS)) != MSA_OK) return st;
  if ((st = check_cache(v_cache, VALUES)) != MSA_OK) return st;
  if (k_cache->dtype != v_cache->dtype || k_cache->num_pages != v_cache->num_pages) return MSA_ERR_INVALID_ARG;
  if (batch->rows_per_req > MSA_MAX_ROWS && k_cache->dtype == MSA_F32) return MSA_ERR_UNSUPPORTED;
  if (!q || !sel_blocks || !sel_count || !out || !workspace) return MSA_ERR_INVALID_ARG;
  if (topk < 1 || topk > MSA_MAX_TOPK) return MSA_ERR_INVALID_ARG;
  if ((st = query_dtype_ok(q_dtype, k_cache)) != MSA_OK) return st;
  if (!finite_pos(sm_scale) || (q_dtype == MSA_FP8_E4M3 && !finite_pos(q_scale))) return MSA_ERR_INVALID_ARG;
  if (workspace_bytes < msa_workspace_bytes(batch, topk)) return MSA_ERR_WORKSPACE;
  return msa_launch_sparse_decode(batch, q, q_dtype, q_scale, sm_scale, k_cache, v_cache, sel_blocks, sel_count,
                                  topk, out, workspace, workspace_bytes, stream) == 0
             ? MSA_OK
             : MSA_ERR_HIP;
}

int msa_sparse_decode_noalloc(const msa_batch* batch, const void* q, int32_t q_dtype, float q_scale, float sm_scale,
                              const msa_cache* k_cache, const msa_cache* v_cache, const int32_t* sel_blocks,
                              const int32_t* sel_count, int32_t topk, float* out, hipStream_t stream) {
  int st;
  if ((st = check_batch(batch, MSA_MAX_PREFILL_ROWS)) != MSA_OK) return st;
  if ((st = check_cache(k_cache, KEYS)) != MSA_OK) return st;
  if ((st = check_cache(v_cache, VALUES)) != MSA_OK) return st;
  if (k_cache->dtype != v_cache->dtype || k_cache->num_pages != v_cache->num_pages) return MSA_ERR_INVALID_ARG;
  if (batch->rows_per_req > MSA_MAX_ROWS && k_cache->dtype == MSA_F32) return MSA_ERR_UNSUPPORTED;
  if (!q || !sel_blocks || !sel_count || !out) return MSA_ERR_INVALID_ARG;
  if (topk < 1 || topk > MSA_MAX_TOPK) return MSA_ERR_INVALID_ARG;
  if ((st = query_dtype_ok(q_dtype, k_cache)) != MSA_OK) return st;
  if (!finite_pos(sm_scale) || (q_dtype == MSA_FP8_E4M3 && !finite_pos(q_scale))) return MSA_ERR_INVALID_ARG;
  const size_t need = k_cache->dtype == MSA_F32 ? msa_decode_partials_bytes(batch, topk)
                                               : msa_split_partials_bytes(batch);
  if (need > (size_t)MSA_NOALLOC_SCRATCH_BYTES) return MSA_ERR_WORKSPACE;
  return msa_launch_sparse_decode_noalloc(batch, q, q_dtype, q_scale, sm_scale, k_cache, v_cache, sel_blocks,
                                          sel_count, topk, out, stream) == 0
             ? MSA_OK
             : MSA_ERR_HIP;
}

int msa_select_decode(const msa_batch* batch, const float* block_scores, int32_t topk, const void* q,
                      int32_t q_dtype, float q_scale, float sm_scale, const msa_cache* k_cache,
                      const msa_cache* v_cache, int32_t* sel_blocks, int32_t* sel_count, float* out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  int st;
  if ((st = check_batch(batch, MSA_MAX_PREFILL_ROWS)) != MSA_OK) return st;
  if ((st = check_cache(k_cache, KEYS)) != MSA_OK) return st;
  if ((st = check_cache(v_cache, VALUES)) != MSA_OK) return st;
  if (k_cache->dtype == MSA_F32 || v_cache->dtype != k_cache->dtype) return MSA_ERR_UNSUPPORTED;
  if (k_cache->num_pages != v_cache->num_pages) return MSA_ERR_INVALID_ARG;
  if (!block_scores || !q || !sel_blocks || !sel_count || !out) return MSA_ERR_INVALID_ARG;
  if (topk < 1 || topk > MSA_MAX_TOPK) return MSA_ERR_INVALID_ARG;
  if (q_dtype != MSA_FP8_E4M3) return MSA_ERR_UNSUPPORTED;
  if (!finite_pos(sm_scale) || !finite_pos(q_scale)) return MSA_ERR_INVALID_ARG;
  if (workspace && workspace_bytes < msa_workspace_bytes(batch, topk)) return MSA_ERR_WORKSPACE;
  return msa_launch_select_decode(batch, block_scores, topk, q, q_scale, sm_scale, k_cache, v_cache, sel_blocks,
                                  sel_count, out, workspace, workspace ? workspace_bytes : 0, stream) == 0
             ? MSA_OK
             : MSA_ERR_HIP;
}

int msa_page_owner(const msa_batch* batch, int32_t num_pages, int32_t* page_owner, hipStream_t stream) {
  int st;
  if ((st = check_batch(batch, MSA_MAX_PREFILL_ROWS)) != MSA_OK) return st;
  if (num_pages < 1 || !page_owner) return MSA_ERR_INVALID_ARG;
  if ((int64_t)batch->num_reqs * batch->max_pages_per_req >= (int64_t)1 << 31) return MSA_ERR_INVALID_ARG;
  return msa_launch_page_owner(batch, num_pages, page_owner, stream) == 0 ? MSA_OK : MSA_ERR_HIP;
}

int msa_insert_index_score(const msa_batch* batch, const float* k_new, const float* v_new, const float* idx_new,
                           const void* q_idx, int32_t q_dtype, float q_scale, const msa_cache* k_cache,
                           const msa_cache* v_cache, const msa_cache* idx_cache, float* block_scores,
                           float* token_scores, hipStream_t stream) {
  int st;
  if ((st = check_batch(batch)) != MSA_OK) return st;
  if ((st = check_cache(k_cache, KEYS)) != MSA_OK) return st;
  if ((st = check_cache(v_cache, VALUES)) != MSA_OK) return st;
  if ((st = check_cache(idx_cache, INDEX)) != MSA_OK) return st;
  for (const msa_cache* c : {k_cache, v_cache, idx_cache})
    if (c->dtype == MSA_F32 || c->dtype != k_cache->dtype) return MSA_ERR_UNSUPPORTED;
  if (k_cache->num_pages != v_cache->num_pages) return MSA_ERR_INVALID_ARG;
  if (!k_new || !v_new || !idx_new || !q_idx || !block_scores) return MSA_ERR_INVALID_ARG;
  if (q_dtype != MSA_FP8_E4M3) return MSA_ERR_UNSUPPORTED;
  if (!finite_pos(q_scale)) return MSA_ERR_INVALID_ARG;
  return msa_launch_insert_index_score(batch, k_new, v_new, idx_new, q_idx, q_scale, k_cache, v_cache, idx_cache,
                                       block_scores, token_scores, stream) == 0
             ? MSA_OK
             : MSA_ERR_HIP;
}

int msa_debug_stream_read(const void* src, int64_t bytes, int32_t workgroups, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink || bytes < 0 || bytes % 16 != 0 || ((uintptr_t)src & 15) != 0) return MSA_ERR_INVALID_ARG;
  if (workgroups < 1 || workgroups > 65535) return MSA_ERR_INVALID_ARG;
  if (bytes == 0) return MSA_OK;
  return msa_launch_stream_read(src, bytes, workgroups, sink, stream) == 0 ? MSA_OK : MSA_ERR_HIP;
}

const char* msa_status_str(int status) {
  switch (status) {
    case MSA_OK: return "ok";
    case MSA_ERR_INVALID_ARG: return "invalid argument";
    case MSA_ERR_UNSUPPORTED: return "unsupported dtype or layout";
    case MSA_ERR_WORKSPACE: return "workspace too small";
    case MSA_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

int msa_debug_dequant(const msa_cache* cache, const int32_t* pages, int32_t n_pages, int32_t mode, float* out,
                      hipStream_t stream) {
  if (!cache || !cache->pages || cache->num_heads < 1 || cache->num_pages < 1) return MSA_ERR_INVALID_ARG;
  if (cache->dtype != MSA_NVFP4 && cache->dtype != MSA_FP8_E4M3 && cache->dtype != MSA_F32) return MSA_ERR_UNSUPPORTED;
  if (cache->dtype == MSA_F32 && cache->layout != MSA_TOKEN_MAJOR) return MSA_ERR_UNSUPPORTED;
  if (cache->layout == MSA_HALF_ROWS && cache->dtype != MSA_FP8_E4M3) return MSA_ERR_UNSUPPORTED;
  if (cache->layout != MSA_TOKEN_MAJOR && cache->layout != MSA_DIM_MAJOR && cache->layout != MSA_HALF_ROWS)
    return MSA_ERR_INVALID_ARG;
  if (n_pages < 0 || (n_pages > 0 && (!pages || !out)) || (mode != 0 && mode != 1)) return MSA_ERR_INVALID_ARG;
  if (n_pages == 0) return MSA_OK;
  return msa_launch_debug_dequant(cache, pages, n_pages, mode, out, stream) == 0 ? MSA_OK : MSA_ERR_HIP;
}

}  // extern "C"
