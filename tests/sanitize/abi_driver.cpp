// Sanitizer run of the C ABI's host-side validation (test infrastructure,
// built by tests/test_sanitizers.py with g++ -fsanitize=address,undefined).
// msa_api.hip is compiled as plain C++ for the host against stub launchers
// that only count calls, so every entry point's argument checks run without a
// GPU: good arguments must reach their launcher once, bad ones must return
// the documented status and launch nothing.
#include "../../block_sparse_attention_index_amd/csrc/msa_api.hip"

#include <algorithm>
#include <cstdio>
#include <limits>

static int launches = 0;
#define STUB(name, ...)                 \
  extern "C" int name(__VA_ARGS__) {    \
    ++launches;                         \
    return 0;                           \
  }
STUB(msa_launch_qkv_insert, const QkvArgs*, hipStream_t)
STUB(msa_launch_kv_insert, const float*, const float*, const float*, const int64_t*, int32_t, const msa_cache*,
     const msa_cache*, const msa_cache*, hipStream_t)
STUB(msa_launch_quantize_e4m3, const float*, int64_t, float, uint8_t*, hipStream_t)
STUB(msa_launch_debug_dequant, const msa_cache*, const int32_t*, int32_t, int32_t, float*, hipStream_t)
STUB(msa_launch_index_score, const msa_batch*, const void*, int32_t, float, const msa_cache*, float*, float*,
     hipStream_t)
STUB(msa_launch_insert_index_score, const msa_batch*, const float*, const float*, const float*, const void*, float,
     const msa_cache*, const msa_cache*, const msa_cache*, float*, float*, hipStream_t)
STUB(msa_launch_topk, const msa_batch*, const float*, int32_t, int32_t, int32_t*, int32_t*, hipStream_t)
STUB(msa_launch_select_decode, const msa_batch*, const float*, int32_t, const void*, float, float, const msa_cache*,
     const msa_cache*, int32_t*, int32_t*, float*, void*, size_t, hipStream_t)
STUB(msa_launch_sparse_decode_noalloc, const msa_batch*, const void*, int32_t, float, float, const msa_cache*,
     const msa_cache*, const int32_t*, const int32_t*, int32_t, float*, hipStream_t)
STUB(msa_launch_stream_read, const void*, int64_t, int32_t, uint32_t*, hipStream_t)
STUB(msa_launch_page_owner, const msa_batch*, int32_t, int32_t*, hipStream_t)
STUB(msa_launch_sparse_decode, const msa_batch*, const void*, int32_t, float, float, const msa_cache*,
     const msa_cache*, const int32_t*, const int32_t*, int32_t, float*, void*, size_t, hipStream_t)
extern "C" size_t msa_prefill_block_bytes(const msa_batch* b, int32_t topk) {  // any size for prefill chunks
  return b->rows_per_req > MSA_MAX_ROWS ? (size_t)b->num_reqs * b->rows_per_req * topk * 4 * 2112 : 0;
}
extern "C" size_t msa_decode_partials_bytes(const msa_batch* b, int32_t topk) {
  return (size_t)b->num_reqs * 4 * (size_t)b->rows_per_req * 8 * (size_t)topk * 130 * 4;
}
extern "C" size_t msa_split_partials_bytes(const msa_batch* b) {  // the split rule for 256 CUs
  const size_t rows = (size_t)b->num_reqs * b->rows_per_req * 4;
  const size_t S = rows * 4 <= 256 ? 4 : (rows * 2 <= 256 ? 2 : 1);
  return S > 1 ? rows * S * 1040 * 4 : 0;
}

static int failures = 0;
static void expect(int got, int want, int want_launches, const char* what) {
  if (got != want || launches != want_launches) {
    std::fprintf(stderr, "%s: status %d (want %d), launches %d (want %d)\n", what, got, want, launches, want_launches);
    ++failures;
  }
  launches = 0;
}

int main() {
  alignas(16) char buf[64];
  void* p = buf;  // never dereferenced by the validation
  const int32_t* ip = reinterpret_cast<const int32_t*>(buf);
  msa_cache kc{MSA_NVFP4, MSA_TOKEN_MAJOR, 4, 16, 0.01f, p}, vc{MSA_NVFP4, MSA_DIM_MAJOR, 4, 16, 0.01f, p};
  msa_cache ic{MSA_NVFP4, MSA_TOKEN_MAJOR, 1, 16, 0.01f, p};
  msa_batch bt{2, 1, 8, 0, ip, ip};
  float* f = reinterpret_cast<float*>(buf);
  int32_t* i32 = reinterpret_cast<int32_t*>(buf);
  const int64_t* slots = reinterpret_cast<const int64_t*>(buf);
  const float nan = std::numeric_limits<float>::quiet_NaN(), inf = std::numeric_limits<float>::infinity();

  // insert
  expect(msa_kv_insert_nvfp4(f, f, f, slots, 3, &kc, &vc, &ic, nullptr), MSA_OK, 1, "insert ok");
  expect(msa_kv_insert_nvfp4(f, f, f, slots, 0, &kc, &vc, &ic, nullptr), MSA_OK, 0, "insert n=0");
  expect(msa_kv_insert_nvfp4(f, f, f, nullptr, 3, &kc, &vc, &ic, nullptr), MSA_ERR_INVALID_ARG, 0, "insert no slots");
  expect(msa_kv_insert_nvfp4(f, nullptr, f, slots, 3, &kc, &vc, &ic, nullptr), MSA_ERR_INVALID_ARG, 0, "insert v/cache");
  expect(msa_kv_insert_nvfp4(f, f, f, slots, -1, &kc, &vc, &ic, nullptr), MSA_ERR_INVALID_ARG, 0, "insert n<0");
  msa_cache bad = kc;
  bad.tensor_scale = nan;
  expect(msa_kv_insert_nvfp4(f, nullptr, nullptr, slots, 3, &bad, nullptr, nullptr, nullptr), MSA_ERR_INVALID_ARG, 0,
         "insert nan scale");
  bad = kc;
  bad.layout = MSA_DIM_MAJOR;
  expect(msa_kv_insert_nvfp4(f, nullptr, nullptr, slots, 3, &bad, nullptr, nullptr, nullptr), MSA_ERR_UNSUPPORTED, 0,
         "insert key layout");
  bad = kc;
  bad.layout = 77;
  expect(msa_kv_insert(f, nullptr, nullptr, slots, 3, &bad, nullptr, nullptr, nullptr), MSA_ERR_INVALID_ARG, 0,
         "insert bogus layout");
  bad = kc;
  bad.dtype = MSA_F32;
  expect(msa_kv_insert_nvfp4(f, nullptr, nullptr, slots, 3, &bad, nullptr, nullptr, nullptr), MSA_ERR_UNSUPPORTED, 0,
         "insert_nvfp4 f32");
  bad.dtype = 9;
  expect(msa_kv_insert(f, nullptr, nullptr, slots, 3, &bad, nullptr, nullptr, nullptr), MSA_ERR_UNSUPPORTED, 0,
         "insert dtype 9");

  // index score
  expect(msa_index_score(&bt, p, MSA_FP8_E4M3, 1.0f, &ic, f, nullptr, nullptr), MSA_OK, 1, "index ok");
  expect(msa_index_score(nullptr, p, MSA_FP8_E4M3, 1.0f, &ic, f, nullptr, nullptr), MSA_ERR_INVALID_ARG, 0,
         "index null batch");
  expect(msa_index_score(&bt, p, MSA_F32, 1.0f, &ic, f, nullptr, nullptr), MSA_ERR_UNSUPPORTED, 0, "index q dtype");
  expect(msa_index_score(&bt, p, MSA_FP8_E4M3, -1.0f, &ic, f, nullptr, nullptr), MSA_ERR_INVALID_ARG, 0,
         "index q_scale");
  msa_batch b2 = bt;
  b2.rows_per_req = MSA_MAX_PREFILL_ROWS + 1;
  expect(msa_index_score(&b2, p, MSA_FP8_E4M3, 1.0f, &ic, f, nullptr, nullptr), MSA_ERR_INVALID_ARG, 0, "index R");
  b2 = bt;
  b2.num_reqs = 65536;
  expect(msa_index_score(&b2, p, MSA_FP8_E4M3, 1.0f, &ic, f, nullptr, nullptr), MSA_ERR_INVALID_ARG, 0, "index B");
  b2 = bt;
  b2.shared_prefix_pages = 9;
  expect(msa_index_score(&b2, p, MSA_FP8_E4M3, 1.0f, &ic, f, nullptr, nullptr), MSA_ERR_INVALID_ARG, 0, "prefix");
  b2 = bt;
  b2.num_reqs = 1 << 20, b2.rows_per_req = 8192;
  expect(msa_index_score(&b2, p, MSA_FP8_E4M3, 1.0f, &ic, f, nullptr, nullptr), MSA_ERR_INVALID_ARG, 0, "rows overflow");

  // owner map: its builder, and a batch that carries one
  int32_t* own = reinterpret_cast<int32_t*>(buf);
  expect(msa_page_owner(&bt, 16, own, nullptr), MSA_OK, 1, "page_owner ok");
  expect(msa_page_owner(&bt, 0, own, nullptr), MSA_ERR_INVALID_ARG, 0, "page_owner no pages");
  expect(msa_page_owner(&bt, 16, nullptr, nullptr), MSA_ERR_INVALID_ARG, 0, "page_owner null");
  expect(msa_page_owner(nullptr, 16, own, nullptr), MSA_ERR_INVALID_ARG, 0, "page_owner null batch");
  b2 = bt;
  b2.num_reqs = 65535, b2.max_pages_per_req = 40000;
  expect(msa_page_owner(&b2, 16, own, nullptr), MSA_ERR_INVALID_ARG, 0, "page_owner entry overflow");
  b2.page_owner = own;
  expect(msa_index_score(&b2, p, MSA_FP8_E4M3, 1.0f, &ic, f, nullptr, nullptr), MSA_ERR_INVALID_ARG, 0,
         "index owner entry overflow");
  b2 = bt;
  b2.page_owner = own;
  expect(msa_index_score(&b2, p, MSA_FP8_E4M3, 1.0f, &ic, f, nullptr, nullptr), MSA_OK, 1, "index with owner");
  expect(msa_insert_index_score(&b2, f, f, f, p, MSA_FP8_E4M3, 1.0f, &kc, &vc, &ic, f, nullptr, nullptr), MSA_OK, 1,
         "insert_index with owner");

  // selection
  expect(msa_block_maxpool_topk(&bt, f, 0, 16, i32, i32, nullptr), MSA_OK, 1, "topk ok");
  expect(msa_block_maxpool_topk(&bt, f, 0, 0, i32, i32, nullptr), MSA_ERR_INVALID_ARG, 0, "topk 0");
  expect(msa_block_maxpool_topk(&bt, f, 0, 65, i32, i32, nullptr), MSA_ERR_INVALID_ARG, 0, "topk 65");
  expect(msa_block_maxpool_topk(&bt, f, 2, 16, i32, i32, nullptr), MSA_ERR_INVALID_ARG, 0, "token flag");

  // attention
  const size_t ws = msa_workspace_bytes(&bt, 16);
  expect(ws == std::max(msa_decode_partials_bytes(&bt, 16), msa_split_partials_bytes(&bt)) ? MSA_OK : -99, MSA_OK, 0,
         "workspace size");
  expect(msa_workspace_bytes(nullptr, 16) == 0 ? MSA_OK : -99, MSA_OK, 0, "workspace size of no batch");
  {  // a prefill chunk: the block-major route's partials, and no per-block F32 partials
    msa_batch pb = bt;
    pb.rows_per_req = 64;
    const size_t pws = msa_workspace_bytes(&pb, 16);
    expect(pws == msa_prefill_block_bytes(&pb, 16) && pws > 0 ? MSA_OK : -99, MSA_OK, 0, "prefill workspace size");
    expect(msa_sparse_decode(&pb, p, MSA_FP8_E4M3, 1.0f, 0.088f, &kc, &vc, i32, i32, 16, f, p, pws, nullptr), MSA_OK,
           1, "prefill decode ok");
    expect(msa_sparse_decode(&pb, p, MSA_FP8_E4M3, 1.0f, 0.088f, &kc, &vc, i32, i32, 16, f, p, pws - 1, nullptr),
           MSA_ERR_WORKSPACE, 0, "prefill decode workspace");
  }
  expect(msa_sparse_decode(&bt, p, MSA_FP8_E4M3, 1.0f, 0.088f, &kc, &vc, i32, i32, 16, f, p, ws, nullptr), MSA_OK, 1,
         "decode ok");
  expect(msa_sparse_decode(&bt, p, MSA_FP8_E4M3, 1.0f, 0.088f, &kc, &vc, i32, i32, 16, f, p, ws - 1, nullptr),
         MSA_ERR_WORKSPACE, 0, "decode workspace");
  expect(msa_sparse_decode(&bt, p, MSA_FP8_E4M3, 1.0f, inf, &kc, &vc, i32, i32, 16, f, p, ws, nullptr),
         MSA_ERR_INVALID_ARG, 0, "decode sm_scale");
  expect(msa_sparse_decode(&bt, p, MSA_FP8_E4M3, 1.0f, 0.088f, &vc, &kc, i32, i32, 16, f, p, ws, nullptr),
         MSA_ERR_UNSUPPORTED, 0, "decode swapped layouts");
  expect(msa_select_decode(&bt, f, 16, p, MSA_FP8_E4M3, 1.0f, 0.088f, &kc, &vc, i32, i32, f, nullptr, 0, nullptr),
         MSA_OK, 1, "select_decode without workspace");
  expect(msa_select_decode(&bt, f, 16, p, MSA_FP8_E4M3, 1.0f, 0.088f, &kc, &vc, i32, i32, f, p, ws, nullptr), MSA_OK,
         1, "select_decode with workspace");
  expect(msa_select_decode(&bt, f, 16, p, MSA_FP8_E4M3, 1.0f, 0.088f, &kc, &vc, i32, i32, f, p, ws - 1, nullptr),
         MSA_ERR_WORKSPACE, 0, "select_decode small workspace");
  expect(msa_select_decode(&bt, f, 16, p, MSA_FP8_E4M3, 1.0f, 0.088f, &kc, &vc, i32, nullptr, f, nullptr, 0, nullptr),
         MSA_ERR_INVALID_ARG, 0, "select_decode no counts");
  expect(msa_sparse_decode_noalloc(&bt, p, MSA_FP8_E4M3, 1.0f, 0.088f, &kc, &vc, i32, i32, 16, f, nullptr), MSA_OK, 1,
         "noalloc ok");
  b2 = bt;
  b2.num_reqs = 4000;  // NVFP4: no scratch memory, any batch
  expect(msa_sparse_decode_noalloc(&b2, p, MSA_FP8_E4M3, 1.0f, 0.088f, &kc, &vc, i32, i32, 16, f, nullptr), MSA_OK, 1,
         "noalloc nvfp4 large batch");
  msa_cache k32{MSA_F32, MSA_TOKEN_MAJOR, 4, 16, 1.0f, p};
  msa_cache v32{MSA_F32, MSA_TOKEN_MAJOR, 4, 16, 1.0f, p};
  expect(msa_sparse_decode_noalloc(&b2, p, MSA_F32, 1.0f, 0.088f, &k32, &v32, i32, i32, 16, f, nullptr),
         MSA_ERR_WORKSPACE, 0, "noalloc f32 beyond the scratch array");
  expect(msa_sparse_decode_noalloc(&bt, p, MSA_F32, 1.0f, 0.088f, &k32, &v32, i32, i32, 16, f, nullptr), MSA_OK, 1,
         "noalloc f32 ok");
  expect(msa_sparse_decode_noalloc(&bt, p, MSA_FP8_E4M3, 1.0f, 0.088f, &kc, &vc, i32, nullptr, 16, f, nullptr),
         MSA_ERR_INVALID_ARG, 0, "noalloc no counts");
  expect(msa_select_decode(&bt, f, 16, p, MSA_FP8_E4M3, 1.0f, 0.088f, &k32, &k32, i32, i32, f, nullptr, 0, nullptr),
         MSA_ERR_UNSUPPORTED, 0, "select_decode f32");

  // fused insert + index
  expect(msa_insert_index_score(&bt, f, f, f, p, MSA_FP8_E4M3, 1.0f, &kc, &vc, &ic, f, nullptr, nullptr), MSA_OK, 1,
         "insert_index ok");
  b2 = bt;
  b2.rows_per_req = 9;
  expect(msa_insert_index_score(&b2, f, f, f, p, MSA_FP8_E4M3, 1.0f, &kc, &vc, &ic, f, nullptr, nullptr),
         MSA_ERR_INVALID_ARG, 0, "insert_index R=9");

  // projection, query quantiser, dequantiser, status text
  const uint16_t* u16 = reinterpret_cast<const uint16_t*>(buf);
  uint8_t* u8 = reinterpret_cast<uint8_t*>(buf);
  expect(msa_qkv_project_insert(u16, u16, 4, 512, f, 1e-6f, f, 16, ip, slots, 1.0f, u8, u8, &kc, &vc, &ic, nullptr,
                                nullptr),
         MSA_OK, 1, "qkv ok");
  expect(msa_qkv_project_insert(u16, u16, 4, 300, f, 1e-6f, f, 16, ip, slots, 1.0f, u8, u8, &kc, &vc, &ic, nullptr,
                                nullptr),
         MSA_ERR_INVALID_ARG, 0, "qkv hidden");
  expect(msa_qkv_project_insert(u16, u16, 4, 512, f, nan, f, 16, ip, slots, 1.0f, u8, u8, &kc, &vc, &ic, nullptr,
                                nullptr),
         MSA_ERR_INVALID_ARG, 0, "qkv eps");
  expect(msa_quantize_e4m3(f, 10, 1.0f, u8, nullptr), MSA_OK, 1, "e4m3 ok");
  expect(msa_quantize_e4m3(f, 10, 0.0f, u8, nullptr), MSA_ERR_INVALID_ARG, 0, "e4m3 scale");
  expect(msa_debug_dequant(&kc, ip, 2, 0, f, nullptr), MSA_OK, 1, "dequant ok");
  expect(msa_debug_dequant(&kc, ip, 2, 2, f, nullptr), MSA_ERR_INVALID_ARG, 0, "dequant mode");
  uint32_t* sink = reinterpret_cast<uint32_t*>(buf);
  expect(msa_debug_stream_read(buf, 64, 4, sink, nullptr), MSA_OK, 1, "stream ok");
  expect(msa_debug_stream_read(buf, 60, 4, sink, nullptr), MSA_ERR_INVALID_ARG, 0, "stream size");
  expect(msa_debug_stream_read(buf + 4, 64, 4, sink, nullptr), MSA_ERR_INVALID_ARG, 0, "stream alignment");
  expect(msa_debug_stream_read(buf, 64, 0, sink, nullptr), MSA_ERR_INVALID_ARG, 0, "stream grid");
  for (int s = -6; s <= 2; ++s) launches += msa_status_str(s)[0] == '\0';
  expect(MSA_OK, MSA_OK, 0, "status text");

  if (failures) return 1;
  std::printf("abi sanitizer run ok\n");
  return 0;
}
