/*
 * msa.h -- C ABI of the MI355X (gfx950) MiniMax Sparse Attention decode path.
 *
 * The method (cited by page title and section):
 *  - vLLM's MiniMax-M3.1-Flash day-0 post, Chinese edition (agentlenshq.com),
 *    section "MiniMax 稀疏注意力的工作原理" (how MSA works): the KV cache is cut
 *    into 128-token blocks; a lightweight indexer scores every cached key
 *    with one index query per GQA group against a single shared index-key
 *    head; scores are max-pooled to one per block; exact attention runs only
 *    over the top-16 blocks, the latest block always kept, so each query
 *    sees at most 2,048 keys.
 *  - the same post, "MiniMax-M3.1 架构的变化": the KV cache (keys, values and
 *    index keys) is NVFP4; "NVIDIA Blackwell MSA 内核优化": queries stay FP8;
 *    "通过查表实现的 NVFP4 MSA 内核": E4M3 scales and E2M1 magnitudes.
 *  - "MiniMax goes sparse" (atlascloud.ai), section 1, Step 1 (index branch,
 *    block max pool, TopK per layer and GQA group) and Step 2 (every query
 *    head of a group attends to the group's blocks).
 *  - The spke.com Japanese rendering of the vLLM post, section "MSA入門", says
 *    the same as the first bullet.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked (host).  The caller owns
 *    every buffer (inputs, outputs, workspaces); the library keeps no state,
 *    allocates nothing and never synchronises.  Calls are asynchronous on
 *    `stream` and may be captured into a HIP graph (no memset nodes).
 *  - Host-side argument errors return a negative msa_status synchronously
 *    and launch nothing.  A failed launch returns MSA_ERR_HIP.
 *  - Device data the host cannot see (block tables, context lengths, slot
 *    mappings) is read defensively: a context length above
 *    max_pages_per_req*128 is clamped, a page id outside [0, num_pages) makes
 *    that page read as masked and a slot outside the pool is skipped.  Results
 *    for such inputs are unspecified but no access leaves the buffers.
 *  - Batch semantics: request b has ctx_lens[b] = L_b cached tokens, its R
 *    new query rows included; row r sits at position p = L_b - R + r and
 *    sees tokens 0..p.  Logical block j of request b is the physical page
 *    block_table[b * max_pages_per_req + j]; page = selection block = 128
 *    tokens.  Rows with p < 0 see nothing.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = -1, /* null pointer, bad size or shape           */
  MSA_ERR_UNSUPPORTED = -2, /* valid but not implemented (dtype, layout)  */
  MSA_ERR_WORKSPACE = -3,   /* workspace smaller than the size query says */
  MSA_ERR_HIP = -4          /* a HIP launch or runtime call failed        */
} msa_status;

typedef enum { MSA_F32 = 0, MSA_FP8_E4M3 = 1, MSA_NVFP4 = 2 } msa_dtype;

typedef enum { MSA_TOKEN_MAJOR = 0, MSA_DIM_MAJOR = 1, MSA_HALF_ROWS = 2 } msa_layout;

#define MSA_PAGE_TOKENS 128
#define MSA_HEAD_DIM 128
#define MSA_HEADS_PER_GROUP 8
#define MSA_MAX_ROWS 8
#define MSA_MAX_PREFILL_ROWS 8192
#define MSA_MAX_TOPK 64
#define MSA_NVFP4_GROUP 16
#define MSA_NVFP4_SLAB_BYTES 9216
#define MSA_F32_SLAB_BYTES 65536
#define MSA_FP8_SLAB_BYTES 16384
#define MSA_QKV_HEADS 45
#define MSA_NOALLOC_SCRATCH_BYTES (4 << 20)

/*
 * One paged cache tensor of one layer.  Page p, head h is the slab at
 * pages + (p * num_heads + h) * slab_bytes.  Slab layouts:
 *   MSA_F32 (token-major only): float [128 tokens][128 dims], 65,536 B.
 *   MSA_FP8_E4M3, 16,384 B per slab: one E4M3 byte per element, value =
 *   e4m3 * tensor_scale (the pages' FP8 cache: 128 B of index keys and
 *   1,024 B of K+V per token and layer; one FP32 scale per cache tensor).
 *     MSA_TOKEN_MAJOR (keys): [128 tokens][128 dims].
 *     MSA_DIM_MAJOR (values): [128 dims][128 tokens].
 *     MSA_HALF_ROWS (index keys): [8 chunks of 16 tokens][2 halves][16
 *       tokens][64 dims]: token t, dim d at (t/16)*2048 + (d/64)*1024 +
 *       (t%16)*64 + d%64.  One 1 KB half is exactly what a 64-lane load of
 *       the indexer's FP8 matrix operand reads (16 tokens x 64 dims), so every
 *       load uses whole cache lines.
 * Required layouts: keys MSA_TOKEN_MAJOR; values MSA_DIM_MAJOR (NVFP4, FP8)
 * or MSA_TOKEN_MAJOR (F32); index keys MSA_TOKEN_MAJOR (NVFP4, F32) or
 * MSA_HALF_ROWS (FP8).  Any other combination is MSA_ERR_UNSUPPORTED.
 *   MSA_NVFP4, 9,216 B per slab.  Element value = (e2m1 * e4m3_scale) *
 *   tensor_scale; one E4M3 scale per 16 consecutive dims of a token (the
 *   block size that the pages' 34,560-vs-61,440 B per token fixes).
 *     MSA_TOKEN_MAJOR (keys, index keys): codes [128 tokens][64 B] (byte i of
 *       a token holds dim 2i in its low nibble, 2i+1 in its high nibble),
 *       then scales [128 tokens][8 B] (byte j: dims 16j..16j+15).
 *     MSA_DIM_MAJOR (values): codes [128 dims][64 B] (byte i of a dim holds
 *       token 2i in its low nibble, 2i+1 in its high nibble), then scales
 *       [8 groups][128 tokens].  Same quantisation groups as token-major; the
 *       bytes are placed so that the attention kernel's P.V matrix-core
 *       operand reads 8 consecutive tokens of one dim as one dword.
 * Keys and index keys must be MSA_TOKEN_MAJOR, values MSA_DIM_MAJOR when
 * NVFP4 (MSA_TOKEN_MAJOR when F32).  tensor_scale must be finite and > 0.
 */
typedef struct {
  int32_t dtype;      /* msa_dtype: MSA_NVFP4 or MSA_F32                  */
  int32_t layout;     /* msa_layout                                        */
  int32_t num_heads;  /* 4 for keys and values, 1 for index keys           */
  int32_t num_pages;  /* physical page pool size (>= 1)                    */
  float tensor_scale; /* per-tensor FP32 scale of an NVFP4 cache; 1 for F32 */
  void* pages;        /* device, num_pages * num_heads * slab bytes        */
} msa_cache;

/*
 * One decode step's batch (the struct itself is host memory).
 * shared_prefix_pages = P > 0 declares that entries 0..P-1 of every
 * block-table row name the same physical pages (a prefix every request
 * shares).  With an NVFP4 index cache the indexer then reads each of those
 * pages once and scores it for all B*R*4 index queries together, on the
 * matrix cores, and scans only pages P.. per request; the pages are taken
 * from row 0 of the table, and rows whose other entries differ get row 0's
 * scores (undefined results, not checked on the device).  Contexts shorter
 * than the prefix are fine (invisible tokens are masked as usual).  With an
 * F32 index cache P is not used.  0 <= P <= max_pages_per_req.
 *
 * page_owner (may be NULL) lets the decode scan (msa_index_score and
 * msa_insert_index_score with an NVFP4 or FP8 index cache, R <= MSA_MAX_ROWS,
 * no token_scores, P = 0) read the index pool in physical page order instead of
 * walking each request's table row.  Entry p names the block that page p
 * holds, b * max_pages_per_req + j where block_table[b][j] == p.  Required:
 * for every request b and every block j below the page of its first new row
 * (j < floor(max(L_b - R, 0) / 128)), page_owner[block_table[b][j]] names
 * (b, j); other entries may hold anything (-1 for a free page), since an entry
 * counts only if the table row it names points back at the page.  Such a call
 * reads every page of the index pool once, in use or not, and sets the
 * entries of the pages that hold the step's new rows, so a decode loop whose
 * tables only grow keeps the map current by itself; msa_page_owner builds it
 * from scratch (after the batch's requests change).  Pages of old blocks must
 * not be shared between requests (a page can name one owner).  Other calls
 * and the other cases ignore it.  B * max_pages_per_req must stay below 2^31
 * when it is set.
 */
typedef struct {
  int32_t num_reqs;            /* B >= 1                                        */
  int32_t rows_per_req;        /* R: 1..MSA_MAX_ROWS (decode, speculative rows); up to
                                  MSA_MAX_PREFILL_ROWS (a prefill chunk) where a call
                                  says so                                        */
  int32_t max_pages_per_req;   /* row stride of block_table (>= 1)              */
  int32_t shared_prefix_pages; /* P: leading table entries shared by every row, 0 if none */
  const int32_t* block_table;  /* device [B][max_pages_per_req] physical page ids */
  const int32_t* ctx_lens;     /* device [B] L_b, new rows included              */
  int32_t* page_owner;         /* device [index cache num_pages] or NULL: the block
                                  table's inverse, see below                     */
} msa_batch;

/*
 * Step 0: write n new tokens into the caches.  k, v: [n][4][128] FP32,
 * idx_k: [n][128] FP32, slot_mapping: [n] slot = page * 128 + offset, slots
 * distinct.  Any of k / v / idx_k may be NULL (with its cache NULL) to skip
 * that cache.  NVFP4 quantisation of each 16-dim group, FP32 round-to-
 * nearest-even at every step (the pages state no recipe; this amax recipe is
 * the reading taken): s = E4M3_sat((amax/6)/tensor_scale); s == 0 -> all
 * codes +0; else code_i = sign(x_i) | E2M1_sat(|x_i / (s*tensor_scale)|).
 * F32 caches store the values unchanged.  The pages fuse this into the QKV
 * GEMM epilogue (vLLM post, "QKV GEMM + norm + RoPE + KV 插入融合"); here it
 * is a kernel of its own.
 */
int msa_kv_insert(const float* k, const float* v, const float* idx_k, const int64_t* slot_mapping, int32_t n,
                  const msa_cache* k_cache, const msa_cache* v_cache, const msa_cache* idx_cache,
                  hipStream_t stream);

/* Same as msa_kv_insert, restricted to NVFP4 caches (MSA_ERR_UNSUPPORTED otherwise). */
int msa_kv_insert_nvfp4(const float* k, const float* v, const float* idx_k, const int64_t* slot_mapping,
                        int32_t n, const msa_cache* k_cache, const msa_cache* v_cache,
                        const msa_cache* idx_cache, hipStream_t stream);

/*
 * The projection that produces a step's new rows, fused with step 0 (vLLM
 * post, "QKV GEMM + norm + RoPE + KV 插入融合": the GEMM's epilogue takes the
 * FP32 accumulators head by head, applies norm and RoPE to the queries and
 * index queries, quantises K, V and the index key to NVFP4 and writes them
 * into the caches; the projected rows never reach HBM).
 *   x: [n][hidden] BF16 hidden states; w: BF16 projection weights in 32-k
 *   blocks, w[h][k/32][r][k%32] = W[128 h + r][k], where output column c is
 *   sum_k x[t][k] W[c][k] (a layout the weights are packed into once; each
 *   16-row operand of the matrix cores is then one contiguous 1 KB).  Columns
 *   are 45 heads of 128: query heads 0..31, key heads 32..35, value heads 36..39,
 *   index queries 40..43 (one per group), index key 44.  hidden: a multiple
 *   of 256, at most 65536.  The products accumulate in FP32.
 * The pages state no norm or rotary detail; the reading taken: for every
 * head but the values, y = h / sqrt(mean(h^2) + eps) * norm_weight[kind][d]
 * over the head's 128 values (kind 0 queries, 1 keys, 2 index queries,
 * 3 index key; norm_weight: [4][128] FP32), then rotate-half rotary
 * embedding: for i < 64, with c = rope_cos_sin[p][i], s = rope_cos_sin[p][64+i]
 * (rope_cos_sin: [rope_rows][128] FP32, p = positions[t]),
 *   out_i = y_i c - y_{i+64} s,  out_{i+64} = y_{i+64} c + y_i s.
 * Values are stored as projected.  Queries go to q_out [n][32][128] and index
 * queries to q_idx_out [n][4][128] as E4M3(out / q_scale); keys, values and
 * the index key go to slot_mapping[t] of the three NVFP4 caches by the
 * quantiser of msa_kv_insert.  A token whose position lies outside
 * [0, rope_rows) is skipped: nothing of it is written.  A token whose slot
 * lies outside the page pools writes its queries but no cache bytes.
 * pre_quant (may be NULL; a test aid): [n][45][128] FP32, the values just
 * before quantisation.  Every cache must be NVFP4 (MSA_ERR_UNSUPPORTED).
 * n: at most 64 * 65535 rows.
 */
int msa_qkv_project_insert(const uint16_t* x, const uint16_t* w, int32_t n, int32_t hidden,
                           const float* norm_weight, float eps, const float* rope_cos_sin, int32_t rope_rows,
                           const int32_t* positions, const int64_t* slot_mapping, float q_scale, uint8_t* q_out,
                           uint8_t* q_idx_out, const msa_cache* k_cache, const msa_cache* v_cache,
                           const msa_cache* idx_cache, float* pre_quant, hipStream_t stream);

/* FP32 -> FP8 E4M3 (OCP) query bytes: out[i] = E4M3_sat_RNE(x[i] / scale), NaN -> 0x7F|sign.
 * Queries stay FP8 while the cache is NVFP4 (vLLM post, Blackwell section). scale > 0. */
int msa_quantize_e4m3(const float* x, int64_t n, float scale, uint8_t* out, hipStream_t stream);

/*
 * Steps 1+2: indexer scores and 128-token block max-pool (vLLM post, "how
 * MSA works"; "MiniMax goes sparse", Step 1).  For every row (b, r), group
 * g in 0..3 and block j: block_scores[((b*R + r)*4 + g)*max_pages + j] =
 * max over tokens t <= p of block j of q_idx[b][r][g] . K_idx[t], or -inf
 * where the block holds no visible token (also for j beyond the context).
 * q_idx: [B][R][4][128], FP8 E4M3 bytes (times q_scale) with an NVFP4 index
 * cache, or FP32 with an F32 cache.  token_scores (may be NULL; a test aid):
 * [B][R][4][max_pages*128] per-token scores, -inf for invisible tokens.
 * Prefill: with an NVFP4 or FP8 index cache R may be up to
 * MSA_MAX_PREFILL_ROWS (the rows of a prompt chunk at positions L_b - R ..
 * L_b - 1); every page of a request is then scored for all its R*4 index
 * queries as one dense matrix-core product (the pages' indexer prefill, vLLM
 * post, "MSA 预填充").
 */
int msa_index_score(const msa_batch* batch, const void* q_idx, int32_t q_dtype, float q_scale,
                    const msa_cache* idx_cache, float* block_scores, float* token_scores, hipStream_t stream);

/*
 * Builds batch->page_owner's content from the block table into page_owner
 * (device [num_pages], num_pages = the index cache's pool size): every entry
 * -1, then entry block_table[b][j] = b * max_pages_per_req + j for the blocks
 * j < ceil(L_b / 128) of every request whose page id lies in [0, num_pages)
 * (a page named by two blocks keeps one of them).  Two kernels on stream; the
 * batch's own page_owner field is not read.  MSA_ERR_INVALID_ARG for a bad
 * batch, num_pages < 1, a NULL page_owner, or B * max_pages_per_req >= 2^31.
 */
int msa_page_owner(const msa_batch* batch, int32_t num_pages, int32_t* page_owner, hipStream_t stream);

/*
 * Steps 0+1+2 in one launch (NVFP4 caches, FP8 index queries): the step's
 * new tokens are written into the caches, then the index scores are computed
 * with them included.  The new tokens of request b are its last R positions,
 * L_b - R .. L_b - 1 (positions below 0 are skipped), at the slots its
 * block-table row gives them: k_new, v_new [B][R][4][128] FP32, idx_new
 * [B][R][128] FP32, row r of request b at position L_b - R + r.  They are
 * quantised and stored exactly as msa_kv_insert_nvfp4 stores them (keys and
 * index keys token-major, values dim-major), a token whose page id is outside
 * the pool is not written, and block_scores / token_scores come out as
 * msa_index_score computes them after that insert.  The pages holding new
 * tokens must not be shared between requests: in particular every new row
 * lies past the shared prefix, L_b - R >= 128 * shared_prefix_pages
 * (otherwise the result is undefined).  The pages fuse the insert
 * into the QKV GEMM epilogue (vLLM post, "QKV GEMM + norm + RoPE + KV 插入融合");
 * here the workgroup that scores a new token's page writes the token first.
 */
int msa_insert_index_score(const msa_batch* batch, const float* k_new, const float* v_new, const float* idx_new,
                           const void* q_idx, int32_t q_dtype, float q_scale, const msa_cache* k_cache,
                           const msa_cache* v_cache, const msa_cache* idx_cache, float* block_scores,
                           float* token_scores, hipStream_t stream);

/*
 * Step 3: block selection (vLLM post, "how MSA works").  For each (b, r, g)
 * with n visible blocks: all blocks if n <= topk; otherwise the latest block
 * n-1 plus the topk-1 best of the others by score, ties to the lower block
 * index, NaN below every number.  sel_blocks [B][R][4][topk] ascending
 * logical block ids, -1 padded; sel_count [B][R][4].  scores are block
 * scores [B][R][4][max_pages] (scores_are_token_level = 0) or token scores
 * [B][R][4][max_pages*128] that are max-pooled first (= 1).  1 <= topk <= 64.
 * R up to MSA_MAX_PREFILL_ROWS.
 */
int msa_block_maxpool_topk(const msa_batch* batch, const float* scores, int32_t scores_are_token_level,
                           int32_t topk, int32_t* sel_blocks, int32_t* sel_count, hipStream_t stream);

/*
 * Workspace bytes msa_sparse_decode (and msa_select_decode, when given one)
 * needs for this batch and topk, on the current device (host call; 0 for an
 * invalid batch).  F32 caches keep per-block partial results there; NVFP4 and
 * FP8 caches keep the partials of rows whose selected blocks are spread over
 * 2 or 4 workgroups, which a batch gets when one workgroup per (request,
 * row, group) would leave that many times the CUs idle (at most one float
 * partial of 8 x 130 values per workgroup the device's CUs can hold).  For a
 * prefill chunk (R > MSA_MAX_ROWS, max_pages_per_req <= 8192) it is the size
 * of the block-major route's state: one partial per (request, row, group,
 * rank) -- 8 x 128 FP16 outputs and 8 x 2 floats, 2,112 bytes -- plus the
 * per-block row lists, about B x R x 4 x topk x 2.2 KB (1.1 GB for 4 chunks
 * of 2,048 rows at topk 16); with a wider table, 0.
 */
size_t msa_workspace_bytes(const msa_batch* batch, int32_t topk);

/*
 * Step 4: exact GQA softmax attention over the selected blocks (vLLM post,
 * "how MSA works"; spke.com "MSA入門" Fig. 1 caption; "MiniMax goes sparse",
 * Step 2).  Query head h belongs to group g = h / 8 and attends, for row r,
 * to the tokens t <= p of the blocks sel_blocks[b][r][g][0..sel_count):
 *   out[b][r][h] = sum_t softmax_t(sm_scale * q_h . K_g[t]) V_g[t].
 * q: [B][R][4*8][128], FP8 E4M3 bytes (times q_scale) with NVFP4 caches or
 * FP32 with F32 caches.  out: [B][R][32][128] FP32; rows with no selected
 * block get zeros.  workspace: device, >= msa_workspace_bytes() (per-block
 * partial results of the F32 route, and of NVFP4 / FP8 rows split over
 * several workgroups, merged by a second launch in a fixed order; no initial
 * contents needed).  Two calls that share a workspace must not run
 * concurrently.
 * With NVFP4 or FP8 caches R may be up to MSA_MAX_PREFILL_ROWS (each row of a
 * prefill chunk attends to its own selection).  Chunks whose workspace holds
 * msa_workspace_bytes() (> 0) go block-major: every selected block is
 * dequantised once for all the rows that chose it, each (row, rank) writes a
 * partial, and a second launch merges each row's partials in rank order
 * (bitwise reproducible; the result differs from the one-workgroup-per-row
 * form that smaller workspaces take by rounding only).
 */
int msa_sparse_decode(const msa_batch* batch, const void* q, int32_t q_dtype, float q_scale, float sm_scale,
                      const msa_cache* k_cache, const msa_cache* v_cache, const int32_t* sel_blocks,
                      const int32_t* sel_count, int32_t topk, float* out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * attention as msa_sparse_decode, same arguments without the workspace, same
 * results.  Scratch memory comes from a fixed array inside the library, one
 * per GPU, of MSA_NOALLOC_SCRATCH_BYTES (4 MiB), held from the first call on
 * a GPU until the process ends; the call itself allocates nothing.  F32
 * caches keep the partial results of every selected block there: an F32
 * batch needing more than that size returns MSA_ERR_WORKSPACE (4 MiB holds 15
 * one-row requests at topk 16).  NVFP4 and FP8 caches keep only the partials
 * of split rows (at most 8 x 130 floats per workgroup the CUs can hold, about
 * 1 MiB on 256 CUs), so every batch fits.  Every call on a GPU shares that
 * GPU's array, and nothing in it needs initial contents (each call writes
 * every partial it reads).  Two calls that may overlap on one GPU (different
 * streams, or different host threads) race and must not be issued.  Errors as
 * msa_sparse_decode; a failed device query returns MSA_ERR_HIP.
 */
int msa_sparse_decode_noalloc(const msa_batch* batch, const void* q, int32_t q_dtype, float q_scale, float sm_scale,
                              const msa_cache* k_cache, const msa_cache* v_cache, const int32_t* sel_blocks,
                              const int32_t* sel_count, int32_t topk, float* out, hipStream_t stream);

/*
 * Steps 3+4 in one launch (NVFP4 caches, FP8 queries): the selection of
 * msa_block_maxpool_topk (from block scores) and the attention of
 * msa_sparse_decode, per (request, group) in one workgroup, so the selected
 * sets never make a round trip through memory between the two steps.
 * sel_blocks / sel_count are written as msa_block_maxpool_topk writes them;
 * out as msa_sparse_decode writes it.  workspace (device, may be NULL; else
 * at least msa_workspace_bytes() bytes, MSA_ERR_WORKSPACE otherwise): with
 * it, a batch that would leave CUs idle spreads each row's selected blocks
 * over several workgroups and merges their partial results in a second
 * launch, and a prefill chunk runs the selection launch and then the
 * block-major route; out then equals msa_sparse_decode's bit for bit.
 * Without it, one workgroup per row.
 */
int msa_select_decode(const msa_batch* batch, const float* block_scores, int32_t topk, const void* q,
                      int32_t q_dtype, float q_scale, float sm_scale, const msa_cache* k_cache,
                      const msa_cache* v_cache, int32_t* sel_blocks, int32_t* sel_count, float* out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * Measurement aid, not a step of the path: read `bytes` bytes of device
 * memory at src (16-byte aligned, bytes a multiple of 16) with the streaming
 * 16-byte loads the index scan uses, spread over `workgroups` workgroups of
 * 256 threads (1..65535) that each read one contiguous share.  Nothing is
 * written except, with negligible probability, one word of sink (device,
 * 4 bytes).  Its rate is the practical HBM read ceiling the index scan is
 * reported against.
 */
int msa_debug_stream_read(const void* src, int64_t bytes, int32_t workgroups, uint32_t* sink, hipStream_t stream);

/* Static text for a status code (host call). */
const char* msa_status_str(int status);

/*
 * Test aid: dequantise whole pages to FP32, out [n_pages][num_heads][128
 * tokens][128 dims], each element the single FP32 rounding of (e2m1 * scale)
 * * tensor_scale.  mode 0 decodes as the indexer does (FP32 scale), mode 1
 * as the attention kernel does (E2M1 and scale in FP16, product in FP16).
 */
int msa_debug_dequant(const msa_cache* cache, const int32_t* pages, int32_t n_pages, int32_t mode, float* out,
                      hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
