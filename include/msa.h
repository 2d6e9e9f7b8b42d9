/*
 * msa.h -- C ABI of libmsa: MiniMax-M3 block-sparse attention over a paged
 * KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The method is described on three vLLM API documentation pages, cited here
 * by title and section:
 *   [FI]  vllm.models.minimax_m3.nvidia.sparse_attention_flashinfer
 *   [NV4] vllm.models.minimax_m3.amd.sparse_attention_nvfp4
 *   [SPA] vllm.models.minimax_m3.amd.ops.sparse_pa
 *
 * Each query token attends only to the 128-token KV blocks named in its
 * top-k row, clipped causally: ids past the token's own block are dropped and
 * the own block is attended up to the token's position ([SPA]
 * _write_sparse_block_table_row_from_values).
 *
 * Conventions shared by every call:
 *  - Every pointer argument is a DEVICE pointer owned by the caller, unless
 *    stated otherwise.  The library never allocates, frees or synchronises;
 *    work is enqueued on `stream` (0 = the null stream).
 *  - All host-visible arguments are validated before any HIP call; on error
 *    nothing is launched and msa_last_error() describes the problem.
 *    Values held in device memory (ids, lengths) are not read on the host.
 *  - Empty work (no rows / no keys) returns MSA_OK and launches nothing,
 *    as [SPA] minimax_m3_insert_index_cache does on empty input.
 *  - A sparse block is 128 tokens; pages hold 16 tokens; a block spans
 *    `block_page_stride` page ids (8 when K and V are separate planes, 16
 *    when one buffer holds both sides of a block), [SPA]
 *    minimax_m3_sparse_block_page_stride.  Physical page ids and byte
 *    offsets are 64-bit, [NV4] supported_kv_cache_layouts.
 *  - Rows of a top-k table must hold distinct non-negative ids (-1 pads).
 *    Repeated ids are outside the contract (the printed routine counts them
 *    twice); the library stays in bounds but the result is unspecified.
 *  - Block-table entries naming pages outside the cache (negative, or past
 *    num_pages) are skipped by every kernel: such a block adds nothing.
 *  - Launch log: while the environment variable MSA_LOG is set to a value
 *    other than "0" (read at each launch), every kernel launch writes one
 *    line to stderr, "[msa] <kernel> ...", with its launch shape (workgroups,
 *    waves, splits, query tile).  Validation failures are not logged; they
 *    are reported through msa_last_error().
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_API __attribute__((visibility("default")))

typedef enum msa_status {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARGUMENT = 1,   /* a value a caller must fix ([SPA] ValueError / assertion) */
  MSA_ERR_UNSUPPORTED = 2,        /* a valid shape / dtype the library does not serve */
  MSA_ERR_WORKSPACE_TOO_SMALL = 3,
  MSA_ERR_HIP = 4                 /* a HIP launch failed; see msa_last_error() */
} msa_status_t;

typedef enum msa_dtype {
  MSA_BF16 = 0,
  MSA_FP16 = 1,
  MSA_FP8_E4M3FN = 2,   /* OCP E4M3FN: max 448, NaN = S.1111.111 */
  MSA_NVFP4 = 3,        /* e2m1 codes + one E4M3FN scale per 16 elements */
  MSA_FP32 = 4
} msa_dtype_t;

/* How a cache's pages are laid out (msa_kv_cache_t.kv_layout). */
typedef enum msa_kv_layout {
  MSA_KV_PAGE16 = 0,    /* 16-token pages: K and V planes, or NVFP4 head slots */
  MSA_KV_ROWS128 = 1    /* 128-token pages with K|V-interleaved token rows */
} msa_kv_layout_t;

/*
 * One layer's paged K/V cache.  [FI] MiniMaxM3SparseFlashInferImpl.forward
 * (K and V views of the cache, fp8 view with per-tensor scales);
 * [NV4] customize_spec (NVFP4: two head slots per kv head, packed data plus
 * block scales, bytes laid out for the kernel).
 *
 * kv_layout MSA_KV_PAGE16 (0, the default):
 * kv_dtype MSA_BF16 / MSA_FP8_E4M3FN: K and V are planes of pages
 *   [page][num_kv_heads][16 tokens][head_dim] elements, page p at byte
 *   p * page_stride_bytes of its buffer.  With block_page_stride 8, block b
 *   owns pages 8b..8b+7 of k_pages (K) and of v_pages (V).  With stride 16,
 *   block b owns pages 16b..16b+15: K in 16b..16b+7 of k_pages, V in
 *   16b+8..16b+15 of v_pages (usually the same buffer).
 * kv_dtype MSA_NVFP4 (head_dim 128): one buffer k_pages of pages
 *   [page][2 * num_kv_heads slots][9 * head_dim bytes]; slot 2g is K and
 *   slot 2g+1 is V of kv head g; v_pages is ignored.  A slot holds 16
 *   tokens: 1024 bytes of e2m1 codes (code byte c of a token holds elements
 *   2c, low nibble, and 2c+1), then 128 E4M3FN scale bytes (scale u covers
 *   elements 16u..16u+15).
 *     K slot, token-major: code byte c of token t at t*64 + c; scale u at
 *       1024 + t*8 + u.
 *     V slot, tokens in groups of 4: code byte c of token t at
 *       ((t/4*16 + c/4)*4 + t%4)*4 + c%4; scale u at 1024 + (t/4*8 + u)*4 + t%4
 *       (the decode reads one token group's 8 elements and their 4 scales
 *       with one load each).
 *
 * kv_layout MSA_KV_ROWS128 (bf16 / fp8 only; [FI] MiniMaxM3SparseFlashInfer-
 *   Backend.supported_kv_cache_layouts: the head-major LBHNC cache the SM90
 *   kernels read): one buffer k_pages of pages
 *   [page][num_kv_heads][128 tokens][2 * head_dim] elements, each token row
 *   holding its K (elements 0 .. head_dim - 1) then its V; page p at byte
 *   p * page_stride_bytes, a multiple of 16 rows (16 * 2 * head_dim
 *   elements; a stride above the page size packs other data, e.g. other
 *   layers, between pages).  Page b is sparse block b, so
 *   block_page_stride must be 8: page-16 id 8b + j (the table builder's ids)
 *   names rows 16j .. 16j + 15 of page b.  v_pages is NULL or
 *   k_pages + head_dim elements (the V view of the same buffer).
 *
 * k_scale / v_scale: device fp32 scalars (NULL = 1.0).  fp8: the
 *   per-tensor dequant multipliers; NVFP4: the per-tensor global scales.
 *   They fold exactly into the softmax scale and the output scale
 *   ([FI] forward: a per-tensor K descale multiplies every logit and a
 *   per-tensor V descale every output, so both move out of the kernel's inner loop).
 * num_pages: pages each buffer holds (MSA_KV_ROWS128: 128-token pages).
 *   Blocks whose pages fall outside [0, num_pages) are skipped (they add
 *   nothing), so a bad table cannot make the attend read out of bounds.
 */
typedef struct msa_kv_cache {
  int32_t kv_dtype;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_page_stride;
  const void* k_pages;
  const void* v_pages;
  int64_t page_stride_bytes;
  int64_t num_pages;
  const float* k_scale;
  const float* v_scale;
  int32_t kv_layout;   /* msa_kv_layout_t */
} msa_kv_cache_t;

/* Thread-local description of the last error returned on this thread. */
MSA_API const char* msa_last_error(void);

/*
 * Page-16 sparse block table, one row per query token.
 * [SPA] _write_sparse_block_table_row_from_values,
 * minimax_m3_build_sparse_block_table_decode / _prefill.
 *
 * topk [total_q][topk_k] int32 (row stride topk_row_stride elements):
 *   logical 128-token block ids, -1 padded, one index head shared by all
 *   attention heads.
 * block_table [num_reqs][bt_cols] int32 (row stride bt_row_stride): a
 *   request's logical block -> physical block id.
 * Row positions, one of two modes:
 *   decode  (query_req_id == NULL): total_q must equal num_reqs *
 *     decode_query_len (the [SPA] decode builder's assertion); row i belongs
 *     to request i / dql at position seq_lens[r] - dql + i % dql
 *     (right-aligned, [FI] forward);
 *   prefill (query_req_id and query_abs_pos non-NULL, [total_q] int32 each):
 *     rows with a negative position or a request id outside [0, num_reqs)
 *     are padding.
 * Per row: causal length = max(pos + 1, 0), own block = pos / 128; an id is
 * kept if 0 <= id <= own block and id < bt_cols.  Kept earlier ("full")
 * blocks fill the slots first, in row order, then the own ("tail") block.
 * Slot s holds block_table[r][id] * block_page_stride + j at 8s + j
 * (j < 8); the rest of the row, up to 8 * topk_k, is zero.
 * sparse_ctx[i] = 128 * full + tail tokens (pos + 1 - 128 * own) when the
 * own block is kept, else min(128 * kept, causal length).
 * Outputs: sparse_bt [total_q][8 * topk_k] int32 (row stride
 * sbt_row_stride >= 8 * topk_k), sparse_ctx [total_q] int32.
 */
MSA_API msa_status_t msa_build_sparse_block_table(
    const int32_t* topk, int64_t topk_row_stride, int32_t topk_k, int32_t total_q,
    const int32_t* block_table, int64_t bt_row_stride, int32_t bt_cols, int32_t num_reqs,
    const int32_t* seq_lens, int32_t decode_query_len,
    const int32_t* query_req_id, const int32_t* query_abs_pos,
    int32_t block_page_stride,
    int32_t* sparse_bt, int64_t sbt_row_stride, int32_t* sparse_ctx,
    hipStream_t stream);

/*
 * Request id and absolute position of each prefill token.
 * [NV4] MiniMaxM3SparseRocmNvfp4MetadataBuilder.build
 * (minimax_m3_query_token_positions; its body is not printed).
 * Token t of request r (cu_seqlens_q[r] <= t < cu_seqlens_q[r+1]) sits at
 * context_lens[r] + t - cu_seqlens_q[r]; tokens t >= cu_seqlens_q[num_reqs]
 * (up to total_q) are padding: request 0, position -1.
 * cu_seqlens_q [num_reqs + 1], context_lens [num_reqs] int32 in;
 * query_req_id, query_abs_pos [total_q] int32 out.
 */
MSA_API msa_status_t msa_query_token_positions(
    const int32_t* cu_seqlens_q, const int32_t* context_lens, int32_t num_reqs, int32_t total_q,
    int32_t* query_req_id, int32_t* query_abs_pos, hipStream_t stream);

/*
 * Bytes of workspace msa_sparse_decode can use for split-K partials.
 * Passing fewer (or NULL) is allowed: the call then uses fewer splits.
 */
MSA_API size_t msa_decode_workspace_size(int32_t total_q, int32_t num_q_heads, int32_t head_dim,
                                         int32_t topk_k);

/*
 * Block-sparse GQA decode, decode_query_len >= 1 tokens per request.
 * [FI] MiniMaxM3SparseFlashInferImpl.forward (msa_sparse_decode_attention:
 * q, K/V cache, top-k, page table, seqused_k, seqlen_q, causal, softmax
 * scale, v scale, out); [NV4] MiniMaxM3SparseRocmNvfp4Impl.forward
 * (the NVFP4 decode with k_scale / v_scale and decode_query_len).
 *
 * q, out [num_reqs * decode_query_len][num_q_heads][head_dim] bf16,
 * contiguous (q_dtype must be MSA_BF16).  Query head h reads kv head
 * h / (num_q_heads / num_kv_heads).  Row positions, top-k clipping and
 * table lookup as in msa_build_sparse_block_table (decode mode).
 * out = softmax(softmax_scale * k_scale * q K^T over the row's tokens) V
 *       * v_scale, with K, V the stored codes; a row with no tokens gets 0.
 * Compute: matrix-core inputs in bf16 for q K^T (fp16 for NVFP4, where
 * e2m1 x E4M3 products are exact) and in fp16 for P V on fp8 / NVFP4 pages
 * (bf16 on bf16 pages); fp32 accumulation and softmax; output rounded to
 * nearest even.
 * topk_k <= 1024; head_dim 64 or 128 (NVFP4: 128);
 * num_q_heads / num_kv_heads <= 16.
 */
MSA_API msa_status_t msa_sparse_decode(
    const void* q, int32_t q_dtype, int32_t num_reqs, int32_t decode_query_len, int32_t num_q_heads,
    const msa_kv_cache_t* kv,
    const int32_t* topk, int64_t topk_row_stride, int32_t topk_k,
    const int32_t* block_table, int64_t bt_row_stride, int32_t bt_cols,
    const int32_t* seq_lens,
    float softmax_scale, void* out,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * msa_sparse_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, math and output as
 * msa_sparse_decode given a full workspace; the split-K partials go to a
 * fixed device array of msa_decode_noalloc_scratch_bytes() bytes that the
 * library holds on each GPU until the process ends.  The call itself
 * allocates nothing.  Every call on one GPU shares that GPU's array, so calls
 * that overlap in time on one GPU (other streams, other threads) race and
 * must be serialised by the caller; calls on one stream are ordered.  A
 * decode whose partials would not fit returns MSA_ERR_WORKSPACE_TOO_SMALL
 * (with the split count the decode picks, <= 16 query heads per kv head and
 * head_dim <= 128, they always fit).  The first call on a device looks the
 * array up (hipGetSymbolAddress), so make it outside graph capture.
 */
MSA_API msa_status_t msa_sparse_decode_noalloc(
    const void* q, int32_t q_dtype, int32_t num_reqs, int32_t decode_query_len, int32_t num_q_heads,
    const msa_kv_cache_t* kv,
    const int32_t* topk, int64_t topk_row_stride, int32_t topk_k,
    const int32_t* block_table, int64_t bt_row_stride, int32_t bt_cols,
    const int32_t* seq_lens,
    float softmax_scale, void* out, hipStream_t stream);

/* Size of msa_sparse_decode_noalloc's per-device scratch array, in bytes. */
MSA_API size_t msa_decode_noalloc_scratch_bytes(void);

/*
 * Bytes of workspace msa_sparse_prefill can use: 32 * (total_q +
 * ceil(total_q / 32)), 0 for total_q <= 0.  A query tile's row order takes
 * as many bytes as the tile has rows (32, 48 or 64), so this covers every
 * tile of any split of total_q rows into requests at 6 to 8 query heads per
 * kv head, and every tile of splits with at most about half as many
 * requests as rows at 4 or 5.  The other arguments are accepted for
 * symmetry with msa_decode_workspace_size and not used.
 */
MSA_API size_t msa_prefill_workspace_size(int32_t total_q, int32_t num_q_heads, int32_t head_dim,
                                          int32_t topk_k);

/*
 * Block-sparse ragged causal prefill.
 * [FI] MiniMaxM3SparseFlashInferImpl.forward (msa_sparse_attention:
 * q, K/V cache, top-k, cu_seqlens_q, causal, softmax scale, page table,
 * seqused_k, v scale, out); [NV4] MiniMaxM3SparseRocmNvfp4Impl.forward
 * (the prefill with per-token request ids and positions).
 *
 * q, out [total_q][num_q_heads][head_dim] bf16, contiguous.  Rows
 * cu_seqlens_q[r] .. cu_seqlens_q[r+1]-1 are request r's new tokens, at
 * positions seq_lens[r] - (cu_seqlens_q[r+1] - cu_seqlens_q[r]) + local
 * offset (seq_lens counts the new tokens); rows before cu_seqlens_q[0] and
 * rows >= cu_seqlens_q[num_reqs] are padding and get 0.  cu_seqlens_q must
 * be non-decreasing; rows it names at or past total_q are not computed.
 * Same math, page formats and limits as
 * msa_sparse_decode (bf16, fp8 e4m3fn or NVFP4 pages; NVFP4 computes in
 * fp16).
 *
 * workspace: device memory the call may overwrite (no alignment needed), or
 * NULL.  At 4 to 8 query heads per kv head the call first writes one row
 * order per query tile there (rows with alike top-k rows share matrix
 * tiles, which saves products); tiles past what workspace_bytes holds keep
 * their natural order.  Any size gives the same results up to rounding;
 * the output does not depend on what the workspace held before the call.
 */
MSA_API msa_status_t msa_sparse_prefill(
    const void* q, int32_t q_dtype, int32_t total_q, int32_t num_q_heads,
    const msa_kv_cache_t* kv,
    const int32_t* topk, int64_t topk_row_stride, int32_t topk_k,
    const int32_t* block_table, int64_t bt_row_stride, int32_t bt_cols, int32_t num_reqs,
    const int32_t* cu_seqlens_q, const int32_t* seq_lens,
    float softmax_scale, void* out,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One layer's whole batch in one call: decode rows first, then prefill rows.
 * [FI] MiniMaxM3SparseFlashInferImpl.forward: the first num_decode_tokens
 * tokens are the decode tokens (their requests, block table and lengths),
 * the rest are prefill tokens (cu_seqlens_q, block table and lengths of the
 * prefill requests); the top-k rows are token-major over the whole batch.
 *
 * q, out [num_tokens][num_q_heads][head_dim] bf16, contiguous; topk
 * [num_tokens][topk_row_stride].  Rows [0, num_decode_tokens) go through
 * msa_sparse_decode (num_decode_tokens / decode_query_len requests), rows
 * [num_decode_tokens, num_tokens) through msa_sparse_prefill with
 * prefill_cu_seqlens_q counted from the first prefill row; either part may
 * be empty.  Both parts are validated before anything is enqueued; then
 * they run in that order on `stream`, with no host synchronisation (the call
 * can be captured into a HIP graph).  workspace serves both parts in turn
 * (the decode's split-K partials, then the prefill's row orders): the larger
 * of msa_decode_workspace_size and msa_prefill_workspace_size is room for
 * both.
 */
MSA_API msa_status_t msa_sparse_attention(
    const void* q, int32_t q_dtype, int32_t num_tokens, int32_t num_q_heads,
    const msa_kv_cache_t* kv,
    const int32_t* topk, int64_t topk_row_stride, int32_t topk_k,
    int32_t num_decode_tokens, int32_t decode_query_len,
    const int32_t* decode_block_table, int64_t decode_bt_row_stride, int32_t decode_bt_cols,
    const int32_t* decode_seq_lens,
    int32_t num_prefill_reqs,
    const int32_t* prefill_block_table, int64_t prefill_bt_row_stride, int32_t prefill_bt_cols,
    const int32_t* prefill_cu_seqlens_q, const int32_t* prefill_seq_lens,
    float softmax_scale, void* out,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Scatter index keys into the key-only side cache.
 * [SPA] minimax_m3_insert_index_cache: keys [N, D] into a cache [B, T, D]
 * through one int64 slot per key; empty input returns at once; the cache's
 * last dimension must be contiguous.  Slot s (int64) goes to block s / T,
 * position s % T; negative slots (padding) and slots >= B*T are skipped.
 * dtype gives the element size (MSA_BF16 / MSA_FP16: 2 bytes, MSA_FP32: 4,
 * MSA_FP8_E4M3FN: 1); strides are in elements.
 */
MSA_API msa_status_t msa_insert_index_cache(
    const void* index_k, int64_t k_stride0, int64_t k_stride1, int32_t n, int32_t d, int32_t dtype,
    void* index_cache, int64_t c_stride0, int64_t c_stride1, int64_t c_stride2,
    int32_t num_blocks, int32_t cache_block_size,
    const int64_t* slot_mapping, int64_t slot_stride, hipStream_t stream);

/*
 * Test hook: every row's K and V in sparse-table order, as an attend's own
 * gather and dequant produce its matrix operands.  [NV4] customize_spec (the
 * two NVFP4 head slots, codes plus block scales) and [FI]
 * MiniMaxM3SparseFlashInferImpl.forward (the fp8 view and its per-tensor
 * scales); the table is msa_build_sparse_block_table's
 * ([SPA] _write_sparse_block_table_row_from_values).
 *
 * sparse_bt [total_q][sbt_width] int32 (row stride sbt_row_stride), page-16
 * ids; sparse_ctx [total_q] int32.  Token t < sparse_ctx[i] of row i lies in
 * slot t / 128, whose physical block is sparse_bt[i][8 * (t / 128)] /
 * block_page_stride, at offset t % 128 of the block.
 * path 0: the decode attend's gather (chunk addressing, page loads masked at
 *   the context, in-register conversion to the operand types);
 * path 1: the prefill attend's staging (the block copied into LDS, fp8 /
 *   NVFP4 converted there).
 * k_out, v_out [total_q][16 * sbt_width][num_kv_heads][head_dim] fp32: the
 * operand element (bf16 / fp8 / e2m1 x E4M3 block scale, exact in the
 * operand type) times k_scale or v_scale, rounded to nearest fp32.  Tokens at
 * or past sparse_ctx[i], and blocks outside [0, num_pages), give zero (an
 * NVFP4 V element past the context may be -0: its scale is cleared, its
 * unwritten code keeps its sign).
 * sbt_width: a multiple of 8, at most 8 * 1024.
 */
MSA_API msa_status_t msa_debug_gather_dequant(
    const msa_kv_cache_t* kv, const int32_t* sparse_bt, int64_t sbt_row_stride, const int32_t* sparse_ctx,
    int32_t total_q, int32_t sbt_width, int32_t path, float* k_out, float* v_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
