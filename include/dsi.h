/*
 * dsi.h — C ABI of the MI355X (gfx950) DeepSeek Sparse Attention "lightning
 * indexer" hot path.
 *
 * What the path computes is defined on three web pages:
 *   P1 = "V4.1 索引器接入稀疏 MQA logits" (summary of vLLM PR 56254): the
 *        hierarchical (candidate-block) indexer — motivation, implementation
 *        breakdown, key source snippets (candidate expansion kernel, row
 *        metadata), review highlights.
 *   P2 = "修复 DSV4 FlashInfer 稀疏 MLA 在打包 KV 布局下的地址错误" (summary of
 *        vLLM PR 47493): packed-pool block span and the slot remap.
 *   P3 = "DeepSeek V3.2 稀疏注意力 DSA 推理流程图解": cost table, per-layer data
 *        flow, the six indexer steps ①–⑥, the prefill/decode table, pitfalls.
 *
 * Conventions shared by every call
 *   - Fixed shapes: H = 64 indexer heads, D = 128 dims, one 132-byte K cache
 *     row per token = 128 FP8 codes followed by the fp32 scale (P3 cost
 *     table and data flow 1).  Token i of a cache block sits at byte i*132 of
 *     the block.
 *   - FP8 is OCP E4M3FN (max 448) stored as uint8; bf16 is stored as its
 *     uint16 bit pattern.  Leading dimensions ("ld") and strides are in
 *     elements of the array they describe, byte strides say "_bytes".
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates, frees or keeps a pointer after the call returns.
 *   - Each call only enqueues work on `stream` (0 = the default stream) and
 *     returns; it never reads device memory from the host and never
 *     synchronises, so every call may be captured into a HIP graph.
 *   - Arguments known on the host are validated before any HIP call; a
 *     failed check returns a negative status and enqueues nothing (checked
 *     up front, never a slower fallback: P1 review highlights).  Values that
 *     live on the device (row ranges, lengths, candidate ids, block-table
 *     entries) are preconditions; where one is out of range the call still
 *     touches no memory outside the buffers described by its arguments, and
 *     the affected outputs are as documented per call.
 *   - Calls that overlap on one stream are ordered; the library holds no
 *     global state, so calls on different streams are independent — with one
 *     exception: dsi_topk_select_noalloc works in a device array the library
 *     keeps per GPU.
 */
#ifndef DSI_H
#define DSI_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported entry points (the library builds with hidden default visibility). */
#define DSI_API __attribute__((visibility("default")))

#define DSI_HEADS 64
#define DSI_HEAD_DIM 128
#define DSI_ROW_BYTES 132
#define DSI_MAX_TOPK 2048

/* Status codes. */
#define DSI_OK 0
#define DSI_EINVAL (-1)       /* null pointer, negative size, ld/stride smaller than the row */
#define DSI_EUNSUPPORTED (-2) /* a parameter outside what the kernels support (listed per call) */
#define DSI_EALIGN (-3)       /* a pointer or byte stride without the required alignment */
#define DSI_ELAUNCH (-4)      /* the HIP launch itself failed */
#define DSI_EWORKSPACE (-5)   /* workspace missing or smaller than dsi_topk_workspace_bytes() */

/* Element type of the logits given to dsi_topk_select. */
#define DSI_F32 0
#define DSI_BF16 1

/* Human-readable text for a status code (static storage, never NULL). */
DSI_API const char* dsi_status_string(int status);

/* ABI version, bumped on any signature or semantic change. */
DSI_API int dsi_abi_version(void);

/*
 * k quantization fused with cache insertion (P3 step ⑤: k is quantized as it
 * is written into the indexer cache; row layout per P3 data flow 1).
 *   k            bf16 [n][k_ld], first 128 values of each row used.
 *   slot_mapping int64 [n]: destination slot of row i; slot = block*block_size
 *                + offset.  A negative slot, or one at or beyond
 *                num_blocks*block_size, is skipped (padding token).
 *   pool         uint8, num_blocks blocks of block_stride_bytes; token
 *                `offset` of block `block` is the 132 bytes at
 *                block*block_stride_bytes + offset*132.
 * Per token: amax = max|k|, scale = max(amax, 1e-4) / 448 (IEEE fp32
 * division), code[d] = E4M3FN(k[d] / scale) rounded to nearest even and
 * saturated to +-448; the row holds the 128 codes then the fp32 scale.
 * Errors: EINVAL (null with n > 0, n < 0, k_ld < 128, block_size < 1,
 * num_blocks < 0, block_stride_bytes < block_size*132); EALIGN (k not 4-byte
 * aligned or k_ld odd, pool or block_stride_bytes not a multiple of 4).
 */
DSI_API int dsi_k_quant_and_cache(const uint16_t* k, int64_t n, int64_t k_ld, const int64_t* slot_mapping, uint8_t* pool,
                          int64_t num_blocks, int32_t block_size, int64_t block_stride_bytes, hipStream_t stream);

/*
 * Dense prefill indexer logits over gathered K (P3 step ⑥ and the
 * prefill/decode table: prefill gathers the history K, then scores):
 *   logits[t][s] = kscale[s] * sum_h w[t][h] * sum_d q[t][h][d] * k[s][d]
 * for s in [max(row_ks[t],0), min(row_ke[t],S)), with q and k the decoded FP8
 * values (the q scale is folded into w, P3 step ④).  No other entry of
 * `logits` is written.
 *   q      e4m3 [T][64][128] contiguous, 16-byte aligned.
 *   w      bf16 [T][64] contiguous, 8-byte aligned.
 *   k_rows [S][132] contiguous cache rows, 16-byte aligned.
 *   row_ks, row_ke int32 [T].
 *   logits fp32 [T][ld], ld >= S.
 * The FP8 codes are decoded exactly to f16 and contracted on the f16 matrix
 * cores with fp32 accumulation (gfx950's FP8-operand matrix instructions
 * truncate their internal sums); the head reduction is fp32.  Errors: EINVAL (null with T,S > 0, T < 0, S < 0,
 * ld < S); EALIGN.
 */
DSI_API int dsi_mqa_logits_prefill(const uint8_t* q, const uint16_t* w, int32_t T, const uint8_t* k_rows, int32_t S,
                           const int32_t* row_ks, const int32_t* row_ke, float* logits, int64_t ld,
                           hipStream_t stream);

/*
 * Paged decode indexer logits straight from the cache, no gather (P3
 * prefill/decode table).  Request b has context length context_lens[b] = L
 * and next_n query rows (the multi-token draft of P3 "MTP"); row b*next_n+i
 * scores tokens s in [0, min(L - next_n + i + 1, max_context_len)) with the
 * formula of dsi_mqa_logits_prefill, reading token s at
 *   pool + block_table[b*bt_ld + s/block_size]*block_stride_bytes
 *        + (s % block_size)*132.
 * No other entry of `logits` is written.  A token whose page id is outside
 * [0, num_blocks), or whose block index s/block_size >= bt_width, scores
 * -inf.
 *   q [B*next_n][64][128] (16-byte aligned), w bf16 [B*next_n][64] (8-byte
 *   aligned), context_lens int32 [B], pool (16-byte aligned),
 *   block_table int32 [B][bt_ld], logits fp32 [B*next_n][ld],
 *   ld >= max_context_len.
 * Errors: EINVAL (nulls, B < 0, ld < max_context_len, bt_ld < bt_width,
 * block_stride_bytes < block_size*132); EUNSUPPORTED (next_n not in 1..4,
 * block_size not a positive multiple of 16, B > 65535); EALIGN (q, pool,
 * block_stride_bytes not multiples of 16, w not 8-byte aligned).
 */
DSI_API int dsi_paged_mqa_logits_decode(const uint8_t* q, const uint16_t* w, int32_t B, int32_t next_n,
                                const int32_t* context_lens, const uint8_t* pool, int64_t num_blocks,
                                int32_t block_size, int64_t block_stride_bytes, const int32_t* block_table,
                                int64_t bt_ld, int32_t bt_width, int32_t max_context_len, float* logits, int64_t ld,
                                hipStream_t stream);

/* Workspace bytes dsi_paged_mqa_topk_decode(_mxfp4) needs for these sizes (0 = none). */
DSI_API size_t dsi_paged_mqa_topk_decode_workspace_bytes(int32_t B, int32_t next_n, int32_t max_context_len,
                                                         int32_t k);

/*
 * The decode indexer step in one call: the logits of dsi_paged_mqa_logits_decode
 * (same arguments, same `logits` output), then their top-k into the index table
 * main attention reads (P3 data flow 2 and the prefill/decode table: decode scores
 * the paged cache directly, then keeps the k best positions per query row).  Row
 * b*next_n+i selects from its own columns [0, min(L - next_n + i + 1,
 * max_context_len)) with the rules of dsi_topk_select: out[r][0 .. m) holds the
 * positions of m = min(k, finite values) largest logits in any order, then -1.
 * With one row per request and rows long enough to be split (more than 16384
 * columns, fewer than 512 rows), the decode kernel also counts the top-k's
 * first-digit histograms while it writes the logits, which saves the top-k one
 * launch and one read of the logits.
 *   out int32 [B*next_n][out_ld], out_ld >= k; workspace of
 *   dsi_paged_mqa_topk_decode_workspace_bytes(B, next_n, max_context_len, k)
 *   bytes, 16-byte aligned, used by this call only.
 * Errors: those of dsi_paged_mqa_logits_decode; EUNSUPPORTED (k not in 1..2048);
 * EINVAL (out_ld < k, out NULL); EWORKSPACE; EALIGN (out, workspace).
 */
DSI_API int dsi_paged_mqa_topk_decode(const uint8_t* q, const uint16_t* w, int32_t B, int32_t next_n,
                                      const int32_t* context_lens, const uint8_t* pool, int64_t num_blocks,
                                      int32_t block_size, int64_t block_stride_bytes, const int32_t* block_table,
                                      int64_t bt_ld, int32_t bt_width, int32_t max_context_len, float* logits,
                                      int64_t ld, int32_t k, int32_t* out, int64_t out_ld, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/*
 * dsi_paged_mqa_topk_decode on the MXFP4 cache: the logits of
 * dsi_paged_mqa_logits_decode_mxfp4 (68-byte rows), then the same top-k.
 * Errors: as dsi_paged_mqa_topk_decode, with the MXFP4 row stride rules.
 */
DSI_API int dsi_paged_mqa_topk_decode_mxfp4(const uint8_t* q, const uint16_t* w, int32_t B, int32_t next_n,
                                            const int32_t* context_lens, const uint8_t* pool, int64_t num_blocks,
                                            int32_t block_size, int64_t block_stride_bytes,
                                            const int32_t* block_table, int64_t bt_ld, int32_t bt_width,
                                            int32_t max_context_len, float* logits, int64_t ld, int32_t k,
                                            int32_t* out, int64_t out_ld, void* workspace, size_t workspace_bytes,
                                            hipStream_t stream);

/*
 * Workspace bytes dsi_topk_select needs for these sizes (0 = none; pass any
 * pointer or NULL then).
 */
DSI_API size_t dsi_topk_workspace_bytes(int32_t rows, int32_t max_width, int32_t k);

/*
 * Per-row top-k selection into the index table consumed by main attention
 * (P3 data flow 2: the k best positions per query row, int32, -1 = empty
 * slot; P3 pitfalls: positions are request-relative; P1: the compressed-space
 * top-k runs on bf16 logits directly).
 * For row r, let V be the FINITE values in columns [max(start,0),
 * min(row_ends[r], max_width)), start = row_starts ? row_starts[r] : 0.
 * out[r][0 .. m) holds the columns (minus start) of m = min(k, |V|) largest
 * members of V, in no particular order; out[r][m .. k) = -1.  Among values
 * that tie at the selection boundary any subset may be chosen.
 *   logits  fp32 or bf16 (dtype = DSI_F32 / DSI_BF16) [rows][ld], 4-byte
 *           aligned rows for fp32.
 *   out     int32 [rows][out_ld], out_ld >= k.
 * Errors: EINVAL (nulls, rows < 0, max_width < 0, ld < max_width,
 * out_ld < k); EUNSUPPORTED (k not in 1..2048, unknown dtype);
 * EWORKSPACE.
 */
DSI_API int dsi_topk_select(const void* logits, int32_t dtype, int64_t ld, int32_t rows, const int32_t* row_starts,
                    const int32_t* row_ends, int32_t max_width, int32_t k, int32_t* out, int64_t out_ld,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Size of the device array dsi_topk_select_noalloc works in (one per GPU). */
#define DSI_TOPK_NOALLOC_MAX_BYTES (16u << 20)

/*
 * dsi_topk_select for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops that forbid allocation): the same selection, rules
 * and errors, with the workspace taken from a device array of
 * DSI_TOPK_NOALLOC_MAX_BYTES that the library holds on each GPU it runs on until
 * the process ends.  The call itself allocates and frees nothing; on its first
 * call on a GPU it looks up that GPU's array (a symbol-address query).  Every
 * call on one GPU works in the same array and leaves its contents behind, so
 * calls that overlap on one GPU (on different streams, or captured graphs
 * replayed concurrently) race and give undefined results; calls ordered on one
 * stream are safe.  Sizes whose workspace (dsi_topk_workspace_bytes) exceeds the
 * array return DSI_EWORKSPACE before any HIP call.
 */
DSI_API int dsi_topk_select_noalloc(const void* logits, int32_t dtype, int64_t ld, int32_t rows,
                                    const int32_t* row_starts, const int32_t* row_ends, int32_t max_width,
                                    int32_t k, int32_t* out, int64_t out_ld, hipStream_t stream);

/*
 * Candidate expansion of the hierarchical indexer (P1 key source snippets:
 * the per-row expansion kernel and its wrapper).  With ratio =
 * candidate_block_size / sparse_block_kv, per row:
 *   flatten: candidate c -> sparse blocks c*ratio .. c*ratio+ratio-1;
 *   keep ids in [0, ceil(max(ke-ks,0)/sbk)); sort ascending, duplicates kept;
 *   add the anchor floor(ks/sbk); pad the tail with the last kept id (or the
 *   anchor when none is kept);
 *   end = (n-1)*sbk + min(max(ke - (last*sbk + ks), 1), sbk), 0 when n = 0.
 *   cand int32 [rows][cand_ld] (column slices allowed), row_ks/row_ke int32
 *   with element strides ks_stride/ke_stride, sparse_indices int32
 *   [rows][si_ld] (first num_candidates*ratio columns written), end int32
 *   with element stride end_stride.
 * Preconditions: 0 <= ks, ke < 2^31 - sparse_block_kv (int32 arithmetic).
 * Errors: EINVAL (nulls, rows < 0, num_candidates < 1, cand_ld <
 * num_candidates, si_ld < num_candidates*ratio, strides < 1);
 * EUNSUPPORTED (ratio not 1 or 2 or not exact, sparse_block_kv not a power
 * of two in 8..128, num_candidates*ratio > 1024).
 */
DSI_API int dsi_expand_candidates(const int32_t* cand, int64_t cand_ld, int32_t rows, int32_t num_candidates,
                          const int32_t* row_ks, int64_t ks_stride, const int32_t* row_ke, int64_t ke_stride,
                          int32_t candidate_block_size, int32_t sparse_block_kv, int32_t* sparse_indices,
                          int64_t si_ld, int32_t* end, int64_t end_stride, hipStream_t stream);

/*
 * Sparse MQA logits on the candidate columns only (P1 motivation and
 * implementation: consumer layers score only the candidate blocks into bf16
 * logits [rows, num_sparse_blocks*sparse_block_kv]).  Column c of row r is
 * token tok = sparse_indices[r][c/sbk]*sbk + c%sbk; when c < end[r] and
 * row_ks[r] <= tok < row_ke[r] it holds the logit of that token (formula of
 * dsi_mqa_logits_prefill) rounded once to bf16 (nearest even), otherwise
 * bf16 -inf (0xFF80).  Every column of every row is written.
 *   K source: block_table == NULL -> k_src is gathered rows [num_k][132]
 *     (a token >= num_k scores -inf); otherwise k_src is a paged pool of
 *     num_k blocks and row r reads block_table[req*bt_ld + tok/block_size]
 *     with req = row_to_req ? row_to_req[r] : r, the table having num_reqs
 *     rows (a req outside [0,num_reqs), a block index >= bt_width or a page
 *     id outside [0,num_k) scores -inf).
 *   q, w as dsi_mqa_logits_prefill with `rows` rows; sparse_indices int32
 *   [rows][si_ld]; end, row_ks, row_ke int32 [rows]; out bf16 [rows][ld],
 *   ld >= num_sparse_blocks*sparse_block_kv.
 * Errors: EINVAL (nulls, rows < 0, num_sparse_blocks < 1, si_ld <
 * num_sparse_blocks, ld too small, bt_ld < bt_width); EUNSUPPORTED
 * (sparse_block_kv not a power of two in 8..128, block_size not a positive
 * multiple of sparse_block_kv and of 8, rows > 65535); EALIGN (q, k_src, block stride not
 * multiples of 16, w not 8-byte aligned).
 */
DSI_API int dsi_sparse_mqa_logits(const uint8_t* q, const uint16_t* w, int32_t rows, const int32_t* row_ks,
                          const int32_t* row_ke, const int32_t* sparse_indices, int64_t si_ld,
                          int32_t num_sparse_blocks, const int32_t* end, int32_t sparse_block_kv,
                          const uint8_t* k_src, int64_t num_k, const int32_t* block_table, int64_t bt_ld,
                          int32_t bt_width, int32_t num_reqs, const int32_t* row_to_req, int32_t block_size,
                          int64_t block_stride_bytes, uint16_t* logits_bf16, int64_t ld, hipStream_t stream);

/*
 * The per-step schedule of the sparse columns (P1 key source snippets and
 * implementation breakdown: the row metadata of the sparse logits is computed
 * once per step and reused by every later consumer layer, as the expansion is;
 * the layers share the block tables and differ only in their K).  For row r
 * and sparse block j (tokens tok0 + o, o < sparse_block_kv, tok0 =
 * sparse_indices[r][j]*sparse_block_kv) one 8-byte entry: the byte offset of
 * the block's first token's row in the K source divided by 4, and the range
 * [lo, hi) of o whose columns dsi_sparse_mqa_logits would score (c < end[r],
 * row_ks[r] <= tok < row_ke[r], tok >= 0, the row inside the source as that
 * call checks it), packed base | lo << 32 | hi << 40; 0xFFFFFFFF with
 * lo = hi = 0 when none.  row_bytes: 132 (FP8 rows, for
 * dsi_sparse_mqa_logits_scheduled) or 68 (MXFP4 rows, for its _mxfp4 form).
 * Every other argument is that of dsi_sparse_mqa_logits(_mxfp4), with the same
 * checks and errors.
 *   schedule uint64 [rows][num_sparse_blocks] (dsi_sparse_schedule_bytes),
 *   8-byte aligned.
 */
DSI_API size_t dsi_sparse_schedule_bytes(int32_t rows, int32_t num_sparse_blocks);
DSI_API int dsi_sparse_schedule(int32_t rows, const int32_t* row_ks, const int32_t* row_ke,
                                const int32_t* sparse_indices, int64_t si_ld, int32_t num_sparse_blocks,
                                const int32_t* end, int32_t sparse_block_kv, int32_t row_bytes, int64_t num_k,
                                const int32_t* block_table, int64_t bt_ld, int32_t bt_width, int32_t num_reqs,
                                const int32_t* row_to_req, int32_t block_size, int64_t block_stride_bytes,
                                uint64_t* schedule, hipStream_t stream);

/*
 * dsi_sparse_mqa_logits with the columns' sources taken from a schedule
 * (dsi_sparse_schedule with row_bytes 132): the same bf16 logits, -inf where
 * the schedule has no valid column.  k_src is the K source (gathered rows or
 * paged pool, as the schedule was built for) of k_src_bytes bytes; a column
 * whose row would extend past k_src_bytes scores -inf, so a schedule cannot
 * lead outside the source.  One schedule serves every layer of a step.
 * Errors: EINVAL (nulls, rows < 0, num_sparse_blocks < 1, ld too small,
 * k_src_bytes < 0); EUNSUPPORTED (sparse_block_kv not a power of two in
 * 8..128, rows > 65535, k_src_bytes >= 2^34); EALIGN (q, k_src 16-byte, w,
 * schedule 8-byte aligned).
 */
DSI_API int dsi_sparse_mqa_logits_scheduled(const uint8_t* q, const uint16_t* w, int32_t rows,
                                            const uint64_t* schedule, int32_t num_sparse_blocks,
                                            int32_t sparse_block_kv, const uint8_t* k_src, int64_t k_src_bytes,
                                            uint16_t* logits_bf16, int64_t ld, hipStream_t stream);

/* dsi_sparse_mqa_logits_scheduled on MXFP4 rows (schedule built with row_bytes 68). */
DSI_API int dsi_sparse_mqa_logits_scheduled_mxfp4(const uint8_t* q, const uint16_t* w, int32_t rows,
                                                  const uint64_t* schedule, int32_t num_sparse_blocks,
                                                  int32_t sparse_block_kv, const uint8_t* k_src, int64_t k_src_bytes,
                                                  uint16_t* logits_bf16, int64_t ld, hipStream_t stream);

/*
 * Sparse column -> request-local position (P1 implementation breakdown: the
 * compressed-space top-k is mapped back to context positions):
 *   out[r][j] = (sparse_indices[r][c/sbk] - floor(row_ks[r]/sbk))*sbk + c%sbk
 * for c = col[r][j] >= 0; -1 stays -1, as does c >= num_sparse_blocks*sbk.
 * out may alias col (same pointer and ld).
 * Errors: EINVAL (nulls, rows < 0, k < 0, lds smaller than k or
 * num_sparse_blocks); EUNSUPPORTED (sparse_block_kv < 1, rows > 65535).
 */
DSI_API int dsi_topk_remap(const int32_t* col, int64_t col_ld, int32_t rows, int32_t k, const int32_t* sparse_indices,
                   int64_t si_ld, int32_t num_sparse_blocks, const int32_t* row_ks, int32_t sparse_block_kv,
                   int32_t* out, int64_t out_ld, hipStream_t stream);

/*
 * Request-local position -> physical cache slot (P3 pitfalls: decode converts
 * the indexer's request-relative positions into paged-cache slots; P2 key
 * source snippets: in a packed pool a slot is block*block_span + offset, -1
 * stays -1):
 *   out[r][j] = block_table[req*bt_ld + p/block_size]*block_span
 *               + p%block_size
 * for p = idx[r][j] >= 0 and req = row_to_req ? row_to_req[r] : r; -1 for
 * p < 0, p/block_size >= bt_width, or req outside [0, num_reqs) (the rows of
 * block_table).  block_span = block stride / 132 (equal
 * to block_size for an unpacked pool).  out may alias idx.
 * Errors: EINVAL (nulls, rows < 0, k < 0, lds < k, bt_ld < bt_width);
 * EUNSUPPORTED (block_size < 1, block_span < block_size, rows > 65535).
 */
DSI_API int dsi_req_index_to_global_slot(const int32_t* idx, int64_t idx_ld, int32_t rows, int32_t k,
                                 const int32_t* row_to_req, const int32_t* block_table, int64_t bt_ld,
                                 int32_t bt_width, int32_t num_reqs, int32_t block_size, int32_t block_span, int32_t* out,
                                 int64_t out_ld, hipStream_t stream);

/*
 * Prefill K gather: the history K of a prefill chunk's requests copied out of
 * the paged cache into contiguous 132-byte rows, the input of
 * dsi_mqa_logits_prefill and of the gathered form of dsi_sparse_mqa_logits
 * (P3 prefill/decode table: prefill collects the history K before scoring,
 * decode reads the cache where it lies; P1 implementation breakdown: the
 * indexer's forward chains the prefill K gather with paged decode).
 * The requests lie end to end: request r owns rows [cu_seq_lens[r],
 * cu_seq_lens[r+1]) of k_rows and its row cu_seq_lens[r] + p is its token p,
 * read from
 *   pool + block_table[r*bt_ld + p/block_size]*block_stride_bytes
 *        + (p % block_size)*132
 * and copied byte for byte.  Rows that no request owns, and tokens whose
 * block index p/block_size >= bt_width or whose page id is outside
 * [0, num_blocks), are written as zero rows.  Exactly rows [0, S) are written.
 *   pool         paged cache, num_blocks blocks of block_stride_bytes.
 *   block_table  int32 [num_reqs][bt_ld]: the chunk's requests' tables.
 *   cu_seq_lens  int32 [num_reqs + 1], non-decreasing (precondition: with
 *                decreasing entries the rows they touch are unspecified, but
 *                no memory outside the arguments is read or written).
 *   k_rows       [S][132] output, 16-byte aligned.
 * Errors: EINVAL (nulls with S > 0, S < 0, num_reqs < 0, num_blocks < 0,
 * block_size < 1, bt_width < 0, bt_ld < bt_width, block_stride_bytes <
 * block_size*132); EUNSUPPORTED (S > 2^31 - 129); EALIGN (k_rows not 16-byte
 * aligned, pool or block_stride_bytes not multiples of 4).
 */
DSI_API int dsi_gather_prefill_k(const uint8_t* pool, int64_t num_blocks, int32_t block_size,
                                 int64_t block_stride_bytes, const int32_t* block_table, int64_t bt_ld,
                                 int32_t bt_width, const int32_t* cu_seq_lens, int32_t num_reqs, uint8_t* k_rows,
                                 int32_t S, hipStream_t stream);

/*
 * q preparation in one pass (P3 indexer steps ③ and ④, P3 pitfalls; P1
 * implementation breakdown: the fused q kernel writes bf16 head weights, the
 * fp32 result rounded once).  For token t and head h, with x the 128 bf16
 * values of q widened to fp32 and p = positions[t]:
 *   RoPE on dims 0..63 only: frequency i (0..31) rotates the pair (a, b) =
 *     (i, i+32), or (2i, 2i+1) when interleave != 0, by c = cos_sin[p][i],
 *     s = cos_sin[p][32+i]:  a' = a*c - b*s,  b' = b*c + a*s
 *     (each product and sum one fp32 rounding, no fused multiply-add);
 *   scale = max(amax, 1e-4)/448, q8[t][h][d] = E4M3FN(x[d]/scale) (IEEE
 *     division, nearest even, saturating) — the k quantization rule;
 *   w_out[t][h] = bf16(((w[t][h] * scale) * softmax_scale) * head_scale),
 *     fp32 products, rounded to bf16 once (nearest even).
 * A position outside [0, max_pos) gives zero codes and a zero weight.
 *   q          bf16 [T][q_ld], head h at elements h*128 .. h*128+127;
 *              16-byte aligned, q_ld a multiple of 8.
 *   positions  int64 [T].
 *   cos_sin    fp32 [max_pos][64]: the 32 cosines, then the 32 sines;
 *              16-byte aligned.
 *   w          bf16 [T][w_ld], the raw head weights.
 *   q8         e4m3 [T][64][128] contiguous (8-byte aligned): the input of
 *              the logits calls.  w_out bf16 [T][64] contiguous.
 * Errors: EINVAL (nulls with T > 0, T < 0, q_ld < 8192, w_ld < 64,
 * max_pos < 1); EALIGN.
 */
DSI_API int dsi_q_rope_quant(const uint16_t* q, int64_t q_ld, int32_t T, const int64_t* positions,
                             const float* cos_sin, int64_t max_pos, int32_t interleave, const uint16_t* w,
                             int64_t w_ld, float softmax_scale, float head_scale, uint8_t* q8, uint16_t* w_out,
                             hipStream_t stream);

/*
 * One rank's top-k candidates under context parallelism (P3 pitfalls: with a
 * request's context split across ranks, each rank keeps only its local top-k
 * candidates, and those, not the score matrix, are exchanged).  For row r and
 * j < k, with p = idx[r][j] (a selection relative to the row's start, as
 * dsi_topk_select emits it) and start = row_starts ? max(row_starts[r], 0) : 0:
 *   vals[r][j] = logits[r][start + p],
 *   gidx[r][j] = p*index_scale + index_offset   (int32, wrapping),
 * and (-inf, -1) where p < 0 or start + p >= max_width.  The scale and offset
 * map the rank's columns to positions in the whole context: 1 and the slice's
 * first position for contiguous slices, R and the rank for round-robin ones.
 *   logits fp32 [rows][ld], ld >= max_width; idx int32 [rows][idx_ld];
 *   vals fp32 [rows][vals_ld]; gidx int32 [rows][gidx_ld]; lds >= k.
 * Errors: EINVAL (nulls with rows, k > 0; negative sizes; lds too small);
 * EUNSUPPORTED (rows > 65535); EALIGN (pointers not 4-byte aligned).
 */
DSI_API int dsi_topk_values(const float* logits, int64_t ld, int32_t rows, const int32_t* row_starts, int32_t max_width,
                            const int32_t* idx, int64_t idx_ld, int32_t k, int32_t index_scale, int32_t index_offset,
                            float* vals, int64_t vals_ld, int32_t* gidx, int64_t gidx_ld, hipStream_t stream);

/* Workspace bytes dsi_topk_merge needs (0 for empty sizes). */
DSI_API size_t dsi_topk_merge_workspace_bytes(int32_t rows, int32_t num_lists, int32_t k_in);

/*
 * Merge of the ranks' exchanged candidate lists into the global top-k (P3
 * pitfalls: the global top-k is chosen from the local candidates; exact, as a
 * token of the global top-k is in the local top-k of the rank holding it).
 * Row r of list l holds k_in (value, global index) pairs at
 * l*list_stride + r*row_ld in `vals` and `gidx` (an all-gather of every rank's
 * dsi_topk_values output gives list_stride = rows*row_ld).  Pairs with a
 * negative index or a non-finite value are ignored.  out[r][0 .. m) holds the
 * global indices of the m = min(k, #valid) largest values, in no particular
 * order (ties at the boundary broken either way), then -1.
 *   out int32 [rows][out_ld], out_ld >= k; workspace of
 *   dsi_topk_merge_workspace_bytes(rows, num_lists, k_in) bytes, 16-byte
 *   aligned, used by this call only.
 * Errors: EINVAL (nulls, rows < 0, num_lists < 1, k_in < 1, row_ld < k_in,
 * out_ld < k); EUNSUPPORTED (k not in 1..2048, num_lists*k_in >= 2^31,
 * rows > 65535); EWORKSPACE; EALIGN.
 */
DSI_API int dsi_topk_merge(const float* vals, const int32_t* gidx, int64_t list_stride, int64_t row_ld,
                           int32_t num_lists, int32_t rows, int32_t k_in, int32_t k, int32_t* out, int64_t out_ld,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The MXFP4 indexer cache (P1 motivation and implementation: the V4.1 sparse
 * indexer reads an MXFP4 indexer cache, checked at start-up, and scores FP8 q
 * against FP4 k).  The pages name the format only; it is the OCP
 * Microscaling format — FP4 E2M1 elements (magnitudes 0, .5, 1, 1.5, 2, 3, 4,
 * 6) sharing one E8M0 scale 2^(E-127) per 32 — in 68-byte rows: 64 bytes of
 * codes (element 2i in the low nibble of byte i, 2i+1 in the high nibble),
 * then the 4 scale bytes of dims 32j..32j+31.  Token i of a block sits at
 * byte i*68 of the block.
 *
 * k quantization into that cache, fused with insertion (as
 * dsi_k_quant_and_cache, same arguments; rows of 68 bytes).  Per block of 32:
 * shared exponent se = floor(log2(amax)) - 2 clamped to [-127, 127] (-127
 * for an all-zero block), scale byte se + 127, codes FP4(x * 2^-se) rounded
 * to nearest even and saturated at +-6 (a value that rounds to zero keeps
 * its sign).
 * Errors: EINVAL (null with n > 0, n < 0, k_ld < 128, block_size < 1,
 * num_blocks < 0, block_stride_bytes < block_size*68); EALIGN (k not 4-byte
 * aligned or k_ld odd, pool or block_stride_bytes not multiples of 4).
 */
DSI_API int dsi_k_quant_and_cache_mxfp4(const uint16_t* k, int64_t n, int64_t k_ld, const int64_t* slot_mapping,
                                        uint8_t* pool, int64_t num_blocks, int32_t block_size,
                                        int64_t block_stride_bytes, hipStream_t stream);

/*
 * Sparse MQA logits on the MXFP4 cache: dsi_sparse_mqa_logits with every key
 * row read as a 68-byte MXFP4 row (gathered rows [num_k][68] when block_table
 * is NULL, else the paged pool).  The key's value is code * 2^(E-127) of its
 * block; everything else (columns, masking, bf16 rounding, -inf) is as in
 * dsi_sparse_mqa_logits.  Decoded values are exact in bf16 for block scales
 * with E <= 252 (larger ones overflow, as they do in fp32).
 * Errors: as dsi_sparse_mqa_logits, with block_stride_bytes >= block_size*68.
 */
DSI_API int dsi_sparse_mqa_logits_mxfp4(const uint8_t* q, const uint16_t* w, int32_t rows, const int32_t* row_ks,
                                        const int32_t* row_ke, const int32_t* sparse_indices, int64_t si_ld,
                                        int32_t num_sparse_blocks, const int32_t* end, int32_t sparse_block_kv,
                                        const uint8_t* k_src, int64_t num_k, const int32_t* block_table,
                                        int64_t bt_ld, int32_t bt_width, int32_t num_reqs, const int32_t* row_to_req,
                                        int32_t block_size, int64_t block_stride_bytes, uint16_t* logits_bf16,
                                        int64_t ld, hipStream_t stream);

/*
 * Paged decode logits on the MXFP4 cache (P1 motivation and implementation:
 * the V4.1 indexer cache holds MXFP4 keys; P3 prefill/decode table: decode
 * reads the paged cache directly): dsi_paged_mqa_logits_decode with token s
 * read as a 68-byte MXFP4 row (dsi_k_quant_and_cache_mxfp4's layout) at
 *   pool + block_table[b*bt_ld + s/block_size]*block_stride_bytes
 *        + (s % block_size)*68,
 * whose value is code * 2^(E-127) of its 32-dim block; no per-token scale
 * follows.  Rows, ranges, -inf for absent pages and every other rule are those
 * of dsi_paged_mqa_logits_decode.  The codes are decoded exactly to bf16 and
 * contracted on the bf16 matrix cores with fp32 accumulation.
 * Errors: as dsi_paged_mqa_logits_decode, with block_stride_bytes >=
 * block_size*68 (and a multiple of 16).
 */
DSI_API int dsi_paged_mqa_logits_decode_mxfp4(const uint8_t* q, const uint16_t* w, int32_t B, int32_t next_n,
                                              const int32_t* context_lens, const uint8_t* pool, int64_t num_blocks,
                                              int32_t block_size, int64_t block_stride_bytes,
                                              const int32_t* block_table, int64_t bt_ld, int32_t bt_width,
                                              int32_t max_context_len, float* logits, int64_t ld,
                                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSI_H */
