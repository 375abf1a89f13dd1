/*
 * CPU oracle for the DeepSeek Sparse Attention "lightning indexer" hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with the
 * HIP library; both sides receive the same input bytes and nothing else.
 *
 * Plain, slow, single-threaded C.  Floating point is fp32 on the dequantized
 * FP8 values (the precision the problem statement fixes); build with
 * -O2 -ffp-contract=off and never with fast-math, so every product and sum is
 * one IEEE fp32 operation in the order written below.
 *
 * Sources (the three web pages this indexer is described on):
 *   P1 = "V4.1 索引器接入稀疏 MQA logits" (summary of vLLM PR 56254):
 *        sections "功能与动机" (motivation), "实现拆解" (implementation),
 *        "关键源码片段" (key source snippets: the candidate-expansion kernel
 *        and the row metadata), "评论区精华" (review), "风险与影响" (risks).
 *   P2 = "修复 DSV4 FlashInfer 稀疏 MLA 在打包 KV 布局下的地址错误" (summary
 *        of vLLM PR 47493): "实现拆解" and "关键源码片段" (packed block span
 *        and the index remap device function).
 *   P3 = "DeepSeek V3.2 稀疏注意力 DSA 推理流程图解": the cost table
 *        ("打分器为什么开销小"), the per-layer data flow
 *        ("一层里的数据是怎么流的"), the six indexer steps
 *        ("Indexer内部到底做了什么", steps ①–⑥) and the pitfalls
 *        ("几个容易踩的点").
 *
 * Parity pins: every function here is checked by the CPU test suite against
 * something other than itself (library routines, closed forms, brute force,
 * hand-derived cases, invariants).  See the test files for each pin.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_H 64   /* indexer heads (P3, step ①: 64 heads of 128 dims) */
#define ORC_D 128  /* head dim; one shared 128-d k per token (P3, step ①) */
#define ORC_ROW 132 /* cache row: 128 FP8 codes + fp32 scale (P3, data flow 1) */

/* ------------------------------------------------------------------------ */
/* O0 codecs                                                                 */
/* ------------------------------------------------------------------------ */

/* OCP FP8 E4M3FN (P3 cost table and step ④ say "FP8"; the layout is the
 * 8-bit e4m3 format with no infinities, max 448).  Closed form per field. */
float orc_e4m3_decode(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  float v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexpf((float)m, -9); /* subnormal: m * 2^-9 */
  else
    v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
  return s ? -v : v;
}

/* Nearest e4m3 code to a finite x, ties to the code with the even mantissa,
 * saturating to +-448.  The non-negative finite codes 0x00..0x7E decode to
 * strictly increasing values, so the nearest code is one of the two codes
 * that bracket |x|: a binary search finds the largest code not above |x|,
 * then the nearer of it and its successor is taken.  The sign of x is kept,
 * so a negative value that rounds to zero gives -0 (0x80). */
uint8_t orc_e4m3_encode(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x), dlo, dhi;
  int lo = 0, hi = 0x7E;
  if (a >= 448.0) return sign | 0x7E;
  while (lo < hi) { /* largest code c with decode(c) <= a */
    int mid = (lo + hi + 1) / 2;
    if ((double)orc_e4m3_decode((uint8_t)mid) <= a)
      lo = mid;
    else
      hi = mid - 1;
  }
  dlo = a - (double)orc_e4m3_decode((uint8_t)lo);
  dhi = (double)orc_e4m3_decode((uint8_t)(lo + 1)) - a;
  if (dhi < dlo || (dhi == dlo && ((lo + 1) & 1) == 0)) lo = lo + 1;
  return sign | (uint8_t)lo;
}

static uint32_t f32_bits(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return u;
}

/* bf16 with round-to-nearest-even on the fp32 bit pattern (finite or inf). */
uint16_t orc_bf16_rne(float x) {
  uint32_t u = f32_bits(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float x;
  memcpy(&x, &u, 4);
  return x;
}

/* ------------------------------------------------------------------------ */
/* O1 k quantization fused with cache insertion (P3 step ⑤; 132-byte row,   */
/* P3 data flow 1).  The pages name the operation and its arguments only;    */
/* the per-token scale rule max(amax, 1e-4)/448 with IEEE division and the   */
/* row layout (codes, then the fp32 scale, token i of a block at i*132) are  */
/* the readings recorded with the design.                                    */
/* ------------------------------------------------------------------------ */
void orc_k_quant_and_cache(const uint16_t* k, int64_t n, int64_t k_ld, const int64_t* slot_mapping,
                           uint8_t* pool, int32_t block_size, int64_t block_stride) {
  int64_t i;
  int d;
  for (i = 0; i < n; i++) {
    int64_t slot = slot_mapping[i];
    float x[ORC_D], amax = 0.0f, scale;
    uint8_t* row;
    if (slot < 0) continue; /* padding token: nothing written */
    for (d = 0; d < ORC_D; d++) {
      x[d] = orc_bf16_to_f32(k[i * k_ld + d]);
      if (fabsf(x[d]) > amax) amax = fabsf(x[d]);
    }
    scale = (amax > 1e-4f ? amax : 1e-4f) / 448.0f;
    row = pool + (slot / block_size) * block_stride + (slot % block_size) * ORC_ROW;
    for (d = 0; d < ORC_D; d++) row[d] = orc_e4m3_encode(x[d] / scale);
    memcpy(row + ORC_D, &scale, 4); /* little-endian fp32 */
  }
}

/* ------------------------------------------------------------------------ */
/* O2 indexer logits (P3 step ⑥):                                            */
/*   logits[t,s] = sum_h w[t,h] * (q[t,h] . k[s])                            */
/* with q the FP8 codes (their scale already folded into w, P3 step ④) and   */
/* k[s] = decode(codes) * scale of its cache row.  No activation: the page   */
/* states the score as this linear weighted sum.                             */
/* ------------------------------------------------------------------------ */

/* q row decoded and transposed to [d][h], so the head loop is innermost.
 * Each head's dot product is still summed over d in ascending order, one
 * fp32 multiply and one fp32 add per term; only independent accumulators are
 * interleaved, nothing is reassociated. */
static void decode_q_row(const uint8_t* q, const uint16_t* w, float qt[ORC_D][ORC_H], float wf[ORC_H]) {
  int h, d;
  for (h = 0; h < ORC_H; h++) {
    wf[h] = orc_bf16_to_f32(w[h]);
    for (d = 0; d < ORC_D; d++) qt[d][h] = orc_e4m3_decode(q[h * ORC_D + d]);
  }
}

/* The logit of one query row against one decoded key vector kd[128]. */
static float logit_kd(float qt[ORC_D][ORC_H], const float wf[ORC_H], const float kd[ORC_D]) {
  float dot[ORC_H], acc = 0.0f;
  int h, d;
  for (h = 0; h < ORC_H; h++) dot[h] = 0.0f;
  for (d = 0; d < ORC_D; d++)
    for (h = 0; h < ORC_H; h++) dot[h] = dot[h] + qt[d][h] * kd[d];
  for (h = 0; h < ORC_H; h++) acc = acc + wf[h] * dot[h];
  return acc;
}

static float logit_one(float qt[ORC_D][ORC_H], const float wf[ORC_H], const uint8_t* krow) {
  float kd[ORC_D], kscale;
  int d;
  memcpy(&kscale, krow + ORC_D, 4);
  for (d = 0; d < ORC_D; d++) kd[d] = orc_e4m3_decode(krow[d]) * kscale;
  return logit_kd(qt, wf, kd);
}

/* Prefill over gathered K rows (P3 prefill/decode table: prefill gathers the
 * history K first).  Row t scores s in [ks[t], ke[t]); every other column in
 * [0, S) gets -inf. */
void orc_mqa_logits_gathered(const uint8_t* q, const uint16_t* w, int32_t rows, const uint8_t* k_rows, int32_t S,
                             const int32_t* ks, const int32_t* ke, float* logits, int64_t ld) {
  float qt[ORC_D][ORC_H]; /* 32 KB on the caller's stack: concurrent calls from several threads stay independent */
  float wf[ORC_H];
  int32_t t, s;
  for (t = 0; t < rows; t++) {
    decode_q_row(q + (int64_t)t * ORC_H * ORC_D, w + (int64_t)t * ORC_H, qt, wf);
    for (s = 0; s < S; s++) {
      float* o = logits + (int64_t)t * ld + s;
      if (s >= ks[t] && s < ke[t])
        *o = logit_one(qt, wf, k_rows + (int64_t)s * ORC_ROW);
      else
        *o = -INFINITY;
    }
  }
}

/* Decode straight from the paged cache, no gather (P3 prefill/decode table).
 * Request b has context length L_b and next_n query rows; row b*next_n + i
 * sees tokens [0, L_b - next_n + i + 1) (the draft rows of a multi-token
 * step, P3 "MTP / nextn"; the reading is recorded with the design).  Token s
 * of request b lives at pool + bt[b][s / bs] * block_stride + (s % bs) * 132.
 * Columns in [0, width) outside the row's range get -inf. */
void orc_mqa_logits_paged(const uint8_t* q, const uint16_t* w, int32_t B, int32_t next_n, const int32_t* context_lens,
                          const uint8_t* pool, int32_t block_size, int64_t block_stride, const int32_t* block_table,
                          int64_t bt_ld, int32_t width, float* logits, int64_t ld) {
  float qt[ORC_D][ORC_H]; /* 32 KB on the caller's stack: concurrent calls from several threads stay independent */
  float wf[ORC_H];
  int32_t b, i, s;
  for (b = 0; b < B; b++) {
    for (i = 0; i < next_n; i++) {
      int64_t r = (int64_t)b * next_n + i;
      int32_t ke = context_lens[b] - next_n + i + 1;
      decode_q_row(q + r * ORC_H * ORC_D, w + r * ORC_H, qt, wf);
      for (s = 0; s < width; s++) {
        float* o = logits + r * ld + s;
        if (s >= 0 && s < ke) {
          int32_t page = block_table[(int64_t)b * bt_ld + s / block_size];
          const uint8_t* krow = pool + (int64_t)page * block_stride + (int64_t)(s % block_size) * ORC_ROW;
          *o = logit_one(qt, wf, krow);
        } else {
          *o = -INFINITY;
        }
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* O3 top-k selection (P3 data flow 2: the k = 2048 highest-scoring tokens   */
/* per query row go into an int32 table where -1 marks an empty slot; P3     */
/* pitfalls: the indexer emits request-relative positions).                  */
/* Definition: among finite values in [start, end), the k largest; emitted   */
/* as col - start in the order (value desc, col asc), then -1.               */
/* ------------------------------------------------------------------------ */
typedef struct {
  float v;
  int32_t c;
} orc_vc;

static int cmp_vc(const void* a, const void* b) {
  const orc_vc* x = (const orc_vc*)a;
  const orc_vc* y = (const orc_vc*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->c > y->c) - (x->c < y->c);
}

static void topk_row(const float* vals, int32_t start, int32_t end, int32_t k, int32_t* out, orc_vc* buf) {
  int32_t c, n = 0, j;
  for (c = start; c < end; c++) {
    float v = vals[c];
    if (isfinite(v)) {
      buf[n].v = v;
      buf[n].c = c;
      n++;
    }
  }
  qsort(buf, (size_t)n, sizeof(orc_vc), cmp_vc);
  for (j = 0; j < k; j++) out[j] = j < n ? buf[j].c - start : -1;
}

/* Returns 0, or -1 if the scratch allocation fails. */
int orc_topk_select_f32(const float* x, int64_t ld, int32_t rows, const int32_t* starts, const int32_t* ends,
                        int32_t max_width, int32_t k, int32_t* out, int64_t out_ld) {
  int32_t r;
  orc_vc* buf = (orc_vc*)malloc(sizeof(orc_vc) * (size_t)(max_width > 0 ? max_width : 1));
  if (!buf) return -1;
  for (r = 0; r < rows; r++) {
    int32_t st = starts ? starts[r] : 0;
    int32_t en = ends[r];
    if (en > max_width) en = max_width;
    if (st < 0) st = 0;
    topk_row(x + (int64_t)r * ld, st, en, k, out + (int64_t)r * out_ld, buf);
  }
  free(buf);
  return 0;
}

/* bf16 rows (P1: the compressed-space top-k runs on the bf16 sparse logits
 * directly).  Each value is decoded exactly to fp32 first. */
int orc_topk_select_bf16(const uint16_t* x, int64_t ld, int32_t rows, const int32_t* starts, const int32_t* ends,
                         int32_t max_width, int32_t k, int32_t* out, int64_t out_ld) {
  int32_t r, c;
  float* row = (float*)malloc(sizeof(float) * (size_t)(max_width > 0 ? max_width : 1));
  orc_vc* buf = (orc_vc*)malloc(sizeof(orc_vc) * (size_t)(max_width > 0 ? max_width : 1));
  if (!row || !buf) {
    free(row);
    free(buf);
    return -1;
  }
  for (r = 0; r < rows; r++) {
    int32_t st = starts ? starts[r] : 0;
    int32_t en = ends[r];
    if (en > max_width) en = max_width;
    if (st < 0) st = 0;
    for (c = 0; c < max_width; c++) row[c] = orc_bf16_to_f32(x[(int64_t)r * ld + c]);
    topk_row(row, st, en, k, out + (int64_t)r * out_ld, buf);
  }
  free(row);
  free(buf);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O4 request-local position -> physical cache slot (P3 pitfalls: decode     */
/* converts the indexer's request-relative positions to paged-cache slots;   */
/* P2 key source snippets: with a packed pool the slot is                    */
/* block * block_span + offset, and -1 stays -1).                            */
/* ------------------------------------------------------------------------ */
void orc_req_index_to_global_slot(const int32_t* idx, int64_t idx_ld, int32_t rows, int32_t k,
                                  const int32_t* row_to_req, const int32_t* block_table, int64_t bt_ld,
                                  int32_t block_size, int32_t block_span, int32_t* out, int64_t out_ld) {
  int32_t r, j;
  for (r = 0; r < rows; r++) {
    int32_t req = row_to_req ? row_to_req[r] : r;
    for (j = 0; j < k; j++) {
      int32_t p = idx[(int64_t)r * idx_ld + j];
      int32_t v = -1;
      if (p >= 0) v = block_table[(int64_t)req * bt_ld + p / block_size] * block_span + p % block_size;
      out[(int64_t)r * out_ld + j] = v;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* O6 candidate expansion (P1 key source snippets: the per-row expansion     */
/* kernel and its wrapper).  Per row: flatten each candidate block into      */
/* `ratio` sparse blocks, keep ids in [0, ceil((ke-ks)/sbk)), sort ascending */
/* without removing duplicates, add the row anchor floor(ks/sbk), pad the    */
/* tail with the last valid id, and count the valid sparse columns `end`.    */
/* int32 arithmetic wraps as two's complement (done in uint32 here).         */
/* ------------------------------------------------------------------------ */
static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

static int32_t wrap_add(int32_t a, int32_t b) { return (int32_t)((uint32_t)a + (uint32_t)b); }
static int32_t wrap_mul(int32_t a, int32_t b) { return (int32_t)((uint32_t)a * (uint32_t)b); }

/* Returns 0, -1 on a bad ratio, -2 if scratch allocation fails. */
int orc_expand_candidates(const int32_t* cand, int64_t cand_ld, int32_t rows, int32_t num_candidates,
                          const int32_t* row_ks, int64_t ks_stride, const int32_t* row_ke, int64_t ke_stride,
                          int32_t candidate_block_size, int32_t sparse_block_kv, int32_t* sparse_indices,
                          int64_t si_ld, int32_t* end, int64_t end_stride) {
  int32_t ratio = candidate_block_size / sparse_block_kv;
  int32_t S = num_candidates * ratio, r, j, sbk = sparse_block_kv;
  int32_t* flat;
  int32_t* sorted;
  if (ratio * sparse_block_kv != candidate_block_size || (ratio != 1 && ratio != 2)) return -1;
  flat = (int32_t*)malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
  sorted = (int32_t*)malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
  if (!flat || !sorted) {
    free(flat);
    free(sorted);
    return -2;
  }
  for (r = 0; r < rows; r++) {
    int32_t ks = row_ks[(int64_t)r * ks_stride];
    int32_t ke = row_ke[(int64_t)r * ke_stride];
    int32_t kv = wrap_add(ke, -ks), maxb, base, n = 0, last = -1, pad;
    if (kv < 0) kv = 0;
    maxb = wrap_add(kv, sbk - 1) / sbk;
    /* flatten: a candidate block c covers sparse blocks c*ratio .. c*ratio+ratio-1 */
    for (j = 0; j < num_candidates; j++) {
      int32_t c = cand[(int64_t)r * cand_ld + j];
      if (ratio == 1) {
        flat[j] = c;
      } else {
        flat[2 * j] = wrap_mul(c, 2);
        flat[2 * j + 1] = wrap_add(wrap_mul(c, 2), 1);
      }
    }
    /* filter to this row's range, keeping duplicates */
    for (j = 0; j < S; j++)
      if (flat[j] >= 0 && flat[j] < maxb) {
        sorted[n++] = flat[j];
        if (flat[j] > last) last = flat[j];
      }
    qsort(sorted, (size_t)n, sizeof(int32_t), cmp_i32);
    base = ks / sbk;
    pad = n > 0 ? wrap_add(last, base) : base;
    for (j = 0; j < S; j++) sparse_indices[(int64_t)r * si_ld + j] = j < n ? wrap_add(sorted[j], base) : pad;
    /* only the last block can be partial; every earlier one is a full block */
    if (n > 0) {
      int32_t last_start = wrap_add(wrap_mul(last, sbk), ks);
      int32_t fill = wrap_add(ke, -last_start);
      if (fill < 1) fill = 1;
      if (fill > sbk) fill = sbk;
      end[(int64_t)r * end_stride] = wrap_add(wrap_mul(n - 1, sbk), fill);
    } else {
      end[(int64_t)r * end_stride] = 0;
    }
  }
  free(flat);
  free(sorted);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O7 sparse MQA logits (P1 motivation and implementation: the consumer      */
/* indexer scores only the candidate blocks, into bf16 logits of width       */
/* num_sparse_blocks * sbk).  Column c of row r is token                     */
/* si[r][c / sbk] * sbk + c % sbk; it is scored (O2) when c < end[r] and the */
/* token lies in [ks, ke), rounded once to bf16; every other column is       */
/* bf16 -inf.  K source: gathered rows [S][132] when block_table is NULL,    */
/* else the paged pool through block_table[row_to_req[r]].  out_f32 = 1      */
/* writes unrounded fp32 instead (used only by the selection invariant).     */
/* ------------------------------------------------------------------------ */
void orc_sparse_mqa_logits(const uint8_t* q, const uint16_t* w, int32_t rows, const int32_t* row_ks,
                           const int32_t* row_ke, const int32_t* sparse_indices, int64_t si_ld,
                           int32_t num_sparse_blocks, const int32_t* end, int32_t sparse_block_kv,
                           const uint8_t* k_src, const int32_t* block_table, int64_t bt_ld, const int32_t* row_to_req,
                           int32_t block_size, int64_t block_stride, int32_t out_f32, void* out, int64_t ld) {
  float qt[ORC_D][ORC_H]; /* 32 KB on the caller's stack: concurrent calls from several threads stay independent */
  float wf[ORC_H];
  int32_t r, c, width = num_sparse_blocks * sparse_block_kv;
  for (r = 0; r < rows; r++) {
    int32_t ks = row_ks[r], ke = row_ke[r], e = end[r];
    decode_q_row(q + (int64_t)r * ORC_H * ORC_D, w + (int64_t)r * ORC_H, qt, wf);
    for (c = 0; c < width; c++) {
      int32_t tok = sparse_indices[(int64_t)r * si_ld + c / sparse_block_kv] * sparse_block_kv + c % sparse_block_kv;
      float v = -INFINITY;
      if (c < e && tok >= ks && tok < ke) {
        const uint8_t* krow;
        if (block_table) {
          int32_t req = row_to_req ? row_to_req[r] : r;
          int32_t page = block_table[(int64_t)req * bt_ld + tok / block_size];
          krow = k_src + (int64_t)page * block_stride + (int64_t)(tok % block_size) * ORC_ROW;
        } else {
          krow = k_src + (int64_t)tok * ORC_ROW;
        }
        v = logit_one(qt, wf, krow);
      }
      if (out_f32)
        ((float*)out)[(int64_t)r * ld + c] = v;
      else
        ((uint16_t*)out)[(int64_t)r * ld + c] = isfinite(v) ? orc_bf16_rne(v) : (uint16_t)0xFF80;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* O8 sparse column -> request-local position (P1 implementation: the top-k */
/* over sparse columns is mapped back to context positions).  With block    */
/* span sbk and the row anchor floor(ks/sbk):                                */
/*   pos = (si[r][c / sbk] - floor(ks / sbk)) * sbk + c % sbk, -1 stays -1.  */
/* ------------------------------------------------------------------------ */
void orc_topk_remap(const int32_t* col, int64_t col_ld, int32_t rows, int32_t k, const int32_t* sparse_indices,
                    int64_t si_ld, const int32_t* row_ks, int32_t sparse_block_kv, int32_t* out, int64_t out_ld) {
  int32_t r, j;
  for (r = 0; r < rows; r++) {
    int32_t base = row_ks[r] / sparse_block_kv;
    for (j = 0; j < k; j++) {
      int32_t c = col[(int64_t)r * col_ld + j];
      int32_t v = -1;
      if (c >= 0)
        v = (sparse_indices[(int64_t)r * si_ld + c / sparse_block_kv] - base) * sparse_block_kv + c % sparse_block_kv;
      out[(int64_t)r * out_ld + j] = v;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* O9 prefill K gather (P3 prefill/decode table: a prefill chunk first      */
/* collects its requests' history K out of the paged cache and then scores  */
/* it, while decode reads the cache where it lies; P1 implementation        */
/* breakdown: the indexer's forward chains the prefill K gather with the    */
/* paged decode path).  The requests of the chunk are laid end to end:      */
/* request r owns output rows [cu[r], cu[r+1]) and its row cu[r] + p is its */
/* token p, found through row r of the block table.  The output is the     */
/* cache rows copied byte for byte; rows that no request owns, and tokens   */
/* whose block index or page id is out of range, are zero rows.             */
/* ------------------------------------------------------------------------ */
void orc_gather_prefill_k(const uint8_t* pool, int64_t num_blocks, int32_t block_size, int64_t block_stride,
                          const int32_t* block_table, int64_t bt_ld, int32_t bt_width, const int32_t* cu,
                          int32_t num_reqs, uint8_t* out, int32_t S) {
  int32_t r, p;
  memset(out, 0, (size_t)S * ORC_ROW);
  for (r = 0; r < num_reqs; r++) {
    for (p = 0; p < cu[r + 1] - cu[r]; p++) {
      int64_t row = (int64_t)cu[r] + p;
      int32_t blk = p / block_size, page;
      if (row < 0 || row >= S || blk >= bt_width) continue;
      page = block_table[(int64_t)r * bt_ld + blk];
      if (page < 0 || page >= num_blocks) continue;
      memcpy(out + row * ORC_ROW, pool + (int64_t)page * block_stride + (int64_t)(p % block_size) * ORC_ROW, ORC_ROW);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* O10 q preparation: RoPE, FP8 quantization and weight fold in one pass     */
/* (P3 indexer steps ③ and ④: rotary position embedding on the first 64 of  */
/* the 128 dims only, then one FP8 scale per 128 values of q, and the q     */
/* scale multiplied into the head weights together with the softmax and    */
/* head scales, weights * q_scale * softmax_scale * head_scale in that      */
/* order; P3 pitfalls: the indexer's RoPE has its own interleave switch;    */
/* P1 implementation breakdown: the fused q kernel writes the weights as    */
/* bf16 directly, the fp32 result rounded once).                            */
/* RoPE on frequency i (0..31) rotates the pair (a, b) = (i, i+32) when not */
/* interleaved, (2i, 2i+1) when interleaved, by the angle whose cosine and  */
/* sine are cos_sin[pos][i] and cos_sin[pos][32+i]:                         */
/*   a' = a*cos - b*sin,  b' = b*cos + a*sin   (each op one fp32 rounding). */
/* Quantization uses the k rule: scale = max(amax, 1e-4)/448, codes =       */
/* E4M3(x/scale).  A position outside [0, max_pos) gives zero codes and a   */
/* zero weight.                                                             */
/* ------------------------------------------------------------------------ */
void orc_q_rope_quant(const uint16_t* q, const int64_t* positions, int32_t T, const float* cos_sin, int64_t max_pos,
                      int32_t interleave, const uint16_t* w, float softmax_scale, float head_scale, uint8_t* q8,
                      uint16_t* w_out) {
  int32_t t, h, i, d;
  for (t = 0; t < T; t++) {
    int64_t pos = positions[t];
    for (h = 0; h < ORC_H; h++) {
      const uint16_t* src = q + ((int64_t)t * ORC_H + h) * ORC_D;
      uint8_t* dst = q8 + ((int64_t)t * ORC_H + h) * ORC_D;
      float x[ORC_D], amax = 0.0f, scale, wf;
      if (pos < 0 || pos >= max_pos) {
        memset(dst, 0, ORC_D);
        w_out[(int64_t)t * ORC_H + h] = 0;
        continue;
      }
      for (d = 0; d < ORC_D; d++) x[d] = orc_bf16_to_f32(src[d]);
      for (i = 0; i < 32; i++) {
        int a = interleave ? 2 * i : i, b = interleave ? 2 * i + 1 : i + 32;
        float c = cos_sin[pos * 64 + i], s = cos_sin[pos * 64 + 32 + i];
        float xa = x[a], xb = x[b];
        x[a] = xa * c - xb * s;
        x[b] = xb * c + xa * s;
      }
      for (d = 0; d < ORC_D; d++)
        if (fabsf(x[d]) > amax) amax = fabsf(x[d]);
      scale = (amax > 1e-4f ? amax : 1e-4f) / 448.0f;
      for (d = 0; d < ORC_D; d++) dst[d] = orc_e4m3_encode(x[d] / scale);
      wf = orc_bf16_to_f32(w[(int64_t)t * ORC_H + h]);
      wf = wf * scale;
      wf = wf * softmax_scale;
      wf = wf * head_scale;
      w_out[(int64_t)t * ORC_H + h] = orc_bf16_rne(wf);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* O11 one rank's top-k candidates under context parallelism (P3 pitfalls:  */
/* with the context split across ranks, each rank keeps only its local      */
/* top-k candidates, and those, not the score matrix, are exchanged).       */
/* Entry j of row r: the rank-local selection p = idx[r][j] (relative to    */
/* the row's start, as dsi_topk_select emits it) becomes the pair           */
/*   value = logits[r][start + p],  global index = p*scale + offset;        */
/* an empty slot (p < 0) or a column at or past max_width gives (-inf, -1). */
/* ------------------------------------------------------------------------ */
void orc_topk_values(const float* logits, int64_t ld, int32_t rows, const int32_t* starts, int32_t max_width,
                     const int32_t* idx, int64_t idx_ld, int32_t k, int32_t index_scale, int32_t index_offset,
                     float* vals, int64_t vals_ld, int32_t* gidx, int64_t gidx_ld) {
  int32_t r, j;
  for (r = 0; r < rows; r++) {
    int32_t st = starts ? starts[r] : 0;
    if (st < 0) st = 0;
    for (j = 0; j < k; j++) {
      int32_t p = idx[(int64_t)r * idx_ld + j];
      float* v = vals + (int64_t)r * vals_ld + j;
      int32_t* g = gidx + (int64_t)r * gidx_ld + j;
      if (p < 0 || (int64_t)st + p >= max_width) {
        *v = -INFINITY;
        *g = -1;
      } else {
        *v = logits[(int64_t)r * ld + st + p];
        *g = (int32_t)((int64_t)p * index_scale + index_offset);
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* O12 merge of the ranks' candidate lists into the global top-k (P3        */
/* pitfalls: the global top-k is chosen from the exchanged local            */
/* candidates; it is exact because a token in the global top-k is also in   */
/* the local top-k of the rank that holds it).  Row r of list l holds k_in  */
/* (value, global index) pairs at l*list_stride + r*row_ld.  Pairs with a   */
/* negative index or a non-finite value are ignored; the output is the      */
/* indices of the k largest values, in the order (value desc, index asc),   */
/* then -1.  Returns 0, or -1 if the scratch allocation fails.              */
/* ------------------------------------------------------------------------ */
int orc_topk_merge(const float* vals, const int32_t* gidx, int64_t list_stride, int64_t row_ld, int32_t num_lists,
                   int32_t rows, int32_t k_in, int32_t k, int32_t* out, int64_t out_ld) {
  int32_t r, l, j, n;
  orc_vc* buf = (orc_vc*)malloc(sizeof(orc_vc) * (size_t)(num_lists * k_in > 0 ? num_lists * k_in : 1));
  if (!buf) return -1;
  for (r = 0; r < rows; r++) {
    n = 0;
    for (l = 0; l < num_lists; l++) {
      for (j = 0; j < k_in; j++) {
        int64_t a = (int64_t)l * list_stride + (int64_t)r * row_ld + j;
        if (gidx[a] >= 0 && isfinite(vals[a])) {
          buf[n].v = vals[a];
          buf[n].c = gidx[a];
          n++;
        }
      }
    }
    qsort(buf, (size_t)n, sizeof(orc_vc), cmp_vc);
    for (j = 0; j < k; j++) out[(int64_t)r * out_ld + j] = j < n ? buf[j].c : -1;
  }
  free(buf);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O13 the MXFP4 indexer cache (P1 motivation and implementation: the V4.1  */
/* sparse indexer runs on an MXFP4 indexer cache, checked at start-up, and  */
/* scores FP8 q against FP4 k).  The pages name the format only; it is the  */
/* OCP Microscaling format: FP4 E2M1 elements (sign, 2 exponent bits with   */
/* bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no inf or */
/* NaN) sharing one E8M0 scale 2^(E-127) per block of 32.  The row layout   */
/* is a reading: 64 bytes of codes (element 2i in the low nibble of byte i, */
/* 2i+1 in the high nibble), then the 4 scale bytes of dims 32j..32j+31:    */
/* 68 bytes per token.                                                      */
/* ------------------------------------------------------------------------ */
#define ORC_ROW4 68

float orc_fp4_decode(uint8_t c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  float v = e == 0 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
  return s ? -v : v;
}

/* Nearest FP4 code to a finite x, ties to the even code (mantissa bit 0),
 * saturating at +-6; the sign is kept (a negative value that rounds to 0
 * gives -0, code 8). */
uint8_t orc_fp4_encode(float x) {
  uint8_t sign = signbit(x) ? 8 : 0, best = 0;
  double a = fabs((double)x), bd = INFINITY;
  int c;
  if (a >= 6.0) return sign | 7;
  for (c = 0; c < 8; c++) {
    double d = fabs(a - (double)orc_fp4_decode((uint8_t)c));
    if (d < bd || (d == bd && (c & 1) == 0)) {
      bd = d;
      best = (uint8_t)c;
    }
  }
  return sign | best;
}

/* Shared exponent of one block of 32 (OCP MX conversion): floor(log2(amax))
 * minus 2, the exponent of FP4's largest value, clamped to E8M0's range
 * [-127, 127]; an all-zero block takes -127. */
static int mx_shared_exp(const float* x) {
  float amax = 0.0f;
  int i, e, se;
  for (i = 0; i < 32; i++)
    if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
  if (amax == 0.0f) return -127;
  (void)frexpf(amax, &e); /* amax = f * 2^e, f in [0.5, 1): floor(log2 amax) = e - 1 */
  se = e - 1 - 2;
  return se < -127 ? -127 : se > 127 ? 127 : se;
}

void orc_k_quant_and_cache_mxfp4(const uint16_t* k, int64_t n, int64_t k_ld, const int64_t* slot_mapping,
                                 uint8_t* pool, int32_t block_size, int64_t block_stride) {
  int64_t i;
  int d, j;
  for (i = 0; i < n; i++) {
    int64_t slot = slot_mapping[i];
    float x[ORC_D];
    uint8_t* row;
    if (slot < 0) continue;
    row = pool + (slot / block_size) * block_stride + (slot % block_size) * ORC_ROW4;
    for (d = 0; d < ORC_D; d++) x[d] = orc_bf16_to_f32(k[i * k_ld + d]);
    memset(row, 0, 64);
    for (j = 0; j < 4; j++) {
      int se = mx_shared_exp(x + 32 * j);
      row[64 + j] = (uint8_t)(se + 127);
      for (d = 32 * j; d < 32 * j + 32; d++) {
        uint8_t c = orc_fp4_encode(ldexpf(x[d], -se));
        row[d / 2] |= (uint8_t)((d & 1) ? c << 4 : c);
      }
    }
  }
}

/* Decoded key of an MXFP4 row: code value times its block's 2^(E-127). */
static void decode_row_mxfp4(const uint8_t* krow, float kd[ORC_D]) {
  int d;
  for (d = 0; d < ORC_D; d++) {
    uint8_t c = (d & 1) ? (uint8_t)(krow[d / 2] >> 4) : (uint8_t)(krow[d / 2] & 15);
    kd[d] = ldexpf(orc_fp4_decode(c), (int)krow[64 + d / 32] - 127);
  }
}

/* O14 sparse MQA logits on the MXFP4 cache: O7 with the key rows read as   */
/* MXFP4 (68-byte rows, gathered [S][68] or paged), FP8 q as before.        */
void orc_sparse_mqa_logits_mxfp4(const uint8_t* q, const uint16_t* w, int32_t rows, const int32_t* row_ks,
                                 const int32_t* row_ke, const int32_t* sparse_indices, int64_t si_ld,
                                 int32_t num_sparse_blocks, const int32_t* end, int32_t sparse_block_kv,
                                 const uint8_t* k_src, const int32_t* block_table, int64_t bt_ld,
                                 const int32_t* row_to_req, int32_t block_size, int64_t block_stride, int32_t out_f32,
                                 void* out, int64_t ld) {
  float qt[ORC_D][ORC_H]; /* 32 KB on the caller's stack: concurrent calls from several threads stay independent */
  float wf[ORC_H], kd[ORC_D];
  int32_t r, c, width = num_sparse_blocks * sparse_block_kv;
  for (r = 0; r < rows; r++) {
    int32_t ks = row_ks[r], ke = row_ke[r], e = end[r];
    decode_q_row(q + (int64_t)r * ORC_H * ORC_D, w + (int64_t)r * ORC_H, qt, wf);
    for (c = 0; c < width; c++) {
      int32_t tok = sparse_indices[(int64_t)r * si_ld + c / sparse_block_kv] * sparse_block_kv + c % sparse_block_kv;
      float v = -INFINITY;
      if (c < e && tok >= ks && tok < ke) {
        const uint8_t* krow;
        if (block_table) {
          int32_t req = row_to_req ? row_to_req[r] : r;
          int32_t page = block_table[(int64_t)req * bt_ld + tok / block_size];
          krow = k_src + (int64_t)page * block_stride + (int64_t)(tok % block_size) * ORC_ROW4;
        } else {
          krow = k_src + (int64_t)tok * ORC_ROW4;
        }
        decode_row_mxfp4(krow, kd);
        v = logit_kd(qt, wf, kd);
      }
      if (out_f32)
        ((float*)out)[(int64_t)r * ld + c] = v;
      else
        ((uint16_t*)out)[(int64_t)r * ld + c] = isfinite(v) ? orc_bf16_rne(v) : (uint16_t)0xFF80;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* O15 paged decode on the MXFP4 cache: O2's decode rows with every key row  */
/* read as a 68-byte MXFP4 row (P1 motivation and implementation: the V4.1   */
/* indexer cache holds MXFP4 keys; decode reads the paged cache directly, P3 */
/* prefill/decode table).  Token s of request b lives at                     */
/* pool + bt[b][s / bs] * block_stride + (s % bs) * 68; a key's value is its  */
/* code times its block's 2^(E-127), and no per-token scale follows.         */
void orc_mqa_logits_paged_mxfp4(const uint8_t* q, const uint16_t* w, int32_t B, int32_t next_n,
                                const int32_t* context_lens, const uint8_t* pool, int32_t block_size,
                                int64_t block_stride, const int32_t* block_table, int64_t bt_ld, int32_t width,
                                float* logits, int64_t ld) {
  float qt[ORC_D][ORC_H]; /* 32 KB on the caller's stack: concurrent calls from several threads stay independent */
  float wf[ORC_H], kd[ORC_D];
  int32_t b, i, s;
  for (b = 0; b < B; b++) {
    for (i = 0; i < next_n; i++) {
      int64_t r = (int64_t)b * next_n + i;
      int32_t ke = context_lens[b] - next_n + i + 1;
      decode_q_row(q + r * ORC_H * ORC_D, w + r * ORC_H, qt, wf);
      for (s = 0; s < width; s++) {
        float* o = logits + r * ld + s;
        if (s < ke) {
          int32_t page = block_table[(int64_t)b * bt_ld + s / block_size];
          decode_row_mxfp4(pool + (int64_t)page * block_stride + (int64_t)(s % block_size) * ORC_ROW4, kd);
          *o = logit_kd(qt, wf, kd);
        } else {
          *o = -INFINITY;
        }
      }
    }
  }
}
