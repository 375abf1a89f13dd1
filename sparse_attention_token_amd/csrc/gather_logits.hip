// Indexer logits over gathered key sets: paged decode (P3 prefill/decode table of
// "DeepSeek V3.2 稀疏注意力 DSA 推理流程图解": decode scores straight from the
// paged cache, no gather) and the hierarchical path's sparse columns (P1 "V4.1
// 索引器接入稀疏 MQA logits", motivation and implementation: consumer layers score
// only the candidate blocks, into bf16 logits).
//
// Both are a stream of 132-byte K rows scored against one to four query rows:
// HBM/L2-bound.  A workgroup gathers 256 keys (segments of 16, or 8, consecutive
// tokens that are contiguous in memory) into LDS with 16-byte loads — all issued
// before any is used — then each wavefront scores 4 groups of 16 keys on the
// matrix cores, decoding the FP8 codes to f16 as it reads them (common.h), and
// writes its outputs.  Query rows are held two at a time (next_n 3 and 4 take a
// second pass over the staged keys).  Block-table entries are read
// once per segment into LDS.  Out-of-range table entries or page ids never
// produce an access outside the pool: those keys score -inf.
#include "common.h"

namespace dsi {
namespace {

constexpr int kKeys = 256;                   // keys per workgroup
constexpr int kChunks16 = kKeys * kRow / 16;  // 2112 sixteen-byte chunks
constexpr int kLoads = (kChunks16 + 255) / 256;

// Load up to 16 bytes at p, stopping at `limit` bytes from `base` (dword granular).
__device__ __forceinline__ uint4 load_bounded(const uint8_t* base, int64_t off, int64_t limit) {
  if (off + 16 <= limit) return *reinterpret_cast<const uint4*>(base + off);
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < 4; j++)
    if (off + 4 * j + 4 <= limit) w[j] = *reinterpret_cast<const uint32_t*>(base + off + 4 * j);
  return uint4{w[0], w[1], w[2], w[3]};
}

// Gather segments of `seg_tokens` rows (byte offsets in s_base, -1 = absent) into LDS.
__device__ __forceinline__ void gather_keys(uint8_t* s_codes, float* s_scale, const int64_t* s_base,
                                            const uint8_t* src, int64_t limit, int seg_tokens, int tid) {
  const int cps = seg_tokens * kRow / 16;  // chunks per segment (132 or 66)
  uint4 v[kLoads];
  bool ok[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; j++) {
    const int c = tid + j * 256;
    ok[j] = false;
    if (c < kChunks16) {
      const int seg = c / cps, cc = c - seg * cps;
      const int64_t base = s_base[seg];
      if (base >= 0) {
        v[j] = load_bounded(src, base + cc * 16, limit);
        ok[j] = true;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kLoads; j++) {
    const int c = tid + j * 256;
    if (ok[j]) {
      const int seg = c / cps, cc = c - seg * cps;
      scatter_chunk(s_codes, s_scale, seg * seg_tokens, cc, v[j]);
    }
  }
}

// ------------------------------------------------------------------ paged decode
// grid = (ceil(max_context_len / 256), B); R = 1 (next_n 1) or 2 (rows taken in pairs).
template <int R>
__global__ __launch_bounds__(256) void paged_decode_kernel(
    const uint8_t* __restrict__ q, const uint16_t* __restrict__ w, int next_n, const int* __restrict__ context_lens,
    const uint8_t* __restrict__ pool, int64_t num_blocks, int block_size, int64_t block_stride,
    const int* __restrict__ block_table, int64_t bt_ld, int bt_width, int max_ctx, float* __restrict__ logits,
    int64_t ld) {
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[kKeys * kLdsKeyStride];
  __shared__ float s_scale[kKeys];
  __shared__ int64_t s_base[16];

  const int b = blockIdx.y, tok0 = blockIdx.x * kKeys;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = context_lens[b];
  const int Lc = min(L, max_ctx);  // the last row of the request sees [0, L)
  if (tok0 >= Lc) return;

  if (tid < 16) {
    const int s = tok0 + 16 * tid;
    int64_t base = -1;
    if (s < Lc) {
      const int blk = s / block_size;
      if (blk < bt_width) {
        const int page = block_table[(int64_t)b * bt_ld + blk];
        if (page >= 0 && page < num_blocks) base = (int64_t)page * block_stride + (int64_t)(s % block_size) * kRow;
      }
    }
    s_base[tid] = base;
  }
  __syncthreads();
  gather_keys(s_codes, s_scale, s_base, pool, num_blocks * block_stride, 16, tid);
  __syncthreads();

  const int n = lane & 15, g = lane >> 4;
  constexpr int KPB = 4 / R;  // key groups per batch of four outputs
  for (int r0 = 0; r0 < next_n; r0 += R) {
    QFrag qf[R];
    WFrag wf[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
      const int64_t row = (int64_t)b * next_n + min(r0 + r, next_n - 1);
      load_q(qf[r], q + row * kHeads * kDim, lane);
      load_w(wf[r], w + row * kHeads, lane);
    }
#pragma unroll
    for (int batch = 0; batch < R; batch++) {
      KFrag kb[KPB];
#pragma unroll
      for (int kgi = 0; kgi < KPB; kgi++)
        load_kfrag_fp8(kb[kgi], s_codes + (wave + 4 * (batch * KPB + kgi)) * 16 * kLdsKeyStride, lane);
      // output j: row j / KPB of the pair, key group j % KPB of the batch
      constexpr int orow[4] = {0, R == 1 ? 0 : 0, R == 1 ? 0 : 1, R == 1 ? 0 : 1};
      constexpr int okg[4] = {0, R == 1 ? 1 : 1, R == 1 ? 2 : 0, R == 1 ? 3 : 1};
      float part[4];
      score4(qf, wf, kb, orow, okg, part);
      const float v = transpose_reduce4(part, lane);
      const int r = r0 + g / KPB, kgi = g % KPB;
      const int grp = wave + 4 * (batch * KPB + kgi);
      const int kslot = grp * 16 + n;
      const int tok = tok0 + kslot;
      if (r < next_n) {
        const int ke = min(L - next_n + r + 1, max_ctx);
        if (tok < ke)
          logits[((int64_t)b * next_n + r) * ld + tok] =
              s_base[grp] >= 0 ? v * s_scale[kslot] : -INFINITY;
      }
    }
  }
}

// ------------------------------------------------------------------ sparse columns
// grid = (ceil(width / 256), rows); one query row per workgroup.
__global__ __launch_bounds__(256) void sparse_logits_kernel(
    const uint8_t* __restrict__ q, const uint16_t* __restrict__ w, const int* __restrict__ row_ks,
    const int* __restrict__ row_ke, const int* __restrict__ sparse_indices, int64_t si_ld, int width,
    const int* __restrict__ end, int sbk, const uint8_t* __restrict__ k_src, int64_t num_k,
    const int* __restrict__ block_table, int64_t bt_ld, int bt_width, int num_reqs,
    const int* __restrict__ row_to_req, int block_size, int64_t block_stride, uint16_t* __restrict__ out,
    int64_t ld) {
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[kKeys * kLdsKeyStride];
  __shared__ float s_scale[kKeys];
  __shared__ int64_t s_base[32];
  __shared__ int s_tok[32];

  const int r = blockIdx.y, c0 = blockIdx.x * kKeys;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = sbk < 16 ? sbk : 16;  // tokens per contiguous segment
  const int nseg = kKeys / G;
  const int ks = row_ks[r], ke = row_ke[r], e = end[r];
  const bool paged = block_table != nullptr;
  const int64_t limit = paged ? num_k * block_stride : num_k * kRow;

  if (tid < nseg) {
    const int c = c0 + tid * G;
    int64_t base = -1;
    int tok = -1;
    if (c < width && c < e) {
      tok = sparse_indices[(int64_t)r * si_ld + c / sbk] * sbk + c % sbk;
      if (tok >= 0) {
        if (!paged) {
          if (tok < num_k) base = (int64_t)tok * kRow;
        } else {
          const int req = row_to_req ? row_to_req[r] : r;
          const int blk = tok / block_size;
          if (blk < bt_width && req >= 0 && req < num_reqs) {
            const int page = block_table[(int64_t)req * bt_ld + blk];
            if (page >= 0 && page < num_k) base = (int64_t)page * block_stride + (int64_t)(tok % block_size) * kRow;
          }
        }
      }
    }
    s_base[tid] = base;
    s_tok[tid] = tok;
  }

  QFrag qf;
  WFrag wf;
  load_q(qf, q + (int64_t)r * kHeads * kDim, lane);
  load_w(wf, w + (int64_t)r * kHeads, lane);
  __syncthreads();
  gather_keys(s_codes, s_scale, s_base, k_src, limit, G, tid);
  __syncthreads();

  const int n = lane & 15, g = lane >> 4;
  KFrag kb[4];
#pragma unroll
  for (int kgi = 0; kgi < 4; kgi++) load_kfrag_fp8(kb[kgi], s_codes + (wave + 4 * kgi) * 16 * kLdsKeyStride, lane);
  QFrag qa[1] = {qf};
  WFrag wa[1] = {wf};
  constexpr int orow[4] = {0, 0, 0, 0};
  constexpr int okg[4] = {0, 1, 2, 3};
  float part[4];
  score4(qa, wa, kb, orow, okg, part);
  const float v = transpose_reduce4(part, lane);
  const int grp = wave + 4 * g;
  const int kslot = grp * 16 + n;
  const int c = c0 + kslot;
  if (c < width) {
    const int seg = kslot / G;
    const int tok = s_tok[seg] + (kslot - seg * G);
    const bool valid = c < e && s_base[seg] >= 0 && tok >= ks && tok < ke && (paged || tok < num_k);
    out[(int64_t)r * ld + c] = valid ? f32_to_bf16_rne(v * s_scale[kslot]) : (uint16_t)0xFF80u;
  }
}

}  // namespace
}  // namespace dsi

extern "C" int dsi_paged_mqa_logits_decode(const uint8_t* q, const uint16_t* w, int32_t B, int32_t next_n,
                                           const int32_t* context_lens, const uint8_t* pool, int64_t num_blocks,
                                           int32_t block_size, int64_t block_stride_bytes,
                                           const int32_t* block_table, int64_t bt_ld, int32_t bt_width,
                                           int32_t max_context_len, float* logits, int64_t ld, hipStream_t stream) {
  using namespace dsi;
  if (B < 0 || max_context_len < 0 || ld < max_context_len || num_blocks < 0 || bt_width < 0 || bt_ld < bt_width)
    return DSI_EINVAL;
  if (next_n < 1 || next_n > 4 || block_size < 16 || (block_size % 16) != 0) return DSI_EUNSUPPORTED;
  if (block_stride_bytes < (int64_t)block_size * kRow) return DSI_EINVAL;
  if (B == 0 || max_context_len == 0) return DSI_OK;
  if (!q || !w || !context_lens || !pool || !block_table || !logits) return DSI_EINVAL;
  if (B > 65535) return DSI_EUNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(pool) & 15) ||
      (block_stride_bytes & 15) || (reinterpret_cast<uintptr_t>(w) & 7) || (reinterpret_cast<uintptr_t>(logits) & 3))
    return DSI_EALIGN;
  const dim3 grid((unsigned)((max_context_len + kKeys - 1) / kKeys), (unsigned)B);
  if (next_n == 1)
    hipLaunchKernelGGL(paged_decode_kernel<1>, grid, dim3(256), 0, stream, q, w, next_n, context_lens, pool,
                       num_blocks, block_size, block_stride_bytes, block_table, bt_ld, bt_width, max_context_len,
                       logits, ld);
  else
    hipLaunchKernelGGL(paged_decode_kernel<2>, grid, dim3(256), 0, stream, q, w, next_n, context_lens, pool,
                       num_blocks, block_size, block_stride_bytes, block_table, bt_ld, bt_width, max_context_len,
                       logits, ld);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}

extern "C" int dsi_sparse_mqa_logits(const uint8_t* q, const uint16_t* w, int32_t rows, const int32_t* row_ks,
                                     const int32_t* row_ke, const int32_t* sparse_indices, int64_t si_ld,
                                     int32_t num_sparse_blocks, const int32_t* end, int32_t sparse_block_kv,
                                     const uint8_t* k_src, int64_t num_k, const int32_t* block_table, int64_t bt_ld,
                                     int32_t bt_width, int32_t num_reqs, const int32_t* row_to_req, int32_t block_size,
                                     int64_t block_stride_bytes, uint16_t* logits_bf16, int64_t ld,
                                     hipStream_t stream) {
  using namespace dsi;
  const int sbk = sparse_block_kv;
  if (sbk < 8 || sbk > 128 || (sbk & (sbk - 1))) return DSI_EUNSUPPORTED;
  if (rows < 0 || num_sparse_blocks < 1 || si_ld < num_sparse_blocks || num_k < 0) return DSI_EINVAL;
  const int64_t width = (int64_t)num_sparse_blocks * sbk;
  if (width > 0x7FFFFFFF || ld < width) return DSI_EINVAL;
  const bool paged = block_table != nullptr;
  if (paged) {
    if (bt_width < 0 || bt_ld < bt_width || num_reqs < 0) return DSI_EINVAL;
    if (block_size < 8 || (block_size % sbk) != 0 || (block_size % 8) != 0) return DSI_EUNSUPPORTED;
    if (block_stride_bytes < (int64_t)block_size * kRow) return DSI_EINVAL;
    if (block_stride_bytes & 15) return DSI_EALIGN;
  }
  if (rows == 0) return DSI_OK;
  if (!q || !w || !row_ks || !row_ke || !sparse_indices || !end || !k_src || !logits_bf16) return DSI_EINVAL;
  if ((reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(k_src) & 15) ||
      (reinterpret_cast<uintptr_t>(w) & 7) || (reinterpret_cast<uintptr_t>(logits_bf16) & 1))
    return DSI_EALIGN;
  if (rows > 65535) return DSI_EUNSUPPORTED;
  const dim3 grid((unsigned)((width + kKeys - 1) / kKeys), (unsigned)rows);
  hipLaunchKernelGGL(sparse_logits_kernel, grid, dim3(256), 0, stream, q, w, row_ks, row_ke, sparse_indices, si_ld,
                     (int)width, end, sbk, k_src, num_k, block_table, bt_ld, bt_width, num_reqs, row_to_req, block_size,
                     block_stride_bytes, logits_bf16, ld);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}
