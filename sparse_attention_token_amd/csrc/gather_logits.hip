// Indexer logits over gathered key sets: paged decode (P3 prefill/decode table of
// "DeepSeek V3.2 稀疏注意力 DSA 推理流程图解": decode scores straight from the
// paged cache, no gather) and the hierarchical path's sparse columns (P1 "V4.1
// 索引器接入稀疏 MQA logits", motivation and implementation: consumer layers score
// only the candidate blocks, into bf16 logits).
//
// Both stream 132-byte K rows past one to four query rows: HBM/L2-bound.  A
// workgroup gathers 256 keys — segments of 16 (or 8) consecutive tokens, each
// contiguous in memory — straight into LDS with global->LDS DMA loads
// (global_load_lds_dwordx4: no VGPR staging, no LDS write instructions; all 33 KB
// in flight at once).  The segments sit back to back, so key slot k is always the
// 132 bytes at LDS offset 132*k.  Each wavefront then scores 4 groups of 16 keys on
// the matrix cores one group at a time (raw codes read with 4-byte LDS loads and
// decoded to f16 per use, common.h), keeping its register footprint small so that
// several workgroups per CU keep loads in flight.  Block-table entries are read
// once per segment.  Out-of-range table entries or page ids never produce an access
// outside the pool: those keys score -inf.
#include "common.h"

namespace dsi {
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* glob_ptr_t;

constexpr int kKeys = 256;                         // keys per workgroup
constexpr int kGatherBytes = kKeys * kRow;         // 33792 = 33 x 1024
constexpr int kGatherSlabs = kGatherBytes / 1024;  // one DMA instruction of a wavefront fills 1 KB

// Issue the DMA loads of a 256-key gather into s_keys.  s_base[seg] is the byte
// offset in src of segment seg (seg_bytes long) or -1 when absent; limit is the byte
// size of src.  A 16-byte piece that would cross `limit` is copied dword by dword.
__device__ __forceinline__ void gather_keys_dma(uint8_t* s_keys, const int64_t* s_base, const uint8_t* src,
                                                int64_t limit, int seg_bytes, int wave, int lane) {
  for (int i = wave; i < kGatherSlabs; i += 4) {
    const int o = i * 1024 + lane * 16;  // this lane's LDS bytes
    const int seg = o / seg_bytes, within = o - seg * seg_bytes;
    const int64_t base = s_base[seg];
    const int64_t goff = base + within;
    if (base >= 0 && goff + 16 <= limit) {
      __builtin_amdgcn_global_load_lds((glob_ptr_t)(src + goff), (lds_ptr_t)(s_keys + i * 1024), 16, 0, 0);
    } else if (base >= 0 && goff < limit) {
#pragma unroll
      for (int j = 0; j < 4; j++)
        if (goff + 4 * j + 4 <= limit)
          *reinterpret_cast<uint32_t*>(s_keys + o + 4 * j) = *reinterpret_cast<const uint32_t*>(src + goff + 4 * j);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // every load of this wavefront has landed in LDS
}

// B fragments of 16 keys from raw rows at LDS offset 132*k: lane (key n, group g)
// reads its 32 codes as 8 dwords and decodes them.
__device__ __forceinline__ void load_kfrag_raw(KFrag& f, const uint8_t* keys, int lane) {
  const int n = lane & 15, g = lane >> 4;
  const uint32_t* p = reinterpret_cast<const uint32_t*>(keys + n * kRow + g * 32);
  uint32_t x[8];
#pragma unroll
  for (int j = 0; j < 8; j++) x[j] = p[j];
  f.b[0] = e4m3x8_to_f16x8(x[0], x[1]);
  f.b[1] = e4m3x8_to_f16x8(x[2], x[3]);
  f.b[2] = e4m3x8_to_f16x8(x[4], x[5]);
  f.b[3] = e4m3x8_to_f16x8(x[6], x[7]);
}

// One (row, 16-key group) output: 16 MFMAs as 4 interleaved head-tile chains, then
// this lane's 16 heads weighted and summed.
__device__ __forceinline__ float score1(const QFrag& q, const WFrag& w, const KFrag& kb) {
  f32x4 c[4];
#pragma unroll
  for (int hb = 0; hb < 4; hb++) c[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; s++)
#pragma unroll
    for (int hb = 0; hb < 4; hb++) c[hb] = mfma_f16(q.a[hb][s], kb.b[s], c[hb]);
  float acc = 0.f;
#pragma unroll
  for (int hb = 0; hb < 4; hb++)
#pragma unroll
    for (int i = 0; i < 4; i++) acc = fmaf(w.w[hb][i], c[hb][i], acc);
  return acc;
}

__device__ __forceinline__ float key_scale(const uint8_t* s_keys, int kslot) {
  return *reinterpret_cast<const float*>(s_keys + kslot * kRow + kDim);
}

// Stage one q row (64 x 128 codes) into 8 KB of LDS by DMA, permuted into the order
// the A fragments are read: 16-byte unit (hb*2 + p)*64 + lane holds codes
// [32g + 16p, +16) of head hb*16 + n (lane = 16g + n), so each fragment read of a
// wavefront is one contiguous, conflict-free 1 KB.  Issued by one wavefront.
__device__ __forceinline__ void stage_q_dma(uint8_t* s_q, const uint8_t* q_row, int lane) {
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int hb = i >> 1, p = i & 1;
    __builtin_amdgcn_global_load_lds((glob_ptr_t)(q_row + (hb * 16 + n) * kDim + g * 32 + p * 16),
                                     (lds_ptr_t)(s_q + i * 1024), 16, 0, 0);
  }
}

// A fragments of one q row staged by stage_q_dma, decoded to f16.
__device__ __forceinline__ void load_q_lds(QFrag& f, const uint8_t* s_q, int lane) {
  const uint4* p = reinterpret_cast<const uint4*>(s_q) + lane;
#pragma unroll
  for (int hb = 0; hb < 4; hb++) {
    const uint4 x0 = p[(hb * 2 + 0) * 64], x1 = p[(hb * 2 + 1) * 64];
    f.a[hb][0] = e4m3x8_to_f16x8(x0.x, x0.y);
    f.a[hb][1] = e4m3x8_to_f16x8(x0.z, x0.w);
    f.a[hb][2] = e4m3x8_to_f16x8(x1.x, x1.y);
    f.a[hb][3] = e4m3x8_to_f16x8(x1.z, x1.w);
  }
}

// ------------------------------------------------------------------ paged decode
// grid = (ceil(max_context_len / 256), B).  Dynamic LDS: the 256 gathered keys, then
// up to two of the request's q rows (8 KB each), all loaded by DMA and waited for
// once.  Rows are then scored one after the other against the staged keys (rows 2
// and 3 of a four-row request are staged after the first two are done).
__global__ __launch_bounds__(256) void paged_decode_kernel(
    const uint8_t* __restrict__ q, const uint16_t* __restrict__ w, int next_n, const int* __restrict__ context_lens,
    const uint8_t* __restrict__ pool, int64_t num_blocks, int block_size, int64_t block_stride,
    const int* __restrict__ block_table, int64_t bt_ld, int bt_width, int max_ctx, float* __restrict__ logits,
    int64_t ld) {
  extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];
  uint8_t* s_keys = s_dyn;
  uint8_t* s_q = s_dyn + kGatherBytes;
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
  // q rows of this request, two at a time: waves 0 and 1 stage rows 0 and 1
  if (wave < min(next_n, 2)) stage_q_dma(s_q + wave * 8192, q + ((int64_t)b * next_n + wave) * kHeads * kDim, lane);
  __syncthreads();
  gather_keys_dma(s_keys, s_base, pool, num_blocks * block_stride, 16 * kRow, wave, lane);
  __syncthreads();

  const int n = lane & 15, g = lane >> 4;
  const int grp = wave + 4 * g;  // after the transpose-reduce lane group g owns key group wave + 4g
  const int kslot = grp * 16 + n;
  const int tok = tok0 + kslot;
  const float ks = key_scale(s_keys, kslot);
  const bool present = s_base[grp] >= 0;
  for (int row = 0; row < next_n; row++) {
    if (row == 2) {  // rows 2 and 3 replace rows 0 and 1 in LDS
      __syncthreads();
      if (wave < next_n - 2)
        stage_q_dma(s_q + wave * 8192, q + ((int64_t)b * next_n + 2 + wave) * kHeads * kDim, lane);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    QFrag qf;
    WFrag wf;
    load_q_lds(qf, s_q + (row & 1) * 8192, lane);
    load_w(wf, w + ((int64_t)b * next_n + row) * kHeads, lane);
    float part[4];
#pragma unroll
    for (int kg = 0; kg < 4; kg++) {
      KFrag kb;
      load_kfrag_raw(kb, s_keys + (wave + 4 * kg) * 16 * kRow, lane);
      part[kg] = score1(qf, wf, kb);
      __builtin_amdgcn_sched_barrier(0);  // one key group in flight: a small register footprint
    }
    const float v = transpose_reduce4(part, lane);
    const int ke = min(L - next_n + row + 1, max_ctx);
    if (tok < ke) logits[((int64_t)b * next_n + row) * ld + tok] = present ? v * ks : -INFINITY;
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
  __shared__ __attribute__((aligned(16))) uint8_t s_keys[kGatherBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_q[8192];
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
  if (wave == 0) stage_q_dma(s_q, q + (int64_t)r * kHeads * kDim, lane);
  __syncthreads();
  gather_keys_dma(s_keys, s_base, k_src, limit, G * kRow, wave, lane);
  WFrag wf;
  load_w(wf, w + (int64_t)r * kHeads, lane);
  __syncthreads();
  QFrag qf;
  load_q_lds(qf, s_q, lane);

  const int n = lane & 15, g = lane >> 4;
  float part[4];
#pragma unroll
  for (int kg = 0; kg < 4; kg++) {
    KFrag kb;
    load_kfrag_raw(kb, s_keys + (wave + 4 * kg) * 16 * kRow, lane);
    part[kg] = score1(qf, wf, kb);
    __builtin_amdgcn_sched_barrier(0);
  }
  const float v = transpose_reduce4(part, lane);
  const int grp = wave + 4 * g;
  const int kslot = grp * 16 + n;
  const int c = c0 + kslot;
  if (c < width) {
    const int seg = kslot / G;
    const int tok = s_tok[seg] + (kslot - seg * G);
    const bool valid = c < e && s_base[seg] >= 0 && tok >= ks && tok < ke && (paged || tok < num_k);
    out[(int64_t)r * ld + c] = valid ? f32_to_bf16_rne(v * key_scale(s_keys, kslot)) : (uint16_t)0xFF80u;
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
  const size_t lds = (size_t)kGatherBytes + (size_t)(next_n < 2 ? next_n : 2) * 8192;
  hipLaunchKernelGGL(paged_decode_kernel, grid, dim3(256), lds, stream, q, w, next_n, context_lens, pool, num_blocks,
                     block_size, block_stride_bytes, block_table, bt_ld, bt_width, max_context_len, logits, ld);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}

extern "C" int dsi_sparse_mqa_logits(const uint8_t* q, const uint16_t* w, int32_t rows, const int32_t* row_ks,
                                     const int32_t* row_ke, const int32_t* sparse_indices, int64_t si_ld,
                                     int32_t num_sparse_blocks, const int32_t* end, int32_t sparse_block_kv,
                                     const uint8_t* k_src, int64_t num_k, const int32_t* block_table, int64_t bt_ld,
                                     int32_t bt_width, int32_t num_reqs, const int32_t* row_to_req,
                                     int32_t block_size, int64_t block_stride_bytes, uint16_t* logits_bf16,
                                     int64_t ld, hipStream_t stream) {
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
                     (int)width, end, sbk, k_src, num_k, block_table, bt_ld, bt_width, num_reqs, row_to_req,
                     block_size, block_stride_bytes, logits_bf16, ld);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}
