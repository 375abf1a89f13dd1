// Integer index steps of the indexer path:
//  - candidate expansion of the hierarchical indexer (P1 "V4.1 索引器接入稀疏 MQA
//    logits", key source snippets: flatten candidate blocks, keep those in the row's
//    range, sort ascending without dedupe, anchor, pad with the last id, count the
//    valid sparse columns);
//  - sparse column -> request-local position (P1 implementation breakdown);
//  - request-local position -> physical cache slot (P3 "DeepSeek V3.2 稀疏注意力 DSA
//    推理流程图解", pitfalls; P2 "修复 DSV4 FlashInfer 稀疏 MLA 在打包 KV 布局下的地址
//    错误", key source snippets: block * block_span + offset, -1 kept).
// int32 arithmetic wraps (two's complement) like the description's tensor ops.
#include "common.h"

namespace dsi {
namespace {

constexpr int kMaxSparse = 1024;  // num_candidates * ratio

// log2(d) when d is a power of two, else -1.
inline int pow2_shift(int d) { return d > 0 && (d & (d - 1)) == 0 ? __builtin_ctz((unsigned)d) : -1; }
constexpr int kInt32Big = 0x7FFFFFFF;

__device__ __forceinline__ int wrap_add(int a, int b) { return (int)((unsigned)a + (unsigned)b); }
__device__ __forceinline__ int wrap_mul(int a, int b) { return (int)((unsigned)a * (unsigned)b); }

// One workgroup per row.  Sorting is a rank sort: element i lands at
// #{j : v_j < v_i} + #{j < i : v_j == v_i}, which is stable and needs no
// barriers beyond the load.  Invalid ids carry the key 2^31-1 and sort last.
__global__ __launch_bounds__(256) void expand_kernel(const int* __restrict__ cand, int64_t cand_ld, int K, int ratio,
                                                     const int* __restrict__ row_ks, int64_t ks_stride,
                                                     const int* __restrict__ row_ke, int64_t ke_stride, int sbk,
                                                     int* __restrict__ si, int64_t si_ld, int* __restrict__ end,
                                                     int64_t end_stride) {
  __shared__ int s_val[kMaxSparse];
  __shared__ int s_sorted[kMaxSparse];
  __shared__ int s_n, s_last;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int S = K * ratio;
  const int ks = row_ks[(int64_t)r * ks_stride], ke = row_ke[(int64_t)r * ke_stride];
  int kv = wrap_add(ke, -ks);
  if (kv < 0) kv = 0;
  const int maxb = wrap_add(kv, sbk - 1) / sbk;
  if (tid == 0) {
    s_n = 0;
    s_last = -1;
  }
  __syncthreads();
  int my_n = 0, my_last = -1;
  for (int i = tid; i < S; i += 256) {
    const int c = cand[(int64_t)r * cand_ld + (ratio == 1 ? i : (i >> 1))];
    const int id = ratio == 1 ? c : wrap_add(wrap_mul(c, 2), i & 1);
    const bool ok = id >= 0 && id < maxb;
    s_val[i] = ok ? id : kInt32Big;
    if (ok) {
      my_n++;
      my_last = max(my_last, id);
    }
  }
  if (my_n) {
    atomicAdd(&s_n, my_n);
    atomicMax(&s_last, my_last);
  }
  __syncthreads();
  for (int i = tid; i < S; i += 256) {
    const int v = s_val[i];
    int rank = 0;
    for (int j = 0; j < S; j++) {
      const int u = s_val[j];
      rank += (u < v) || (u == v && j < i);
    }
    s_sorted[rank] = v;
  }
  __syncthreads();
  const int n = s_n, last = s_last;
  const int base = ks / sbk;
  const int pad = n > 0 ? wrap_add(last, base) : base;
  for (int j = tid; j < S; j += 256) si[(int64_t)r * si_ld + j] = j < n ? wrap_add(s_sorted[j], base) : pad;
  if (tid == 0) {
    int e = 0;
    if (n > 0) {
      int fill = wrap_add(ke, -wrap_add(wrap_mul(last, sbk), ks));
      fill = min(max(fill, 1), sbk);  // only the last block can be partial
      e = wrap_add(wrap_mul(n - 1, sbk), fill);
    }
    end[(int64_t)r * end_stride] = e;
  }
}

// Four entries per thread (one 16-byte load and store where the rows allow it), the
// divisions by the block size as shifts when it is a power of two (shift >= 0).
constexpr int kIdxPerThread = 4;

__device__ __forceinline__ int div_by(int x, int d, int shift) { return shift >= 0 ? x >> shift : x / d; }
__device__ __forceinline__ int mod_by(int x, int d, int shift) { return shift >= 0 ? x & (d - 1) : x % d; }

template <typename F>
__device__ __forceinline__ void map4(const int* in, int* out, int j0, int k, F&& f) {
  if (j0 + kIdxPerThread <= k && !((reinterpret_cast<uintptr_t>(in + j0) | reinterpret_cast<uintptr_t>(out + j0)) & 15)) {
    const int4 x = *reinterpret_cast<const int4*>(in + j0);
    *reinterpret_cast<int4*>(out + j0) = make_int4(f(x.x), f(x.y), f(x.z), f(x.w));
  } else {
    for (int j = j0; j < min(j0 + kIdxPerThread, k); j++) out[j] = f(in[j]);
  }
}

__global__ __launch_bounds__(256) void remap_kernel(const int* col, int64_t col_ld, int rows, int k,
                                                    const int* __restrict__ si, int64_t si_ld, int width,
                                                    const int* __restrict__ row_ks, int sbk, int sbk_shift, int* out,
                                                    int64_t out_ld) {
  const int r = blockIdx.y;
  const int j0 = (blockIdx.x * 256 + threadIdx.x) * kIdxPerThread;
  if (j0 >= k) return;
  const int base = div_by(row_ks[r], sbk, row_ks[r] >= 0 ? sbk_shift : -1);
  const int* sir = si + (int64_t)r * si_ld;
  map4(col + (int64_t)r * col_ld, out + (int64_t)r * out_ld, j0, k, [&](int c) {
    return c >= 0 && c < width ? (sir[div_by(c, sbk, sbk_shift)] - base) * sbk + mod_by(c, sbk, sbk_shift) : -1;
  });
}

__global__ __launch_bounds__(256) void slot_kernel(const int* idx, int64_t idx_ld, int k,
                                                   const int* __restrict__ row_to_req,
                                                   const int* __restrict__ block_table, int64_t bt_ld, int bt_width,
                                                   int num_reqs, int block_size, int bs_shift, int block_span, int* out,
                                                   int64_t out_ld) {
  const int r = blockIdx.y;
  const int j0 = (blockIdx.x * 256 + threadIdx.x) * kIdxPerThread;
  if (j0 >= k) return;
  const int req = row_to_req ? row_to_req[r] : r;
  const bool req_ok = req >= 0 && req < num_reqs;
  const int* btr = block_table + (int64_t)(req_ok ? req : 0) * bt_ld;
  map4(idx + (int64_t)r * idx_ld, out + (int64_t)r * out_ld, j0, k, [&](int p) {
    if (p < 0 || !req_ok) return -1;
    const int blk = div_by(p, block_size, bs_shift);
    return blk < bt_width ? btr[blk] * block_span + mod_by(p, block_size, bs_shift) : -1;
  });
}

}  // namespace
}  // namespace dsi

extern "C" int dsi_expand_candidates(const int32_t* cand, int64_t cand_ld, int32_t rows, int32_t num_candidates,
                                     const int32_t* row_ks, int64_t ks_stride, const int32_t* row_ke,
                                     int64_t ke_stride, int32_t candidate_block_size, int32_t sparse_block_kv,
                                     int32_t* sparse_indices, int64_t si_ld, int32_t* end, int64_t end_stride,
                                     hipStream_t stream) {
  using namespace dsi;
  const int sbk = sparse_block_kv;
  if (sbk < 8 || sbk > 128 || (sbk & (sbk - 1))) return DSI_EUNSUPPORTED;
  const int ratio = candidate_block_size / sbk;
  if (ratio * sbk != candidate_block_size || (ratio != 1 && ratio != 2)) return DSI_EUNSUPPORTED;
  if (rows < 0 || num_candidates < 1 || cand_ld < num_candidates || si_ld < (int64_t)num_candidates * ratio ||
      ks_stride < 1 || ke_stride < 1 || end_stride < 1)
    return DSI_EINVAL;
  if ((int64_t)num_candidates * ratio > kMaxSparse) return DSI_EUNSUPPORTED;
  if (rows == 0) return DSI_OK;
  if (!cand || !row_ks || !row_ke || !sparse_indices || !end) return DSI_EINVAL;
  hipLaunchKernelGGL(expand_kernel, dim3((unsigned)rows), dim3(256), 0, stream, cand, cand_ld, num_candidates, ratio,
                     row_ks, ks_stride, row_ke, ke_stride, sbk, sparse_indices, si_ld, end, end_stride);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}

extern "C" int dsi_topk_remap(const int32_t* col, int64_t col_ld, int32_t rows, int32_t k,
                              const int32_t* sparse_indices, int64_t si_ld, int32_t num_sparse_blocks,
                              const int32_t* row_ks, int32_t sparse_block_kv, int32_t* out, int64_t out_ld,
                              hipStream_t stream) {
  using namespace dsi;
  if (sparse_block_kv < 1) return DSI_EUNSUPPORTED;
  if (rows < 0 || k < 0 || num_sparse_blocks < 0 || col_ld < k || out_ld < k || si_ld < num_sparse_blocks)
    return DSI_EINVAL;
  const int64_t width = (int64_t)num_sparse_blocks * sparse_block_kv;
  if (width > 0x7FFFFFFF) return DSI_EUNSUPPORTED;
  if (rows == 0 || k == 0) return DSI_OK;
  if (!col || !sparse_indices || !row_ks || !out) return DSI_EINVAL;
  if (rows > 65535) return DSI_EUNSUPPORTED;
  const int per_block = 256 * kIdxPerThread;
  hipLaunchKernelGGL(remap_kernel, dim3((unsigned)((k + per_block - 1) / per_block), (unsigned)rows), dim3(256), 0,
                     stream, col, col_ld, rows, k, sparse_indices, si_ld, (int)width, row_ks, sparse_block_kv,
                     pow2_shift(sparse_block_kv), out, out_ld);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}

extern "C" int dsi_req_index_to_global_slot(const int32_t* idx, int64_t idx_ld, int32_t rows, int32_t k,
                                            const int32_t* row_to_req, const int32_t* block_table, int64_t bt_ld,
                                            int32_t bt_width, int32_t num_reqs, int32_t block_size, int32_t block_span, int32_t* out,
                                            int64_t out_ld, hipStream_t stream) {
  using namespace dsi;
  if (block_size < 1 || block_span < block_size) return DSI_EUNSUPPORTED;
  if (rows < 0 || k < 0 || idx_ld < k || out_ld < k || bt_width < 0 || bt_ld < bt_width || num_reqs < 0)
    return DSI_EINVAL;
  if (rows == 0 || k == 0) return DSI_OK;
  if (!idx || !block_table || !out) return DSI_EINVAL;
  if (rows > 65535) return DSI_EUNSUPPORTED;
  const int per_block = 256 * kIdxPerThread;
  hipLaunchKernelGGL(slot_kernel, dim3((unsigned)((k + per_block - 1) / per_block), (unsigned)rows), dim3(256), 0,
                     stream, idx, idx_ld, k, row_to_req, block_table, bt_ld, bt_width, num_reqs, block_size,
                     pow2_shift(block_size), block_span, out, out_ld);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}
