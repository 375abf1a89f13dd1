// Prefill K gather: the history K of a prefill chunk's requests, copied out of the paged
// indexer cache into contiguous 132-byte rows (P3 "DeepSeek V3.2 稀疏注意力 DSA 推理流程图解",
// prefill/decode table: prefill collects the history K before scoring it, decode reads the
// cache where it lies; P1 "V4.1 索引器接入稀疏 MQA logits", implementation breakdown: the
// indexer's forward chains the prefill K gather with the paged decode path).
//
// Request r owns output rows [cu[r], cu[r+1]); its row cu[r] + p is its token p, i.e. the
// cache row block_table[r][p / block_size] * block_stride + (p % block_size) * 132.
//
// A pure copy, bound by HBM: 132 B read and 132 B written per row.  One workgroup owns 128
// consecutive output rows (32 groups of 4 rows; a group is 528 B = 33 aligned 16-byte
// chunks of the output).  First every thread resolves one row's source (request by
// binary search over the few requests the workgroup's rows span, then the page), then the
// workgroup streams its 16-byte output chunks: a group whose four sources are consecutive
// rows of one page at a 16-byte aligned address (every group of a request that starts on a
// multiple of 4 rows when block_size is a multiple of 4) moves as one 16-byte load per
// chunk; any other group assembles each chunk from four 4-byte loads of its rows.  Rows
// without a source are written as zeros.  The cache rows are read with the non-temporal hint
// (each is read once; 131072 rows: 10.5 -> 9.9 us), the output with the default policy (the
// logits kernel reads it next).
#include "common.h"

namespace dsi {
namespace {

constexpr int kGRows = 128;                    // output rows per workgroup
constexpr int kGGroups = kGRows / 4;           // 4-row groups
constexpr int kGChunks = kGGroups * 33;        // 16-byte chunks per workgroup (528 B per group)
constexpr int kGThreads = 256;
constexpr int kGIters = (kGChunks + kGThreads - 1) / kGThreads;
constexpr uint64_t kNoSrc = ~0ull;

__global__ __launch_bounds__(kGThreads) void gather_prefill_k_kernel(
    const uint8_t* __restrict__ pool, int64_t num_blocks, int32_t block_size, int64_t block_stride,
    const int32_t* __restrict__ block_table, int64_t bt_ld, int32_t bt_width, const int32_t* __restrict__ cu,
    int32_t num_reqs, uint8_t* __restrict__ out, int32_t S) {
  __shared__ uint64_t s_src[kGRows];
  __shared__ int s_fast[kGGroups];
  __shared__ int s_cnt[2];
  const int tid = threadIdx.x;
  const int r0 = (int)blockIdx.x * kGRows;
  const int nrows = min(kGRows, S - r0);
  const int rl = r0 + nrows - 1;

  // Requests spanned by rows r0..rl: #{j : cu[j] <= row} - 1 for the first and last row.
  if (tid < 2) s_cnt[tid] = 0;
  __syncthreads();
  int c0 = 0, c1 = 0;
  for (int j = tid; j <= num_reqs; j += kGThreads) {
    const int v = cu[j];
    c0 += v <= r0;
    c1 += v <= rl;
  }
  if (c0) atomicAdd(&s_cnt[0], c0);
  if (c1) atomicAdd(&s_cnt[1], c1);
  __syncthreads();

  if (tid < kGRows) {
    const int row = r0 + tid;
    uint64_t src = kNoSrc;
    if (tid < nrows && num_reqs > 0) {
      int lo = max(s_cnt[0] - 1, 0);
      int hi = max(min(s_cnt[1] - 1, num_reqs - 1), lo);
      while (lo < hi) {  // last request starting at or before `row`
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= row) lo = mid;
        else hi = mid - 1;
      }
      const int b = cu[lo], e = cu[lo + 1];
      if (b <= row && row < e) {
        const int64_t p = (int64_t)row - b;
        const int64_t blk = p / block_size;
        if (blk < bt_width) {
          const int page = block_table[(int64_t)lo * bt_ld + blk];
          if (page >= 0 && page < num_blocks)
            src = (uint64_t)page * (uint64_t)block_stride + (uint64_t)(p % block_size) * kRow;
        }
      }
    }
    s_src[tid] = src;
  }
  __syncthreads();
  if (tid < kGGroups) {
    const uint64_t a = s_src[4 * tid];
    bool fast = a != kNoSrc && ((reinterpret_cast<uintptr_t>(pool) + a) & 15) == 0;
#pragma unroll
    for (int i = 1; i < 4; i++) fast = fast && s_src[4 * tid + i] == a + (uint64_t)(kRow * i);
    s_fast[tid] = fast;
  }
  __syncthreads();

  const int nbytes = nrows * kRow;
  uint8_t* obase = out + (int64_t)r0 * kRow;
  uint4 v[kGIters];
#pragma unroll
  for (int it = 0; it < kGIters; it++) {
    const int c = tid + it * kGThreads;
    v[it] = make_uint4(0, 0, 0, 0);
    if (c < kGChunks && c * 16 < nbytes) {
      const int g = c / 33, q = c - g * 33;
      if (s_fast[g]) {
        {
          typedef uint32_t v4u __attribute__((ext_vector_type(4)));
          const v4u x = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(pool + s_src[4 * g] + q * 16));
          v[it] = make_uint4(x[0], x[1], x[2], x[3]);
        }
      } else {
        uint32_t d[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
          const int b = q * 16 + 4 * k, rr = b / kRow, o = b - rr * kRow;
          const uint64_t a = s_src[4 * g + rr];
          d[k] = a == kNoSrc ? 0u : __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(pool + a + o));
        }
        v[it] = make_uint4(d[0], d[1], d[2], d[3]);
      }
    }
  }
#pragma unroll
  for (int it = 0; it < kGIters; it++) {
    const int c = tid + it * kGThreads;
    const int off = c * 16;
    if (c >= kGChunks || off >= nbytes) continue;
    if (off + 16 <= nbytes) {
      *reinterpret_cast<uint4*>(obase + off) = v[it];
    } else {  // the output's last rows end inside this chunk (S not a multiple of 4)
      const uint32_t d[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
      for (int k = 0; k < 4 && off + 4 * k < nbytes; k++) *reinterpret_cast<uint32_t*>(obase + off + 4 * k) = d[k];
    }
  }
}

}  // namespace
}  // namespace dsi

extern "C" int dsi_gather_prefill_k(const uint8_t* pool, int64_t num_blocks, int32_t block_size,
                                    int64_t block_stride_bytes, const int32_t* block_table, int64_t bt_ld,
                                    int32_t bt_width, const int32_t* cu_seq_lens, int32_t num_reqs, uint8_t* k_rows,
                                    int32_t S, hipStream_t stream) {
  using namespace dsi;
  if (S < 0 || num_reqs < 0 || num_blocks < 0 || block_size < 1 || bt_width < 0 || bt_ld < bt_width ||
      block_stride_bytes < (int64_t)block_size * kRow)
    return DSI_EINVAL;
  if (S == 0) return DSI_OK;
  if (!pool || !block_table || !cu_seq_lens || !k_rows) return DSI_EINVAL;
  if (S > 0x7FFFFFFF - kGRows) return DSI_EUNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(k_rows) & 15) || (reinterpret_cast<uintptr_t>(pool) & 3) ||
      (block_stride_bytes & 3))
    return DSI_EALIGN;
  const unsigned grid = (unsigned)((S + kGRows - 1) / kGRows);
  hipLaunchKernelGGL(gather_prefill_k_kernel, dim3(grid), dim3(kGThreads), 0, stream, pool, num_blocks, block_size,
                     block_stride_bytes, block_table, bt_ld, bt_width, cu_seq_lens, num_reqs, k_rows, S);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}
