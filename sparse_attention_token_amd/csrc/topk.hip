// Per-row top-k selection into the index table main attention reads (P3 data flow 2
// of "DeepSeek V3.2 稀疏注意力 DSA 推理流程图解": the k best positions per query row
// as int32, -1 for an empty slot; P3 pitfalls: request-relative positions; P1 "V4.1
// 索引器接入稀疏 MQA logits": the compressed-space top-k runs on bf16 logits).
//
// Radix select, no sort: values map to order-preserving unsigned keys (non-finite
// values are dropped); a most-significant-digit-first pass per digit builds an LDS
// histogram of the keys that still match the selected prefix and picks the digit
// where the count from the top reaches k.  After the last digit the k-th largest
// key tau is exact; one more pass writes every key > tau and enough keys == tau,
// each wavefront reserving its output slots with one LDS atomic (ballot + popcount).
// One workgroup of 1024 threads per row; the row is re-read from L2 on each pass.
#include "common.h"

namespace dsi {
namespace {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kHistBins = 2048;

template <bool BF16>
struct KeyOf {
  static __device__ __forceinline__ bool load(const void* row, int i, uint32_t& key) {
    if (BF16) {
      const uint32_t h = reinterpret_cast<const uint16_t*>(row)[i];
      key = bf16_key(h);
      return (h & 0x7F80u) != 0x7F80u;
    } else {
      const uint32_t u = reinterpret_cast<const uint32_t*>(row)[i];
      key = f32_key(u);
      return (u & 0x7F800000u) != 0x7F800000u;
    }
  }
};

// Exclusive suffix sum over threads (thread i gets the sum of `x` of all threads > i).
__device__ __forceinline__ int block_suffix_excl(int x, int* s_wave, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  // inclusive suffix scan within the wave (lanes above contribute)
  int v = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_down(v, off);
    if (lane + off < 64) v += y;
  }
  if (lane == 0) s_wave[wave] = v;  // wave total
  __syncthreads();
  int above = 0;
  for (int j = wave + 1; j < kTkWaves; j++) above += s_wave[j];
  __syncthreads();
  return v - x + above;
}

template <bool BF16>
__global__ __launch_bounds__(kTkThreads) void topk_kernel(const uint8_t* __restrict__ logits, int64_t row_bytes,
                                                          const int* __restrict__ row_starts,
                                                          const int* __restrict__ row_ends, int max_width, int k,
                                                          int* __restrict__ out, int64_t out_ld) {
  __shared__ int s_hist[kHistBins];
  __shared__ int s_wave[kTkWaves];
  __shared__ int s_sel[4];  // digit, count above, total valid
  __shared__ int s_cnt[2];

  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int st = row_starts ? max(row_starts[r], 0) : 0;
  const int en = min(row_ends[r], max_width);
  const int n = max(en - st, 0);
  const void* row = logits + (int64_t)r * row_bytes;
  int* orow = out + (int64_t)r * out_ld;

  constexpr int kPasses = BF16 ? 2 : 3;
  // digit (shift, width) from the most significant end
  const int shifts[3] = {BF16 ? 5 : 21, BF16 ? 0 : 10, 0};
  const int widths[3] = {11, BF16 ? 5 : 11, 10};

  uint32_t prefix = 0;   // selected high bits so far
  int need = k;          // how many still to take at or below the prefix
  int total = 0;
  bool take_all = false;

  for (int p = 0; p < kPasses; p++) {
    const int sh = shifts[p], wd = widths[p];
    const int nb = 1 << wd;
    for (int i = tid; i < nb; i += kTkThreads) s_hist[i] = 0;
    __syncthreads();
    const int hs = sh + wd;  // bits at and above hs are fixed by the prefix
    for (int i = tid; i < n; i += kTkThreads) {
      uint32_t key;
      if (KeyOf<BF16>::load(row, st + i, key)) {
        if (hs >= 32 || (key >> hs) == (prefix >> hs)) atomicAdd(&s_hist[(key >> sh) & (nb - 1)], 1);
      }
    }
    __syncthreads();
    // two bins per thread, counted from the top
    const int b0 = 2 * tid, b1 = 2 * tid + 1;
    const int h0 = b0 < nb ? s_hist[b0] : 0, h1 = b1 < nb ? s_hist[b1] : 0;
    const int above = block_suffix_excl(h0 + h1, s_wave, tid);
    if (p == 0 && tid == 0) s_sel[2] = above + h0 + h1;  // total number of valid values
    if (above < need && need <= above + h0 + h1) {
      if (above + h1 >= need) {
        s_sel[0] = b1;
        s_sel[1] = above;
      } else {
        s_sel[0] = b0;
        s_sel[1] = above + h1;
      }
    }
    __syncthreads();
    if (p == 0) {
      total = s_sel[2];
      if (total <= k) {
        take_all = true;
        break;
      }
    }
    prefix |= (uint32_t)s_sel[0] << sh;
    need -= s_sel[1];
    __syncthreads();
  }

  if (tid < 2) s_cnt[tid] = 0;
  __syncthreads();
  const int n_gt = take_all ? 0 : k - need;  // keys strictly above tau
  const uint32_t tau = prefix;
  for (int i0 = 0; i0 < n; i0 += kTkThreads) {
    const int i = i0 + tid;
    uint32_t key = 0;
    bool valid = i < n && KeyOf<BF16>::load(row, st + i, key);
    const bool gt = valid && (take_all || key > tau);
    const bool eq = valid && !take_all && key == tau;
    const uint64_t mgt = __ballot(gt), meq = __ballot(eq);
    int base_gt = 0, base_eq = 0;
    if (lane == 0) {
      if (mgt) base_gt = atomicAdd(&s_cnt[0], __popcll(mgt));
      if (meq) base_eq = atomicAdd(&s_cnt[1], __popcll(meq));
    }
    base_gt = __shfl(base_gt, 0);
    base_eq = __shfl(base_eq, 0);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (gt) orow[base_gt + __popcll(mgt & below)] = i;
    if (eq) {
      const int pos = base_eq + __popcll(meq & below);
      if (pos < need) orow[n_gt + pos] = i;
    }
  }
  const int m = take_all ? total : k;
  for (int j = m + tid; j < k; j += kTkThreads) orow[j] = -1;
}

}  // namespace
}  // namespace dsi

extern "C" size_t dsi_topk_workspace_bytes(int32_t rows, int32_t max_width, int32_t k) {
  (void)rows;
  (void)max_width;
  (void)k;
  return 0;
}

extern "C" int dsi_topk_select(const void* logits, int32_t dtype, int64_t ld, int32_t rows,
                               const int32_t* row_starts, const int32_t* row_ends, int32_t max_width, int32_t k,
                               int32_t* out, int64_t out_ld, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  using namespace dsi;
  (void)workspace;
  if (dtype != DSI_F32 && dtype != DSI_BF16) return DSI_EUNSUPPORTED;
  if (k < 1 || k > DSI_MAX_TOPK) return DSI_EUNSUPPORTED;
  if (rows < 0 || max_width < 0 || ld < max_width || out_ld < k) return DSI_EINVAL;
  if (workspace_bytes < dsi_topk_workspace_bytes(rows, max_width, k)) return DSI_EWORKSPACE;
  if (rows == 0) return DSI_OK;
  if (!logits || !row_ends || !out) return DSI_EINVAL;
  if (dtype == DSI_F32 && (reinterpret_cast<uintptr_t>(logits) & 3)) return DSI_EALIGN;
  if (dtype == DSI_BF16 && (reinterpret_cast<uintptr_t>(logits) & 1)) return DSI_EALIGN;
  if (reinterpret_cast<uintptr_t>(out) & 3) return DSI_EALIGN;
  const int64_t row_bytes = ld * (dtype == DSI_F32 ? 4 : 2);
  if (dtype == DSI_F32)
    hipLaunchKernelGGL(topk_kernel<false>, dim3((unsigned)rows), dim3(kTkThreads), 0, stream,
                       reinterpret_cast<const uint8_t*>(logits), row_bytes, row_starts, row_ends, max_width, k, out,
                       out_ld);
  else
    hipLaunchKernelGGL(topk_kernel<true>, dim3((unsigned)rows), dim3(kTkThreads), 0, stream,
                       reinterpret_cast<const uint8_t*>(logits), row_bytes, row_starts, row_ends, max_width, k, out,
                       out_ld);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}
