// Top-k under context parallelism (P3 "DeepSeek V3.2 稀疏注意力 DSA 推理流程图解", pitfalls:
// with a request's context split across ranks, each rank keeps its local top-k candidates,
// only those are exchanged, and the global top-k is chosen from them; exact, because a token
// of the global top-k is in the local top-k of the rank that holds it).
//
//  - topk_values_kernel turns one rank's local selection into (value, global index) pairs:
//    the values are read back from the rank's logits at the selected columns, the indices
//    mapped from the rank's columns to the whole context by a scale and an offset.
//  - The merge lays every row's exchanged candidates out as one fp32 row in the caller's
//    workspace (empty or non-finite candidates as NaN, which selection ignores), selects
//    the k largest with the library's own top-k, and maps the selected candidate slots back
//    to their global indices in place.
// Elementwise and gather steps: a few MB per call at the shapes of a decode step.
#include "common.h"

namespace dsi {
namespace {

__global__ __launch_bounds__(256) void topk_values_kernel(const float* __restrict__ logits, int64_t ld,
                                                          const int* __restrict__ row_starts, int max_width,
                                                          const int* __restrict__ idx, int64_t idx_ld, int k,
                                                          int index_scale, int index_offset, float* __restrict__ vals,
                                                          int64_t vals_ld, int* __restrict__ gidx, int64_t gidx_ld) {
  const int r = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
  if (j >= k) return;
  const int st = row_starts ? max(row_starts[r], 0) : 0;
  const int p = idx[(int64_t)r * idx_ld + j];
  float v = -__builtin_inff();
  int g = -1;
  if (p >= 0 && (int64_t)st + p < max_width) {
    v = logits[(int64_t)r * ld + st + p];
    g = (int)((unsigned)p * (unsigned)index_scale + (unsigned)index_offset);
  }
  vals[(int64_t)r * vals_ld + j] = v;
  gidx[(int64_t)r * gidx_ld + j] = g;
}

// Candidate slot c of row r (list c / k_in, entry c % k_in) -> one fp32 row of width
// num_lists * k_in; the row's end (its width) goes to ends[r].
__global__ __launch_bounds__(256) void merge_compose_kernel(const float* __restrict__ vals,
                                                            const int* __restrict__ gidx, int64_t list_stride,
                                                            int64_t row_ld, int k_in, int width,
                                                            float* __restrict__ rows_out, int* __restrict__ ends) {
  const int r = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
  if (c == 0) ends[r] = width;
  if (c >= width) return;
  const int l = c / k_in, j = c - l * k_in;
  const int64_t a = (int64_t)l * list_stride + (int64_t)r * row_ld + j;
  rows_out[(int64_t)r * width + c] = gidx[a] >= 0 ? vals[a] : __builtin_nanf("");
}

__global__ __launch_bounds__(256) void merge_map_kernel(const int* __restrict__ gidx, int64_t list_stride,
                                                        int64_t row_ld, int k_in, int* __restrict__ out,
                                                        int64_t out_ld, int k) {
  const int r = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
  if (j >= k) return;
  int* o = out + (int64_t)r * out_ld + j;
  const int c = *o;
  if (c >= 0) {
    const int l = c / k_in;
    *o = gidx[(int64_t)l * list_stride + (int64_t)r * row_ld + (c - l * k_in)];
  }
}

struct MergeWs {
  int* ends;
  float* rows;
  void* topk;
  size_t topk_bytes;
};

inline size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

inline MergeWs merge_ws(void* base, int rows, int width) {
  uint8_t* p = static_cast<uint8_t*>(base);
  MergeWs w;
  w.ends = reinterpret_cast<int*>(p);
  p += align16((size_t)rows * 4);
  w.rows = reinterpret_cast<float*>(p);
  p += align16((size_t)rows * width * 4);
  w.topk = p;
  w.topk_bytes = dsi_topk_workspace_bytes(rows, width, 1);  // independent of k
  return w;
}

}  // namespace
}  // namespace dsi

extern "C" int dsi_topk_values(const float* logits, int64_t ld, int32_t rows, const int32_t* row_starts,
                               int32_t max_width, const int32_t* idx, int64_t idx_ld, int32_t k, int32_t index_scale,
                               int32_t index_offset, float* vals, int64_t vals_ld, int32_t* gidx, int64_t gidx_ld,
                               hipStream_t stream) {
  using namespace dsi;
  if (rows < 0 || k < 0 || max_width < 0 || ld < max_width || idx_ld < k || vals_ld < k || gidx_ld < k)
    return DSI_EINVAL;
  if (rows == 0 || k == 0) return DSI_OK;
  if (!logits || !idx || !vals || !gidx) return DSI_EINVAL;
  if (rows > 65535) return DSI_EUNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(logits) | reinterpret_cast<uintptr_t>(idx) | reinterpret_cast<uintptr_t>(vals) |
       reinterpret_cast<uintptr_t>(gidx)) & 3)
    return DSI_EALIGN;
  hipLaunchKernelGGL(topk_values_kernel, dim3((unsigned)((k + 255) / 256), (unsigned)rows), dim3(256), 0, stream,
                     logits, ld, row_starts, max_width, idx, idx_ld, k, index_scale, index_offset, vals, vals_ld, gidx,
                     gidx_ld);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}

extern "C" size_t dsi_topk_merge_workspace_bytes(int32_t rows, int32_t num_lists, int32_t k_in) {
  using namespace dsi;
  if (rows <= 0 || num_lists <= 0 || k_in <= 0 || (int64_t)num_lists * k_in > 0x7FFFFFFF) return 0;
  const int width = num_lists * k_in;
  return align16((size_t)rows * 4) + align16((size_t)rows * width * 4) + dsi_topk_workspace_bytes(rows, width, 1);
}

extern "C" int dsi_topk_merge(const float* vals, const int32_t* gidx, int64_t list_stride, int64_t row_ld,
                              int32_t num_lists, int32_t rows, int32_t k_in, int32_t k, int32_t* out, int64_t out_ld,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace dsi;
  if (k < 1 || k > DSI_MAX_TOPK) return DSI_EUNSUPPORTED;
  if (rows < 0 || num_lists < 1 || k_in < 1 || row_ld < k_in || out_ld < k) return DSI_EINVAL;
  if ((int64_t)num_lists * k_in > 0x7FFFFFFF) return DSI_EUNSUPPORTED;
  if (rows == 0) return DSI_OK;
  if (!vals || !gidx || !out) return DSI_EINVAL;
  if (rows > 65535) return DSI_EUNSUPPORTED;
  if (workspace_bytes < dsi_topk_merge_workspace_bytes(rows, num_lists, k_in) || !workspace) return DSI_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(vals) | reinterpret_cast<uintptr_t>(gidx) | reinterpret_cast<uintptr_t>(out)) & 3)
    return DSI_EALIGN;
  if (reinterpret_cast<uintptr_t>(workspace) & 15) return DSI_EALIGN;
  const int width = num_lists * k_in;
  const MergeWs w = merge_ws(workspace, rows, width);
  hipLaunchKernelGGL(merge_compose_kernel, dim3((unsigned)((width + 255) / 256), (unsigned)rows), dim3(256), 0, stream,
                     vals, gidx, list_stride, row_ld, k_in, width, w.rows, w.ends);
  if (hipGetLastError() != hipSuccess) return DSI_ELAUNCH;
  const int st = dsi_topk_select(w.rows, DSI_F32, width, rows, nullptr, w.ends, width, k, out, out_ld, w.topk,
                                 w.topk_bytes, stream);
  if (st != DSI_OK) return st;
  hipLaunchKernelGGL(merge_map_kernel, dim3((unsigned)((k + 255) / 256), (unsigned)rows), dim3(256), 0, stream, gidx,
                     list_stride, row_ld, k_in, out, out_ld, k);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}
