// Top-k of few long rows, split between workgroups: the workspace layout shared by the
// producers of its first-digit histograms and the selection kernels (topk.hip).
//
// A row's selection (P3 data flow 2 of "DeepSeek V3.2 稀疏注意力 DSA 推理流程图解": the k
// best positions per query row, -1 for an empty slot) starts from the histogram of the top
// 11 bits of its order-preserving keys.  Parts of a row are counted separately, each into a
// "slot": by the split path's own histogram kernel (one slot per row slice) or by the paged
// decode kernel while it writes the logits (one slot per workgroup and row it scores).  The
// row's slots are consecutive, [first, last] in its metadata.
//
// Workspace, from its start (16-byte aligned):
//   slots  uint32 [num_slots][1024]: slot s holds bins 2j (low half) and 2j+1 (high half) of
//          word j; a part never exceeds 65535 columns, so the halves never carry;
//   meta   int32  [rows][8]: 0 first slot, 1 last slot, 2 columns written so far, 3 boundary-bin
//          candidates collected so far, 4 slices done (2..4: device-scope atomic counters, zeroed
//          by the writer of the row's first slot);
//   cand   uint64 [rows][kSplitCap]: the row's boundary-bin candidates, key in the low word and
//          column in the high word, written and read only with device-scope atomics (the row's
//          last slice to finish reads every slice's candidates at the point of coherence).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsi {

constexpr int kSplitBins = 2048;          // first digit: the top 11 key bits
constexpr int kSlotWords = kSplitBins / 2;
constexpr int kSlotBytes = kSlotWords * 4;
constexpr int kSplitCap = 12288;          // boundary-bin candidates kept per row
constexpr int kMetaInts = 8;

enum SplitMeta { kMetaFirst = 0, kMetaLast, kMetaCntGt, kMetaCntEq, kMetaDone };

struct SplitWs {
  uint32_t* slots;
  int* meta;
  unsigned long long* cand;
};

__host__ __device__ inline size_t split_ws_bytes(int64_t rows, int64_t num_slots) {
  return (size_t)num_slots * kSlotBytes + (size_t)rows * kMetaInts * 4 + (size_t)rows * kSplitCap * 8;
}

__host__ __device__ inline SplitWs split_ws(void* ws, int64_t rows, int64_t num_slots) {
  uint8_t* p = static_cast<uint8_t*>(ws);
  SplitWs w;
  w.slots = reinterpret_cast<uint32_t*>(p);
  p += (size_t)num_slots * kSlotBytes;
  w.meta = reinterpret_cast<int*>(p);
  p += (size_t)rows * kMetaInts * 4;
  w.cand = reinterpret_cast<unsigned long long*>(p);
  return w;
}

// Where a row's valid columns are: [start, end) from caller arrays (row_starts nullable, both
// clamped to [0, max_width)), or from decode context lengths (row b*next_n + i of a request
// of length L sees [0, min(L - next_n + i + 1, max_width))).
struct RowRange {
  const int* starts;
  const int* ends;
  const int* lens;  // non-null: the decode form
  int next_n;
  int max_width;
  __device__ __forceinline__ void get(int r, int& st, int& en) const {
    if (lens) {
      const int b = r / next_n, i = r - b * next_n;
      st = 0;
      en = min(max(lens[b] - next_n + i + 1, 0), max_width);
    } else {
      st = starts ? max(starts[r], 0) : 0;
      en = max(min(ends[r], max_width), st);
    }
  }
};

// fp32 logits: a value's first-digit bin (top 11 bits of its order-preserving key).  Finite values
// have bins in [4, 2044); -inf, +inf and NaN fall in bins 0..3 and 2044..2047, which the selection
// ignores, so a producer may count every column of a row's range.
__device__ __forceinline__ uint32_t f32_first_bin(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return key >> 21;
}

// dsi_topk_select after its argument checks: every row's range from `range`, fp32 or bf16 logits
// [rows][ld], the workspace of dsi_topk_workspace_bytes(rows, max_width, k).
int topk_dispatch(const void* logits, bool bf16, int64_t ld, int rows, const RowRange& range, int max_width, int k,
                  int* out, int64_t out_ld, void* workspace, hipStream_t stream);

// Selection over slots already written (by the paged decode kernel): the split path's selection
// launch, on `stream`.  Rows are fp32.  G = workgroups per row.
int launch_split_select(const float* logits, int64_t ld, int rows, const RowRange& range, int k, int* out,
                        int64_t out_ld, void* ws, int64_t num_slots, int G, hipStream_t stream);

// Workgroups per row of the split path for `rows` fp32 rows of up to max_width columns (its slices
// hold at most 8192 columns); 1 when the rows are not split.
int split_groups_f32(int rows, int max_width);

}  // namespace dsi
