// Dense prefill indexer logits over gathered K (P3 step ⑥ and the prefill/decode
// table of "DeepSeek V3.2 稀疏注意力 DSA 推理流程图解": prefill gathers the history
// K, then scores every history token for every query token).
//
// The contraction [T*64, 128] x [128, S] runs on the matrix cores with the FP8 codes
// decoded exactly to f16 (see common.h for why and how); the head-weighted sum is the
// epilogue.  A workgroup owns 8 query rows (two per wavefront, q decoded once and
// held in VGPRs) and a chunk of 1024 keys, streamed through LDS in double-buffered
// tiles of 64 keys that are decoded to f16 as they are staged (each staged key is
// then read by all 8 rows); tiles wholly outside the rows' [ks, ke) ranges are never
// loaded, so causal work above the diagonal is skipped.  Consecutive workgroups on
// one XCD share the same rows (their q in that XCD's L2); K (132 B per key) is
// re-read from L2 by each row tile.
#include "common.h"

namespace dsi {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfRowsPerWave = 2;
constexpr int kPfRows = kPfWaves * kPfRowsPerWave;  // query rows per workgroup
constexpr int kTileKeys = 64;                        // keys per LDS tile
constexpr int kChunkTiles = 16;                      // tiles per workgroup
constexpr int kChunkKeys = kTileKeys * kChunkTiles;
constexpr int kTileChunks16 = kTileKeys * kRow / 16;  // 528 sixteen-byte chunks per full tile
constexpr int kLoadsPerThread = (kTileChunks16 + 255) / 256;

struct TileRegs {
  uint4 v[kLoadsPerThread];
  uint32_t tail;  // one dword of a tile whose byte size is not a multiple of 16
};

__device__ __forceinline__ void load_tile(TileRegs& r, const uint8_t* k_rows, int key0, int nkeys, int tid) {
  const int bytes = nkeys * kRow;
  const int full = bytes >> 4;
  const uint8_t* base = k_rows + (int64_t)key0 * kRow;
#pragma unroll
  for (int j = 0; j < kLoadsPerThread; j++) {
    int c = tid + j * 256;
    if (c < full) r.v[j] = *reinterpret_cast<const uint4*>(base + c * 16);
  }
  int tail_words = (bytes & 15) >> 2;
  if (tid < tail_words) r.tail = *reinterpret_cast<const uint32_t*>(base + full * 16 + tid * 4);
}

__device__ __forceinline__ void store_tile(const TileRegs& r, uint8_t* codes, float* scale, int nkeys, int tid) {
  const int bytes = nkeys * kRow;
  const int full = bytes >> 4;
#pragma unroll
  for (int j = 0; j < kLoadsPerThread; j++) {
    int c = tid + j * 256;
    if (c < full) {
      scatter_word_f16(codes, scale, c * 4 + 0, r.v[j].x);
      scatter_word_f16(codes, scale, c * 4 + 1, r.v[j].y);
      scatter_word_f16(codes, scale, c * 4 + 2, r.v[j].z);
      scatter_word_f16(codes, scale, c * 4 + 3, r.v[j].w);
    }
  }
  int tail_words = (bytes & 15) >> 2;
  if (tid < tail_words) scatter_word_f16(codes, scale, full * 4 + tid, r.tail);
}

__global__ __launch_bounds__(256) void prefill_logits_kernel(
    const uint8_t* __restrict__ q, const uint16_t* __restrict__ w, int T, const uint8_t* __restrict__ k_rows, int S,
    const int* __restrict__ row_ks, const int* __restrict__ row_ke, float* __restrict__ logits, int64_t ld,
    int n_chunks) {
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[2][kTileKeys * kLdsKeyStrideF16];
  __shared__ float s_scale[2][kTileKeys];

  // Workgroups are dealt to the 8 XCDs round-robin; renumber so that the chunks
  // of one row tile run on the same XCD.
  const int nwg = gridDim.x;
  int id = blockIdx.x;
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  const int rt = id / n_chunks, chunk = id - rt * n_chunks;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t_first = rt * kPfRows;

  // Union of the workgroup's row ranges, clipped to this chunk.
  int lo = 0x7FFFFFFF, hi = 0;
#pragma unroll
  for (int i = 0; i < kPfRows; i++) {
    int t = t_first + i;
    if (t < T) {
      int a = max(row_ks[t], 0), b = min(row_ke[t], S);
      if (a < b) {
        lo = min(lo, a);
        hi = max(hi, b);
      }
    }
  }
  const int c_lo = max(chunk * kChunkKeys, lo);
  const int c_hi = min(chunk * kChunkKeys + kChunkKeys, hi);
  if (c_lo >= c_hi) return;  // uniform across the workgroup
  const int tile_first = c_lo / kTileKeys, tile_end = (c_hi + kTileKeys - 1) / kTileKeys;

  // This wavefront's rows: q fragments, weights and ranges.
  QFrag qf[kPfRowsPerWave];
  WFrag wf[kPfRowsPerWave];
  int rks[kPfRowsPerWave], rke[kPfRowsPerWave], trow[kPfRowsPerWave];
#pragma unroll
  for (int r = 0; r < kPfRowsPerWave; r++) {
    int t = t_first + wave * kPfRowsPerWave + r;
    trow[r] = t;
    int tc = min(t, T - 1);
    load_q(qf[r], q + (int64_t)tc * kHeads * kDim, lane);
    load_w(wf[r], w + (int64_t)tc * kHeads, lane);
    rks[r] = t < T ? max(row_ks[t], 0) : 0;
    rke[r] = t < T ? min(row_ke[t], S) : 0;
  }

  TileRegs regs;
  {
    int key0 = tile_first * kTileKeys;
    int nk = min(kTileKeys, S - key0);
    load_tile(regs, k_rows, key0, nk, tid);
    store_tile(regs, s_codes[0], s_scale[0], nk, tid);
  }
  __syncthreads();

  const int n = lane & 15, g = lane >> 4;
  for (int tile = tile_first; tile < tile_end; tile++) {
    const int buf = (tile - tile_first) & 1;
    const bool has_next = tile + 1 < tile_end;
    const int nkey0 = (tile + 1) * kTileKeys;
    const int nnk = has_next ? min(kTileKeys, S - nkey0) : 0;
    if (has_next) load_tile(regs, k_rows, nkey0, nnk, tid);

    const int key0 = tile * kTileKeys;
    // 4 key groups of 16 per tile, taken two at a time with both rows: four outputs per lane.
#pragma unroll
    for (int pair = 0; pair < 2; pair++) {
      float part[4];
#pragma unroll
      for (int kg = 0; kg < 2; kg++) {
        KFrag kb;
        load_kfrag_f16(kb, s_codes[buf] + (pair * 2 + kg) * 16 * kLdsKeyStrideF16, lane);
#pragma unroll
        for (int r = 0; r < kPfRowsPerWave; r++) part[r * 2 + kg] = score_partial(qf[r], wf[r], kb);
      }
      const float v = transpose_reduce4(part, lane);
      // lane group g owns output j = g: row g>>1, key group pair*2 + (g&1)
      const int r = g >> 1;
      const int kslot = (pair * 2 + (g & 1)) * 16 + n;
      const int key = key0 + kslot;
      const int rk = r ? rks[1] : rks[0], re = r ? rke[1] : rke[0], t = r ? trow[1] : trow[0];
      if (key >= rk && key < re) logits[(int64_t)t * ld + key] = v * (s_scale[buf][kslot] * kF16Unscale);
    }

    if (has_next) store_tile(regs, s_codes[buf ^ 1], s_scale[buf ^ 1], nnk, tid);
    __syncthreads();
  }
}

}  // namespace
}  // namespace dsi

extern "C" int dsi_mqa_logits_prefill(const uint8_t* q, const uint16_t* w, int32_t T, const uint8_t* k_rows,
                                      int32_t S, const int32_t* row_ks, const int32_t* row_ke, float* logits,
                                      int64_t ld, hipStream_t stream) {
  using namespace dsi;
  if (T < 0 || S < 0 || ld < S) return DSI_EINVAL;
  if (T == 0 || S == 0) return DSI_OK;
  if (!q || !w || !k_rows || !row_ks || !row_ke || !logits) return DSI_EINVAL;
  if ((reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(k_rows) & 15) ||
      (reinterpret_cast<uintptr_t>(w) & 7) || (reinterpret_cast<uintptr_t>(logits) & 3))
    return DSI_EALIGN;
  const int row_tiles = (T + kPfRows - 1) / kPfRows;
  const int n_chunks = (S + kChunkKeys - 1) / kChunkKeys;
  const int64_t grid = (int64_t)row_tiles * n_chunks;
  if (grid > 0x7FFFFFFF) return DSI_EUNSUPPORTED;
  hipLaunchKernelGGL(prefill_logits_kernel, dim3((unsigned)grid), dim3(256), 0, stream, q, w, T, k_rows, S, row_ks,
                     row_ke, logits, ld, n_chunks);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}
