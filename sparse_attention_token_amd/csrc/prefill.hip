// Dense prefill indexer logits over gathered K (P3 step ⑥ and the prefill/decode
// table of "DeepSeek V3.2 稀疏注意力 DSA 推理流程图解": prefill gathers the history
// K, then scores every history token for every query token).
//
// The contraction [T*64, 128] x [128, S] runs on the matrix cores with the FP8 codes
// decoded exactly to f16 (common.h); the head-weighted sum is the epilogue.
//
// A workgroup owns 8 query rows, one per wavefront (its q decoded once into VGPRs),
// and a chunk of 1024 keys streamed through LDS in double-buffered tiles of 64 keys.
// Each tile is loaded as 4-byte words (consecutive lanes take consecutive words, so
// the decoded 8-byte LDS writes of a wavefront are contiguous and conflict-free),
// decoded to f16 once, and read by all 8 rows.  Per tile a wavefront runs one batch:
// its row against the tile's 4 groups of 16 keys (64 MFMAs in 16 independent chains),
// then one 4x4 transpose-reduce and one coalesced 256-byte store.  Tiles wholly
// outside the rows' [ks, ke) ranges are never loaded, so causal work above the
// diagonal is skipped.  Workgroups are renumbered so that the chunks of one row tile
// run on the same XCD (their q stays in that XCD's L2); K (132 B per key) is re-read
// from L2 by each row tile.
#include "common.h"

namespace dsi {
namespace {

constexpr int kPfThreads = 512;
constexpr int kPfRows = kPfThreads / 64;  // one query row per wavefront
constexpr int kTileKeys = 64;             // keys per LDS tile
constexpr int kChunkTiles = 16;           // tiles per workgroup
constexpr int kChunkKeys = kTileKeys * kChunkTiles;
constexpr int kTileWords = kTileKeys * kRow / 4;  // 2112 dwords per full tile
constexpr int kWordsPerThread = (kTileWords + kPfThreads - 1) / kPfThreads;
constexpr int kTileLdsBytes = kTileKeys * kLdsKeyStrideF16 + kTileKeys * 4;  // f16 rows, then the fp32 scales
constexpr int kScaleOffset = kTileKeys * kLdsKeyStrideF16;
constexpr int kOutRow[4] = {0, 0, 0, 0};
constexpr int kOutKg[4] = {0, 1, 2, 3};

__global__ __launch_bounds__(kPfThreads) void prefill_logits_kernel(
    const uint8_t* __restrict__ q, const uint16_t* __restrict__ w, int T, const uint8_t* __restrict__ k_rows, int S,
    const int* __restrict__ row_ks, const int* __restrict__ row_ke, float* __restrict__ logits, int64_t ld,
    int n_chunks) {
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[2][kTileLdsBytes];

  const int nwg = gridDim.x;
  int id = blockIdx.x;
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);  // chunks of a row tile on one XCD
  const int rt = id / n_chunks, chunk = id - rt * n_chunks;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t_first = rt * kPfRows;

  // Union of the workgroup's row ranges, clipped to this chunk.
  int lo = 0x7FFFFFFF, hi = 0;
#pragma unroll
  for (int i = 0; i < kPfRows; i++) {
    const int t = t_first + i;
    if (t < T) {
      const int a = max(row_ks[t], 0), b = min(row_ke[t], S);
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

  // This thread's staging words: the same positions in every tile.
  int lds_off[kWordsPerThread];
  bool is_code[kWordsPerThread];
#pragma unroll
  for (int j = 0; j < kWordsPerThread; j++) {
    const int d = tid + j * kPfThreads;
    const int row = d / 33, word = d - row * 33;
    is_code[j] = word < 32;
    lds_off[j] = word < 32 ? row * kLdsKeyStrideF16 + word * 8 : kScaleOffset + row * 4;
  }

  // This wavefront's row.
  const int t = t_first + wave;
  const int tc = min(t, T - 1);
  QFrag qf[1];
  WFrag wf[1];
  load_q(qf[0], q + (int64_t)tc * kHeads * kDim, lane);
  load_w(wf[0], w + (int64_t)tc * kHeads, lane);
  const int rks = t < T ? max(row_ks[t], 0) : 0;
  const int rke = t < T ? min(row_ke[t], S) : 0;

  uint32_t regs[kWordsPerThread];
  auto load_tile = [&](int tile) {
    const int nwords = min(kTileKeys, S - tile * kTileKeys) * (kRow / 4);
    const uint32_t* src = reinterpret_cast<const uint32_t*>(k_rows + (int64_t)tile * kTileKeys * kRow);
#pragma unroll
    for (int j = 0; j < kWordsPerThread; j++) {
      const int d = tid + j * kPfThreads;
      if (d < nwords) regs[j] = src[d];
    }
  };
  auto store_tile = [&](int tile, uint8_t* dst) {
    const int nwords = min(kTileKeys, S - tile * kTileKeys) * (kRow / 4);
#pragma unroll
    for (int j = 0; j < kWordsPerThread; j++) {
      const int d = tid + j * kPfThreads;
      if (d < nwords) {
        if (is_code[j])
          *reinterpret_cast<uint2*>(dst + lds_off[j]) = e4m3x4_to_f16x4(regs[j]);
        else
          *reinterpret_cast<uint32_t*>(dst + lds_off[j]) = regs[j];
      }
    }
  };

  load_tile(tile_first);
  store_tile(tile_first, s_tile[0]);
  __syncthreads();

  const int n = lane & 15, g = lane >> 4;
  for (int tile = tile_first; tile < tile_end; tile++) {
    const int buf = (tile - tile_first) & 1;
    const bool has_next = tile + 1 < tile_end;
    if (has_next) load_tile(tile + 1);

    const uint8_t* cur = s_tile[buf];
    KFrag kb[4];
#pragma unroll
    for (int kg = 0; kg < 4; kg++) load_kfrag_f16(kb[kg], cur + kg * 16 * kLdsKeyStrideF16, lane);
    float part[4];
    score4(qf, wf, kb, kOutRow, kOutKg, part);
    const float v = transpose_reduce4(part, lane);
    // lane group g owns key group g: keys g*16 + n of the tile
    const int kslot = g * 16 + n;
    const int key = tile * kTileKeys + kslot;
    if (key >= rks && key < rke)
      logits[(int64_t)t * ld + key] = v * reinterpret_cast<const float*>(cur + kScaleOffset)[kslot];

    if (has_next) store_tile(tile + 1, s_tile[buf ^ 1]);
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
  hipLaunchKernelGGL(prefill_logits_kernel, dim3((unsigned)grid), dim3(kPfThreads), 0, stream, q, w, T, k_rows, S,
                     row_ks, row_ke, logits, ld, n_chunks);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}
