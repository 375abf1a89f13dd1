// Dense prefill indexer logits over gathered K (P3 step ⑥ and the prefill/decode table of
// "DeepSeek V3.2 稀疏注意力 DSA 推理流程图解": prefill gathers the history K, then scores
// every history token for every query token).
//
// The contraction [T*64, 128] x [128, S] runs on the matrix cores with the FP8 codes
// decoded exactly to f16 (common.h); the head-weighted sum is the epilogue.
//
// Matrix instruction: v_mfma_f32_16x16x32_f16.  On random FP8 operands the chip is at its
// power limit, and this form draws less energy per flop than the 32x32x16 one: its clock
// stays higher by more than it loses in issue rate.
//   A = 16 heads x 32 dims of q   (lane l: head l%16, 8 dims of lane group g = l/16)
//   B = 32 dims x 16 keys of K    (lane l: key  l%16, the same 8 dims)
//   C = 16 heads x 16 keys, lane l holds heads 4g + i (i < 4) of key l%16.
// Lane group g owns dims [32g, 32g+32) of the 128 and feeds 8 of them to each of four
// slices; A and B use the same assignment, so the sum over dims is complete.  Four head
// blocks cover the 64 heads and a 32-key group is two 16-key blocks: after its 32 MFMAs each
// lane holds 16 heads of each of two keys, and the head-weighted sums are 32 FMAs.  The other
// three lane groups hold the other 48 heads of the same keys: for a 64-key half tile, two
// v_permlane32_swap and one v_permlane16_swap exchange the four groups' partial sums of the
// half's two 32-key groups, and three adds leave each lane with one key of the half.
//
// A workgroup of 8 wavefronts (one per CU) owns 8 query rows, one per wavefront, its q
// decoded once into VGPRs, and a share of the keys streamed through LDS in double-buffered
// 128-key tiles: each tile is staged once (each wavefront loads an eighth of every row's
// codes), decoded to f16 once and read by all 8 rows.  Tiles wholly outside the rows'
// [ks, ke) ranges are never loaded, so causal work above the diagonal is skipped; the tiles
// a row tile does need are split evenly between its workgroups.  K (132 B per key) is
// re-read from L2 by each row tile.
#include "common.h"

namespace dsi {
namespace {

constexpr int kPfThreads = 512;
constexpr int kPfRows = kPfThreads / 64;  // one query row per wavefront
constexpr int kGroups = 4;                // 32-key groups per tile
constexpr int kTileKeys = 32 * kGroups;   // keys per LDS tile
constexpr int kChunkTiles = 32;           // tiles per workgroup at most (S sets the split count)
constexpr int kChunkKeys = kTileKeys * kChunkTiles;
constexpr int kScaleOffset = kTileKeys * kLdsKeyStrideF16;  // f16 rows, then the fp32 scales
constexpr int kTileLdsBytes = kScaleOffset + kTileKeys * 4;
constexpr int kRowsPerLane = kTileKeys / 64;  // staging: lane r of wave p takes rows r + 64j,
constexpr int kStageDims = kDim / kPfRows;     // dims [kStageDims*p, kStageDims*(p+1))
static_assert(kStageDims % 16 == 0, "staging moves whole 16-byte pieces");

// This lane's A fragments of one query row: head block hb (heads 16hb + l%16), slice s
// (dims 32g + 8s + [0, 8)), decoded from the codes as loaded.
struct Q16 {
  f16x8 a[4][4];
};

__device__ __forceinline__ void load_q16_codes(uint4 (&x)[4][2], const uint8_t* q_row, int lane) {
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int hb = 0; hb < 4; hb++) {
    const uint4* p = reinterpret_cast<const uint4*>(q_row + (hb * 16 + n) * kDim + g * 32);
    x[hb][0] = p[0];
    x[hb][1] = p[1];
  }
}

__device__ __forceinline__ void decode_q16(Q16& f, const uint4 (&x)[4][2]) {
#pragma unroll
  for (int hb = 0; hb < 4; hb++)
#pragma unroll
    for (int j = 0; j < 2; j++) {
      f.a[hb][2 * j] = e4m3x8_to_f16x8(x[hb][j].x, x[hb][j].y);
      f.a[hb][2 * j + 1] = e4m3x8_to_f16x8(x[hb][j].z, x[hb][j].w);
    }
}

// The weights of the 16 heads this lane holds in C: w[hb][i] is head 16hb + 4g + i.
struct W16 {
  float w[4][4];
};

__device__ __forceinline__ void load_w16_raw(uint2 (&x)[4], const uint16_t* w_row, int lane) {
  const int g = lane >> 4;
#pragma unroll
  for (int hb = 0; hb < 4; hb++) x[hb] = *reinterpret_cast<const uint2*>(w_row + hb * 16 + g * 4);
}

__device__ __forceinline__ void decode_w16(W16& f, const uint2 (&x)[4]) {
#pragma unroll
  for (int hb = 0; hb < 4; hb++) {
    f.w[hb][0] = bf16_to_f32(x[hb].x & 0xFFFFu);
    f.w[hb][1] = bf16_to_f32(x[hb].x >> 16);
    f.w[hb][2] = bf16_to_f32(x[hb].y & 0xFFFFu);
    f.w[hb][3] = bf16_to_f32(x[hb].y >> 16);
  }
}

// B fragments of one 32-key group from the f16 tile: key block kb (keys 16kb + l%16), slice s
// (dims 32g + 8s + [0, 8)).
struct K16 {
  f16x8 b[2][4];
};

constexpr int kF16PerRow = kLdsKeyStrideF16 / 16;  // f16x8 units per LDS key row

__device__ __forceinline__ const f16x8* k16_base(const uint8_t* keys, int lane) {
  return reinterpret_cast<const f16x8*>(keys + (lane & 15) * kLdsKeyStrideF16 + (lane >> 4) * 64);
}

// All eight fragments of one group (after a barrier, when nothing else can run).
__device__ __forceinline__ void load_k16(K16& f, const uint8_t* keys, int lane) {
  const f16x8* p = k16_base(keys, lane);
#pragma unroll
  for (int kb = 0; kb < 2; kb++)
#pragma unroll
    for (int s = 0; s < 4; s++) f.b[kb][s] = p[kb * 16 * kF16PerRow + s];
}

// Accumulators of one group: head block hb x key block kb.
struct Acc16 {
  f32x4 x[4][2];
};

// One 32-key group on the matrix cores, with the previous group's head sums and other work
// threaded between its 32 MFMAs in a fixed order (sched_barrier fences keep the compiler from
// regrouping them).  Step i issues MFMA i (slice i/8, key block (i/4)%2, head block i%4) into
// x, then FMA i of the head sums of y (the previous group's accumulators: key block i/16, head
// block (i/4)%4, head 4g + i%4), then, after the last MFMA of a slice and key block has read
// it, that fragment of the next group (when kLoadNext), and on even steps extra(i/2).  acc[0]
// + acc[1] is key block 0's sum, acc[2] + acc[3] key block 1's.
template <bool kLoadNext, typename Extra>
__device__ __forceinline__ void group_phase(Acc16& x, const Q16& q, K16& kb, const uint8_t* next, int lane,
                                            const W16& w, const Acc16& y, float (&acc)[4], Extra&& extra) {
  const f16x8* np = k16_base(next, lane);
#pragma unroll
  for (int j = 0; j < 4; j++) acc[j] = 0.f;
#pragma unroll
  for (int i = 0; i < 32; i++) {
    const int s = i >> 3, kk = (i >> 2) & 1, hb = i & 3;
    x.x[hb][kk] = mfma_f16(q.a[hb][s], kb.b[kk][s], s == 0 ? f32x4{} : x.x[hb][kk]);
    __builtin_amdgcn_sched_barrier(0);
    {
      const int k2 = i >> 4, h2 = (i >> 2) & 3, e = i & 3;
      acc[2 * k2 + (i & 1)] = fmaf(w.w[h2][e], y.x[h2][k2][e], acc[2 * k2 + (i & 1)]);
    }
    if (kLoadNext && hb == 3) kb.b[kk][s] = np[kk * 16 * kF16PerRow + s];
    if ((i & 1) == 0) extra(i >> 1);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The full sums of a 64-key half tile from its two groups' partial sums (gXkY: group X, key
// block Y; each over the 16 heads of this lane's group).  The first swap pairs lane groups
// {0, 2} and {1, 3} of each group; the second pairs the two results.  Lane l ends with key
// half_key(l) of the half.
__device__ __forceinline__ float combine_groups(float g0k0, float g0k1, float g1k0, float g1k1) {
  const auto u = __builtin_amdgcn_permlane32_swap(__float_as_uint(g0k0), __float_as_uint(g0k1), false, false);
  const auto v = __builtin_amdgcn_permlane32_swap(__float_as_uint(g1k0), __float_as_uint(g1k1), false, false);
  const float y0 = __uint_as_float(u[0]) + __uint_as_float(u[1]);
  const float y1 = __uint_as_float(v[0]) + __uint_as_float(v[1]);
  const auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(y0), __float_as_uint(y1), false, false);
  return __uint_as_float(z[0]) + __uint_as_float(z[1]);
}

// 16-lane row 0: group 0 keys 0..15; row 1: group 1 keys 0..15 (32..47 of the half); row 2:
// group 0 keys 16..31; row 3: group 1 keys 16..31.
__device__ __forceinline__ int half_key(int lane) { return (lane & 15) + 16 * ((lane >> 5) & 1) + 32 * ((lane >> 4) & 1); }

__global__ __launch_bounds__(kPfThreads, 1) void prefill_logits_kernel(
    const uint8_t* __restrict__ q, const uint16_t* __restrict__ w, int T, const uint8_t* __restrict__ k_rows, int S,
    const int* __restrict__ row_ks, const int* __restrict__ row_ke, float* __restrict__ logits, int64_t ld,
    int n_parts) {
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[2][kTileLdsBytes];

  // Workgroup -> (part, row tile): parts outermost and row tiles in descending order, so the
  // larger causal row tiles are dispatched first, and the parts of one row tile (which share
  // its q) land on the same XCD whenever the row-tile count is a multiple of the 8 XCDs.
  const int row_tiles = (T + kPfRows - 1) / kPfRows;
  const int part = blockIdx.x / row_tiles;
  const int rt = row_tiles - 1 - (int)(blockIdx.x - part * row_tiles);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront: row values live in SGPRs
  const int t_first = rt * kPfRows;

  // Union of the workgroup's row ranges; this workgroup takes an equal share (part `part` of
  // n_parts) of the tiles that cover it.  The range loads have uniform addresses and no
  // branches between them, so they are issued together as scalar loads: two 8-word loads when
  // all eight rows exist, else one load per row (rows past T repeat row T-1 and are ignored).
  const int t = t_first + wave;  // this wavefront's row
  int lo = 0x7FFFFFFF, hi = 0, rks = 0, rke = 0;
  {
    int a[kPfRows], b[kPfRows];
    if (t_first + kPfRows <= T) {
#pragma unroll
      for (int i = 0; i < kPfRows; i++) {
        a[i] = row_ks[t_first + i];
        b[i] = row_ke[t_first + i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < kPfRows; i++) {
        const int ti = min(t_first + i, T - 1);
        a[i] = row_ks[ti];
        b[i] = row_ke[ti];
      }
    }
#pragma unroll
    for (int i = 0; i < kPfRows; i++) {
      const int x = max(a[i], 0), y = min(b[i], S);
      const bool real = t_first + i < T;
      const bool use = real && x < y;
      lo = use ? min(lo, x) : lo;
      hi = use ? max(hi, y) : hi;
      rks = i == wave ? (real ? x : 0) : rks;
      rke = i == wave ? (real ? y : 0) : rke;
    }
  }
  if (lo >= hi) return;  // uniform across the workgroup
  const int t0 = lo / kTileKeys, nt = (hi + kTileKeys - 1) / kTileKeys - t0;
  const int tile_first = t0 + part * nt / n_parts, tile_end = t0 + (part + 1) * nt / n_parts;
  if (tile_first >= tile_end) return;

  // The row's q codes and weights are requested here and decoded only after the first tile's
  // loads are issued (below), so the two round trips to memory overlap.
  const int tc = min(t, T - 1);
  uint4 q_codes[4][2];
  uint2 w_raw[4];
  load_q16_codes(q_codes, q + (int64_t)tc * kHeads * kDim, lane);
  load_w16_raw(w_raw, w + (int64_t)tc * kHeads, lane);

  // Output: a raw buffer over this row's logits whose record size ends at the row's range
  // end; a lane whose key is below the range start (or below this workgroup's first tile)
  // gets an offset past the end, so the hardware drops its store and the pipelined loop
  // below has no branches.
  const int key_lo = max(rks, tile_first * kTileKeys);
  const __amdgpu_buffer_rsrc_t out_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(logits + (int64_t)tc * ld, (short)0, rke * 4, 0x00020000);
  auto store_logit = [&](int key, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), out_rsrc, key >= key_lo ? key * 4 : 0x7FFFFFFC, 0, 0);
  };

  // Staging: lane r of wavefront p loads the codes [16p, 16p+16) of rows r + 64j of the tile
  // (one 16-byte load per row), decodes them and writes 32 bytes of f16; the row's scale is
  // copied by every wavefront of the same parity (same value).  Writes by consecutive lanes
  // go to consecutive rows, 272 bytes apart, so they are conflict-free.  Rows past the end of
  // a partial tile repeat its last row; their keys are never stored.
  constexpr int kLoads = kStageDims / 16;  // 16-byte loads per row
  constexpr int kVecs = kStageDims / 8;    // f16x8 writes per row
  uint4 regs[kRowsPerLane][kLoads];
  uint32_t sreg;
  auto load_piece = [&](int tile, int i) {  // i < kRowsPerLane*kLoads: one 16-byte load; then the scale
    const int last = min(kTileKeys, S - tile * kTileKeys) - 1;
    const uint8_t* src = k_rows + (int64_t)tile * kTileKeys * kRow;
    if (i < kRowsPerLane * kLoads) {
      const int j = i / kLoads, c = i % kLoads;
      const uint32_t off = __umul24((uint32_t)min(lane + 64 * j, last), (uint32_t)kRow) + wave * kStageDims + 16 * c;
      regs[j][c] = *reinterpret_cast<const uint4*>(src + off);
    } else if (i == kRowsPerLane * kLoads) {
      sreg = *reinterpret_cast<const uint32_t*>(src + __umul24((uint32_t)min(lane + 64 * (wave & 1), last), (uint32_t)kRow) + kDim);
    }
  };
  auto store_piece = [&](uint8_t* dst, int i) {  // i < kRowsPerLane*kVecs: one f16x8 (4 conversions); then the scale
    if (i < kRowsPerLane * kVecs) {
      const int j = i / kVecs, c = i % kVecs;
      const uint4& x = regs[j][c >> 1];
      const uint32_t lo = (c & 1) ? x.z : x.x, hi = (c & 1) ? x.w : x.y;
      reinterpret_cast<f16x8*>(dst + (lane + 64 * j) * kLdsKeyStrideF16 + wave * (2 * kStageDims))[c] =
          e4m3x8_to_f16x8(lo, hi);
    } else if (i == kRowsPerLane * kVecs) {
      reinterpret_cast<uint32_t*>(dst + kScaleOffset)[lane + 64 * (wave & 1)] = sreg;
    }
  };

#pragma unroll
  for (int i = 0; i <= kRowsPerLane * kLoads; i++) load_piece(tile_first, i);
  __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the first decode waits
  Q16 qf;
  W16 wf;
  decode_q16(qf, q_codes);
  decode_w16(wf, w_raw);
#pragma unroll
  for (int i = 0; i <= kRowsPerLane * kVecs; i++) store_piece(s_tile[0], i);
  __syncthreads();

  // Software pipeline over 32-key groups.  While the matrix cores run group g, the wavefront
  // computes the head sums of group g-1, loads the B fragments of group g+1 slice by slice
  // and does its share of staging the next tile (global loads during the first group,
  // decode and LDS writes during the third).  The tile's one barrier sits before its last
  // group, whose fragments are already in registers, so the next tile's first fragments
  // load under that group's MFMAs.  The head sums of a tile's last group are taken during
  // the next tile's first group, so the matrix work never waits for an epilogue.
  Acc16 xa = {}, xb = {};
  float acc[4];
  float pe0 = 0.f, pe1 = 0.f;  // head sums of group 0 or 2 (key blocks 0 and 1), waiting for their partner
  const int hk = half_key(lane);
  float scale_lo = 0.f;  // scale of key hk of the current tile
  float scale_hi = 0.f;  // scale of key 64 + hk of the previous tile
  K16 kb;
  load_k16(kb, s_tile[0], lane);
  for (int tile = tile_first; tile < tile_end; tile++) {
    const int buf = (tile - tile_first) & 1;
    const uint8_t* cur = s_tile[buf];
    uint8_t* nxt = s_tile[buf ^ 1];
    const float* scale = reinterpret_cast<const float*>(cur + kScaleOffset);
    const int next_tile = min(tile + 1, tile_end - 1);

    // group 0 -> xa; head sums of the previous tile's group 3; global loads of the next tile
    group_phase<true>(xa, qf, kb, cur + 32 * kLdsKeyStrideF16, lane, wf, xb, acc, [&](int i) {
      if (i >= 2 && i <= 2 + kRowsPerLane * kLoads) load_piece(next_tile, i - 2);
      if (i == 12) scale_lo = scale[hk];
    });
    store_logit((tile - 1) * kTileKeys + 64 + hk, combine_groups(pe0, pe1, acc[0] + acc[1], acc[2] + acc[3]) * scale_hi);

    // group 1 -> xb; head sums of group 0
    group_phase<true>(xb, qf, kb, cur + 64 * kLdsKeyStrideF16, lane, wf, xa, acc, [&](int) {});
    pe0 = acc[0] + acc[1];
    pe1 = acc[2] + acc[3];

    // group 2 -> xa; head sums of group 1; decode the next tile into the other buffer
    group_phase<true>(xa, qf, kb, cur + 96 * kLdsKeyStrideF16, lane, wf, xb, acc, [&](int i) {
      if (i >= 2 && i <= 2 + kRowsPerLane * kVecs) store_piece(nxt, i - 2);
      if (i == 12) scale_hi = scale[64 + hk];
    });
    const float v_lo = combine_groups(pe0, pe1, acc[0] + acc[1], acc[2] + acc[3]) * scale_lo;
    // Every wavefront is done with this tile's buffer (group 3's fragments and both scale
    // halves are in registers) and has written its part of the next tile.
    __syncthreads();

    // group 3 -> xb; head sums of group 2; fragments of the next tile's group 0
    store_logit(tile * kTileKeys + hk, v_lo);
    group_phase<true>(xb, qf, kb, nxt, lane, wf, xa, acc, [&](int) {});
    pe0 = acc[0] + acc[1];
    pe1 = acc[2] + acc[3];
  }
  // head sums of the last tile's group 3
#pragma unroll
  for (int j = 0; j < 4; j++) acc[j] = 0.f;
#pragma unroll
  for (int kk = 0; kk < 2; kk++)
#pragma unroll
    for (int hb = 0; hb < 4; hb++)
#pragma unroll
      for (int e = 0; e < 4; e++) acc[2 * kk + (e & 1)] = fmaf(wf.w[hb][e], xb.x[hb][kk][e], acc[2 * kk + (e & 1)]);
  store_logit((tile_end - 1) * kTileKeys + 64 + hk, combine_groups(pe0, pe1, acc[0] + acc[1], acc[2] + acc[3]) * scale_hi);
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
  const int n_parts = (S + kChunkKeys - 1) / kChunkKeys;  // each row tile's key range is split n_parts ways
  const int64_t grid = (int64_t)row_tiles * n_parts;
  if (grid > 0x7FFFFFFF) return DSI_EUNSUPPORTED;
  hipLaunchKernelGGL(prefill_logits_kernel, dim3((unsigned)grid), dim3(kPfThreads), 0, stream, q, w, T, k_rows, S,
                     row_ks, row_ke, logits, ld, n_parts);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}
