// Per-row top-k selection into the index table main attention reads (P3 data flow 2
// of "DeepSeek V3.2 稀疏注意力 DSA 推理流程图解": the k best positions per query row
// as int32, -1 for an empty slot; P3 pitfalls: request-relative positions; P1 "V4.1
// 索引器接入稀疏 MQA logits": the compressed-space top-k runs on bf16 logits).
//
// Radix select, no sort.  Values map to order-preserving unsigned keys (non-finite
// values are dropped).  One workgroup per row — 1024 threads for rows longer than
// 16K columns, else 256 threads with a smaller LDS footprint so that several rows
// share a CU — and the row is read twice, with 16-byte loads, four per thread in
// flight:
//   pass 1 builds an LDS histogram of the top 11 key bits and finds the bin b1 where
//          the count from the top reaches k;
//   pass 2 writes every column whose bin is above b1 and collects the columns of bin
//          b1 (key, column) into LDS;
// the remaining key bits (21 for fp32, 5 for bf16) are then resolved on those
// candidates in LDS, digit by digit, and the selected candidates written.  Output
// slots are reserved per wavefront (ballot + popcount, one LDS atomic).  A row whose
// boundary bin holds more candidates than LDS can keep (heavy ties) resolves the
// remaining digits with passes over the row instead.
#include "common.h"

namespace dsi {
namespace {

constexpr int kHistBins = 2048;
constexpr int kUnroll = 4;  // 16-byte loads in flight per thread
constexpr int kShortRow = 16384;  // rows up to this width use the small configuration

// Workgroup size and the number of boundary-bin candidates kept in LDS.
template <int THREADS, int CAP>
struct Cfg {
  static constexpr int kThreads = THREADS;
  static constexpr int kWaves = THREADS / 64;
  static constexpr int kCap = CAP;
  static constexpr int kBinsPerThread = kHistBins / THREADS;
};
using LongRows = Cfg<1024, 12288>;  // 96 KB of candidates
using ShortRows = Cfg<256, 2048>;   // 16 KB of candidates

template <bool BF16>
struct Keys {
  static constexpr int kBits = BF16 ? 16 : 32;
  static constexpr int kElemBytes = BF16 ? 2 : 4;
  static constexpr int kPerVec = 16 / kElemBytes;
  static constexpr int kTopShift = kBits - 11;  // first digit: the top 11 bits
  static __device__ __forceinline__ bool key(uint32_t raw, uint32_t& k) {
    if (BF16) {
      k = bf16_key(raw);
      return (raw & 0x7F80u) != 0x7F80u;
    } else {
      k = f32_key(raw);
      return (raw & 0x7F800000u) != 0x7F800000u;
    }
  }
  static __device__ __forceinline__ uint32_t elem(const uint4& v, int i) {
    const uint32_t w = i / (4 / kElemBytes) == 0 ? v.x : i / (4 / kElemBytes) == 1 ? v.y
                       : i / (4 / kElemBytes) == 2 ? v.z : v.w;
    return BF16 ? ((i & 1) ? (w >> 16) : (w & 0xFFFFu)) : w;
  }
  static __device__ __forceinline__ uint32_t load1(const uint8_t* row, int c) {
    return BF16 ? (uint32_t) reinterpret_cast<const uint16_t*>(row)[c] : reinterpret_cast<const uint32_t*>(row)[c];
  }
};

// Visit every column of [st, en) once: f(active, column, raw bits).  Every lane of
// the workgroup calls f the same number of times (active = false for padding), so
// f may use wavefront ballots.  Columns between 16-byte boundaries use 16-byte loads,
// kUnroll per thread at a time; the unaligned head and tail use element loads.
template <bool BF16, int THREADS, typename F>
__device__ __forceinline__ void scan_row(const uint8_t* row, int st, int en, int tid, F&& f) {
  using K = Keys<BF16>;
  constexpr int E = K::kPerVec;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row) + (uintptr_t)st * K::kElemBytes;
  int c0 = st + (int)(((16 - (addr & 15)) & 15) / K::kElemBytes);
  if (c0 > en) c0 = en;
  const int nvec = (en - c0) / E;
  const int c1 = c0 + nvec * E;
  // head and tail (fewer than E columns each)
  {
    const int nh = c0 - st, nt = en - c1;
    const bool ah = tid < nh, at = tid < nt;
    const int ch = st + tid, ct = c1 + tid;
    f(ah, ch, ah ? K::load1(row, ch) : 0u);
    f(at, ct, at ? K::load1(row, ct) : 0u);
  }
  const uint4* vec = reinterpret_cast<const uint4*>(row + (size_t)c0 * K::kElemBytes);
  for (int base = 0; base < nvec; base += THREADS * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      const int vi = base + u * THREADS + tid;
      if (vi < nvec) v[u] = vec[vi];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      const int vi = base + u * THREADS + tid;
      const bool a = vi < nvec;
#pragma unroll
      for (int e = 0; e < E; e++) f(a, c0 + vi * E + e, a ? K::elem(v[u], e) : 0u);
    }
  }
}

// Reserve consecutive slots for the lanes whose pred is set; returns this lane's slot.
__device__ __forceinline__ int wave_reserve(bool pred, int* counter, int lane) {
  const uint64_t m = __ballot(pred);
  int base = 0;
  if (lane == 0 && m) base = atomicAdd(counter, __popcll(m));
  base = __shfl(base, 0);
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  return base + __popcll(m & below);
}

// Exclusive suffix sum over threads (thread i gets the sum of `x` of all threads > i).
template <int WAVES>
__device__ __forceinline__ int block_suffix_excl(int x, int* s_wave, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  int v = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_down(v, off);
    if (lane + off < 64) v += y;
  }
  if (lane == 0) s_wave[wave] = v;
  __syncthreads();
  int above = 0;
  for (int j = wave + 1; j < WAVES; j++) above += s_wave[j];
  __syncthreads();
  return v - x + above;
}

// Given an LDS histogram of nb bins (already filled), find the bin where the count
// from the top reaches `need`.  Writes the bin and the count strictly above it to
// s_sel[0..1]; s_sel[2] = total count.  Each thread owns kBinsPerThread consecutive
// bins.  Call with all threads; ends synchronised.
template <typename C>
__device__ __forceinline__ void select_bin(const int* hist, int nb, int need, int* s_wave, int* s_sel, int tid) {
  constexpr int BPT = C::kBinsPerThread;
  int h[BPT], local = 0;
#pragma unroll
  for (int j = 0; j < BPT; j++) {
    const int bin = tid * BPT + j;
    h[j] = bin < nb ? hist[bin] : 0;
    local += h[j];
  }
  const int above = block_suffix_excl<C::kWaves>(local, s_wave, tid);
  if (tid == 0) s_sel[2] = above + local;
  if (above < need && need <= above + local) {
    int acc = above;
#pragma unroll
    for (int j = BPT - 1; j >= 0; j--) {
      if (acc + h[j] >= need) {
        s_sel[0] = tid * BPT + j;
        s_sel[1] = acc;
        break;
      }
      acc += h[j];
    }
  }
  __syncthreads();
}

template <bool BF16, typename C>
__global__ __launch_bounds__(C::kThreads) void topk_kernel(const uint8_t* __restrict__ logits, int64_t row_bytes,
                                                          const int* __restrict__ row_starts,
                                                          const int* __restrict__ row_ends, int max_width, int k,
                                                          int* __restrict__ out, int64_t out_ld) {
  using K = Keys<BF16>;
  __shared__ int s_hist[kHistBins];
  constexpr int kTkThreads = C::kThreads, kCandCap = C::kCap;
  __shared__ uint32_t s_ckey[kCandCap];
  __shared__ int s_ccol[kCandCap];
  __shared__ int s_wave[C::kWaves];
  __shared__ int s_sel[4];
  __shared__ int s_cnt[4];  // 0: written above the boundary, 1: candidates, 2: written from candidates

  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int st = row_starts ? max(row_starts[r], 0) : 0;
  const int en = max(min(row_ends[r], max_width), st);
  const uint8_t* row = logits + (int64_t)r * row_bytes;
  int* orow = out + (int64_t)r * out_ld;

  for (int i = tid; i < kHistBins; i += kTkThreads) s_hist[i] = 0;
  if (tid < 4) s_cnt[tid] = 0;
  __syncthreads();

  // pass 1: histogram of the top 11 key bits
  scan_row<BF16, kTkThreads>(row, st, en, tid, [&](bool a, int, uint32_t raw) {
    uint32_t key;
    if (a && K::key(raw, key)) atomicAdd(&s_hist[key >> K::kTopShift], 1);
  });
  __syncthreads();
  select_bin<C>(s_hist, kHistBins, k, s_wave, s_sel, tid);
  const int total = s_sel[2];

  if (total <= k) {  // every valid value is selected
    scan_row<BF16, kTkThreads>(row, st, en, tid, [&](bool a, int c, uint32_t raw) {
      uint32_t key;
      const bool take = a && K::key(raw, key);
      const int pos = wave_reserve(take, &s_cnt[0], lane);
      if (take && pos < k) orow[pos] = c - st;
    });
    for (int j = total + tid; j < k; j += kTkThreads) orow[j] = -1;
    return;
  }

  const uint32_t b1 = (uint32_t)s_sel[0];
  const int above1 = s_sel[1];
  // pass 2: columns above the boundary bin are selected; the boundary bin's are candidates
  scan_row<BF16, kTkThreads>(row, st, en, tid, [&](bool a, int c, uint32_t raw) {
    uint32_t key = 0;
    const bool valid = a && K::key(raw, key);
    const uint32_t d = key >> K::kTopShift;
    const bool gt = valid && d > b1, eq = valid && d == b1;
    const int pos = wave_reserve(gt, &s_cnt[0], lane);
    if (gt && pos < k) orow[pos] = c - st;
    const int slot = wave_reserve(eq, &s_cnt[1], lane);
    if (eq && slot < kCandCap) {
      s_ckey[slot] = key;
      s_ccol[slot] = c;
    }
  });
  __syncthreads();
  const int m = s_cnt[1];
  int need = k - above1;

  // remaining digits below the top 11 bits: fp32 (11, 10), bf16 (5)
  constexpr int kLow = K::kTopShift;
  const int nd = BF16 ? 1 : 2;
  const int shifts[2] = {BF16 ? 0 : 10, 0};
  const int widths[2] = {BF16 ? 5 : 11, 10};
  uint32_t prefix = b1 << kLow;  // known high bits of the threshold key
  const bool in_lds = m <= kCandCap;
  for (int p = 0; p < nd; p++) {
    const int sh = shifts[p], wd = widths[p], nb = 1 << wd;
    const int hs = sh + wd;  // bits at and above hs are fixed by `prefix`
    for (int i = tid; i < nb; i += kTkThreads) s_hist[i] = 0;
    __syncthreads();
    if (in_lds) {
      for (int i = tid; i < m; i += kTkThreads) {
        const uint32_t key = s_ckey[i];
        if ((key >> hs) == (prefix >> hs)) atomicAdd(&s_hist[(key >> sh) & (nb - 1)], 1);
      }
    } else {
      scan_row<BF16, kTkThreads>(row, st, en, tid, [&](bool a, int, uint32_t raw) {
        uint32_t key;
        if (a && K::key(raw, key) && (key >> hs) == (prefix >> hs)) atomicAdd(&s_hist[(key >> sh) & (nb - 1)], 1);
      });
    }
    __syncthreads();
    select_bin<C>(s_hist, nb, need, s_wave, s_sel, tid);
    prefix |= (uint32_t)s_sel[0] << sh;
    need -= s_sel[1];
    __syncthreads();
  }
  // tau = prefix: select the boundary-bin keys above tau, and `need` of those equal to it
  const int base = above1;  // slots [0, above1) hold the columns above the boundary bin
  const int n_above_tau = (k - base) - need;
  if (in_lds) {
    for (int i0 = 0; i0 < m; i0 += kTkThreads) {
      const int i = i0 + tid;
      const bool a = i < m;
      const uint32_t key = a ? s_ckey[i] : 0u;
      const bool gt = a && key > prefix, eq = a && key == prefix;
      const int pg = wave_reserve(gt, &s_cnt[2], lane);
      if (gt && base + pg < k) orow[base + pg] = s_ccol[i] - st;
      const int pe = wave_reserve(eq, &s_cnt[3], lane);
      if (eq && pe < need && base + n_above_tau + pe < k) orow[base + n_above_tau + pe] = s_ccol[i] - st;
    }
  } else {
    scan_row<BF16, kTkThreads>(row, st, en, tid, [&](bool a, int c, uint32_t raw) {
      uint32_t key = 0;
      const bool valid = a && K::key(raw, key) && (key >> kLow) == b1;
      const bool gt = valid && key > prefix, eq = valid && key == prefix;
      const int pg = wave_reserve(gt, &s_cnt[2], lane);
      if (gt && base + pg < k) orow[base + pg] = c - st;
      const int pe = wave_reserve(eq, &s_cnt[3], lane);
      if (eq && pe < need && base + n_above_tau + pe < k) orow[base + n_above_tau + pe] = c - st;
    });
  }
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
  const uint8_t* src = reinterpret_cast<const uint8_t*>(logits);
  const bool small = max_width <= kShortRow;
  if (dtype == DSI_F32) {
    if (small)
      hipLaunchKernelGGL((topk_kernel<false, ShortRows>), dim3((unsigned)rows), dim3(ShortRows::kThreads), 0, stream,
                         src, row_bytes, row_starts, row_ends, max_width, k, out, out_ld);
    else
      hipLaunchKernelGGL((topk_kernel<false, LongRows>), dim3((unsigned)rows), dim3(LongRows::kThreads), 0, stream,
                         src, row_bytes, row_starts, row_ends, max_width, k, out, out_ld);
  } else {
    if (small)
      hipLaunchKernelGGL((topk_kernel<true, ShortRows>), dim3((unsigned)rows), dim3(ShortRows::kThreads), 0, stream,
                         src, row_bytes, row_starts, row_ends, max_width, k, out, out_ld);
    else
      hipLaunchKernelGGL((topk_kernel<true, LongRows>), dim3((unsigned)rows), dim3(LongRows::kThreads), 0, stream,
                         src, row_bytes, row_starts, row_ends, max_width, k, out, out_ld);
  }
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}
