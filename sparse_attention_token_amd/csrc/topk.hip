// Per-row top-k selection into the index table main attention reads (P3 data flow 2
// of "DeepSeek V3.2 稀疏注意力 DSA 推理流程图解": the k best positions per query row
// as int32, -1 for an empty slot; P3 pitfalls: request-relative positions; P1 "V4.1
// 索引器接入稀疏 MQA logits": the compressed-space top-k runs on bf16 logits).
//
// Radix select, no sort.  Values map to order-preserving unsigned keys (non-finite
// values are dropped).  Three shapes, by row width and row count:
//   * rows of at most 16K columns (fp32) or 16K (bf16): one 256-thread workgroup per row
//     reads the row once into registers (topk_reg_kernel below);
//   * longer rows, when there are enough of them to fill the CUs: one 1024-thread
//     workgroup per row reads the row twice — pass 1 builds an LDS histogram of the top
//     11 key bits and finds the bin b1 where the count from the top reaches k; pass 2
//     writes every column whose bin is above b1 and collects the columns of bin b1 (key,
//     column) into LDS; the remaining key bits (21 for fp32, 5 for bf16) are resolved on
//     those candidates, digit by digit (by passes over the row when the boundary bin
//     outgrows LDS).  Output slots are reserved per wavefront (ballot + popcount, one LDS
//     atomic);
//   * few long rows are split between workgroups of 8192 columns, in two launches that
//     communicate through the caller's workspace: per-slice histograms; then every slice
//     sums its row's histograms, finds the boundary bin, writes its columns above it at
//     positions reserved by one atomic per workgroup and appends its boundary-bin columns to
//     a per-row candidate list, and the row's last slice to finish resolves the candidates as
//     above.  The paged decode kernel can count the histograms while it writes the logits,
//     which leaves one launch (topk_split.h).
#include <algorithm>
#include <mutex>

#include "common.h"
#include "topk_split.h"

namespace dsi {
namespace {

constexpr int kHistBins = kSplitBins;
constexpr int kShortRow = 16384;  // rows up to this width are held in registers, one workgroup per row

// Workgroup size and the number of boundary-bin candidates kept in LDS.
// Histograms may keep kCopies lane-interleaved copies of every bin (bin b, copy lane %
// kCopies at b * kCopies + copy); select_bin sums the copies.  One copy where the histogram
// shares LDS with much else (more copies cost occupancy); two in the split path's slice
// step, where lanes alternate between them so that neighbouring lanes with equal bins do not
// collide (measured faster there).
template <int THREADS, int CAP, int COPIES>
struct Cfg {
  static constexpr int kThreads = THREADS;
  static constexpr int kWaves = THREADS / 64;
  static constexpr int kCap = CAP;
  static constexpr int kCopies = COPIES;
  static constexpr int kBinsPerThread = kHistBins / THREADS;
};
using LongRows = Cfg<1024, 12288, 1>;  // 96 KB of candidates

template <int C>
__device__ __forceinline__ void hist_add(int* h, uint32_t bin, int lane) {
  atomicAdd(&h[bin * C + (lane & (C - 1))], 1);
}

template <bool BF16>
struct Keys {
  static constexpr int kUnroll = BF16 ? 2 : 4;  // 16-byte loads in flight per thread: 16 elements
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

// Visit every column of [st, en) once, in batches: f(n, active[], column[], raw[]) with
// n = 2 (the unaligned head and tail, fewer than 16 bytes each, element loads) and then
// n = UNROLL x (values per 16 bytes) per round of 16-byte loads (UNROLL per thread and round; 16 fp32 or bf16 values
// by default).  Every lane of the workgroup makes the same calls (active = false for padding), so f may use
// wavefront ballots.  Constructing the reader issues the head, the tail and the first round's loads, so a kernel can
// put them in flight before other work and visit the row later; the next round's loads are issued before a round is
// visited.
template <bool BF16, int THREADS, int UNROLL = Keys<BF16>::kUnroll>
struct RowReader {
  using K = Keys<BF16>;
  static constexpr int E = K::kPerVec;
  static constexpr int kUnroll = UNROLL;
  static constexpr int N = kUnroll * E;
  const uint4* vec;
  int c0, c1, nvec, st, tid;
  bool hact[2];
  uint32_t hraw[2];
  uint4 v[kUnroll];

  __device__ __forceinline__ RowReader(const uint8_t* row, int st_, int en, int tid_) : st(st_), tid(tid_) {
    const uintptr_t addr = reinterpret_cast<uintptr_t>(row) + (uintptr_t)st * K::kElemBytes;
    c0 = st + (int)(((16 - (addr & 15)) & 15) / K::kElemBytes);
    if (c0 > en) c0 = en;
    nvec = (en - c0) / E;
    c1 = c0 + nvec * E;
    vec = reinterpret_cast<const uint4*>(row + (size_t)c0 * K::kElemBytes);
    load(0);
    const int nh = c0 - st, nt = en - c1;
    hact[0] = tid < nh;
    hact[1] = tid < nt;
    hraw[0] = hact[0] ? K::load1(row, st + tid) : 0u;
    hraw[1] = hact[1] ? K::load1(row, c1 + tid) : 0u;
  }
  __device__ __forceinline__ void load(int base) {
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      const int vi = base + u * THREADS + tid;
      if (vi < nvec) v[u] = vec[vi];
    }
  }
  template <typename F>
  __device__ __forceinline__ void run(F&& f) {
    {
      const int col[2] = {st + tid, c1 + tid};
      f(hact, col, hraw);
    }
    for (int base = 0; base < nvec; base += THREADS * kUnroll) {
      uint4 cur[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; u++) cur[u] = v[u];
      if (base + THREADS * kUnroll < nvec) load(base + THREADS * kUnroll);
      bool act[N];
      int col[N];
      uint32_t raw[N];
#pragma unroll
      for (int u = 0; u < kUnroll; u++) {
        const int vi = base + u * THREADS + tid;
        const bool a = vi < nvec;
#pragma unroll
        for (int e = 0; e < E; e++) {
          act[u * E + e] = a;
          col[u * E + e] = c0 + vi * E + e;
          raw[u * E + e] = a ? K::elem(cur[u], e) : 0u;
        }
      }
      f(act, col, raw);
    }
  }
};

template <bool BF16, int THREADS, typename F>
__device__ __forceinline__ void scan_row(const uint8_t* row, int st, int en, int tid, F&& f) {
  RowReader<BF16, THREADS> rd(row, st, en, tid);
  rd.run(f);
}

// Reserve consecutive slots for the set predicates of a batch, one LDS atomic per
// wavefront: pos[i] is this lane's slot for element i (meaningful where pred[i]).
// Slots follow the element order of the batch, lanes in order within an element.
template <int N>
__device__ __forceinline__ void reserve_batch(const bool (&pred)[N], int* counter, int lane, int (&pos)[N]) {
  uint64_t m[N];
  int total = 0;
#pragma unroll
  for (int i = 0; i < N; i++) {
    m[i] = __ballot(pred[i]);
    total += __popcll(m[i]);
  }
  int base = 0;
  if (total) {  // uniform
    if (lane == 0) base = atomicAdd(counter, total);
    base = __builtin_amdgcn_readfirstlane(base);
  }
#pragma unroll
  for (int i = 0; i < N; i++) {
    pos[i] = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m[i] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m[i], 0u));
    base += __popcll(m[i]);
  }
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

// Given an LDS histogram of nb bins (COPIES copies each, already filled), find the bin where the count
// from the top reaches `need`.  Writes the bin and the count strictly above it to
// s_sel[0..1]; s_sel[2] = total count.  Each thread owns kBinsPerThread consecutive
// bins.  Call with all threads; ends synchronised.
template <typename C, int COPIES = C::kCopies>
__device__ __forceinline__ void select_bin(const int* hist, int nb, int need, int* s_wave, int* s_sel, int tid) {
  constexpr int BPT = C::kBinsPerThread;
  int h[BPT], local = 0;
#pragma unroll
  for (int j = 0; j < BPT; j++) {
    const int bin = tid * BPT + j;
    h[j] = 0;
    if (bin < nb)
#pragma unroll
      for (int c = 0; c < COPIES; c++) h[j] += hist[bin * COPIES + c];
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

// Columns [a, b) of slice g of G of a row's range [st, en): contiguous, nearly equal.
__device__ __forceinline__ void slice_range(int st, int en, int g, int G, int& a, int& b) {
  const int64_t w = ((int64_t)en - st + G - 1) / G;
  a = (int)min((int64_t)st + g * w, (int64_t)en);
  b = (int)min((int64_t)a + w, (int64_t)en);
}

// The boundary bin b1 (top 11 key bits) is known, `above1` columns above it are written
// to out[0, above1), and the m columns of bin b1 are in s_ckey/s_ccol (when m <= cap).
// Resolves the remaining key bits (fp32: digits of 10 and 11 bits, bf16: 5) by histograms over
// the candidates — or over the row when m > cap — and writes the k - above1 selected
// boundary-bin columns to out[above1, k).  Call with all threads.
template <bool BF16, typename C>
__device__ __forceinline__ void resolve_boundary(const uint8_t* row, int st, int en, int k, uint32_t b1, int above1,
                                                 int m, int cap, const uint32_t* s_ckey, const int* s_ccol,
                                                 int* s_hist, int* s_wave, int* s_sel, int* s_cnt, int* orow,
                                                 int tid) {
  using K = Keys<BF16>;
  constexpr int kTkThreads = C::kThreads;
  const int lane = tid & 63;
  int need = k - above1;
  constexpr int kLow = K::kTopShift;
  const int nd = BF16 ? 1 : 2;
  const int shifts[2] = {BF16 ? 0 : 11, 0};
  const int widths[2] = {BF16 ? 5 : 10, 11};
  uint32_t prefix = b1 << kLow;  // known high bits of the threshold key
  const bool in_lds = m <= cap;
  for (int p = 0; p < nd; p++) {
    const int sh = shifts[p], wd = widths[p], nb = 1 << wd;
    const int hs = sh + wd;  // bits at and above hs are fixed by `prefix`
    for (int i = tid; i < nb * C::kCopies; i += kTkThreads) s_hist[i] = 0;
    __syncthreads();
    if (in_lds) {
      for (int i = tid; i < m; i += kTkThreads) {
        const uint32_t key = s_ckey[i];
        if ((key >> hs) == (prefix >> hs)) hist_add<C::kCopies>(s_hist, (key >> sh) & (nb - 1), lane);
      }
    } else {
      scan_row<BF16, kTkThreads>(row, st, en, tid, [&](const auto& act, const auto&, const auto& raw) {
        constexpr int n = sizeof(act) / sizeof(act[0]);
#pragma unroll
        for (int i = 0; i < n; i++) {
          uint32_t key;
          if (act[i] && K::key(raw[i], key) && (key >> hs) == (prefix >> hs))
            hist_add<C::kCopies>(s_hist, (key >> sh) & (nb - 1), lane);
        }
      });
    }
    __syncthreads();
    select_bin<C>(s_hist, nb, need, s_wave, s_sel, tid);
    prefix |= (uint32_t)s_sel[0] << sh;
    need -= s_sel[1];
    __syncthreads();
  }
  // tau = prefix: select the boundary-bin keys above tau, and `need` of those equal to it
  const int base = above1;
  const int n_above_tau = (k - base) - need;
  auto emit = [&](const auto& gt, const auto& eq, const auto& col) {
    constexpr int n = sizeof(gt) / sizeof(gt[0]);
    int pg[n], pe[n];
    reserve_batch(gt, &s_cnt[2], lane, pg);
    reserve_batch(eq, &s_cnt[3], lane, pe);
#pragma unroll
    for (int i = 0; i < n; i++) {
      if (gt[i] && base + pg[i] < k) orow[base + pg[i]] = col[i] - st;
      if (eq[i] && pe[i] < need && base + n_above_tau + pe[i] < k) orow[base + n_above_tau + pe[i]] = col[i] - st;
    }
  };
  if (in_lds) {
    for (int i0 = 0; i0 < m; i0 += kTkThreads) {
      const int i = i0 + tid;
      const bool a = i < m;
      const uint32_t key = a ? s_ckey[i] : 0u;
      const bool gt[1] = {a && key > prefix}, eq[1] = {a && key == prefix};
      const int col[1] = {a ? s_ccol[i] : 0};
      emit(gt, eq, col);
    }
  } else {
    scan_row<BF16, kTkThreads>(row, st, en, tid, [&](const auto& act, const auto& col, const auto& raw) {
      constexpr int n = sizeof(act) / sizeof(act[0]);
      bool gt[n], eq[n];
#pragma unroll
      for (int i = 0; i < n; i++) {
        uint32_t key = 0;
        const bool valid = act[i] && K::key(raw[i], key) && (key >> kLow) == b1;
        gt[i] = valid && key > prefix;
        eq[i] = valid && key == prefix;
      }
      emit(gt, eq, col);
    });
  }
}

// ---------------------------------------------------------------- one workgroup per row
template <bool BF16, typename C>
__global__ __launch_bounds__(C::kThreads) void topk_kernel(const uint8_t* __restrict__ logits, int64_t row_bytes,
                                                          RowRange range, int k,
                                                          int* __restrict__ out, int64_t out_ld) {
  using K = Keys<BF16>;
  __shared__ int s_hist[kHistBins * C::kCopies];
  constexpr int kTkThreads = C::kThreads, kCandCap = C::kCap;
  __shared__ uint32_t s_ckey[kCandCap];
  __shared__ int s_ccol[kCandCap];
  __shared__ int s_wave[C::kWaves];
  __shared__ int s_sel[4];
  __shared__ int s_cnt[4];  // 0: written above the boundary, 1: candidates, 2/3: written from candidates

  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  int st, en;
  range.get(r, st, en);
  const uint8_t* row = logits + (int64_t)r * row_bytes;
  int* orow = out + (int64_t)r * out_ld;

  for (int i = tid; i < kHistBins * C::kCopies; i += kTkThreads) s_hist[i] = 0;
  if (tid < 4) s_cnt[tid] = 0;
  __syncthreads();

  // pass 1: histogram of the top 11 key bits
  scan_row<BF16, kTkThreads>(row, st, en, tid, [&](const auto& act, const auto&, const auto& raw) {
    constexpr int n = sizeof(act) / sizeof(act[0]);
#pragma unroll
    for (int i = 0; i < n; i++) {
      uint32_t key;
      if (act[i] && K::key(raw[i], key)) hist_add<C::kCopies>(s_hist, key >> K::kTopShift, lane);
    }
  });
  __syncthreads();
  select_bin<C>(s_hist, kHistBins, k, s_wave, s_sel, tid);
  const int total = s_sel[2];
  const uint32_t b1 = (uint32_t)s_sel[0];
  const int above1 = s_sel[1];
  const bool all = total <= k;  // every valid value is selected

  // pass 2: columns above the boundary bin (or every valid column) are written; the
  // boundary bin's are candidates
  scan_row<BF16, kTkThreads>(row, st, en, tid, [&](const auto& act, const auto& col, const auto& raw) {
    constexpr int n = sizeof(act) / sizeof(act[0]);
    bool gt[n], eq[n];
    uint32_t keys[n];
    int pos[n], slot[n];
#pragma unroll
    for (int i = 0; i < n; i++) {
      uint32_t key = 0;
      const bool valid = act[i] && K::key(raw[i], key);
      const uint32_t d = key >> K::kTopShift;
      gt[i] = valid && (all || d > b1);
      eq[i] = valid && !all && d == b1;
      keys[i] = key;
    }
    reserve_batch(gt, &s_cnt[0], lane, pos);
    reserve_batch(eq, &s_cnt[1], lane, slot);
#pragma unroll
    for (int i = 0; i < n; i++) {
      if (gt[i] && pos[i] < k) orow[pos[i]] = col[i] - st;
      if (eq[i] && slot[i] < kCandCap) {
        s_ckey[slot[i]] = keys[i];
        s_ccol[slot[i]] = col[i];
      }
    }
  });
  if (all) {
    for (int j = total + tid; j < k; j += kTkThreads) orow[j] = -1;
    return;
  }
  __syncthreads();
  resolve_boundary<BF16, C>(row, st, en, k, b1, above1, s_cnt[1], kCandCap, s_ckey, s_ccol, s_hist, s_wave, s_sel,
                            s_cnt, orow, tid);
}

// ---------------------------------------------------------------- rows held in registers
// A row of at most THREADS * VPT 16-byte vectors (plus an unaligned head and tail of fewer
// than 16 bytes each) is read from memory once: thread t keeps vectors i*THREADS + t of the
// row in registers, converted to keys, and every pass runs on them.
//
// Non-finite values and the empty slots past the row fall into histogram bins no finite
// value reaches — the four lowest (negative NaN/inf; key 0 for empty slots) and the four
// highest (positive inf/NaN) — which the bin search ignores.  Output slots are reserved
// once per wavefront: each thread counts its columns above the boundary bin and in it, a
// wavefront prefix sum of the two counts packed into one word (wavefront totals stay below
// 2^16, so the halves never carry into each other) gives every thread its offsets, and two
// LDS atomics per wavefront reserve the ranges.  Columns above the boundary bin go straight
// to their slots (lanes with nothing to write store to a spare slot instead of branching);
// the boundary bin's columns are kept in LDS and resolved there by further key digits, or
// by passes over the row in memory when there are more than the LDS list holds (heavy
// ties).  The keys are laundered between passes so that the compiler recomputes their
// bins instead of keeping a second register per key.  The selected columns are
// assembled in LDS and the finished row is written in one coalesced pass.
template <int THREADS, int VPT, int F32_WAVES = 1>
struct RegCfg {
  static constexpr int kThreads = THREADS;
  static constexpr int kVpt = VPT;
  static constexpr int kF32Waves = F32_WAVES;  // wavefronts per SIMD the fp32 kernel is compiled for (at least)
  static constexpr int kCap = 1024;  // boundary-bin columns kept in LDS
  static constexpr int kWaves = THREADS / 64;
  static constexpr int kCopies = 1;
  static constexpr int kBinsPerThread = kHistBins / THREADS;
};
using RegTiny = RegCfg<256, 4>;    // fp32 rows up to 4096 columns, bf16 rows up to 8192 (fewer VGPRs: more rows
                                   // per CU, e.g. 1056 bf16 rows of 8192 in one round instead of two)
using RegSmall = RegCfg<256, 8, 8>;  // fp32 rows up to 8192 columns, bf16 rows up to 16384.  The fp32 kernel is
                                     // held to 64 VGPRs (a few spills) so that eight rows share a CU instead of
                                     // seven: the 2048 x 8192 prefill top-k measured 26.7 -> 26.2 us.
using RegMid = RegCfg<512, 8>;     // fp32 rows up to 16384 columns (512 threads: half the per-row latency of 256 x 64 keys)

template <bool BF16, typename C>
constexpr int reg_capacity() {
  return C::kThreads * C::kVpt * Keys<BF16>::kPerVec;
}

// Bin search by wavefront 0 alone: lane l sums bins [l*B, l*B + B) of hist (B = nb / 64, or
// bin l when nb < 64), a wavefront suffix sum gives each lane the count above its bins, and
// the lane whose bins hold the `need`-th largest writes s_sel[0] = that bin, s_sel[1] = the
// count strictly above it, s_sel[3] = the count in it, s_sel[2] = the total.  Bins outside
// [lo, hi) count as empty.
// Call with all threads (after the histogram is complete); ends synchronised.
template <int NB>
__device__ __forceinline__ void find_bin_w0(const int* hist, int lo, int hi, int need, int* s_sel, int tid) {
  constexpr int B = NB >= 64 ? NB / 64 : 1;
  if (tid < 64) {
    int h[B], local = 0;
    if (B % 4 == 0) {
#pragma unroll
      for (int j = 0; j < B; j += 4) {
        const int4 x = *reinterpret_cast<const int4*>(hist + tid * B + j);
        h[j] = x.x;
        h[j + 1] = x.y;
        h[j + 2] = x.z;
        h[j + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < B; j++) h[j] = tid * B + j < NB ? hist[tid * B + j] : 0;
    }
#pragma unroll
    for (int j = 0; j < B; j++) {
      const int bin = tid * B + j;
      h[j] = (bin < NB && bin >= lo && bin < hi) ? h[j] : 0;
      local += h[j];
    }
    // suffix sum over lanes: above = sum of `local` over lanes > tid
    int v = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_down(v, off);
      if (tid + off < 64) v += y;
    }
    const int above = v - local;
    if (tid == 0) s_sel[2] = v;
    // the bin j with acc_j < need <= acc_j + h[j], acc_j = above + (bins above j): one
    // lane holds it, found without branches
    int acc = above, sel = -1, sel_acc = 0, sel_cnt = 0;
#pragma unroll
    for (int j = B - 1; j >= 0; j--) {
      const bool hit = acc < need && need <= acc + h[j];
      sel = hit ? tid * B + j : sel;
      sel_acc = hit ? acc : sel_acc;
      sel_cnt = hit ? h[j] : sel_cnt;
      acc += h[j];
    }
    if (sel >= 0) {
      s_sel[0] = sel;
      s_sel[1] = sel_acc;
      s_sel[3] = sel_cnt;
    }
  }
  __syncthreads();
}

// find_bin_w0 for the 2048-bin first digit, spread over all WAVES wavefronts: wavefront q
// owns bins [q*B*64, (q+1)*B*64) (B = 2048 / (64 * WAVES) per lane), the wavefronts' totals
// meet in s_part, and the one holding the `need`-th largest writes s_sel as find_bin_w0 does.
// Call with all threads (after the histogram is complete); ends synchronised.
template <int WAVES>
__device__ __forceinline__ void find_bin_all(const int* hist, int lo, int hi, int need, int* s_part, int* s_sel,
                                             int tid) {
  constexpr int B = kHistBins / (64 * WAVES);
  static_assert(B >= 4 && B % 4 == 0, "whole int4 reads per lane");
  const int lane = tid & 63, wave = tid >> 6;
  const int first = tid * B;  // this lane's first bin (bins ascend with tid)
  int h[B], local = 0;
#pragma unroll
  for (int j = 0; j < B; j += 4) {
    const int4 x = *reinterpret_cast<const int4*>(hist + first + j);
    h[j] = x.x;
    h[j + 1] = x.y;
    h[j + 2] = x.z;
    h[j + 3] = x.w;
  }
#pragma unroll
  for (int j = 0; j < B; j++) {
    const int bin = first + j;
    h[j] = (bin >= lo && bin < hi) ? h[j] : 0;
    local += h[j];
  }
  int v = local;  // suffix sum over the wavefront's lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_down(v, off);
    if (lane + off < 64) v += y;
  }
  if (lane == 0) s_part[wave] = v;  // the wavefront's total
  __syncthreads();
  int above_w = 0, total = 0;
#pragma unroll
  for (int q = 0; q < WAVES; q++) {
    const int t = s_part[q];
    total += t;
    above_w += q > wave ? t : 0;
  }
  if (tid == 0) s_sel[2] = total;
  int acc = above_w + v - local, sel = -1, sel_acc = 0, sel_cnt = 0;
#pragma unroll
  for (int j = B - 1; j >= 0; j--) {
    const bool hit = acc < need && need <= acc + h[j];
    sel = hit ? first + j : sel;
    sel_acc = hit ? acc : sel_acc;
    sel_cnt = hit ? h[j] : sel_cnt;
    acc += h[j];
  }
  if (sel >= 0) {
    s_sel[0] = sel;
    s_sel[1] = sel_acc;
    s_sel[3] = sel_cnt;
  }
  __syncthreads();
}

// Makes the compiler treat the values as redefined here, so that predicates computed from
// them in an earlier unrolled loop are recomputed rather than kept alive (as one 64-bit
// lane mask each) until a later loop.
template <int M>
__device__ __forceinline__ void launder(uint32_t (&a)[M]) {
#pragma unroll
  for (int j = 0; j < M; j++) asm volatile("" : "+v"(a[j]));
}

// Reserve output ranges for one wavefront: this thread has `a` items for range A and `b`
// for range B (each below 2^16 per wavefront); returns the thread's first slots in pa, pb,
// counted from the running totals *ca, *cb (LDS), which grow by the wavefront's sums.
__device__ __forceinline__ void reserve2(int a, int b, int* ca, int* cb, int lane, int& pa, int& pb) {
  const int packed = (a << 16) | b;
  int incl = packed;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  int ba = 0, bb = 0;
  if (lane == 63) {
    ba = atomicAdd(ca, incl >> 16);
    bb = atomicAdd(cb, incl & 0xFFFF);
  }
  ba = __shfl(ba, 63);
  bb = __shfl(bb, 63);
  const int excl = incl - packed;
  pa = ba + (excl >> 16);
  pb = bb + (excl & 0xFFFF);
}

// The boundary bin by passes over the row (heavy ties: more columns than the LDS list holds), out of line so that
// its registers do not burden the common path.  s_hist: kHistBins ints.
template <bool BF16, typename C>
__device__ __forceinline__ void reg_resolve_by_row(const uint8_t* row, int st, int en, int k, uint32_t b1,
                                                             int above1, int m, int* s_hist, int* s_wave, int* s_sel,
                                                             int* s_cnt, int* s_out, int tid) {
  resolve_boundary<BF16, C>(row, st, en, k, b1, above1, m, 0, nullptr, nullptr, s_hist, s_wave, s_sel, s_cnt, s_out,
                            tid);
}

template <bool BF16, typename C>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(BF16 ? 1 : C::kF32Waves))) void
topk_reg_kernel(const uint8_t* __restrict__ logits, int64_t row_bytes,
                                                              RowRange range, int k,
                                                              int* __restrict__ out, int64_t out_ld) {
  using K = Keys<BF16>;
  constexpr int T = C::kThreads, E = K::kPerVec, V = C::kVpt, N = V * E;
  constexpr int kShift = K::kTopShift;
  constexpr int kCap = C::kCap;
  constexpr uint32_t kLoBin = 8;  // finite values have bins in [kLoBin, kHistBins) in this kernel's key form
  static_assert((N + 2) * 64 < 65536, "packed per-wavefront counts must stay below 2^16");
  // Arrays carry 64 spare slots past their end: a lane with nothing to store (or add)
  // writes its own spare slot instead of branching.  LDS is what bounds the rows resident
  // per CU, so buffers are reused once dead: the first-digit histogram becomes the list of
  // selected columns once the boundary bin is known, and the candidate list becomes the
  // histogram of the passes over the row when the boundary bin outgrows it.
  static_assert(DSI_MAX_TOPK == kHistBins, "the selected columns fill the first-digit histogram's storage");
  static_assert(2 * (kCap + 64) >= kHistBins, "the candidate list holds an 11-bit histogram");
  __shared__ __attribute__((aligned(16))) int s_hist[kHistBins + 64];
  int* const s_out = s_hist;  // the selected columns, after the boundary bin is found
  __shared__ __attribute__((aligned(16))) uint32_t s_cand[2 * (kCap + 64)];  // boundary-bin keys, then columns
  uint32_t* const s_ckey = s_cand;
  int* const s_ccol = reinterpret_cast<int*>(s_cand + kCap + 64);
  __shared__ int s_dig[128];  // the boundary bin's further digits
  __shared__ int s_sel[4];
  __shared__ int s_wave[C::kWaves];
  __shared__ int s_cnt[4];  // 0: written, 3: boundary bin; 1/2: resolution

  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  int st, en;
  range.get(r, st, en);
  const uint8_t* row = logits + (int64_t)r * row_bytes;
  int* orow = out + (int64_t)r * out_ld;

  // Head [st, c0) and tail [c1, en): fewer than E columns each, one element per thread;
  // nvec aligned vectors in between (the host guarantees nvec <= T * V).
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row) + (uintptr_t)st * K::kElemBytes;
  const int c0 = min(st + (int)(((16 - (addr & 15)) & 15) / K::kElemBytes), en);
  const int nvec = (en - c0) / E;
  const int c1 = c0 + nvec * E;
  const uint4* vec = reinterpret_cast<const uint4*>(row + (size_t)c0 * K::kElemBytes);
  // Keys; 0 (an ignored bin) for slots outside the row.  bf16 keys are 16 bits: two share a
  // register (key j in half j & 1 of kk[j / 2]), which saves a third of the kernel's VGPRs.
  constexpr int kPack = BF16 ? 2 : 1;
  uint32_t kk[(N + 2) / kPack];
  auto key_at = [&](int j) -> uint32_t {
    if constexpr (BF16)
      return (j & 1) ? (kk[j >> 1] >> 16) : (kk[j >> 1] & 0xFFFFu);
    else
      return kk[j];
  };
  auto set_key = [&](int j, uint32_t v) {  // called for j in increasing order
    if constexpr (BF16) {
      if (j & 1)
        kk[j >> 1] |= v << 16;
      else
        kk[j >> 1] = v;
    } else {
      kk[j] = v;
    }
  };
  // Keys: the order-preserving key plus four first-digit bins, modulo the key width.  Finite
  // values keep their order and land in bins [8, 2048); +inf and +NaN wrap to bins 0..3 and
  // -inf and -NaN stay in 4..7, below every finite value, as do the zero keys of slots outside
  // the row.  Each later test is then one unsigned comparison.
  auto reg_key = [](uint32_t raw) -> uint32_t {
    if constexpr (BF16) {
      const uint32_t t = (raw & 0x8000u) ? 0xFFFFu : 0x8000u;
      return ((raw ^ t) + 0x80u) & 0xFFFFu;
    } else {
      const uint32_t t = (uint32_t)((int32_t)raw >> 31) | 0x80000000u;
      return (raw ^ t) + 0x00800000u;
    }
  };
  // The row's loads are all issued first; the histogram is cleared and the barrier passed while
  // they are in flight (a barrier waits for LDS operations only), and each vector's keys are
  // built and counted as soon as it arrives.  The vectors are read through a buffer record that
  // ends at the row's last whole vector (reads past it return zeros), so the loads carry no
  // branches and the compiler can wait for each one by its position.
  // The head and tail elements go first: waiting for them then does not wait for the vectors.
  const bool ha = tid < c0 - st, ta = tid < en - c1;
  const uint32_t raw_h = ha ? K::load1(row, st + tid) : 0u;
  const uint32_t raw_t = ta ? K::load1(row, c1 + tid) : 0u;
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(vec), (short)0, nvec * 16, 0x00020000);
  uint4 xv[V];
#pragma unroll
  for (int i = 0; i < V; i++) {  // in order: the keys are built in this order
    xv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, (i * T + tid) * 16, 0, 0));
    __builtin_amdgcn_sched_barrier(0);
  }
  // column of kk[j] relative to st
  const int col_base = c0 - st + tid * E;
  auto column = [&](int j) { return j < N ? col_base + (j / E) * T * E + (j % E) : (j == N ? tid : c1 - st + tid); };

  for (int i = tid; i < kHistBins; i += T) s_hist[i] = 0;
  if (tid < 4) s_cnt[tid] = 0;
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);  // no key is built before the barrier (it would wait for its load there)
  // Keys and the first-digit histogram over the row's slots only (whole vectors past the row
  // are skipped by the lanes holding them).
#pragma unroll
  for (int i = 0; i < V; i++) {
    const bool in = i * T + tid < nvec;
#pragma unroll
    for (int e = 0; e < E; e++) set_key(i * E + e, in ? reg_key(K::elem(xv[i], e)) : 0u);
    if (in) {
#pragma unroll
      for (int e = 0; e < E; e++) atomicAdd(&s_hist[key_at(i * E + e) >> kShift], 1);
    }
  }
  set_key(N, ha ? reg_key(raw_h) : 0u);
  set_key(N + 1, ta ? reg_key(raw_t) : 0u);
  if (ha) atomicAdd(&s_hist[key_at(N) >> kShift], 1);
  if (ta) atomicAdd(&s_hist[key_at(N + 1) >> kShift], 1);
  launder(kk);  // the bins are recomputed where needed rather than kept, one register per key
  __syncthreads();
  find_bin_all<C::kWaves>(s_hist, kLoBin, kHistBins, k, s_wave, s_sel, tid);  // its last read of s_hist precedes
                                                                              // its closing barrier
  const int total = s_sel[2];
  const bool all = total <= k;  // every finite value is selected
  const uint32_t b1 = all ? 0xFFFFFFFFu : (uint32_t)s_sel[0];
  const int above1 = all ? total : s_sel[1];
  // Written: key > top (above the boundary bin; every finite value when all are taken).
  // Candidates: key - t_eq < span (the boundary bin; none when all are taken).
  const uint32_t top = all ? (kLoBin << kShift) - 1u : (b1 << kShift) | ((1u << kShift) - 1u);
  const uint32_t t_eq = all ? 0u : b1 << kShift;
  const uint32_t span = all ? 0u : 1u << kShift;

  // Each wavefront counts its columns of both kinds (ballots, scalar sums), reserves one range
  // of each, then writes them in slot order: slot j of every lane, then slot j + 1.  The head
  // and tail slots are skipped by a wavefront none of whose lanes holds one (their keys are 0,
  // neither written nor a candidate): rows that start aligned have no head, and only a few lanes
  // of one wavefront hold a tail.
  const bool any_h = __builtin_amdgcn_ballot_w64(ha) != 0, any_t = __builtin_amdgcn_ballot_w64(ta) != 0;
  auto skip = [&](int j) { return (j == N && !any_h) || (j == N + 1 && !any_t); };
  int cg = 0, ce = 0;
#pragma unroll
  for (int j = 0; j < N + 2; j++) {
    if (skip(j)) continue;
    const uint32_t key = key_at(j);
    cg += __popcll(__builtin_amdgcn_ballot_w64(key > top));
    ce += __popcll(__builtin_amdgcn_ballot_w64(key - t_eq < span));
    __builtin_amdgcn_sched_barrier(0);  // one slot at a time: each mask lives briefly
  }
  asm volatile("" : "+s"(cg), "+s"(ce));  // the sums are complete here, not sunk into the branch below
  int pg = 0, pe = 0;
  if (lane == 0) {
    pg = atomicAdd(&s_cnt[0], cg);
    pe = atomicAdd(&s_cnt[3], ce);
  }
  launder(kk);
  // Byte offsets: each position is the wavefront's base plus the lane's rank among the set
  // lanes of the slot's mask.  A candidate past the list (the boundary bin outgrew it, and the
  // list will not be read) goes to the lane's spare entry instead.
  uint32_t og = (uint32_t)__builtin_amdgcn_readfirstlane(pg) * 4u;
  uint32_t oe = (uint32_t)__builtin_amdgcn_readfirstlane(pe);
  char* const b_out = reinterpret_cast<char*>(s_out);
  char* const b_key = reinterpret_cast<char*>(s_ckey);
  char* const b_col = reinterpret_cast<char*>(s_ccol);
  const uint32_t spare = kCap + lane;
#pragma unroll
  for (int j = 0; j < N + 2; j++) {
    if (skip(j)) continue;
    const uint32_t key = key_at(j);
    const bool gt = key > top;
    const bool eq = key - t_eq < span;
    const uint64_t mg = __builtin_amdgcn_ballot_w64(gt);
    const uint64_t me = __builtin_amdgcn_ballot_w64(eq);
    const int col = column(j);
    const uint32_t rg = __builtin_amdgcn_mbcnt_hi((uint32_t)(mg >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mg, 0u));
    const uint32_t re = __builtin_amdgcn_mbcnt_hi((uint32_t)(me >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)me, oe));
    if (gt) *reinterpret_cast<int*>(b_out + og + rg * 4u) = col;
    if (eq) {
      const uint32_t at = min(re, spare) * 4u;
      *reinterpret_cast<uint32_t*>(b_key + at) = key;
      *reinterpret_cast<int*>(b_col + at) = col;
    }
    og += (uint32_t)__popcll(mg) * 4u;
    oe += (uint32_t)__popcll(me);
    asm volatile("" : "+s"(og));  // kept as a byte offset: one shift-add per address
    __builtin_amdgcn_sched_barrier(0);  // one element at a time: keeps register pressure low
  }
  __syncthreads();
  if (!all) {
    const int m = s_cnt[3];
    const int need = k - above1;
    if (m <= kCap) {
      // Further digits of the key (fp32: three of 7 bits; bf16: 5 bits) by histograms over
      // the boundary bin's columns in LDS.  Narrow digits keep each pass's fixed cost (clear
      // the bins, search them) small: the candidates are a few hundred at most in practice.
      constexpr int kDigits = BF16 ? 1 : 3;
      constexpr int kSh[3] = {BF16 ? 0 : 14, 7, 0};
      constexpr int kWd[3] = {BF16 ? 5 : 7, 7, 7};
      uint32_t prefix = b1 << kShift;
      int rem = need;
      // When the bin a digit selects holds exactly the columns still needed, all of it is
      // taken and the lower digits are skipped: the threshold becomes "every key from the
      // bin's lowest key up" (prefix - 1 as a strict bound, nothing taken at equality).
      bool whole = !BF16 && m == need;  // bf16 has one further digit: nothing to skip (measured)
#pragma unroll
      for (int p = 0; p < kDigits; p++) {
        if (whole) break;  // uniform: from LDS values read after a barrier
        const int sh = kSh[p], nb = 1 << kWd[p], hs = sh + kWd[p];
        for (int i = tid; i < nb; i += T) s_dig[i] = 0;
        __syncthreads();
        for (int i = tid; i < m; i += T) {
          const uint32_t key = s_ckey[i];
          if ((key >> hs) == (prefix >> hs)) atomicAdd(&s_dig[(key >> sh) & (nb - 1)], 1);
        }
        __syncthreads();
        find_bin_w0<(BF16 ? 32 : 128)>(s_dig, 0, nb, rem, s_sel, tid);
        prefix |= (uint32_t)s_sel[0] << sh;
        rem -= s_sel[1];
        whole = !BF16 && s_sel[3] == rem;
      }
      if (whole) {
        prefix -= 1;
        rem = 0;
      }
      // prefix is the threshold key: boundary-bin keys above it are taken, and `rem` of
      // those equal to it
      const int n_above_tau = need - rem;
      for (int i = tid; i < m; i += T) {
        const uint32_t key = s_ckey[i];
        if (key > prefix) {
          s_out[above1 + atomicAdd(&s_cnt[1], 1)] = s_ccol[i];
        } else if (key == prefix) {
          const int t = atomicAdd(&s_cnt[2], 1);
          if (t < rem) s_out[above1 + n_above_tau + t] = s_ccol[i];
        }
      }
    } else {
      // The boundary bin holds more columns than the LDS list: resolve it with passes over
      // the row in memory (heavy ties), writing relative columns into s_out.
      __syncthreads();
      if (tid < 4) s_cnt[tid] = 0;
      __syncthreads();
      // (b1 - 4: the boundary bin in the plain key form that the passes over the row use)
      reg_resolve_by_row<BF16, C>(row, st, en, k, b1 - 4, above1, m, reinterpret_cast<int*>(s_cand), s_wave, s_sel,
                                  s_cnt, s_out, tid);
    }
    __syncthreads();
  }
  const int n = all ? total : k;
  for (int j = tid; j < k; j += T) orow[j] = j < n ? s_out[j] : -1;
}

// ---------------------------------------------------------------- long rows split between workgroups
// Few long rows (decode): each row is cut into G slices of at most 8192 fp32 (16384 bf16)
// columns, one 512-thread workgroup per slice, in up to two launches that communicate through
// the caller's workspace (layout in topk_split.h):
//   1. topk_slice_hist_kernel: each slice's first-digit histogram into its slot — skipped when
//      the paged decode kernel has counted the row's slots while writing its logits;
//   2. topk_split_select_kernel: every slice holds its columns in registers as keys, sums its
//      row's slots (the row's histogram, 4 bins per thread), finds the boundary bin b1, and
//      writes its columns above b1 (every valid column when the row has at most k) at output
//      positions reserved by one device-scope atomic per workgroup; its boundary-bin columns go
//      to the row's candidate list the same way; the row's last slice to finish (a device-scope
//      count of finished slices) resolves the boundary bin from the candidates (or from the
//      row, when it holds more than the list) and pads with -1.
// No workgroup waits for another: the output order is any order, so the shared state is the
// row's counters and candidate list, all accessed with device-scope atomics.
constexpr int kSplitThreads = 512;
constexpr int kSplitVecs = 4;  // 16-byte vectors per thread: 16 fp32 or 32 bf16 columns
using SliceCfg = Cfg<kSplitThreads, 0, 2>;  // two histogram copies in the slice step (measured 26.0 -> 25.6 us)

template <bool BF16>
constexpr int split_slice_cap() {
  return kSplitThreads * kSplitVecs * Keys<BF16>::kPerVec;
}
static_assert(split_slice_cap<true>() < 65536, "slot halves count at most 65535 columns");

// Slice workgroups are numbered so that the G slices of a row run on one XCD (workgroups go to the eight XCDs in
// turn by linear id; row r's resolve workgroup, number r, lands on the same one): the row's slots and candidates
// then meet in that XCD's L2.  Grid: 8 * ceil(rows / 8) * G workgroups; false for the padding.
__device__ __forceinline__ bool split_coords(int G, int rows, int& r, int& g) {
  const int x = (int)blockIdx.x & 7, q = (int)blockIdx.x >> 3;
  g = q % G;
  r = (q / G) * 8 + x;
  return r < rows;
}

__host__ inline unsigned split_grid(int rows, int G) { return (unsigned)(8 * ((rows + 7) / 8) * G); }

// Step 1: the first-digit histogram of each slice into slot r*G + g; slice 0 records the row's slot range and
// clears its counters.
template <bool BF16>
__global__ __launch_bounds__(kSplitThreads) void topk_slice_hist_kernel(const uint8_t* __restrict__ logits,
                                                                       int64_t row_bytes, RowRange range, void* ws,
                                                                       int rows, int G) {
  using K = Keys<BF16>;
  constexpr int kC = SliceCfg::kCopies;
  __shared__ int s_hist[kHistBins * kC];
  const int tid = threadIdx.x, lane = tid & 63;
  int r, g;
  if (!split_coords(G, rows, r, g)) return;
  int st, en;
  range.get(r, st, en);
  int a, b;
  slice_range(st, en, g, G, a, b);
  RowReader<BF16, kSplitThreads> rd(logits + (int64_t)r * row_bytes, a, b, tid);
  for (int i = tid; i < kHistBins * kC; i += kSplitThreads) s_hist[i] = 0;
  __syncthreads();
  rd.run([&](const auto& act, const auto&, const auto& raw) {
    constexpr int n = sizeof(act) / sizeof(act[0]);
#pragma unroll
    for (int i = 0; i < n; i++) {
      uint32_t key;
      if (act[i] && K::key(raw[i], key)) hist_add<kC>(s_hist, key >> K::kTopShift, lane);
    }
  });
  __syncthreads();
  const int64_t slots = (int64_t)rows * G;
  const SplitWs w = split_ws(ws, rows, slots);
  uint32_t* dst = w.slots + ((int64_t)r * G + g) * kSlotWords;
  for (int j = tid; j < kSlotWords; j += kSplitThreads) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int c = 0; c < kC; c++) lo += s_hist[(2 * j) * kC + c], hi += s_hist[(2 * j + 1) * kC + c];
    dst[j] = lo | (hi << 16);
  }
  if (g == 0 && tid == 0) {
    int* meta = w.meta + (int64_t)r * kMetaInts;
    meta[kMetaFirst] = r * G;
    meta[kMetaLast] = r * G + G - 1;
    meta[kMetaCntGt] = 0;
    meta[kMetaCntEq] = 0;
    meta[kMetaDone] = 0;
  }
}

// Step 2 (the last).  Keys in registers as in topk_reg_kernel (invalid columns and empty slots get key 0, a bin no
// finite value reaches); per-thread counts, one workgroup prefix sum of both counts packed in a word (a slice's
// counts stay below 2^16), one atomic per count per workgroup.  Then the boundary bin: every slice appends its
// candidates to the row's list with device-scope atomic stores, waits until they have completed, and counts itself
// done with a device-scope atomic add; the slice that finds itself last (its add returns the count of all the
// others) reads every candidate back with device-scope atomic loads and resolves them in registers by 7-bit digits.
// No workgroup waits for another, and no fence writes the caches back: only the candidates and the counters, all
// accessed with device-scope atomics, cross workgroups.
constexpr int kCandPerThread = kSplitCap / kSplitThreads;  // 24: the resolving slice holds every candidate
static_assert(kCandPerThread * kSplitThreads == kSplitCap, "candidates divide over the threads");
using SplitCfg = Cfg<kSplitThreads, 0, 1>;  // the passes over the row when the boundary bin outgrows the list

// The boundary bin by passes over the row (heavy ties: more columns than the candidate list holds), out of line so
// that its registers do not burden the common path.
template <bool BF16>
__device__ __attribute__((noinline)) void split_resolve_by_row(const uint8_t* row, int st, int en, int k, uint32_t b1,
                                                               int above1, int m, int* s_hist, int* s_part, int* s_sel,
                                                               int* s_cnt, int* orow, int tid) {
  resolve_boundary<BF16, SplitCfg>(row, st, en, k, b1, above1, m, 0, nullptr, nullptr, s_hist, s_part, s_sel, s_cnt,
                                   orow, tid);
}

template <bool BF16>
__global__ __launch_bounds__(kSplitThreads) void topk_split_select_kernel(
    const uint8_t* __restrict__ logits, int64_t row_bytes, RowRange range, int k, int* __restrict__ out,
    int64_t out_ld, void* ws, int rows, int64_t num_slots, int G, int slots_per_row) {
  using K = Keys<BF16>;
  constexpr int T = kSplitThreads, E = K::kPerVec, V = kSplitVecs, N = V * E, W = T / 64;
  constexpr int kShift = K::kTopShift;
  constexpr uint32_t kLoBin = 4, kHiBin = kHistBins - 4;  // finite values have bins in [kLoBin, kHiBin)
  constexpr int kSlotBatch = 16;                          // slot loads in flight per thread
  __shared__ __attribute__((aligned(16))) int s_hist[kHistBins];
  __shared__ int s_sel[4];
  __shared__ int s_part[W];
  __shared__ int s_wsum[W];
  __shared__ int s_base[2];
  __shared__ int s_cnt[4];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int r, g;
  if (!split_coords(G, rows, r, g)) return;
  int st, en;
  range.get(r, st, en);
  int* orow = out + (int64_t)r * out_ld;
  if (en <= st) {  // an empty row: slice 0 pads it
    if (g == 0)
      for (int j = tid; j < k; j += T) orow[j] = -1;
    return;
  }
  int a, b;
  slice_range(st, en, g, G, a, b);
  if (a >= b) return;  // uniform: a slice past the row's end
  const int64_t wid = ((int64_t)en - st + G - 1) / G;
  const int nslices = (int)(((int64_t)en - st + wid - 1) / wid);  // the row's slices that reach the end

  // this slice's keys: head [a, c0) and tail [c1, b) one element per thread, nvec aligned vectors between
  const uint8_t* row = logits + (int64_t)r * row_bytes;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row) + (uintptr_t)a * K::kElemBytes;
  const int c0 = min(a + (int)(((16 - (addr & 15)) & 15) / K::kElemBytes), b);
  const int nvec = (b - c0) / E;
  const int c1 = c0 + nvec * E;
  const uint4* vec = reinterpret_cast<const uint4*>(row + (size_t)c0 * K::kElemBytes);
  constexpr int kPack = BF16 ? 2 : 1;
  uint32_t kk[(N + 2) / kPack];
  auto key_at = [&](int j) -> uint32_t {
    if constexpr (BF16)
      return (j & 1) ? (kk[j >> 1] >> 16) : (kk[j >> 1] & 0xFFFFu);
    else
      return kk[j];
  };
  auto set_key = [&](int j, uint32_t v) {
    if constexpr (BF16) {
      if (j & 1)
        kk[j >> 1] |= v << 16;
      else
        kk[j >> 1] = v;
    } else {
      kk[j] = v;
    }
  };
  uint4 x[V];
#pragma unroll
  for (int i = 0; i < V; i++) {
    const int vi = i * T + tid;
    x[i] = vi < nvec ? vec[vi] : uint4{0u, 0u, 0u, 0u};
  }
  const bool ha = tid < c0 - a, ta = tid < b - c1;
  const uint32_t hraw = ha ? K::load1(row, a + tid) : 0u, traw = ta ? K::load1(row, c1 + tid) : 0u;

  // the row's histogram: the sum of its slots; thread t owns bins 4t .. 4t+3 (two words of every slot); a batch of
  // slots' loads is issued before any is summed
  const SplitWs w = split_ws(ws, rows, num_slots);
  int* meta = w.meta + (int64_t)r * kMetaInts;
  // slots_per_row > 0: row r's slots are r*slots_per_row onwards (known without a load); else its metadata says
  const int s_lo = slots_per_row ? r * slots_per_row : max(meta[kMetaFirst], 0);
  const int s_hi = (int)min(slots_per_row ? (int64_t)r * slots_per_row + slots_per_row - 1 : (int64_t)meta[kMetaLast],
                            num_slots - 1);
  uint32_t h[4] = {0u, 0u, 0u, 0u};
  {
    const uint2* sp = reinterpret_cast<const uint2*>(w.slots) + tid;
    for (int s0 = s_lo; s0 <= s_hi; s0 += kSlotBatch) {
      uint2 y[kSlotBatch];
#pragma unroll
      for (int u = 0; u < kSlotBatch; u++)
        y[u] = s0 + u <= s_hi ? sp[(int64_t)(s0 + u) * (kSlotWords / 2)] : uint2{0u, 0u};
#pragma unroll
      for (int u = 0; u < kSlotBatch; u++) {
        h[0] += y[u].x & 0xFFFFu, h[1] += y[u].x >> 16, h[2] += y[u].y & 0xFFFFu, h[3] += y[u].y >> 16;
      }
    }
  }
  reinterpret_cast<int4*>(s_hist)[tid] = int4{(int)h[0], (int)h[1], (int)h[2], (int)h[3]};
  if (tid < 4) {
    s_sel[tid] = 0;  // stays 0 when the row has at most k values (no bin is selected)
    s_cnt[tid] = 0;
  }
  __syncthreads();
  find_bin_all<W>(s_hist, kLoBin, kHiBin, k, s_part, s_sel, tid);
  const int total = s_sel[2];
  const bool all = total <= k;  // every finite value is selected
  const uint32_t b1 = all ? 0xFFFFFFFFu : (uint32_t)s_sel[0];
  const int above1 = all ? total : s_sel[1];
  const int m = all ? 0 : s_sel[3];
  const bool collect = !all && m <= kSplitCap;

#pragma unroll
  for (int i = 0; i < V; i++) {
    const bool in = i * T + tid < nvec;
#pragma unroll
    for (int e = 0; e < E; e++) {
      uint32_t key;
      const bool ok = K::key(K::elem(x[i], e), key);
      set_key(i * E + e, in && ok ? key : 0u);
    }
  }
  {
    uint32_t key;
    const bool hok = K::key(hraw, key);
    set_key(N, ha && hok ? key : 0u);
    const bool tok = K::key(traw, key);
    set_key(N + 1, ta && tok ? key : 0u);
  }
  // column of kk[j]
  auto column = [&](int j) { return j < N ? c0 + tid * E + (j / E) * T * E + (j % E) : (j == N ? a + tid : c1 + tid); };

  // Keys of non-finite values and empty slots are 0, below every finite value's key (bins >= kLoBin), so
  // "above the boundary" is key > top and "in the boundary bin" is key - t_eq < span (span 0: none collected).
  const uint32_t top = all ? (kLoBin << kShift) - 1u : (b1 << kShift) | ((1u << kShift) - 1u);
  const uint32_t t_eq = all ? 0u : b1 << kShift;
  const uint32_t span = collect ? 1u << kShift : 0u;
  // Each wavefront counts both kinds with ballots; the workgroup's counts (packed gt << 16 | eq: a slice's stay
  // below 2^16) are reserved with one device-scope atomic per kind; then each wavefront writes its columns in slot
  // order (slot j of every lane, then slot j + 1) at mbcnt ranks, so that a store's lanes write consecutive words.
  int cg = 0, ce = 0;
#pragma unroll
  for (int j = 0; j < N + 2; j++) {
    const uint32_t key = key_at(j);
    cg += __popcll(__builtin_amdgcn_ballot_w64(key > top));
    ce += __popcll(__builtin_amdgcn_ballot_w64(key - t_eq < span));
    __builtin_amdgcn_sched_barrier(0);  // one slot at a time: each mask lives briefly
  }
  asm volatile("" : "+s"(cg), "+s"(ce));  // the sums are complete here
  if (lane == 0) s_wsum[wave] = (cg << 16) | ce;
  __syncthreads();
  int before = 0, wg_total = 0;
#pragma unroll
  for (int q = 0; q < W; q++) {
    const int t = s_wsum[q];
    before += q < wave ? t : 0;
    wg_total += t;
  }
  if (tid == 0) {
    s_base[0] = (wg_total >> 16) ? atomicAdd(&meta[kMetaCntGt], wg_total >> 16) : 0;
    s_base[1] = (wg_total & 0xFFFF) ? atomicAdd(&meta[kMetaCntEq], wg_total & 0xFFFF) : 0;
  }
  __syncthreads();
  int pg = __builtin_amdgcn_readfirstlane(s_base[0] + (before >> 16));
  int pe = __builtin_amdgcn_readfirstlane(s_base[1] + (before & 0xFFFF));
  unsigned long long* cand = w.cand + (int64_t)r * kSplitCap;
  // Candidates go to the row's list as device-scope atomic stores (written through to the point where every XCD
  // sees them); the wait below covers their completion before the slice counts itself done.
  launder(kk);
#pragma unroll
  for (int j = 0; j < N + 2; j++) {
    const uint32_t key = key_at(j);
    const bool gt = key > top;
    const bool eq = key - t_eq < span;
    const uint64_t mg = __builtin_amdgcn_ballot_w64(gt);
    const uint64_t me = __builtin_amdgcn_ballot_w64(eq);
    const int col = column(j);
    const int ig = pg + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mg >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mg, 0u));
    const int ie = pe + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(me >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)me, 0u));
    if (gt && ig < k) orow[ig] = col - st;
    if (eq && ie < kSplitCap)
      __hip_atomic_store(cand + ie, ((unsigned long long)(uint32_t)col << 32) | key, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    pg += __popcll(mg);
    pe += __popcll(me);
    __builtin_amdgcn_sched_barrier(0);  // one element at a time: no lane masks kept for later elements
  }
  if (all) {  // uniform: nothing to resolve; slice 0 pads the row
    if (g == 0)
      for (int j = total + tid; j < k; j += T) orow[j] = -1;
    return;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's candidate stores have completed
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&meta[kMetaDone], 1) == nslices - 1;
  __syncthreads();
  if (!s_last) return;  // uniform

  // The row's last slice: the boundary bin b1 holds m columns, need = k - above1 of them are selected.
  const int need = k - above1;
  if (!collect) {  // more than the list holds (heavy ties): passes over the row
    split_resolve_by_row<BF16>(row, st, en, k, b1, above1, m, s_hist, s_part, s_sel, s_cnt, orow, tid);
    return;
  }
  uint32_t ck[kCandPerThread];
  int cc[kCandPerThread];
  const int nj = (m + T - 1) / T;  // uniform: rounds of candidates that hold any
#pragma unroll
  for (int j = 0; j < kCandPerThread; j++) {
    const int i = tid + j * T;
    unsigned long long v = 0;
    if (j < nj && i < m) v = __hip_atomic_load(cand + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ck[j] = (uint32_t)v;  // key 0 (an unused entry) never matches a prefix in bin b1 >= 4
    cc[j] = (int)(v >> 32);
  }
  // Further digits of the key (fp32: three of 7 bits; bf16: 5 bits), each by a histogram over the candidates; when
  // the bin a digit selects holds exactly the columns still needed, all of it is taken and the lower digits are
  // skipped ("every key from the bin's lowest up": prefix - 1 as a strict bound, nothing taken at equality).
  constexpr int kDigits = BF16 ? 1 : 3;
  constexpr int kSh[3] = {BF16 ? 0 : 14, 7, 0};
  constexpr int kWd[3] = {BF16 ? 5 : 7, 7, 7};
  uint32_t prefix = b1 << kShift;
  int rem = need;
  bool whole = !BF16 && m == need;
#pragma unroll
  for (int p = 0; p < kDigits; p++) {
    if (whole) break;  // uniform
    const int sh = kSh[p], nb = 1 << kWd[p], hs = sh + kWd[p];
    __syncthreads();  // the previous digit's bins are no longer read
    for (int i = tid; i < nb; i += T) s_hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kCandPerThread; j++) {
      if (j < nj && (ck[j] >> hs) == (prefix >> hs)) atomicAdd(&s_hist[(ck[j] >> sh) & (nb - 1)], 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    find_bin_w0<(BF16 ? 32 : 128)>(s_hist, 0, nb, rem, s_sel, tid);
    prefix |= (uint32_t)s_sel[0] << sh;
    rem -= s_sel[1];
    whole = !BF16 && s_sel[3] == rem;
  }
  if (whole) {
    prefix -= 1;
    rem = 0;
  }
  const int n_above_tau = need - rem;
#pragma unroll
  for (int j = 0; j < kCandPerThread; j++) {
    const uint32_t key = ck[j];
    if (j >= nj || (key >> kShift) != b1) continue;  // unused entries (j >= nj: uniform)
    if (key > prefix) {
      orow[above1 + atomicAdd(&s_cnt[1], 1)] = cc[j] - st;
    } else if (key == prefix) {
      const int t = atomicAdd(&s_cnt[2], 1);
      if (t < rem) orow[above1 + n_above_tau + t] = cc[j] - st;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Workgroups per row: split long rows when there are too few rows to fill the CUs.
inline int split_count(int rows, int max_width, bool bf16) {
  if (max_width <= kShortRow || rows >= 512) return 1;
  const int cap = bf16 ? split_slice_cap<true>() : split_slice_cap<false>();
  return (int)(((int64_t)max_width + cap - 1) / cap);
}

template <bool BF16>
int launch_select_resolve(const uint8_t* src, int64_t row_bytes, int rows, const RowRange& range, int k, int* out,
                          int64_t out_ld, void* ws, int64_t num_slots, int G, int slots_per_row, hipStream_t stream) {
  hipLaunchKernelGGL(topk_split_select_kernel<BF16>, dim3(split_grid(rows, G)), dim3(kSplitThreads), 0, stream, src,
                     row_bytes, range, k, out, out_ld, ws, rows, num_slots, G, slots_per_row);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}

}  // namespace
}  // namespace dsi

namespace dsi {

int split_groups_f32(int rows, int max_width) { return split_count(rows, max_width, false); }

int launch_split_select(const float* logits, int64_t ld, int rows, const RowRange& range, int k, int* out,
                        int64_t out_ld, void* ws, int64_t num_slots, int G, hipStream_t stream) {
  return launch_select_resolve<false>(reinterpret_cast<const uint8_t*>(logits), ld * 4, rows, range, k, out, out_ld,
                                      ws, num_slots, G, 0, stream);
}

}  // namespace dsi

extern "C" size_t dsi_topk_workspace_bytes(int32_t rows, int32_t max_width, int32_t k) {
  using namespace dsi;
  (void)k;
  if (rows <= 0 || max_width <= 0) return 0;
  // the larger of the fp32 and bf16 split sizes (the dtype is not an argument)
  const int G = std::max(split_count(rows, max_width, false), split_count(rows, max_width, true));
  return G > 1 ? split_ws_bytes(rows, (int64_t)rows * G) : 0;
}

namespace dsi {

int topk_dispatch(const void* logits, bool bf, int64_t ld, int rows, const RowRange& range, int max_width, int k,
                  int* out, int64_t out_ld, void* workspace, hipStream_t stream) {
  const int64_t row_bytes = ld * (bf ? 2 : 4);
  const uint8_t* src = reinterpret_cast<const uint8_t*>(logits);
  const int G = split_count(rows, max_width, bf);
  if (G > 1) {
    const int64_t slots = (int64_t)rows * G;
    const dim3 grid(split_grid(rows, G));
    if (bf) {
      hipLaunchKernelGGL(topk_slice_hist_kernel<true>, grid, dim3(kSplitThreads), 0, stream, src, row_bytes, range,
                         workspace, rows, G);
      return launch_select_resolve<true>(src, row_bytes, rows, range, k, out, out_ld, workspace, slots, G, G, stream);
    }
    hipLaunchKernelGGL(topk_slice_hist_kernel<false>, grid, dim3(kSplitThreads), 0, stream, src, row_bytes, range,
                       workspace, rows, G);
    return launch_select_resolve<false>(src, row_bytes, rows, range, k, out, out_ld, workspace, slots, G, G, stream);
  }
  const dim3 grid((unsigned)rows);
#define DSI_TOPK_REG(B, CFG)                                                                                        \
  hipLaunchKernelGGL((topk_reg_kernel<B, CFG>), grid, dim3(CFG::kThreads), 0, stream, src, row_bytes, range, k, out, \
                     out_ld)
  if (!bf) {
    if (max_width <= reg_capacity<false, RegTiny>())
      DSI_TOPK_REG(false, RegTiny);
    else if (max_width <= reg_capacity<false, RegSmall>())
      DSI_TOPK_REG(false, RegSmall);
    else if (max_width <= reg_capacity<false, RegMid>())
      DSI_TOPK_REG(false, RegMid);
    else
      hipLaunchKernelGGL((topk_kernel<false, LongRows>), grid, dim3(LongRows::kThreads), 0, stream, src, row_bytes,
                         range, k, out, out_ld);
  } else {
    if (max_width <= reg_capacity<true, RegTiny>())
      DSI_TOPK_REG(true, RegTiny);
    else if (max_width <= reg_capacity<true, RegSmall>())
      DSI_TOPK_REG(true, RegSmall);
    else
      hipLaunchKernelGGL((topk_kernel<true, LongRows>), grid, dim3(LongRows::kThreads), 0, stream, src, row_bytes,
                         range, k, out, out_ld);
  }
#undef DSI_TOPK_REG
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}

namespace {

int topk_select_impl(const void* logits, int32_t dtype, int64_t ld, int32_t rows, const int32_t* row_starts,
                     const int32_t* row_ends, int32_t max_width, int32_t k, int32_t* out, int64_t out_ld,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (dtype != DSI_F32 && dtype != DSI_BF16) return DSI_EUNSUPPORTED;
  if (k < 1 || k > DSI_MAX_TOPK) return DSI_EUNSUPPORTED;
  if (rows < 0 || max_width < 0 || ld < max_width || out_ld < k) return DSI_EINVAL;
  const size_t need = dsi_topk_workspace_bytes(rows, max_width, k);
  if (workspace_bytes < need || (need && !workspace)) return DSI_EWORKSPACE;
  if (rows == 0) return DSI_OK;
  if (!logits || !row_ends || !out) return DSI_EINVAL;
  if (dtype == DSI_F32 && (reinterpret_cast<uintptr_t>(logits) & 3)) return DSI_EALIGN;
  if (dtype == DSI_BF16 && (reinterpret_cast<uintptr_t>(logits) & 1)) return DSI_EALIGN;
  if ((reinterpret_cast<uintptr_t>(out) & 3) || (reinterpret_cast<uintptr_t>(workspace) & 15)) return DSI_EALIGN;
  if (rows > 65535) return DSI_EUNSUPPORTED;
  return topk_dispatch(logits, dtype == DSI_BF16, ld, rows, RowRange{row_starts, row_ends, nullptr, 1, max_width},
                       max_width, k, out, out_ld, workspace, stream);
}

// ---------------------------------------------------------------- no-allocation variant
// The workspace of dsi_topk_select_noalloc: one file-scope device array per GPU, held for the
// process's lifetime.  In host code `scratch` names a host-side stand-in, not device memory, so
// the kernels get the array's device address, looked up once per device (with that device
// current) and kept in s_scratch.
constexpr int kMaxDevices = 64;
__device__ __attribute__((aligned(256))) uint8_t scratch[DSI_TOPK_NOALLOC_MAX_BYTES];
std::mutex s_scratch_mu;
void* s_scratch[kMaxDevices];

// The device address of this stream's GPU's array (looked up on first use).
int scratch_for(hipStream_t stream, void** ptr) {
  int dev = -1, cur = -1;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || hipGetDevice(&cur) != hipSuccess) return DSI_ELAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return DSI_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(s_scratch_mu);
  if (!s_scratch[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return DSI_ELAUNCH;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return DSI_ELAUNCH;
    if (e != hipSuccess || !p) return DSI_ELAUNCH;
    s_scratch[dev] = p;
  }
  *ptr = s_scratch[dev];
  return DSI_OK;
}

}  // namespace
}  // namespace dsi

extern "C" int dsi_topk_select(const void* logits, int32_t dtype, int64_t ld, int32_t rows,
                               const int32_t* row_starts, const int32_t* row_ends, int32_t max_width, int32_t k,
                               int32_t* out, int64_t out_ld, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return dsi::topk_select_impl(logits, dtype, ld, rows, row_starts, row_ends, max_width, k, out, out_ld, workspace,
                               workspace_bytes, stream);
}

extern "C" int dsi_topk_select_noalloc(const void* logits, int32_t dtype, int64_t ld, int32_t rows,
                                       const int32_t* row_starts, const int32_t* row_ends, int32_t max_width,
                                       int32_t k, int32_t* out, int64_t out_ld, hipStream_t stream) {
  using namespace dsi;
  if (dtype != DSI_F32 && dtype != DSI_BF16) return DSI_EUNSUPPORTED;
  if (k < 1 || k > DSI_MAX_TOPK) return DSI_EUNSUPPORTED;
  if (rows < 0 || max_width < 0 || ld < max_width || out_ld < k) return DSI_EINVAL;
  const size_t need = dsi_topk_workspace_bytes(rows, max_width, k);
  if (need > (size_t)DSI_TOPK_NOALLOC_MAX_BYTES) return DSI_EWORKSPACE;  // before any HIP call
  void* ws = nullptr;
  if (need) {
    const int st = scratch_for(stream, &ws);
    if (st != DSI_OK) return st;
  }
  return topk_select_impl(logits, dtype, ld, rows, row_starts, row_ends, max_width, k, out, out_ld, ws,
                          need ? (size_t)DSI_TOPK_NOALLOC_MAX_BYTES : 0, stream);
}
