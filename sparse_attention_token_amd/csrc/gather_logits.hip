// Indexer logits over gathered key sets: paged decode (P3 prefill/decode table of
// "DeepSeek V3.2 稀疏注意力 DSA 推理流程图解": decode scores straight from the
// paged cache, no gather) and the hierarchical path's sparse columns (P1 "V4.1
// 索引器接入稀疏 MQA logits", motivation and implementation: consumer layers score
// only the candidate blocks, into bf16 logits).
//
// Both stream 132-byte K rows past one to four query rows.  A workgroup gathers chunks of
// 256 keys straight into LDS with global->LDS DMA loads (global_load_lds_dwordx4: no VGPR
// staging, no LDS write instructions), double-buffered so that the next chunk is in flight
// while one is scored, and scores them on the matrix cores with the query rows decoded in
// VGPRs (common.h's 32x32x16 layout): each wavefront takes 32-key groups in pipelined
// pairs, decoding the FP8 codes from LDS per use.  Out-of-range table entries, page ids
// or tokens never produce an access outside the source: those keys score -inf.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "topk_split.h"

namespace dsi {
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* glob_ptr_t;

// ------------------------------------------------------------------ paged decode
// A workgroup (4 wavefronts) streams segments of up to 16 chunks of 256 keys of one request
// through a ring of LDS buffers: the DMA gathers of the next chunks are in flight while
// one chunk is scored, and the request's q rows stay decoded in VGPRs for the segment.
// Scoring decodes a 32-key group's FP8 codes under the previous group's MFMAs and sums
// heads under the next group's.
// Rows are spread over the wavefronts (1 row: 4 wavefronts share each chunk's keys; 2
// rows: 2 wavefronts per row; 3-4 rows: one wavefront per row, all keys).  Each key row
// lands in LDS as nine 16-byte pieces at a 144-byte stride (bytes 0..127, then 116..131
// so that the scale sits at byte 140 and nothing past the row is read), which makes
// every B-fragment read a conflict-free 16-byte LDS load.
constexpr int kDcChunk = 256;                       // keys per LDS buffer
constexpr int kDcRow = 144;                         // LDS bytes per key
constexpr int kDcBuf = kDcChunk * kDcRow;           // 36864
constexpr int kDcSlabsPerWave = kDcBuf / 1024 / 4;  // 9 DMA instructions per wavefront per chunk
constexpr int kDcJob = 16;                          // chunks per job (16 rather than 8: fewer set-ups,
                                                    // 75.6 -> 71.7 us for 16 requests x 2 rows)
constexpr int kDcSegs = kDcJob * kDcChunk / 16;     // 16-token segments per job

// Issue this wavefront's NP DMA pieces of one chunk: slab i (1 KB of the chunk buffer) is
// slab wave + 4i, lane l's 16 bytes are piece 64*slab + l, read from src_of(piece).  The
// loads are issued as inline assembly (one wait state, then global_load_lds_dwordx4), so the
// compiler does not treat them as writes to the other buffer that the scoring of the current
// chunk has to wait for; the kernel orders them itself with an explicit vmcnt wait and a
// barrier.  The LDS destination of the wavefront's 1 KB goes in M0 through the operand
// constraint "{m0}": the compiler writes M0 itself and knows the statement reads it (M0 is a
// reserved register, so naming it as a clobber would not protect a value the compiler keeps
// there).  Every source address (each needs an LDS read of its key's offset) is computed
// before the first load is issued: the assembly statements are ordered memory operations,
// so interleaving them with those reads cost one LDS round trip per load.  kStream sets the
// loads' non-temporal hint ("nt"): the paged decode reads each page once per call, and the
// hint made its reads of random 8448-byte pages faster; the sparse kernels re-read one
// source from the caches and keep the default policy.
template <bool kStream, int NP, typename SrcOf>
__device__ __forceinline__ void dma_chunk(uint8_t* buf, int wave, int lane, SrcOf&& src_of) {
  const uint8_t* src[NP];
#pragma unroll
  for (int i = 0; i < NP; i++) src[i] = src_of((wave + 4 * i) * 64 + lane);
#pragma unroll
  for (int i = 0; i < NP; i++) {
    const uint32_t lds =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)(buf + (wave + 4 * i) * 1024));
    if constexpr (kStream)
      asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src[i]), "{m0}"(lds) : "memory");
    else
      asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src[i]), "{m0}"(lds) : "memory");
  }
}

// This wavefront's share of one decode chunk: piece s (16 bytes) is key s/9, piece s%9 of
// the key's 132-byte row (bytes 16p, or 116..131 for p = 8); absent segments read the
// pool's first bytes (their keys score -inf).
__device__ __forceinline__ void dc_gather(uint8_t* buf, const int64_t* seg_base, const uint8_t* pool, int wave,
                                          int lane) {
  dma_chunk<true, kDcSlabsPerWave>(buf, wave, lane, [&](int piece) {
    const int key = piece / 9, p = piece - key * 9;
    const int64_t base = seg_base[key >> 4];
    return base >= 0 ? pool + base + (key & 15) * kRow + (p < 8 ? 16 * p : 116) : pool;
  });
}

// Wait until at most `n` of this wavefront's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// wait_vm<kDcSlabsPerWave * (idx / NB) + KS * (idx % NB)>() for a wavefront-uniform idx
// in [0, (NB - 1) * NB): the wait for a chunk's gather when idx / NB gathers of this
// wavefront and the stores of idx % NB scored chunks were issued after it.
template <int NB, int KS, int I = 0>
__device__ __forceinline__ void wait_gather(int idx) {
  if constexpr (I < (NB - 1) * NB) {
    if (idx == I) {
      wait_vm<kDcSlabsPerWave * (I / NB) + KS * (I % NB)>();
      return;
    }
    wait_gather<NB, KS, I + 1>(idx);
  } else {
    wait_vm<0>();
  }
}

// B fragments of one 32-key group from raw rows in a chunk buffer: key l%32, codes
// [64h, 64h+64) as four 16-byte loads, decoded to f16.
__device__ __forceinline__ void load_k32_raw(K32& f, const uint8_t* keys, int lane) {
  const uint4* p = reinterpret_cast<const uint4*>(keys + (lane & 31) * kDcRow + (lane >> 5) * 64);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const uint4 x = p[j];
    f.b[2 * j] = e4m3x8_to_f16x8(x.x, x.y);
    f.b[2 * j + 1] = e4m3x8_to_f16x8(x.z, x.w);
  }
}

// The weights of the 32 heads this lane holds in C, kept as bf16 pairs (16 registers instead
// of 32): weight e of head block hb is head hb*32 + 8*(e/4) + 4h + e%4, and w[hb][e / 2]
// holds weights e (low half) and e + 1 (high half).
struct W32p {
  uint32_t w[2][8];
  __device__ __forceinline__ float get(int hb, int e) const {
    const uint32_t x = w[hb][e >> 1];
    return __uint_as_float((e & 1) ? (x & 0xFFFF0000u) : (x << 16));
  }
};

__device__ __forceinline__ void load_w32p(W32p& f, const uint16_t* w_row, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int hb = 0; hb < 2; hb++)
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const uint2 x = *reinterpret_cast<const uint2*>(w_row + hb * 32 + 8 * b + 4 * h);
      f.w[hb][2 * b] = x.x;
      f.w[hb][2 * b + 1] = x.y;
    }
}

// One 32-key group on the matrix cores with the neighbouring groups' work threaded between
// its 16 MFMAs in a fixed order (sched_barrier fences keep the compiler from regrouping):
// step i issues MFMA i (slice i/2, head block i%2) into x, then two of the 32 FMAs of the
// head sum of y (the previous group's accumulators) when kEpi, then — when kNext — the
// decode of the next group's slices 2j and 2j+1 into kb once MFMA 4j+3 has read them
// (their raw codes are read from LDS two slice pairs ahead), then extra(i).
template <bool kEpi, bool kNext, typename Extra>
__device__ __forceinline__ void dc_phase(f32x16& x0, f32x16& x1, const Q32& q, K32& kb, const uint8_t* next,
                                         int lane, const W32p& w, const f32x16& y0, const f32x16& y1,
                                         float (&acc)[4], Extra&& extra) {
  const uint4* np = reinterpret_cast<const uint4*>(next + (lane & 31) * kDcRow + (lane >> 5) * 64);
  uint4 raw[2];
  if (kNext) {
    raw[0] = np[0];
    raw[1] = np[1];
  }
#pragma unroll
  for (int j = 0; j < 4; j++) acc[j] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int sl = i >> 1;
    if ((i & 1) == 0)
      x0 = mfma32(q.a[0][sl], kb.b[sl], i == 0 ? f32x16{} : x0);
    else
      x1 = mfma32(q.a[1][sl], kb.b[sl], i == 1 ? f32x16{} : x1);
    __builtin_amdgcn_sched_barrier(0);
    if (kEpi) {
#pragma unroll
      for (int e = 2 * i; e < 2 * i + 2; e++) {
        if (e < 16)
          acc[e & 3] = fmaf(w.get(0, e), y0[e], acc[e & 3]);
        else
          acc[e & 3] = fmaf(w.get(1, e - 16), y1[e - 16], acc[e & 3]);
      }
    }
    if (kNext && (i & 3) == 3) {
      const int j = i >> 2;
      kb.b[2 * j] = e4m3x8_to_f16x8(raw[j & 1].x, raw[j & 1].y);
      kb.b[2 * j + 1] = e4m3x8_to_f16x8(raw[j & 1].z, raw[j & 1].w);
      if (j < 2) raw[j] = np[j + 2];  // codes of slices 2j+4 and 2j+5
    }
    extra(i);
    __builtin_amdgcn_sched_barrier(0);
  }
}

__device__ __forceinline__ float dc_acc_sum(const float (&acc)[4]) { return (acc[0] + acc[1]) + (acc[2] + acc[3]); }

// The head sum of one group's accumulators on its own (no MFMAs to hide it behind).
__device__ __forceinline__ float dc_head_sum(const W32p& w, const f32x16& y0, const f32x16& y1) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 16; e++) acc[e & 3] = fmaf(w.get(0, e), y0[e], acc[e & 3]);
#pragma unroll
  for (int e = 0; e < 16; e++) acc[e & 3] = fmaf(w.get(1, e), y1[e], acc[e & 3]);
  return dc_acc_sum(acc);
}

// ------------------------------------------------------------------ MXFP4 key rows
// A 68-byte MXFP4 row lands in LDS as five 16-byte pieces at an 80-byte stride (bytes
// 0..63, then 52..67, so the four scale bytes sit at 76..79; 20 dwords per key keep
// 16-byte reads by 8 consecutive keys on distinct banks).  The block scales differ within
// one 16-dim MFMA step (each lane half feeds its own 32-dim block), so they are applied
// while decoding: the hardware converter turns each FP4 code times its block's 2^(E-127)
// into bf16, exactly, and q's FP8 codes are decoded to bf16, exactly; the contraction runs
// on the bf16 matrix cores with fp32 accumulation (products of 4- and 2-bit significands
// are exact).
constexpr int kMxRow = 68;                          // bytes per MXFP4 key row
constexpr int kMxLds = 80;                          // LDS bytes per key
constexpr int kMxBuf = kDcChunk * kMxLds;           // 20480
constexpr int kMxSlabsPerWave = kMxBuf / 1024 / 4;  // 5 DMA instructions per wavefront per chunk

__device__ __forceinline__ f32x16 mfma32_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// q[row] as bf16 A fragments (load_q32's layout).
struct Q32b {
  bf16x8 a[2][8];
};

__device__ __forceinline__ void load_q32_bf16(Q32b& f, const uint8_t* q_row, int lane) {
  const int m = lane & 31, h = lane >> 5;
#pragma unroll
  for (int hb = 0; hb < 2; hb++) {
    const uint4* p = reinterpret_cast<const uint4*>(q_row + (hb * 32 + m) * kDim + h * 64);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint4 x = p[j];
      f.a[hb][2 * j] = e4m3x8_to_bf16x8(x.x, x.y);
      f.a[hb][2 * j + 1] = e4m3x8_to_bf16x8(x.z, x.w);
    }
  }
}

// Raw B data of one key row for this lane (key l%32, lane half h = dims [64h, 64h+64)):
// the half's 32 code bytes and the scales of its blocks 2h and 2h+1.
struct MxRaw {
  uint4 c0, c1;
  float s0, s1;
};

__device__ __forceinline__ MxRaw load_mx_raw(const uint8_t* keys, int lane) {
  const uint8_t* row = keys + (lane & 31) * kMxLds;
  const int h = lane >> 5;
  MxRaw r;
  r.c0 = *reinterpret_cast<const uint4*>(row + 32 * h);
  r.c1 = *reinterpret_cast<const uint4*>(row + 32 * h + 16);
  const uint32_t sc = *reinterpret_cast<const uint32_t*>(row + 76);
  r.s0 = e8m0_to_f32((sc >> (16 * h)) & 255u);
  r.s1 = e8m0_to_f32((sc >> (16 * h + 8)) & 255u);
  return r;
}

struct K32b {
  bf16x8 b[8];
};

// Slices 2j and 2j+1 (dims 64h + 16j .. +16) of a raw row.
__device__ __forceinline__ void decode_mx_pair(K32b& kb, const MxRaw& r, int j) {
  const uint4& c = j < 2 ? r.c0 : r.c1;
  const float sc = j < 2 ? r.s0 : r.s1;
  const uint32_t w0 = (j & 1) ? c.z : c.x, w1 = (j & 1) ? c.w : c.y;
  kb.b[2 * j] = fp4x8_to_bf16x8(w0, sc);
  kb.b[2 * j + 1] = fp4x8_to_bf16x8(w1, sc);
}

// dc_phase on bf16 operands: MFMA i of the group, two head-sum FMAs of the previous group,
// the next group's slices decoded as MFMAs 4j+3 retire their sources, then extra(i).
template <bool kEpi, bool kNext, typename Extra>
__device__ __forceinline__ void mx_phase(f32x16& x0, f32x16& x1, const Q32b& q, K32b& kb, const uint8_t* next,
                                         int lane, const W32p& w, const f32x16& y0, const f32x16& y1,
                                         float (&acc)[4], Extra&& extra) {
  MxRaw raw;
  if (kNext) raw = load_mx_raw(next, lane);
#pragma unroll
  for (int j = 0; j < 4; j++) acc[j] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int sl = i >> 1;
    if ((i & 1) == 0)
      x0 = mfma32_bf16(q.a[0][sl], kb.b[sl], i == 0 ? f32x16{} : x0);
    else
      x1 = mfma32_bf16(q.a[1][sl], kb.b[sl], i == 1 ? f32x16{} : x1);
    __builtin_amdgcn_sched_barrier(0);
    if (kEpi) {
#pragma unroll
      for (int e = 2 * i; e < 2 * i + 2; e++) {
        if (e < 16)
          acc[e & 3] = fmaf(w.get(0, e), y0[e], acc[e & 3]);
        else
          acc[e & 3] = fmaf(w.get(1, e - 16), y1[e - 16], acc[e & 3]);
      }
    }
    if (kNext && (i & 3) == 3) decode_mx_pair(kb, raw, i >> 2);
    extra(i);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// This wavefront's share of one decode chunk of MXFP4 rows (as dc_gather): piece s is key
// s/5, piece s%5 of its 68-byte row (bytes 16p, or 52..67 for p = 4).
__device__ __forceinline__ void dc_gather_mx(uint8_t* buf, const int64_t* seg_base, const uint8_t* pool, int wave,
                                             int lane) {
  dma_chunk<true, kMxSlabsPerWave>(buf, wave, lane, [&](int piece) {
    const int key = piece / 5, p = piece - key * 5;
    const int64_t base = seg_base[key >> 4];
    return base >= 0 ? pool + base + (key & 15) * kMxRow + (p < 4 ? 16 * p : 52) : pool;
  });
}

// ------------------------------------------------------------------ paged decode kernel
// WPR = wavefronts per row (4, 2 or 1): each scores 256 / WPR keys of every chunk.  NB =
// chunk buffers in LDS: NB - 1 gathers are in flight while one chunk is scored.
// Work split.  persistent = 0: workgroup (x, y) takes chunks [kDcJob x, kDcJob (x + 1)) of request y
// (grid = (ceil(max_context_len / (256 * kDcJob)), B)).  persistent = 1 (B <= kDcMaxReqs): the grid is
// one-dimensional (two workgroups per CU) and workgroup i takes the i-th of gridDim.x equal
// shares of all requests' chunks in request order, as segments of at most kDcJob chunks of
// one request each, so that no CU idles while a few long jobs finish.
constexpr int kDcMaxReqs = 1024;

// MX selects the cache format: false = 132-byte FP8 rows (f16 matrix cores, per-key fp32
// scale), true = 68-byte MXFP4 rows (bf16 matrix cores, block scales applied in decoding).
// HIST (persistent, one row per request): the kernel also counts the first-digit histogram of
// the top-k's split path (topk_split.h) for every request it scores, in LDS as bin pairs, and
// writes it to slot blockIdx.x + b when it leaves request b.  The workgroups taking a
// request's chunks are consecutive and every share is non-empty, so the request's slots are
// consecutive too and no two (workgroup, request) pairs share one: the workgroup holding the
// request's first chunk records the first slot (and clears the request's counters), the one
// holding its last chunk the last slot.  A share is at most 255 chunks (the host sizes the
// grid), so a slot's bin counts fit in 16 bits.
template <int WPR, int NB, bool MX, bool HIST>
__global__ __launch_bounds__(256, NB > 2 ? 1 : 2) void paged_decode_kernel(
    const uint8_t* __restrict__ q, const uint16_t* __restrict__ w, int B, int next_n,
    const int* __restrict__ context_lens, const uint8_t* __restrict__ pool, int64_t num_blocks, int block_size,
    int64_t block_stride, const int* __restrict__ block_table, int64_t bt_ld, int bt_width, int max_ctx,
    float* __restrict__ logits, int64_t ld, int persistent, void* ws, int64_t num_slots) {
  static_assert(!MX || NB == 2, "the MXFP4 ring's waits assume two buffers");
  static_assert(!HIST || WPR == 4, "histograms are counted for one row per request");
  if constexpr (HIST) persistent = 1;  // a compile-time fact here: the per-request grid's code is dropped
  constexpr int kKeysPerWave = kDcChunk / WPR;
  constexpr int kGroups = kKeysPerWave / 32;
  constexpr int kStores = kKeysPerWave / 64;
  constexpr int kRowBytes = MX ? kMxRow : kRow;  // bytes per key in the pool
  constexpr int kLdsRow = MX ? kMxLds : kDcRow;  // bytes per key in LDS
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[NB][MX ? kMxBuf : kDcBuf];
  __shared__ int64_t s_base[kDcSegs];
  __shared__ uint32_t s_hist[HIST ? kSlotWords : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool has_pool = num_blocks > 0;
  auto chunks_of = [&](int L) { return (min(max(L, 0), max_ctx) + kDcChunk - 1) / kDcChunk; };
  if constexpr (HIST)
    for (int j = tid; j < kSlotWords; j += 256) s_hist[j] = 0u;  // ordered before use by run()'s first barrier

  // Score chunks [c_first, c_end) (at most kDcJob) of request b.
  auto run = [&](int b, int c_first, int c_end) {
  const int L = context_lens[b];
  const int Lc = min(L, max_ctx);  // the last row of the request sees [0, L)
  __syncthreads();  // the previous segment's buffers and segment bases are no longer read
  if constexpr (HIST) {
    if (tid == 0) {
      int* meta = split_ws(ws, B, num_slots).meta + (int64_t)b * kMetaInts;
      const int slot = (int)blockIdx.x + b;
      if (c_first == 0) {
        meta[kMetaFirst] = slot;
        meta[kMetaCntGt] = 0;
        meta[kMetaCntEq] = 0;
        meta[kMetaDone] = 0;
      }
      if (c_end == chunks_of(L)) meta[kMetaLast] = slot;
    }
  }

  // Segment bases of the whole job (-1: absent).
  for (int sg = tid; sg < kDcSegs; sg += 256) {
    const int s = (c_first * kDcChunk) + 16 * sg;
    int64_t base = -1;
    if (s < Lc) {
      const int blk = s / block_size;
      if (blk < bt_width) {
        const int page = block_table[(int64_t)b * bt_ld + blk];
        if (page >= 0 && page < num_blocks)
          base = (int64_t)page * block_stride + (int64_t)(s % block_size) * kRowBytes;
      }
    }
    s_base[sg] = base;
  }

  // This wavefront's row and key range within each chunk.
  const int row = wave / WPR;
  const int kbase = (wave % WPR) * kKeysPerWave;
  const bool active = row < next_n;  // 3 rows: the fourth wavefront only gathers
  const int rr = min(row, next_n - 1);
  std::conditional_t<MX, Q32b, Q32> qf;
  W32p wf;
  if constexpr (MX)
    load_q32_bf16(qf, q + ((int64_t)b * next_n + rr) * kHeads * kDim, lane);
  else
    load_q32(qf, q + ((int64_t)b * next_n + rr) * kHeads * kDim, lane);
  load_w32p(wf, w + ((int64_t)b * next_n + rr) * kHeads, lane);
  const int ke = active ? min(L - next_n + rr + 1, max_ctx) : 0;
  const __amdgpu_buffer_rsrc_t out_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      logits + ((int64_t)b * next_n + rr) * ld, (short)0, max(ke, 0) * 4, 0x00020000);
  __syncthreads();  // segment bases visible

  auto gather = [&](int c) {  // chunk c into its buffer
    if (!has_pool) return;
    if constexpr (MX)
      dc_gather_mx(s_buf[(c - c_first) % NB], s_base + (c - c_first) * 16, pool, wave, lane);
    else
      dc_gather(s_buf[(c - c_first) % NB], s_base + (c - c_first) * 16, pool, wave, lane);
  };
  // Score chunk c: this wavefront's keys as kGroups / 2 pairs of 32-key groups, each pair
  // software-pipelined (dc_phase: the first group's MFMAs carry the second group's decode,
  // the second group's MFMAs the first group's head sum).  With two buffers the gather of
  // chunk `next` (if any) is issued whole before the first group: issuing it piece by piece
  // between the first MFMAs (so that a busy vector-memory queue would not hold up the matrix
  // work) measured slower — each DMA instruction then stalled the phase it sat in — in this
  // kernel (65 -> 64 us) and more in the sparse ones (189 -> 176 us, 159 -> 150 us).
  auto score_chunk = [&](int c, const uint8_t* buf, int next) {
    const int64_t* seg = s_base + (c - c_first) * 16;
#pragma unroll
    for (int h = 0; h < kGroups / 2; h++) {
      const uint8_t* keys = buf + (kbase + 64 * h) * kLdsRow;
      if (NB == 2 && h == 0 && next < c_end) gather(next);
      f32x16 a0, a1, b0 = {}, b1 = {};
      float acc[4];
      float scale = 1.0f;  // MXFP4: the block scales are in the decoded values
      if constexpr (MX) {
        K32b kb;
        const MxRaw r0 = load_mx_raw(keys, lane);
#pragma unroll
        for (int j = 0; j < 4; j++) decode_mx_pair(kb, r0, j);
        mx_phase<false, true>(a0, a1, qf, kb, keys + 32 * kLdsRow, lane, wf, b0, b1, acc, [](int) {});
        mx_phase<true, false>(b0, b1, qf, kb, keys, lane, wf, a0, a1, acc, [](int) {});
      } else {
        K32 kb;
        load_k32_raw(kb, keys, lane);
        dc_phase<false, true>(a0, a1, qf, kb, keys + 32 * kLdsRow, lane, wf, b0, b1, acc, [](int) {});
        dc_phase<true, false>(b0, b1, qf, kb, keys, lane, wf, a0, a1, acc, [](int) {});
        scale = *reinterpret_cast<const float*>(buf + (kbase + 64 * h + lane) * kLdsRow + 140);
      }
      const float v = combine_halves(dc_acc_sum(acc), dc_head_sum(wf, b0, b1));
      const int key = kbase + 64 * h + lane;  // key within the chunk
      const float out = seg[key >> 4] >= 0 ? v * scale : -INFINITY;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out), out_rsrc, (c * kDcChunk + key) * 4, 0, 0);
      if constexpr (HIST) {  // every column inside the row's range; non-finite values fall in bins the top-k ignores
        if (c * kDcChunk + key < ke) {
          // word bin/2 of the packed histogram, half bin&1 (bin = f32_first_bin(out) = key >> 21)
          const uint32_t u = __float_as_uint(out);
          const uint32_t k = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
          atomicAdd(&s_hist[k >> 22], 1u + ((k >> 21) & 1u) * 0xFFFFu);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

#pragma unroll
  for (int j = 0; j < NB - 1; j++)
    if (c_first + j < c_end) gather(c_first + j);
  for (int cc = c_first; cc < c_end; cc++) {
    // Wait for chunk cc's gather.  Issued after it by this wavefront: the gathers of the
    // chunks up to cc + NB - 2 that exist, and the stores of the chunks scored since —
    // all of them before the loop when cc's gather was issued in the prologue, else the
    // NB - 1 chunks before cc.
    const int ng = min(c_end - 1 - cc, NB - 2);
    const int ns = min(cc - c_first, NB - 1);
    if (has_pool) {
      if (active)
        wait_gather<NB, kStores>(ng * NB + ns);
      else
        wait_gather<NB, 0>(ng * NB + ns);
    }
    __syncthreads();  // every wavefront's part has landed; and everyone is done with chunk cc - 1's buffer
    if (NB > 2 && cc + NB - 1 < c_end) gather(cc + NB - 1);  // into chunk cc - 1's buffer
    if (active)
      score_chunk(cc, s_buf[(cc - c_first) % NB], cc + NB - 1);
    else if (NB == 2 && cc + NB - 1 < c_end)
      gather(cc + NB - 1);
  }
  };  // run

  // Persistent: every wavefront finds this workgroup's share from all requests' chunk counts
  // (lane l holds requests l, l + 64, ...; a running prefix over them), then walks it.  With fewer
  // chunks than workgroups, only the first `total` take one chunk each: no share is empty.
  int b = B, start = 0, g0 = 0, g1 = 0;  // the request holding chunk g0 and its first global chunk
  if (persistent) {
    const int nblk = (B + 63) / 64;  // uniform
    // lane l holds requests l, l + 64, ...: first the total, then the request holding g0
    int total = 0;
    for (int i = 0; i < nblk; i++) {
      const int r = i * 64 + lane;
      int v = r < B ? chunks_of(context_lens[r]) : 0;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      total += v;
    }
    // Uniform in fact; said so, or the share's loop counts (and every value carried through the
    // loop, the output row's buffer descriptor included) would be treated as per-lane values.
    total = __builtin_amdgcn_readfirstlane(total);
    const int nwg = min((int)gridDim.x, total);
    if ((int)blockIdx.x >= nwg) return;  // uniform: no share
    g0 = (int)((int64_t)blockIdx.x * total / nwg);
    g1 = (int)((int64_t)(blockIdx.x + 1) * total / nwg);
    int carry = 0;
    for (int i = 0; i < nblk && b == B; i++) {
      const int r = i * 64 + lane;
      const int c = r < B ? chunks_of(context_lens[r]) : 0;
      int v = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(v, off);
        if (lane >= off) v += y;
      }
      const uint64_t m = __ballot(carry + v > g0);
      if (m) {
        const int l = __ffsll((unsigned long long)m) - 1;
        b = i * 64 + l;
        start = carry + __shfl(v - c, l);
      }
      carry += __shfl(v, 63);
    }
  } else {
    b = blockIdx.y;
    start = -(int)blockIdx.x * kDcJob;  // local chunk = g0 - start
    g1 = kDcJob;
  }
  b = __builtin_amdgcn_readfirstlane(b);
  int lc = __builtin_amdgcn_readfirstlane(g0 - start);
  int remaining = __builtin_amdgcn_readfirstlane(g1 - g0);
  int counted = -1;  // HIST: the request whose counts s_hist holds
  // HIST: write request rb's counts to its slot and clear them (each word by the thread that owns it)
  auto flush = [&](int rb) {
    __syncthreads();  // every lane's counts are in
    uint32_t* dst = split_ws(ws, B, num_slots).slots + ((int64_t)blockIdx.x + rb) * kSlotWords;
    for (int j = tid; j < kSlotWords; j += 256) {
      dst[j] = s_hist[j];
      s_hist[j] = 0u;
    }
  };
  while (remaining > 0 && b < B) {  // uniform
    const int cb = __builtin_amdgcn_readfirstlane(chunks_of(context_lens[b]));
    const int len = min(remaining, min(cb - lc, kDcJob));
    if (len > 0) {
      if constexpr (HIST) {
        if (counted != b) {
          if (counted >= 0) flush(counted);
          counted = b;
        }
      }
      run(b, lc, lc + len);
    }
    remaining -= max(len, 0);
    lc += max(len, 0);
    if (lc >= cb) {
      if (!persistent) break;
      b++;
      lc = 0;
    }
  }
  if constexpr (HIST)
    if (counted >= 0) flush(counted);
}

// ------------------------------------------------------------------ sparse columns
// The paged-decode machinery on the hierarchical path's candidate columns.  Every row's
// columns form nch = ceil(width / 256) chunks; the grid (two workgroups per CU) takes equal
// shares of all (row, chunk) pairs, as segments of up to kSpJob chunks of one row.  A
// segment starts by computing each of its columns' source offset — the column's token
// through sparse_indices, then the gathered row or the page through the block table, or
// "absent" when the column scores -inf — so blocks, pages and invalid columns need no
// special case later.  It then streams its chunks through the DMA ring and scores them as
// the decode kernel scores one row (four wavefronts x 64 keys per chunk), rounding to bf16.
// Chunks per segment: longer segments pay the segment set-up (offsets, q decode) less often
// (8 instead of 4 chunks: 205 -> 196 us on the hierarchical workload); the FP8 kernel's two
// 36 KB buffers and 8 KB of offsets fill the 160 KB LDS at two workgroups per CU, the MXFP4
// kernel's 20 KB buffers leave room for 32, a whole 8192-column row (178 -> 165 us at 16,
// 144 -> 138 us at 32).
constexpr int kSpJob = 8;
constexpr int kMxJob = 32;
constexpr uint32_t kSpAbsent = 0xFFFFFFFFu;   // source offsets are in 4-byte units

// This wavefront's share of one chunk's gather (as dc_gather, with one source offset per key).
__device__ __forceinline__ void sp_gather(uint8_t* buf, const uint32_t* key_off, const uint8_t* src, int wave,
                                          int lane) {
  dma_chunk<false, kDcSlabsPerWave>(buf, wave, lane, [&](int piece) {
    const int key = piece / 9, p = piece - key * 9;
    const uint32_t off = key_off[key];
    return off != kSpAbsent ? src + (int64_t)off * 4 + (p < 8 ? 16 * p : 116) : src;
  });
}

// Source offsets (4-byte units, kSpAbsent for columns that score -inf) of columns [c0, c0 + n) of row r into s_off,
// for key rows of ROWB bytes: every column follows its token through sparse_indices and, when paged, the block
// table.
template <int ROWB>
__device__ __forceinline__ void fill_offsets(uint32_t* s_off, int r, int c0, int n, int tid, int width, int sbk,
                                             int sbk_shift, const int* row_ks, const int* row_ke, const int* end,
                                             const int* sparse_indices, int64_t si_ld, int64_t num_k,
                                             const int* block_table, int64_t bt_ld, int bt_width, int num_reqs,
                                             const int* row_to_req, int block_size, int64_t block_stride) {
  const bool paged = block_table != nullptr;
  const int ks = row_ks[r], ke = row_ke[r], e = end[r];
  const int req = paged ? (row_to_req ? row_to_req[r] : r) : 0;
  const bool req_ok = !paged || (req >= 0 && req < num_reqs);
  for (int t = tid; t < n; t += 256) {
    const int c = c0 + t;
    uint32_t off = kSpAbsent;
    if (c < width && c < e) {
      const int tok = sparse_indices[(int64_t)r * si_ld + (c >> sbk_shift)] * sbk + (c & (sbk - 1));
      if (tok >= ks && tok < ke && tok >= 0) {
        if (!paged) {
          if (tok < num_k) off = (uint32_t)tok * (ROWB / 4);
        } else {
          const int blk = tok / block_size;
          if (req_ok && blk < bt_width) {
            const int page = block_table[(int64_t)req * bt_ld + blk];
            if (page >= 0 && page < num_k)
              off = (uint32_t)(((int64_t)page * block_stride + (int64_t)(tok % block_size) * ROWB) >> 2);
          }
        }
      }
    }
    s_off[t] = off;
  }
}

template <int JOB>
__global__ __launch_bounds__(256, 2) void sparse_logits_kernel(
    const uint8_t* __restrict__ q, const uint16_t* __restrict__ w, int rows, const int* __restrict__ row_ks,
    const int* __restrict__ row_ke, const int* __restrict__ sparse_indices, int64_t si_ld, int width,
    const int* __restrict__ end, int sbk, const uint8_t* __restrict__ k_src, int64_t num_k,
    const int* __restrict__ block_table, int64_t bt_ld, int bt_width, int num_reqs,
    const int* __restrict__ row_to_req, int block_size, int64_t block_stride, uint16_t* __restrict__ out,
    int64_t ld) {
  constexpr int NB = 2;
  constexpr int kKeysPerWave = kDcChunk / 4;
  constexpr int kGroups = kKeysPerWave / 32;
  constexpr int kStores = kKeysPerWave / 64;
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[NB][kDcBuf];
  __shared__ uint32_t s_off[JOB * kDcChunk];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool has_src = num_k > 0;
  const int sbk_shift = __builtin_ctz(sbk);
  const int nch = (width + kDcChunk - 1) / kDcChunk;
  const int kbase = wave * kKeysPerWave;

  // Score chunks [c_first, c_end) (at most JOB) of row r.
  auto run = [&](int r, int c_first, int c_end) {
    __syncthreads();  // the previous segment's buffers and offsets are no longer read
    fill_offsets<kRow>(s_off, r, c_first * kDcChunk, (c_end - c_first) * kDcChunk, tid, width, sbk, sbk_shift, row_ks,
                       row_ke, end, sparse_indices, si_ld, num_k, block_table, bt_ld, bt_width, num_reqs, row_to_req,
                       block_size, block_stride);
    Q32 qf;
    W32p wf;
    load_q32(qf, q + (int64_t)r * kHeads * kDim, lane);
    load_w32p(wf, w + (int64_t)r * kHeads, lane);
    const __amdgpu_buffer_rsrc_t out_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(out + (int64_t)r * ld, (short)0, width * 2, 0x00020000);
    __syncthreads();  // offsets visible

    auto gather = [&](int c) {
      if (has_src) sp_gather(s_buf[(c - c_first) % NB], s_off + (c - c_first) * kDcChunk, k_src, wave, lane);
    };
    auto score_chunk = [&](int c, const uint8_t* buf, int next) {
      const uint32_t* coff = s_off + (c - c_first) * kDcChunk;
#pragma unroll
      for (int h = 0; h < kGroups / 2; h++) {
        const uint8_t* keys = buf + (kbase + 64 * h) * kDcRow;
        if (h == 0 && next < c_end) gather(next);
        K32 kb;
        load_k32_raw(kb, keys, lane);
        f32x16 a0, a1, b0 = {}, b1 = {};
        float acc[4];
        dc_phase<false, true>(a0, a1, qf, kb, keys + 32 * kDcRow, lane, wf, b0, b1, acc, [](int) {});
        dc_phase<true, false>(b0, b1, qf, kb, keys, lane, wf, a0, a1, acc, [](int) {});
        const float v = combine_halves(dc_acc_sum(acc), dc_head_sum(wf, b0, b1));
        const int key = kbase + 64 * h + lane;  // key within the chunk
        const float scale = *reinterpret_cast<const float*>(buf + key * kDcRow + 140);
        const uint16_t o = coff[key] != kSpAbsent ? f32_to_bf16_rne(v * scale) : (uint16_t)0xFF80u;
        __builtin_amdgcn_raw_buffer_store_b16(o, out_rsrc, (c * kDcChunk + key) * 2, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    gather(c_first);
    for (int cc = c_first; cc < c_end; cc++) {
      // as in the decode kernel: after chunk cc's gather this wavefront issued the stores of
      // the chunk before it (when cc is not the segment's first)
      if (has_src) wait_gather<NB, kStores>(min(cc - c_first, 1));
      __syncthreads();
      score_chunk(cc, s_buf[(cc - c_first) % NB], cc + 1);
    }
  };

  const int64_t total = (int64_t)rows * nch;
  int64_t g = (int64_t)blockIdx.x * total / gridDim.x;
  const int64_t g1 = (int64_t)(blockIdx.x + 1) * total / gridDim.x;
  while (g < g1) {  // uniform
    const int r = (int)(g / nch), lc = (int)(g - (int64_t)r * nch);
    const int len = (int)min((int64_t)min(nch - lc, JOB), g1 - g);
    run(r, lc, lc + len);
    g += len;
  }
}

// ------------------------------------------------------------------ sparse columns, MXFP4 cache
// The same work split and DMA ring on 68-byte MXFP4 key rows (P1 motivation and
// implementation: the V4.1 sparse indexer scores FP8 q against an MXFP4 k cache), with the
// MXFP4 key format below.
// Five 16-byte pieces per 68-byte row: bytes 0..63 and 52..67.
__device__ __forceinline__ void mx_gather(uint8_t* buf, const uint32_t* key_off, const uint8_t* src, int wave,
                                          int lane) {
  dma_chunk<false, kMxSlabsPerWave>(buf, wave, lane, [&](int piece) {
    const int key = piece / 5, p = piece - key * 5;
    const uint32_t off = key_off[key];
    return off != kSpAbsent ? src + (int64_t)off * 4 + (p < 4 ? 16 * p : 52) : src;
  });
}

template <int JOB>
__global__ __launch_bounds__(256, 2) void sparse_logits_mx_kernel(
    const uint8_t* __restrict__ q, const uint16_t* __restrict__ w, int rows, const int* __restrict__ row_ks,
    const int* __restrict__ row_ke, const int* __restrict__ sparse_indices, int64_t si_ld, int width,
    const int* __restrict__ end, int sbk, const uint8_t* __restrict__ k_src, int64_t num_k,
    const int* __restrict__ block_table, int64_t bt_ld, int bt_width, int num_reqs,
    const int* __restrict__ row_to_req, int block_size, int64_t block_stride, uint16_t* __restrict__ out,
    int64_t ld) {
  constexpr int NB = 2;
  constexpr int kKeysPerWave = kDcChunk / 4;
  constexpr int kGroups = kKeysPerWave / 32;
  constexpr int kStores = kKeysPerWave / 64;
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[NB][kMxBuf];
  __shared__ uint32_t s_off[JOB * kDcChunk];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool has_src = num_k > 0;
  const int sbk_shift = __builtin_ctz(sbk);
  const int nch = (width + kDcChunk - 1) / kDcChunk;
  const int kbase = wave * kKeysPerWave;

  auto run = [&](int r, int c_first, int c_end) {
    __syncthreads();  // the previous segment's buffers and offsets are no longer read
    fill_offsets<kMxRow>(s_off, r, c_first * kDcChunk, (c_end - c_first) * kDcChunk, tid, width, sbk, sbk_shift,
                         row_ks, row_ke, end, sparse_indices, si_ld, num_k, block_table, bt_ld, bt_width, num_reqs,
                         row_to_req, block_size, block_stride);
    Q32b qf;
    W32p wf;
    load_q32_bf16(qf, q + (int64_t)r * kHeads * kDim, lane);
    load_w32p(wf, w + (int64_t)r * kHeads, lane);
    const __amdgpu_buffer_rsrc_t out_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(out + (int64_t)r * ld, (short)0, width * 2, 0x00020000);
    __syncthreads();  // offsets visible

    auto gather = [&](int c) {
      if (has_src) mx_gather(s_buf[(c - c_first) % NB], s_off + (c - c_first) * kDcChunk, k_src, wave, lane);
    };
    auto score_chunk = [&](int c, const uint8_t* buf, int next) {
      const uint32_t* coff = s_off + (c - c_first) * kDcChunk;
#pragma unroll
      for (int h = 0; h < kGroups / 2; h++) {
        const uint8_t* keys = buf + (kbase + 64 * h) * kMxLds;
        if (h == 0 && next < c_end) gather(next);
        K32b kb;
        const MxRaw r0 = load_mx_raw(keys, lane);
#pragma unroll
        for (int j = 0; j < 4; j++) decode_mx_pair(kb, r0, j);
        f32x16 a0, a1, b0 = {}, b1 = {};
        float acc[4];
        mx_phase<false, true>(a0, a1, qf, kb, keys + 32 * kMxLds, lane, wf, b0, b1, acc, [](int) {});
        mx_phase<true, false>(b0, b1, qf, kb, keys, lane, wf, a0, a1, acc, [](int) {});
        const float v = combine_halves(dc_acc_sum(acc), dc_head_sum(wf, b0, b1));
        const int key = kbase + 64 * h + lane;  // key within the chunk
        const uint16_t o = coff[key] != kSpAbsent ? f32_to_bf16_rne(v) : (uint16_t)0xFF80u;
        __builtin_amdgcn_raw_buffer_store_b16(o, out_rsrc, (c * kDcChunk + key) * 2, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    gather(c_first);
    for (int cc = c_first; cc < c_end; cc++) {
      if (has_src) wait_gather<NB, kStores>(min(cc - c_first, 1));
      __syncthreads();
      score_chunk(cc, s_buf[(cc - c_first) % NB], cc + 1);
    }
  };

  const int64_t total = (int64_t)rows * nch;
  int64_t g = (int64_t)blockIdx.x * total / gridDim.x;
  const int64_t g1 = (int64_t)(blockIdx.x + 1) * total / gridDim.x;
  while (g < g1) {  // uniform
    const int r = (int)(g / nch), lc = (int)(g - (int64_t)r * nch);
    const int len = (int)min((int64_t)min(nch - lc, JOB), g1 - g);
    run(r, lc, lc + len);
    g += len;
  }
}

// The sparse kernels with a per-step schedule (FP8 or MXFP4 key rows): the columns' sources
// follow from one entry per sparse block, so a segment stages its blocks' entries (at most
// kSgBlk) instead of a source offset per column, and runs up to a whole 8192-column row
// (kSgJob chunks; min(kSgJob, sbk) keeps the entries within kSgBlk).  The columns' offsets are
// derived one chunk at a time into a ring of three chunks: chunk c is scored while chunk c+1's
// gather is in flight and chunk c+2's offsets are written.  A segment's set-up (the entries, q
// and the first gather) is then paid once per row share rather than once per eight chunks.
constexpr int kSgJob = 32;
constexpr int kSgBlk = 256;

template <bool MX>
__global__ __launch_bounds__(256, 2) void sparse_logits_sched_kernel(
    const uint8_t* __restrict__ q, const uint16_t* __restrict__ w, int rows, int width, int sbk,
    const uint8_t* __restrict__ k_src, int64_t has_src_rows, uint16_t* __restrict__ out, int64_t ld,
    const unsigned long long* __restrict__ sched, int64_t src_bytes) {
  constexpr int NB = 2;
  constexpr int kKeysPerWave = kDcChunk / 4;
  constexpr int kGroups = kKeysPerWave / 32;
  constexpr int kStores = kKeysPerWave / 64;
  constexpr int kRowBytes = MX ? kMxRow : kRow;
  constexpr int kLdsRowBytes = MX ? kMxLds : kDcRow;
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[NB][MX ? kMxBuf : kDcBuf];
  __shared__ uint32_t s_off[3][kDcChunk];       // source offsets (4-byte units) of chunks c % 3
  __shared__ unsigned long long s_blk[kSgBlk];  // the segment's schedule entries

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool has_src = has_src_rows > 0;
  const int sbk_shift = __builtin_ctz(sbk);
  const int nch = (width + kDcChunk - 1) / kDcChunk;
  const int nsb = width >> sbk_shift;  // entries per row (the width is a whole number of blocks)
  const int job = min(kSgJob, sbk);    // chunks per segment: job * 256 / sbk <= kSgBlk entries
  const int kbase = wave * kKeysPerWave;

  // Offsets of chunk c's columns, one per thread, from the entries staged from block blk0 on.
  auto fill = [&](int c, int blk0) {
    const int col = c * kDcChunk + tid;
    uint32_t off = kSpAbsent;
    if (col < width) {
      const unsigned long long e = s_blk[(col >> sbk_shift) - blk0];
      const uint32_t base = (uint32_t)e, lo = (uint32_t)(e >> 32) & 0xFFu, hi = (uint32_t)(e >> 40) & 0xFFu;
      const uint32_t o = (uint32_t)(col & (sbk - 1));
      if (base != kSpAbsent && o >= lo && o < hi) {
        const uint32_t x = base + o * (kRowBytes / 4);
        if ((uint64_t)x * 4 + kRowBytes <= (uint64_t)src_bytes) off = x;
      }
    }
    s_off[c % 3][tid] = off;
  };

  // Score chunks [c_first, c_end) (at most job) of row r.
  auto run = [&](int r, int c_first, int c_end) {
    __syncthreads();  // the previous segment's buffers, offsets and entries are no longer read
    const int blk0 = (c_first * kDcChunk) >> sbk_shift;
    const int nblk = min(nsb, (c_end * kDcChunk) >> sbk_shift) - blk0;
    const unsigned long long* srow = sched + (int64_t)r * nsb + blk0;
    for (int i = tid; i < nblk; i += 256) s_blk[i] = srow[i];
    typename std::conditional<MX, Q32b, Q32>::type qf;
    W32p wf;
    if constexpr (MX)
      load_q32_bf16(qf, q + (int64_t)r * kHeads * kDim, lane);
    else
      load_q32(qf, q + (int64_t)r * kHeads * kDim, lane);
    load_w32p(wf, w + (int64_t)r * kHeads, lane);
    const __amdgpu_buffer_rsrc_t out_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(out + (int64_t)r * ld, (short)0, width * 2, 0x00020000);
    __syncthreads();  // entries visible
    fill(c_first, blk0);
    if (c_first + 1 < c_end) fill(c_first + 1, blk0);
    __syncthreads();  // the first two chunks' offsets visible

    auto gather = [&](int c) {
      if (!has_src) return;
      if constexpr (MX)
        mx_gather(s_buf[(c - c_first) % NB], s_off[c % 3], k_src, wave, lane);
      else
        sp_gather(s_buf[(c - c_first) % NB], s_off[c % 3], k_src, wave, lane);
    };
    auto score_chunk = [&](int c, const uint8_t* buf) {
      const uint32_t* coff = s_off[c % 3];
#pragma unroll
      for (int h = 0; h < kGroups / 2; h++) {
        const uint8_t* keys = buf + (kbase + 64 * h) * kLdsRowBytes;
        if (h == 0) {
          if (c + 1 < c_end) gather(c + 1);
          if (c + 2 < c_end) fill(c + 2, blk0);  // chunk c-1's slot: read by nothing after the last barrier
        }
        f32x16 a0, a1, b0 = {}, b1 = {};
        float acc[4];
        float v;
        if constexpr (MX) {
          K32b kb;
          const MxRaw r0 = load_mx_raw(keys, lane);
#pragma unroll
          for (int j = 0; j < 4; j++) decode_mx_pair(kb, r0, j);
          mx_phase<false, true>(a0, a1, qf, kb, keys + 32 * kLdsRowBytes, lane, wf, b0, b1, acc, [](int) {});
          mx_phase<true, false>(b0, b1, qf, kb, keys, lane, wf, a0, a1, acc, [](int) {});
          v = combine_halves(dc_acc_sum(acc), dc_head_sum(wf, b0, b1));
        } else {
          K32 kb;
          load_k32_raw(kb, keys, lane);
          dc_phase<false, true>(a0, a1, qf, kb, keys + 32 * kLdsRowBytes, lane, wf, b0, b1, acc, [](int) {});
          dc_phase<true, false>(b0, b1, qf, kb, keys, lane, wf, a0, a1, acc, [](int) {});
          v = combine_halves(dc_acc_sum(acc), dc_head_sum(wf, b0, b1));
        }
        const int key = kbase + 64 * h + lane;  // key within the chunk
        if constexpr (!MX) v *= *reinterpret_cast<const float*>(buf + key * kDcRow + 140);  // the row's scale
        const uint16_t o = coff[key] != kSpAbsent ? f32_to_bf16_rne(v) : (uint16_t)0xFF80u;
        __builtin_amdgcn_raw_buffer_store_b16(o, out_rsrc, (c * kDcChunk + key) * 2, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    gather(c_first);
    for (int cc = c_first; cc < c_end; cc++) {
      // as in the decode kernel: after chunk cc's gather this wavefront issued the stores of
      // the chunk before it (when cc is not the segment's first)
      if (has_src) wait_gather<NB, kStores>(min(cc - c_first, 1));
      __syncthreads();
      score_chunk(cc, s_buf[(cc - c_first) % NB]);
    }
  };

  const int64_t total = (int64_t)rows * nch;
  int64_t g = (int64_t)blockIdx.x * total / gridDim.x;
  const int64_t g1 = (int64_t)(blockIdx.x + 1) * total / gridDim.x;
  while (g < g1) {  // uniform
    const int r = (int)(g / nch), lc = (int)(g - (int64_t)r * nch);
    const int len = (int)min((int64_t)min(nch - lc, job), g1 - g);
    run(r, lc, lc + len);
    g += len;
  }
}

// ------------------------------------------------------------------ per-step schedule of the sparse columns
// One entry per (row, sparse block j): tokens tok0 + o, o < sbk, with tok0 = sparse_indices[r][j]*sbk, lie in one
// page (the page size is a multiple of sbk) or in one run of gathered rows, so column j*sbk + o reads
// base + o*ROWB/4 (4-byte units).  Its columns are valid for o in [lo, hi): c < end, ks <= tok < ke, tok >= 0, and
// the token's row is in the source (gathered: tok < num_k; paged: the request, block index and page id are in
// range).  An entry packs base | lo << 32 | hi << 40, or kSpAbsent with lo = hi = 0 when no column is valid.
__global__ __launch_bounds__(256) void sparse_schedule_kernel(
    int rows, const int* __restrict__ row_ks, const int* __restrict__ row_ke, const int* __restrict__ sparse_indices,
    int64_t si_ld, int nsb, const int* __restrict__ end, int sbk, int row_bytes, int64_t num_k,
    const int* __restrict__ block_table, int64_t bt_ld, int bt_width, int num_reqs, const int* __restrict__ row_to_req,
    int block_size, int64_t block_stride, unsigned long long* __restrict__ sched) {
  const int r = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows || j >= nsb) return;
  const int64_t tok0 = (int64_t)sparse_indices[(int64_t)r * si_ld + j] * sbk;
  const int64_t lo = std::min<int64_t>(std::max<int64_t>(std::max(row_ks[r], 0) - tok0, 0), sbk);
  int64_t hi = std::min<int64_t>((int64_t)row_ke[r] - tok0, (int64_t)end[r] - (int64_t)j * sbk);
  hi = std::max<int64_t>(std::min<int64_t>(hi, sbk), 0);
  int64_t base = -1;
  if (block_table == nullptr) {
    hi = std::max<int64_t>(std::min<int64_t>(hi, num_k - tok0), 0);
    if (lo < hi) base = tok0 * row_bytes;
  } else if (lo < hi) {  // then tok0 >= 0
    const int req = row_to_req ? row_to_req[r] : r;
    const int64_t blk = tok0 / block_size;
    if (req >= 0 && req < num_reqs && blk < bt_width) {
      const int page = block_table[(int64_t)req * bt_ld + blk];
      if (page >= 0 && page < num_k) base = (int64_t)page * block_stride + (tok0 % block_size) * row_bytes;
    }
  }
  sched[(int64_t)r * nsb + j] = (base >= 0 && lo < hi)
                                    ? ((uint64_t)(base >> 2) | ((uint64_t)lo << 32) | ((uint64_t)hi << 40))
                                    : (uint64_t)kSpAbsent;
}

}  // namespace
}  // namespace dsi

namespace dsi {
namespace {

// Checks shared by both cache formats and by the fused top-k calls.
template <bool MX>
int paged_decode_check(const uint8_t* q, const uint16_t* w, int32_t B, int32_t next_n, const int32_t* context_lens,
                       const uint8_t* pool, int64_t num_blocks, int32_t block_size, int64_t block_stride_bytes,
                       const int32_t* block_table, int64_t bt_ld, int32_t bt_width, int32_t max_context_len,
                       float* logits, int64_t ld) {
  if (B < 0 || max_context_len < 0 || ld < max_context_len || num_blocks < 0 || bt_width < 0 || bt_ld < bt_width)
    return DSI_EINVAL;
  if (next_n < 1 || next_n > 4 || block_size < 16 || (block_size % 16) != 0) return DSI_EUNSUPPORTED;
  if (block_stride_bytes < (int64_t)block_size * (MX ? kMxRow : kRow)) return DSI_EINVAL;
  if (B == 0 || max_context_len == 0) return DSI_OK;
  if (!q || !w || !context_lens || !pool || !block_table || !logits) return DSI_EINVAL;
  if (B > 65535) return DSI_EUNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(pool) & 15) ||
      (block_stride_bytes & 15) || (reinterpret_cast<uintptr_t>(w) & 7) || (reinterpret_cast<uintptr_t>(logits) & 3))
    return DSI_EALIGN;
  return DSI_OK;
}

// Persistent shares pay off where scoring a chunk is cheap (one row per request: the tail of
// unequal jobs dominated); with two or more rows per request the per-request grid measured
// faster.
bool dc_persistent(int B, int next_n) { return B <= kDcMaxReqs && next_n == 1; }

// Persistent grid: two workgroups per CU, and enough that no share exceeds 255 chunks (the
// histogram slots count in 16 bits).
int64_t dc_grid(int B, int64_t max_chunks) {
  const int64_t all = max_chunks * B;
  return std::max<int64_t>(1, std::max(std::min<int64_t>(2 * (int64_t)cu_count(), all), (all + 254) / 255));
}

// Slots the fused call provides: an upper bound of the persistent grid for any device of up to
// 512 CUs, plus one per request (a workgroup's slots are blockIdx.x + request).
int64_t dc_num_slots(int B, int64_t max_chunks) {
  return std::max<int64_t>(1024, (max_chunks * B + 254) / 255) + B;
}

// The fused call counts the histograms in the decode kernel when the top-k takes the split path
// and the decode kernel the persistent one.
bool dc_fused(int B, int next_n, int max_ctx) {
  return dc_persistent(B, next_n) && split_groups_f32(B * next_n, max_ctx) > 1;
}

template <bool MX, bool HIST>
int launch_paged_decode(const uint8_t* q, const uint16_t* w, int32_t B, int32_t next_n, const int32_t* context_lens,
                        const uint8_t* pool, int64_t num_blocks, int32_t block_size, int64_t block_stride_bytes,
                        const int32_t* block_table, int64_t bt_ld, int32_t bt_width, int32_t max_context_len,
                        float* logits, int64_t ld, void* ws, int64_t num_slots, hipStream_t stream) {
  const int64_t max_chunks = (max_context_len + kDcChunk - 1) / kDcChunk;
  const bool persistent = dc_persistent(B, next_n);
  dim3 grid;
  if (persistent) {
    int64_t g = dc_grid(B, max_chunks);
    if (HIST) g = std::min<int64_t>(g, num_slots - B);  // the slots bound the grid (never below the 255-chunk floor)
    grid = dim3((unsigned)g);
  } else {
    grid = dim3((unsigned)((max_chunks + kDcJob - 1) / kDcJob), (unsigned)B);
  }
  const int wpr = next_n == 1 ? 4 : next_n == 2 ? 2 : 1;
  constexpr int kNB = 2;
  if constexpr (HIST) {
    hipLaunchKernelGGL((paged_decode_kernel<4, kNB, MX, true>), grid, dim3(256), 0, stream, q, w, B, next_n,
                       context_lens, pool, num_blocks, block_size, block_stride_bytes, block_table, bt_ld, bt_width,
                       max_context_len, logits, ld, 1, ws, num_slots);
  } else {
    auto k = wpr == 4 ? paged_decode_kernel<4, kNB, MX, false>
             : wpr == 2 ? paged_decode_kernel<2, kNB, MX, false> : paged_decode_kernel<1, kNB, MX, false>;
    hipLaunchKernelGGL(k, grid, dim3(256), 0, stream, q, w, B, next_n, context_lens, pool, num_blocks, block_size,
                       block_stride_bytes, block_table, bt_ld, bt_width, max_context_len, logits, ld,
                       (int)persistent, nullptr, (int64_t)0);
  }
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}

template <bool MX>
int paged_decode(const uint8_t* q, const uint16_t* w, int32_t B, int32_t next_n, const int32_t* context_lens,
                 const uint8_t* pool, int64_t num_blocks, int32_t block_size, int64_t block_stride_bytes,
                 const int32_t* block_table, int64_t bt_ld, int32_t bt_width, int32_t max_context_len, float* logits,
                 int64_t ld, hipStream_t stream) {
  const int st = paged_decode_check<MX>(q, w, B, next_n, context_lens, pool, num_blocks, block_size,
                                        block_stride_bytes, block_table, bt_ld, bt_width, max_context_len, logits, ld);
  if (st != DSI_OK || B == 0 || max_context_len == 0) return st;
  return launch_paged_decode<MX, false>(q, w, B, next_n, context_lens, pool, num_blocks, block_size,
                                        block_stride_bytes, block_table, bt_ld, bt_width, max_context_len, logits, ld,
                                        nullptr, 0, stream);
}

size_t paged_topk_ws_bytes(int32_t B, int32_t next_n, int32_t max_context_len, int32_t k) {
  if (B <= 0 || next_n < 1 || max_context_len <= 0) return 0;
  if (dc_fused(B, next_n, max_context_len))
    return split_ws_bytes((int64_t)B * next_n, dc_num_slots(B, (max_context_len + kDcChunk - 1) / kDcChunk));
  return dsi_topk_workspace_bytes(B * next_n, max_context_len, k);
}

// Decode logits and their top-k in one call: the decode kernel counts the split top-k's
// histograms while it writes the logits (when both take those paths), else the plain decode
// kernel and the top-k of dsi_topk_select, with the rows' ranges taken from the lengths.
template <bool MX>
int paged_topk_decode(const uint8_t* q, const uint16_t* w, int32_t B, int32_t next_n, const int32_t* context_lens,
                      const uint8_t* pool, int64_t num_blocks, int32_t block_size, int64_t block_stride_bytes,
                      const int32_t* block_table, int64_t bt_ld, int32_t bt_width, int32_t max_context_len,
                      float* logits, int64_t ld, int32_t k, int32_t* out, int64_t out_ld, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  const int st = paged_decode_check<MX>(q, w, B, next_n, context_lens, pool, num_blocks, block_size,
                                        block_stride_bytes, block_table, bt_ld, bt_width, max_context_len, logits, ld);
  if (st != DSI_OK) return st;
  if (k < 1 || k > DSI_MAX_TOPK) return DSI_EUNSUPPORTED;
  if (out_ld < k) return DSI_EINVAL;
  const size_t need = paged_topk_ws_bytes(B, next_n, max_context_len, k);
  if (ws_bytes < need || (need && !ws)) return DSI_EWORKSPACE;
  if (B == 0) return DSI_OK;
  if (!out || !context_lens) return DSI_EINVAL;
  if ((reinterpret_cast<uintptr_t>(out) & 3) || (reinterpret_cast<uintptr_t>(ws) & 15)) return DSI_EALIGN;
  const int rows = B * next_n;
  const RowRange range{nullptr, nullptr, context_lens, next_n, max_context_len};
  if (dc_fused(B, next_n, max_context_len)) {
    const int64_t slots = dc_num_slots(B, (max_context_len + kDcChunk - 1) / kDcChunk);
    const int r = launch_paged_decode<MX, true>(q, w, B, next_n, context_lens, pool, num_blocks, block_size,
                                                block_stride_bytes, block_table, bt_ld, bt_width, max_context_len,
                                                logits, ld, ws, slots, stream);
    if (r != DSI_OK) return r;
    return launch_split_select(logits, ld, rows, range, k, out, out_ld, ws, slots,
                               split_groups_f32(rows, max_context_len), stream);
  }
  if (max_context_len > 0) {
    const int r = launch_paged_decode<MX, false>(q, w, B, next_n, context_lens, pool, num_blocks, block_size,
                                                 block_stride_bytes, block_table, bt_ld, bt_width, max_context_len,
                                                 logits, ld, nullptr, 0, stream);
    if (r != DSI_OK) return r;
  }
  return topk_dispatch(logits, false, ld, rows, range, max_context_len, k, out, out_ld, ws, stream);
}

}  // namespace
}  // namespace dsi

extern "C" int dsi_paged_mqa_logits_decode(const uint8_t* q, const uint16_t* w, int32_t B, int32_t next_n,
                                           const int32_t* context_lens, const uint8_t* pool, int64_t num_blocks,
                                           int32_t block_size, int64_t block_stride_bytes,
                                           const int32_t* block_table, int64_t bt_ld, int32_t bt_width,
                                           int32_t max_context_len, float* logits, int64_t ld, hipStream_t stream) {
  return dsi::paged_decode<false>(q, w, B, next_n, context_lens, pool, num_blocks, block_size, block_stride_bytes,
                                  block_table, bt_ld, bt_width, max_context_len, logits, ld, stream);
}

extern "C" int dsi_paged_mqa_logits_decode_mxfp4(const uint8_t* q, const uint16_t* w, int32_t B, int32_t next_n,
                                                 const int32_t* context_lens, const uint8_t* pool,
                                                 int64_t num_blocks, int32_t block_size, int64_t block_stride_bytes,
                                                 const int32_t* block_table, int64_t bt_ld, int32_t bt_width,
                                                 int32_t max_context_len, float* logits, int64_t ld,
                                                 hipStream_t stream) {
  return dsi::paged_decode<true>(q, w, B, next_n, context_lens, pool, num_blocks, block_size, block_stride_bytes,
                                 block_table, bt_ld, bt_width, max_context_len, logits, ld, stream);
}

extern "C" size_t dsi_paged_mqa_topk_decode_workspace_bytes(int32_t B, int32_t next_n, int32_t max_context_len,
                                                            int32_t k) {
  return dsi::paged_topk_ws_bytes(B, next_n, max_context_len, k);
}

extern "C" int dsi_paged_mqa_topk_decode(const uint8_t* q, const uint16_t* w, int32_t B, int32_t next_n,
                                         const int32_t* context_lens, const uint8_t* pool, int64_t num_blocks,
                                         int32_t block_size, int64_t block_stride_bytes, const int32_t* block_table,
                                         int64_t bt_ld, int32_t bt_width, int32_t max_context_len, float* logits,
                                         int64_t ld, int32_t k, int32_t* out, int64_t out_ld, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  return dsi::paged_topk_decode<false>(q, w, B, next_n, context_lens, pool, num_blocks, block_size, block_stride_bytes,
                                       block_table, bt_ld, bt_width, max_context_len, logits, ld, k, out, out_ld,
                                       workspace, workspace_bytes, stream);
}

extern "C" int dsi_paged_mqa_topk_decode_mxfp4(const uint8_t* q, const uint16_t* w, int32_t B, int32_t next_n,
                                               const int32_t* context_lens, const uint8_t* pool, int64_t num_blocks,
                                               int32_t block_size, int64_t block_stride_bytes,
                                               const int32_t* block_table, int64_t bt_ld, int32_t bt_width,
                                               int32_t max_context_len, float* logits, int64_t ld, int32_t k,
                                               int32_t* out, int64_t out_ld, void* workspace, size_t workspace_bytes,
                                               hipStream_t stream) {
  return dsi::paged_topk_decode<true>(q, w, B, next_n, context_lens, pool, num_blocks, block_size, block_stride_bytes,
                                      block_table, bt_ld, bt_width, max_context_len, logits, ld, k, out, out_ld,
                                      workspace, workspace_bytes, stream);
}

extern "C" int dsi_sparse_mqa_logits(const uint8_t* q, const uint16_t* w, int32_t rows, const int32_t* row_ks,
                                     const int32_t* row_ke, const int32_t* sparse_indices, int64_t si_ld,
                                     int32_t num_sparse_blocks, const int32_t* end, int32_t sparse_block_kv,
                                     const uint8_t* k_src, int64_t num_k, const int32_t* block_table, int64_t bt_ld,
                                     int32_t bt_width, int32_t num_reqs, const int32_t* row_to_req,
                                     int32_t block_size, int64_t block_stride_bytes, uint16_t* logits_bf16,
                                     int64_t ld, hipStream_t stream) {
  using namespace dsi;
  const int sbk = sparse_block_kv;
  if (sbk < 8 || sbk > 128 || (sbk & (sbk - 1))) return DSI_EUNSUPPORTED;
  if (rows < 0 || num_sparse_blocks < 1 || si_ld < num_sparse_blocks || num_k < 0) return DSI_EINVAL;
  const int64_t width = (int64_t)num_sparse_blocks * sbk;
  if (width > 0x7FFFFFFF || ld < width) return DSI_EINVAL;
  const bool paged = block_table != nullptr;
  if (paged) {
    if (bt_width < 0 || bt_ld < bt_width || num_reqs < 0) return DSI_EINVAL;
    if (block_size < 8 || (block_size % sbk) != 0 || (block_size % 8) != 0) return DSI_EUNSUPPORTED;
    if (block_stride_bytes < (int64_t)block_size * kRow) return DSI_EINVAL;
    if (block_stride_bytes & 15) return DSI_EALIGN;
  }
  if (rows == 0) return DSI_OK;
  if (!q || !w || !row_ks || !row_ke || !sparse_indices || !end || !k_src || !logits_bf16) return DSI_EINVAL;
  if ((reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(k_src) & 15) ||
      (reinterpret_cast<uintptr_t>(w) & 7) || (reinterpret_cast<uintptr_t>(logits_bf16) & 1))
    return DSI_EALIGN;
  if (rows > 65535) return DSI_EUNSUPPORTED;
  // source offsets are kept in 4-byte units in 32 bits
  const int64_t src_bytes = paged ? num_k * block_stride_bytes : num_k * kRow;
  if (src_bytes >= ((int64_t)1 << 34)) return DSI_EUNSUPPORTED;
  const int64_t nch = (width + kDcChunk - 1) / kDcChunk;
  const int64_t slots = 2 * (int64_t)cu_count();
  const dim3 grid((unsigned)std::max<int64_t>(1, std::min<int64_t>(slots, nch * rows)));
  hipLaunchKernelGGL((sparse_logits_kernel<kSpJob>), grid, dim3(256), 0, stream, q, w, rows, row_ks, row_ke,
                     sparse_indices, si_ld, (int)width, end, sbk, k_src, num_k, block_table, bt_ld, bt_width, num_reqs,
                     row_to_req, block_size, block_stride_bytes, logits_bf16, ld);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}

extern "C" int dsi_sparse_mqa_logits_mxfp4(const uint8_t* q, const uint16_t* w, int32_t rows, const int32_t* row_ks,
                                           const int32_t* row_ke, const int32_t* sparse_indices, int64_t si_ld,
                                           int32_t num_sparse_blocks, const int32_t* end, int32_t sparse_block_kv,
                                           const uint8_t* k_src, int64_t num_k, const int32_t* block_table,
                                           int64_t bt_ld, int32_t bt_width, int32_t num_reqs,
                                           const int32_t* row_to_req, int32_t block_size, int64_t block_stride_bytes,
                                           uint16_t* logits_bf16, int64_t ld, hipStream_t stream) {
  using namespace dsi;
  const int sbk = sparse_block_kv;
  if (sbk < 8 || sbk > 128 || (sbk & (sbk - 1))) return DSI_EUNSUPPORTED;
  if (rows < 0 || num_sparse_blocks < 1 || si_ld < num_sparse_blocks || num_k < 0) return DSI_EINVAL;
  const int64_t width = (int64_t)num_sparse_blocks * sbk;
  if (width > 0x7FFFFFFF || ld < width) return DSI_EINVAL;
  const bool paged = block_table != nullptr;
  if (paged) {
    if (bt_width < 0 || bt_ld < bt_width || num_reqs < 0) return DSI_EINVAL;
    if (block_size < 8 || (block_size % sbk) != 0 || (block_size % 8) != 0) return DSI_EUNSUPPORTED;
    if (block_stride_bytes < (int64_t)block_size * kMxRow) return DSI_EINVAL;
    if (block_stride_bytes & 15) return DSI_EALIGN;
  }
  if (rows == 0) return DSI_OK;
  if (!q || !w || !row_ks || !row_ke || !sparse_indices || !end || !k_src || !logits_bf16) return DSI_EINVAL;
  if ((reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(k_src) & 15) ||
      (reinterpret_cast<uintptr_t>(w) & 7) || (reinterpret_cast<uintptr_t>(logits_bf16) & 1))
    return DSI_EALIGN;
  if (rows > 65535) return DSI_EUNSUPPORTED;
  const int64_t src_bytes = paged ? num_k * block_stride_bytes : num_k * kMxRow;
  if (src_bytes >= ((int64_t)1 << 34)) return DSI_EUNSUPPORTED;
  const int64_t nch = (width + kDcChunk - 1) / kDcChunk;
  const int64_t slots = 2 * (int64_t)cu_count();
  const dim3 grid((unsigned)std::max<int64_t>(1, std::min<int64_t>(slots, nch * rows)));
  hipLaunchKernelGGL((sparse_logits_mx_kernel<kMxJob>), grid, dim3(256), 0, stream, q, w, rows, row_ks, row_ke,
                     sparse_indices, si_ld, (int)width, end, sbk, k_src, num_k, block_table, bt_ld, bt_width, num_reqs,
                     row_to_req, block_size, block_stride_bytes, logits_bf16, ld);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}

extern "C" size_t dsi_sparse_schedule_bytes(int32_t rows, int32_t num_sparse_blocks) {
  return rows > 0 && num_sparse_blocks > 0 ? (size_t)rows * num_sparse_blocks * 8 : 0;
}

extern "C" int dsi_sparse_schedule(int32_t rows, const int32_t* row_ks, const int32_t* row_ke,
                                   const int32_t* sparse_indices, int64_t si_ld, int32_t num_sparse_blocks,
                                   const int32_t* end, int32_t sparse_block_kv, int32_t row_bytes, int64_t num_k,
                                   const int32_t* block_table, int64_t bt_ld, int32_t bt_width, int32_t num_reqs,
                                   const int32_t* row_to_req, int32_t block_size, int64_t block_stride_bytes,
                                   uint64_t* schedule, hipStream_t stream) {
  using namespace dsi;
  const int sbk = sparse_block_kv;
  if (sbk < 8 || sbk > 128 || (sbk & (sbk - 1))) return DSI_EUNSUPPORTED;
  if (row_bytes != kRow && row_bytes != kMxRow) return DSI_EUNSUPPORTED;
  if (rows < 0 || num_sparse_blocks < 1 || si_ld < num_sparse_blocks || num_k < 0) return DSI_EINVAL;
  const bool paged = block_table != nullptr;
  if (paged) {
    if (bt_width < 0 || bt_ld < bt_width || num_reqs < 0) return DSI_EINVAL;
    if (block_size < 8 || (block_size % sbk) != 0 || (block_size % 8) != 0) return DSI_EUNSUPPORTED;
    if (block_stride_bytes < (int64_t)block_size * row_bytes) return DSI_EINVAL;
    if (block_stride_bytes & 15) return DSI_EALIGN;
  }
  if (rows == 0) return DSI_OK;
  if (!row_ks || !row_ke || !sparse_indices || !end || !schedule) return DSI_EINVAL;
  if (reinterpret_cast<uintptr_t>(schedule) & 7) return DSI_EALIGN;
  if (rows > 65535) return DSI_EUNSUPPORTED;
  const int64_t src_bytes = paged ? num_k * block_stride_bytes : num_k * row_bytes;
  if (src_bytes >= ((int64_t)1 << 34)) return DSI_EUNSUPPORTED;  // offsets are kept in 4-byte units in 32 bits
  const dim3 grid((unsigned)((num_sparse_blocks + 255) / 256), (unsigned)rows);
  hipLaunchKernelGGL(sparse_schedule_kernel, grid, dim3(256), 0, stream, rows, row_ks, row_ke, sparse_indices, si_ld,
                     num_sparse_blocks, end, sbk, row_bytes, num_k, block_table, bt_ld, bt_width, num_reqs,
                     row_to_req, block_size, block_stride_bytes, reinterpret_cast<unsigned long long*>(schedule));
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}

namespace dsi {
namespace {

template <bool MX>
int sparse_scheduled(const uint8_t* q, const uint16_t* w, int32_t rows, const uint64_t* schedule,
                     int32_t num_sparse_blocks, int32_t sparse_block_kv, const uint8_t* k_src, int64_t k_src_bytes,
                     uint16_t* logits_bf16, int64_t ld, hipStream_t stream) {
  const int sbk = sparse_block_kv;
  if (sbk < 8 || sbk > 128 || (sbk & (sbk - 1))) return DSI_EUNSUPPORTED;
  if (rows < 0 || num_sparse_blocks < 1 || k_src_bytes < 0) return DSI_EINVAL;
  const int64_t width = (int64_t)num_sparse_blocks * sbk;
  if (width > 0x7FFFFFFF || ld < width) return DSI_EINVAL;
  if (rows == 0) return DSI_OK;
  if (!q || !w || !schedule || !logits_bf16 || (!k_src && k_src_bytes > 0)) return DSI_EINVAL;
  if ((reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(k_src) & 15) ||
      (reinterpret_cast<uintptr_t>(w) & 7) || (reinterpret_cast<uintptr_t>(logits_bf16) & 1) ||
      (reinterpret_cast<uintptr_t>(schedule) & 7))
    return DSI_EALIGN;
  if (rows > 65535) return DSI_EUNSUPPORTED;
  if (k_src_bytes >= ((int64_t)1 << 34)) return DSI_EUNSUPPORTED;
  const int64_t nch = (width + kDcChunk - 1) / kDcChunk;
  const int64_t slots = 2 * (int64_t)cu_count();
  const dim3 grid((unsigned)std::max<int64_t>(1, std::min<int64_t>(slots, nch * rows)));
  const int64_t has_src = k_src_bytes > 0 ? 1 : 0;  // the kernels gather only when the source has rows
  const unsigned long long* sched = reinterpret_cast<const unsigned long long*>(schedule);
  hipLaunchKernelGGL(sparse_logits_sched_kernel<MX>, grid, dim3(256), 0, stream, q, w, rows, (int)width, sbk, k_src,
                     has_src, logits_bf16, ld, sched, k_src_bytes);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}

}  // namespace
}  // namespace dsi

extern "C" int dsi_sparse_mqa_logits_scheduled(const uint8_t* q, const uint16_t* w, int32_t rows,
                                               const uint64_t* schedule, int32_t num_sparse_blocks,
                                               int32_t sparse_block_kv, const uint8_t* k_src, int64_t k_src_bytes,
                                               uint16_t* logits_bf16, int64_t ld, hipStream_t stream) {
  return dsi::sparse_scheduled<false>(q, w, rows, schedule, num_sparse_blocks, sparse_block_kv, k_src, k_src_bytes,
                                      logits_bf16, ld, stream);
}

extern "C" int dsi_sparse_mqa_logits_scheduled_mxfp4(const uint8_t* q, const uint16_t* w, int32_t rows,
                                                     const uint64_t* schedule, int32_t num_sparse_blocks,
                                                     int32_t sparse_block_kv, const uint8_t* k_src,
                                                     int64_t k_src_bytes, uint16_t* logits_bf16, int64_t ld,
                                                     hipStream_t stream) {
  return dsi::sparse_scheduled<true>(q, w, rows, schedule, num_sparse_blocks, sparse_block_kv, k_src, k_src_bytes,
                                     logits_bf16, ld, stream);
}
