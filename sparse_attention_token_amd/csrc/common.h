// Device helpers shared by the gfx950 indexer kernels.
//
// Scoring layout (used by every logits kernel).  The indexer score of P3 step ⑥
// ("DeepSeek V3.2 稀疏注意力 DSA 推理流程图解") is a 64-head x 128-dim contraction of
// FP8 values followed by a per-head weighted sum.
//
// Matrix instruction.  The FP8 codes are decoded exactly to f16 and contracted with
// v_mfma_f32_16x16x32_f16.  gfx950's FP8-operand MFMAs (16x16x128 f8f6f4 and
// 16x16x32 fp8) were measured to drop product bits about 13 binades below the largest
// product of their internal sum, with a one-sided (truncating) error that reaches
// ~0.1 on indexer logits — beyond the path's 1e-3 (1 + |ref|) bar — while the f16
// MFMA sums the same products exactly.  Every E4M3FN value is a normal f16 (2^-9 to
// 448), so the decode (v_cvt_scalef32_pk_f16_fp8 with scale 1, two codes per
// instruction) is exact.
//
// Operands of one MFMA (k = 32 dims of a 128-dim slice):
//   A = 16 heads x 32 dims of q   (lane l: head l%16, 8 dims of lane group g = l/16)
//   B = 32 dims x 16 keys of K    (lane l: key  l%16, the same 8 dims)
//   C = 16 heads x 16 keys, lane l holds heads 4*(l/16)+i, i<4, of key l%16.
// Lane group g owns dims [32g, 32g+32) of the 128 and feeds 8 of them to each of the
// four slices; A and B use the same assignment, so the sum over dims is complete.
// Four head tiles cover the 64 heads, so after the MFMAs each lane holds 16 heads of
// one key; the head-weighted sum is 16 FMAs per lane followed by a sum over the four
// lane groups.  That cross-lane sum is done for four (row, key-group) outputs at once
// as a 4x4 transpose-reduce: two exchange stages (lane^32, lane^16), after which each
// lane group owns one output.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsi.h"

namespace dsi {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kHeads = 64;
constexpr int kDim = 128;
constexpr int kRow = 132;              // bytes per cache row
constexpr int kLdsKeyStride = 144;     // LDS bytes per FP8 key row: 128 codes + pad; 36 dwords = 4 mod 32
                                       // banks, so 16-byte reads by 8 consecutive keys are conflict-free
constexpr int kLdsKeyStrideF16 = 272;  // LDS bytes per f16 key row: 256 + pad, 68 dwords = 4 mod 32 banks

__device__ __forceinline__ f32x4 mfma_f16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round-to-nearest-even fp32 -> bf16 on the bit pattern (finite or inf).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// fp32 -> OCP E4M3FN code: round to nearest even, saturate to +-448, keep the
// sign of the input (also for results that round to zero).  Derived from the
// format: a normal e4m3 value keeps 3 of the 23 fp32 mantissa bits and has a
// biased exponent 120 below fp32's; below 2^-6 the format is the grid m*2^-9.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // |x| >= 448 (and inf/nan, never produced here)
  if (a >= 0x3C800000u) {                      // |x| >= 2^-6: normal range
    uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);  // round the 20 dropped mantissa bits to nearest even
    return sign | ((r >> 20) - (120u << 3));
  }
  float m = rintf(__uint_as_float(a) * 512.0f);  // exact scaling, then nearest-even integer 0..8
  return sign | (uint32_t)m;
}

// Four fp32 -> four E4M3FN codes (one dword, little-endian) on the hardware converter
// (v_cvt_pk_fp8_f32): nearest even, sign kept for results that round to zero.  On every
// fp32 input with |x| <= 464 it returns exactly what f32_to_e4m3 does (checked on the
// device over all such bit patterns); callers keep |x| in that range.
__device__ __forceinline__ uint32_t e4m3x4_hw(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// x / s rounded to nearest even, given y = RN(1/s): q = RN(x*y) is faithful, the remainder
// x - q*s is exact in one fused multiply-add, and RN(q + remainder*y) is the correctly
// rounded quotient whenever it is a normal number (Markstein's theorem; Handbook of
// Floating-Point Arithmetic, division by fused multiply-add).  The sign is copied from x, so
// a quotient that underflows keeps the sign an IEEE division gives it.  One IEEE division
// per row (for y) replaces one per element.
__device__ __forceinline__ float div_rn_by(float x, float s, float y) {
  const float q = __fmul_rn(x, y);
  const float r = __builtin_fmaf(-q, s, x);
  return __builtin_copysignf(__builtin_fmaf(r, y, q), x);
}

// Four E4M3FN codes (one dword, little-endian) -> four f16 (two dwords), exact.
__device__ __forceinline__ uint2 e4m3x4_to_f16x4(uint32_t x) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false);  // codes 0, 1
  const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true);   // codes 2, 3
  return uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 2^(E-127) as an fp32 (E = 0 gives the subnormal 2^-127): an MXFP4 block's E8M0 scale.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) { return __uint_as_float(e ? e << 23 : 0x00400000u); }

// Eight FP4 E2M1 codes (one dword, element 2i in the low nibble of byte i) times `scale` -> bf16 on the
// hardware converter (v_cvt_scalef32_pk_bf16_fp4): exact for every code and every scale 2^(E-127) with E <= 252
// (checked on the device over all of them).
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t x, float scale) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, scale, 0);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, scale, 1);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, scale, 2);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, scale, 3);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Eight E4M3 codes (two dwords) -> bf16, exact (v_cvt_scalef32_pk_bf16_fp8 at scale 1).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t x0, uint32_t x1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Eight codes (two dwords) -> one f16x8 operand.
__device__ __forceinline__ f16x8 e4m3x8_to_f16x8(uint32_t x0, uint32_t x1) {
  const uint2 a = e4m3x4_to_f16x4(x0), b = e4m3x4_to_f16x4(x1);
  return __builtin_bit_cast(f16x8, (u32x4{a.x, a.y, b.x, b.y}));
}

// Order-preserving unsigned keys (larger value <-> larger key).
__device__ __forceinline__ uint32_t f32_key(uint32_t u) { return (u & 0x80000000u) ? ~u : (u | 0x80000000u); }
__device__ __forceinline__ uint32_t bf16_key(uint32_t h) { return (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u); }

// 4x4 transpose-reduce across the lane groups g = lane/16.  v[j], j = 0..3, are
// this lane's partial sums of four outputs; on return the lane holds the full
// sum of output j = g (summed over the four lane groups of its column).
__device__ __forceinline__ float transpose_reduce4(const float v[4], int lane) {
  const bool hi = lane >= 32;        // g in {2,3}
  const bool odd = (lane >> 4) & 1;  // g in {1,3}
  float s0 = hi ? v[0] : v[2];
  float s1 = hi ? v[1] : v[3];
  float r0 = __shfl_xor(s0, 32);
  float r1 = __shfl_xor(s1, 32);
  float k0 = (hi ? v[2] : v[0]) + r0;  // output 2*hi + 0
  float k1 = (hi ? v[3] : v[1]) + r1;  // output 2*hi + 1
  float s = odd ? k0 : k1;
  float r = __shfl_xor(s, 16);
  return (odd ? k1 : k0) + r;
}

// A-operand fragments of one query row: four 16-head tiles x four 32-dim slices.
struct QFrag {
  f16x8 a[4][4];
};

// Load q[row] (64 x 128 codes, contiguous) and decode it into this lane's A fragments:
// lane (head n, group g) reads the codes [32g, 32g+32) of head hb*16+n; slice s takes 8.
__device__ __forceinline__ void load_q(QFrag& f, const uint8_t* q_row, int lane) {
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int hb = 0; hb < 4; hb++) {
    const uint4* p = reinterpret_cast<const uint4*>(q_row + (hb * 16 + n) * kDim + g * 32);
    const uint4 x0 = p[0], x1 = p[1];
    f.a[hb][0] = e4m3x8_to_f16x8(x0.x, x0.y);
    f.a[hb][1] = e4m3x8_to_f16x8(x0.z, x0.w);
    f.a[hb][2] = e4m3x8_to_f16x8(x1.x, x1.y);
    f.a[hb][3] = e4m3x8_to_f16x8(x1.z, x1.w);
  }
}

// This lane's 16 head weights of one row: heads hb*16 + 4*(lane/16) + i.
struct WFrag {
  float w[4][4];
};

__device__ __forceinline__ void load_w(WFrag& f, const uint16_t* w_row, int lane) {
  const int g = lane >> 4;
#pragma unroll
  for (int hb = 0; hb < 4; hb++) {
    uint2 x = *reinterpret_cast<const uint2*>(w_row + hb * 16 + g * 4);
    f.w[hb][0] = bf16_to_f32(x.x & 0xFFFFu);
    f.w[hb][1] = bf16_to_f32(x.x >> 16);
    f.w[hb][2] = bf16_to_f32(x.y & 0xFFFFu);
    f.w[hb][3] = bf16_to_f32(x.y >> 16);
  }
}

// B-operand fragments for 16 keys: four 32-dim slices.
struct KFrag {
  f16x8 b[4];
};

// From FP8 key rows in LDS (kLdsKeyStride apart): read this lane's 32 codes and decode.
__device__ __forceinline__ void load_kfrag_fp8(KFrag& f, const uint8_t* keys, int lane) {
  const int n = lane & 15, g = lane >> 4;
  const uint4* p = reinterpret_cast<const uint4*>(keys + n * kLdsKeyStride + g * 32);
  const uint4 x0 = p[0], x1 = p[1];
  f.b[0] = e4m3x8_to_f16x8(x0.x, x0.y);
  f.b[1] = e4m3x8_to_f16x8(x0.z, x0.w);
  f.b[2] = e4m3x8_to_f16x8(x1.x, x1.y);
  f.b[3] = e4m3x8_to_f16x8(x1.z, x1.w);
}

// From key rows already decoded to f16 in LDS (kLdsKeyStrideF16 apart).
__device__ __forceinline__ void load_kfrag_f16(KFrag& f, const uint8_t* keys, int lane) {
  const int n = lane & 15, g = lane >> 4;
  const f16x8* p = reinterpret_cast<const f16x8*>(keys + n * kLdsKeyStrideF16 + g * 64);
#pragma unroll
  for (int s = 0; s < 4; s++) f.b[s] = p[s];
}

// Head-weighted partials of four (row, 16-key group) outputs at once: out j uses
// q[rows[j]] and kb[kgs[j]].  The 64 MFMAs run as 16 independent accumulator chains
// (4 outputs x 4 head tiles) taken slice by slice, so consecutive MFMAs never wait on
// each other; then each lane weights and sums its 16 heads per output.
template <int NQ, int NK>
__device__ __forceinline__ void score4(const QFrag (&q)[NQ], const WFrag (&w)[NQ], const KFrag (&kb)[NK],
                                       const int (&rows)[4], const int (&kgs)[4], float (&part)[4]) {
  f32x4 c[4][4];
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int hb = 0; hb < 4; hb++) c[j][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; s++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int hb = 0; hb < 4; hb++) c[j][hb] = mfma_f16(q[rows[j]].a[hb][s], kb[kgs[j]].b[s], c[j][hb]);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    float acc = 0.f;
#pragma unroll
    for (int hb = 0; hb < 4; hb++)
#pragma unroll
      for (int i = 0; i < 4; i++) acc = fmaf(w[rows[j]].w[hb][i], c[j][hb][i], acc);
    part[j] = acc;
  }
}

// Copy one 16-byte chunk of a contiguous run of 132-byte cache rows into the FP8
// LDS key layout: dword d of the run belongs to row d/33, word d%33 (word 32 is
// the fp32 scale).  `chunk` is the chunk index within the run, `key0` the LDS key
// slot of the run's first row.
__device__ __forceinline__ void scatter_chunk(uint8_t* lds_codes, float* lds_scale, int key0, int chunk,
                                              const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; j++) {
    int d = chunk * 4 + j;
    int row = d / 33, word = d - row * 33;
    if (word < 32)
      *reinterpret_cast<uint32_t*>(lds_codes + (key0 + row) * kLdsKeyStride + word * 4) = w[j];
    else
      lds_scale[key0 + row] = __uint_as_float(w[j]);
  }
}


// ---------------------------------------------------------------------------
// 32x32x16 layout (v_mfma_f32_32x32x16_f16), used where a wavefront scores one query row
// against 32-key groups:
//   A = 32 heads x 16 dims of q   (lane l: head l%32, 8 dims of lane half h = l/32)
//   B = 16 dims x 32 keys of K    (lane l: key  l%32, the same 8 dims)
//   C = 32 heads x 32 keys, lane l holds heads 8*(i/4) + 4*h + i%4 (i < 16) of key l%32.
// Lane half h owns dims [64h, 64h+64) of the 128 and feeds 8 of them to each of eight
// slices.  Two head blocks cover the 64 heads, so 16 MFMAs leave each lane 32 heads of one
// key: the head-weighted sum is 32 FMAs, and the other lane half holds the other 32 heads.
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// q[row] decoded into this lane's A fragments: head hb*32 + l%32, dims [64h + 8s, +8) for
// slice s.
struct Q32 {
  f16x8 a[2][8];
};

// The codes behind load_q32's fragments, as loaded (so that a caller can issue other loads
// before decoding them).
__device__ __forceinline__ void load_q32_codes(uint4 (&x)[2][4], const uint8_t* q_row, int lane) {
  const int m = lane & 31, h = lane >> 5;
#pragma unroll
  for (int hb = 0; hb < 2; hb++) {
    const uint4* p = reinterpret_cast<const uint4*>(q_row + (hb * 32 + m) * kDim + h * 64);
#pragma unroll
    for (int j = 0; j < 4; j++) x[hb][j] = p[j];
  }
}

__device__ __forceinline__ void decode_q32(Q32& f, const uint4 (&x)[2][4]) {
#pragma unroll
  for (int hb = 0; hb < 2; hb++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      f.a[hb][2 * j] = e4m3x8_to_f16x8(x[hb][j].x, x[hb][j].y);
      f.a[hb][2 * j + 1] = e4m3x8_to_f16x8(x[hb][j].z, x[hb][j].w);
    }
}

__device__ __forceinline__ void load_q32(Q32& f, const uint8_t* q_row, int lane) {
  uint4 x[2][4];
  load_q32_codes(x, q_row, lane);
  decode_q32(f, x);
}

// The weights of the 32 heads this lane holds in C: w[hb][i] is head hb*32 + 8*(i/4) + 4h + i%4.
struct W32 {
  float w[2][16];
};

// The bf16 weights behind load_w32's values, as loaded.
__device__ __forceinline__ void load_w32_raw(uint2 (&x)[2][4], const uint16_t* w_row, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int hb = 0; hb < 2; hb++)
#pragma unroll
    for (int b = 0; b < 4; b++) x[hb][b] = *reinterpret_cast<const uint2*>(w_row + hb * 32 + 8 * b + 4 * h);
}

__device__ __forceinline__ void decode_w32(W32& f, const uint2 (&x)[2][4]) {
#pragma unroll
  for (int hb = 0; hb < 2; hb++)
#pragma unroll
    for (int b = 0; b < 4; b++) {
      f.w[hb][4 * b + 0] = bf16_to_f32(x[hb][b].x & 0xFFFFu);
      f.w[hb][4 * b + 1] = bf16_to_f32(x[hb][b].x >> 16);
      f.w[hb][4 * b + 2] = bf16_to_f32(x[hb][b].y & 0xFFFFu);
      f.w[hb][4 * b + 3] = bf16_to_f32(x[hb][b].y >> 16);
    }
}

__device__ __forceinline__ void load_w32(W32& f, const uint16_t* w_row, int lane) {
  uint2 x[2][4];
  load_w32_raw(x, w_row, lane);
  decode_w32(f, x);
}

// B fragments of one 32-key group from the f16 tile: key l%32, dims [64h + 8s, +8).
struct K32 {
  f16x8 b[8];
};

// Sum of the two lane halves for two 32-key groups at once: on return lane l holds the
// full sum of key l of the 64-key tile (group l/32, key l%32).
__device__ __forceinline__ float combine_halves(float g0, float g1) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(g0), __float_as_uint(g1), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace dsi
