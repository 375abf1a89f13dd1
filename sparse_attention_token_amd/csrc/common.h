// Device helpers shared by the gfx950 indexer kernels.
//
// The indexer score of P3 step ⑥ ("DeepSeek V3.2 稀疏注意力 DSA 推理流程图解") is a 64-head x
// 128-dim contraction of FP8 values followed by a per-head weighted sum.
//
// Matrix instructions.  The FP8 codes are decoded exactly to f16 (or bf16) and contracted on
// the f16 (bf16) matrix instructions.  gfx950's FP8-operand MFMAs (16x16x128 f8f6f4 and
// 16x16x32 fp8) were measured to drop product bits about 13 binades below the largest product
// of their internal sum, with a one-sided (truncating) error that reaches ~0.1 on indexer
// logits — beyond the path's 1e-3 (1 + |ref|) bar — while the f16 MFMA sums the same products
// exactly.  Every E4M3FN value is a normal f16 (2^-9 to 448), so the decode
// (v_cvt_scalef32_pk_f16_fp8 with scale 1, two codes per instruction) is exact.
//
// Two operand layouts: the dense prefill kernel's v_mfma_f32_16x16x32_f16 (described in
// prefill.hip) and the one-row scoring kernels' v_mfma_f32_32x32x16_f16 (below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsi.h"

namespace dsi {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Compute units of the current device (queried once per device), for sizing persistent grids.
inline int cu_count() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] <= 0) {
    int n = 0;
    cached[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cached[dev];
}

constexpr int kHeads = 64;
constexpr int kDim = 128;
constexpr int kRow = 132;              // bytes per cache row
constexpr int kLdsKeyStrideF16 = 272;  // LDS bytes per f16 key row: 256 + pad, 68 dwords = 4 mod 32 banks

// The 16x16x32 f16 matrix instruction (the dense prefill kernel's; its operand layout is described there).
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

__device__ __forceinline__ void load_q32(Q32& f, const uint8_t* q_row, int lane) {
  const int m = lane & 31, h = lane >> 5;
#pragma unroll
  for (int hb = 0; hb < 2; hb++) {
    const uint4* p = reinterpret_cast<const uint4*>(q_row + (hb * 32 + m) * kDim + h * 64);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint4 x = p[j];
      f.a[hb][2 * j] = e4m3x8_to_f16x8(x.x, x.y);
      f.a[hb][2 * j + 1] = e4m3x8_to_f16x8(x.z, x.w);
    }
  }
}

// B fragments of one 32-key group: key l%32, dims [64h + 8s, +8).
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
