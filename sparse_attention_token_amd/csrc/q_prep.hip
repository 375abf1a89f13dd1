// q preparation in one pass: rotary position embedding on the first 64 of the 128 dims,
// FP8 quantization with one scale per head row of 128 values, and the fold of that scale
// (with the softmax and head scales) into the head weights, written as bf16 (P3 "DeepSeek
// V3.2 稀疏注意力 DSA 推理流程图解", indexer steps ③ and ④ and pitfalls: the indexer's RoPE has
// its own interleave switch; P1 "V4.1 索引器接入稀疏 MQA logits", implementation breakdown:
// the fused q kernel writes the per-head weights as bf16, the fp32 result rounded once).
//
// One workgroup per token; sixteen lanes own a (token, head) row at a time, four heads per
// lane group: lane j holds dims 8j..8j+7 (one 16-byte bf16 load).  Not interleaved,
// frequency i pairs dims i and i+32, i.e. lane j with lane j^4 for j < 8 (one lane
// exchange); interleaved, it pairs dims 2i and 2i+1, inside a lane.  The
// amax is a 16-lane max-reduction.  Every rounding step is the one written in the method
// (fp32 products and sums without contraction into fused multiply-adds, correctly rounded
// divisions — one IEEE division per row for the reciprocal of the scale, then a remainder
// correction per element — nearest-even E4M3 on the hardware converter, bf16), so the codes
// and weights are bit-exact.  HBM-bound: 256 B
// read and 128 B written per head row; the rotary table row is shared by a token's 64
// heads.
#include "common.h"

namespace dsi {
namespace {

constexpr int kQpThreads = 256;
constexpr int kQpHeadsPerGroup = kHeads / (kQpThreads / 16);  // 4: one workgroup per token

// Rotation of one 16-lane group's 8 values per lane (see the file comment for the lane layout).
// Not interleaved, lanes j < 4 hold the first dims of their pairs (a' = a*cos - b*sin) and lanes
// 4..7 the second (b' = b*cos + a*sin); the caller passes s already negated for j < 4, which is
// the same rounding (RN(y*(-s)) = -RN(y*s)), so both take one path.
__device__ __forceinline__ void rope8(float (&x)[8], const float (&c)[8], const float (&s)[8], int j, bool interleave) {
#pragma clang fp contract(off)
  if (!interleave) {
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; e++) y[e] = __shfl_xor(x[e], 4);
    if (j < 8) {
#pragma unroll
      for (int e = 0; e < 8; e++) x[e] = x[e] * c[e] + y[e] * s[e];
    }
  } else if (j < 8) {  // pairs (2m, 2m+1) inside the lane, frequency 4j + m
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const float a = x[2 * m], b = x[2 * m + 1];
      x[2 * m] = a * c[m] - b * s[m];
      x[2 * m + 1] = b * c[m] + a * s[m];
    }
  }
}

// One workgroup per token: 16 groups of 16 lanes, each group four heads (h = group + 16*k), so the
// position and the rotary table row are loaded once per lane and the four q loads are in flight together.
__global__ __launch_bounds__(kQpThreads) void q_rope_quant_kernel(
    const uint16_t* __restrict__ q, int64_t q_ld, const int64_t* __restrict__ positions,
    const float* __restrict__ cos_sin, int64_t max_pos, int32_t interleave, const uint16_t* __restrict__ w,
    int64_t w_ld, float softmax_scale, float head_scale, uint8_t* __restrict__ q8, uint16_t* __restrict__ w_out) {
#pragma clang fp contract(off)
  const int j = threadIdx.x & 15, g = threadIdx.x >> 4;
  const int64_t t = blockIdx.x;
  uint4 raw[kQpHeadsPerGroup];
#pragma unroll
  for (int k = 0; k < kQpHeadsPerGroup; k++)
    raw[k] = *reinterpret_cast<const uint4*>(q + t * q_ld + (g + 16 * k) * kDim + j * 8);
  const int64_t pos = positions[t];
  uint8_t* dst = q8 + t * (kHeads * kDim) + j * 8;
  if (pos < 0 || pos >= max_pos) {
#pragma unroll
    for (int k = 0; k < kQpHeadsPerGroup; k++) {
      *reinterpret_cast<uint2*>(dst + (g + 16 * k) * kDim) = make_uint2(0, 0);
      if (j == 0) w_out[t * kHeads + g + 16 * k] = 0;
    }
    return;
  }
  float c[8] = {}, s[8] = {};
  const float* cs = cos_sin + pos * 64;
  if (j < 8) {
    if (!interleave) {  // lane j, element e: frequency (j & 3) * 8 + e
      const int i0 = (j & 3) * 8;
      const float4 c0 = *reinterpret_cast<const float4*>(cs + i0), c1 = *reinterpret_cast<const float4*>(cs + i0 + 4);
      const float4 s0 = *reinterpret_cast<const float4*>(cs + 32 + i0);
      const float4 s1 = *reinterpret_cast<const float4*>(cs + 36 + i0);
      c[0] = c0.x, c[1] = c0.y, c[2] = c0.z, c[3] = c0.w, c[4] = c1.x, c[5] = c1.y, c[6] = c1.z, c[7] = c1.w;
      s[0] = s0.x, s[1] = s0.y, s[2] = s0.z, s[3] = s0.w, s[4] = s1.x, s[5] = s1.y, s[6] = s1.z, s[7] = s1.w;
      if (j < 4) {
#pragma unroll
        for (int e = 0; e < 8; e++) s[e] = -s[e];
      }
    } else {  // lane j, pair m: frequency 4j + m
      const float4 c0 = *reinterpret_cast<const float4*>(cs + j * 4);
      const float4 s0 = *reinterpret_cast<const float4*>(cs + 32 + j * 4);
      c[0] = c0.x, c[1] = c0.y, c[2] = c0.z, c[3] = c0.w;
      s[0] = s0.x, s[1] = s0.y, s[2] = s0.z, s[3] = s0.w;
    }
  }
  float wraw[kQpHeadsPerGroup];
#pragma unroll
  for (int k = 0; k < kQpHeadsPerGroup; k++) wraw[k] = j == 0 ? bf16_to_f32(w[t * w_ld + g + 16 * k]) : 0.0f;
#pragma unroll
  for (int k = 0; k < kQpHeadsPerGroup; k++) {
    const uint4 r = raw[k];
    float x[8] = {bf16_to_f32(r.x & 0xFFFFu), bf16_to_f32(r.x >> 16), bf16_to_f32(r.y & 0xFFFFu),
                  bf16_to_f32(r.y >> 16),     bf16_to_f32(r.z & 0xFFFFu), bf16_to_f32(r.z >> 16),
                  bf16_to_f32(r.w & 0xFFFFu), bf16_to_f32(r.w >> 16)};
    rope8(x, c, s, j, interleave != 0);
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; e++) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float scale = __fdiv_rn(fmaxf(amax, 1e-4f), 448.0f);
    const float inv = __fdiv_rn(1.0f, scale);
    float z[8];
#pragma unroll
    for (int e = 0; e < 8; e++) z[e] = div_rn_by(x[e], scale, inv);  // |z| <= 448 (1 + 2^-23)
    *reinterpret_cast<uint2*>(dst + (g + 16 * k) * kDim) =
        make_uint2(e4m3x4_hw(z[0], z[1], z[2], z[3]), e4m3x4_hw(z[4], z[5], z[6], z[7]));
    if (j == 0) {
      float wf = wraw[k] * scale;
      wf = wf * softmax_scale;
      wf = wf * head_scale;
      w_out[t * kHeads + g + 16 * k] = f32_to_bf16_rne(wf);
    }
  }
}

}  // namespace
}  // namespace dsi

extern "C" int dsi_q_rope_quant(const uint16_t* q, int64_t q_ld, int32_t T, const int64_t* positions,
                                const float* cos_sin, int64_t max_pos, int32_t interleave, const uint16_t* w,
                                int64_t w_ld, float softmax_scale, float head_scale, uint8_t* q8, uint16_t* w_out,
                                hipStream_t stream) {
  using namespace dsi;
  if (T < 0 || q_ld < (int64_t)kHeads * kDim || w_ld < kHeads || max_pos < 1) return DSI_EINVAL;
  if (T == 0) return DSI_OK;
  if (!q || !positions || !cos_sin || !w || !q8 || !w_out) return DSI_EINVAL;
  if ((reinterpret_cast<uintptr_t>(q) & 15) || (q_ld & 7) || (reinterpret_cast<uintptr_t>(cos_sin) & 15) ||
      (reinterpret_cast<uintptr_t>(positions) & 7) || (reinterpret_cast<uintptr_t>(w) & 1) ||
      (reinterpret_cast<uintptr_t>(q8) & 7) || (reinterpret_cast<uintptr_t>(w_out) & 1))
    return DSI_EALIGN;
  hipLaunchKernelGGL(q_rope_quant_kernel, dim3((unsigned)T), dim3(kQpThreads), 0, stream, q, q_ld, positions, cos_sin,
                     max_pos, interleave, w, w_ld, softmax_scale, head_scale, q8, w_out);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}
