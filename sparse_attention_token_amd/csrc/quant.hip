// k quantization fused with cache insertion (P3 step ⑤ of "DeepSeek V3.2 稀疏注意力
// DSA 推理流程图解": k is quantized to FP8 as it is written into the indexer cache,
// one 132-byte row per token, P3 data flow 1).
//
// One wavefront per token: each lane owns two of the 128 bf16 values; the amax is a
// wavefront max-reduction, the scale max(amax, 1e-4)/448 and every k/scale are IEEE
// fp32 divisions, and each lane writes its two FP8 codes; lane 0 writes the scale.
// HBM-bound: 256 B read + 132 B written per token.
#include "common.h"

namespace dsi {
namespace {

constexpr int kQuantWaves = 4;

__global__ __launch_bounds__(256) void k_quant_kernel(const uint16_t* __restrict__ k, int64_t n, int64_t k_ld,
                                                      const int64_t* __restrict__ slot_mapping,
                                                      uint8_t* __restrict__ pool, int64_t num_slots,
                                                      int32_t block_size, int64_t block_stride) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6);
  if (i >= n) return;
  const int64_t slot = slot_mapping[i];
  if (slot < 0 || slot >= num_slots) return;  // padding token: nothing written
  const uint32_t pair = *reinterpret_cast<const uint32_t*>(k + i * k_ld + 2 * lane);
  const float x0 = bf16_to_f32(pair & 0xFFFFu), x1 = bf16_to_f32(pair >> 16);
  float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float scale = __fdiv_rn(fmaxf(amax, 1e-4f), 448.0f);
  const uint32_t c0 = f32_to_e4m3(__fdiv_rn(x0, scale));
  const uint32_t c1 = f32_to_e4m3(__fdiv_rn(x1, scale));
  uint8_t* row = pool + (slot / block_size) * block_stride + (slot % block_size) * kRow;
  *reinterpret_cast<uint16_t*>(row + 2 * lane) = (uint16_t)(c0 | (c1 << 8));
  if (lane == 0) *reinterpret_cast<float*>(row + kDim) = scale;
}

// MXFP4 (OCP Microscaling: FP4 E2M1 elements, one E8M0 scale 2^(E-127) per 32) into 68-byte
// rows: 64 bytes of codes (element 2i in the low nibble of byte i), then the four scale
// bytes (P1 motivation and implementation: the V4.1 sparse indexer reads an MXFP4 indexer
// cache).  One wavefront per token, lane l holding dims 2l and 2l+1; block j is lanes
// 16j..16j+15.  Shared exponent floor(log2(amax)) - 2 clamped to [-127, 127] (-127 for an
// all-zero block); each element x * 2^-se (exact) rounded to nearest even FP4, saturating
// at 6.
constexpr int kRow4 = 68;

// Nearest-even FP4 E2M1 code of y: the count of the midpoints between consecutive
// magnitudes (0, .5, 1, 1.5, 2, 3, 4, 6) that |y| passes, a tie counting as passed when
// the upper neighbour has the even code; 7 from 5 up (saturation); sign kept.
__device__ __forceinline__ uint32_t f32_to_fp4(float y) {
  const float a = fabsf(y);
  const uint32_t m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return ((__float_as_uint(y) >> 28) & 8u) | m;
}

__global__ __launch_bounds__(256) void k_quant_mxfp4_kernel(const uint16_t* __restrict__ k, int64_t n, int64_t k_ld,
                                                            const int64_t* __restrict__ slot_mapping,
                                                            uint8_t* __restrict__ pool, int64_t num_slots,
                                                            int32_t block_size, int64_t block_stride) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6);
  if (i >= n) return;
  const int64_t slot = slot_mapping[i];
  if (slot < 0 || slot >= num_slots) return;  // padding token: nothing written
  const uint32_t pair = *reinterpret_cast<const uint32_t*>(k + i * k_ld + 2 * lane);
  const float x0 = bf16_to_f32(pair & 0xFFFFu), x1 = bf16_to_f32(pair >> 16);
  float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  int se = -127;
  if (amax > 0.0f) se = min(max(__builtin_amdgcn_frexp_expf(amax) - 3, -127), 127);  // amax = f * 2^e, f in [.5, 1)
  const uint32_t c0 = f32_to_fp4(ldexpf(x0, -se)), c1 = f32_to_fp4(ldexpf(x1, -se));
  uint8_t* row = pool + (slot / block_size) * block_stride + (slot % block_size) * kRow4;
  row[lane] = (uint8_t)(c0 | (c1 << 4));
  if ((lane & 15) == 0) row[64 + (lane >> 4)] = (uint8_t)(se + 127);
}

}  // namespace
}  // namespace dsi

extern "C" int dsi_k_quant_and_cache(const uint16_t* k, int64_t n, int64_t k_ld, const int64_t* slot_mapping,
                                     uint8_t* pool, int64_t num_blocks, int32_t block_size,
                                     int64_t block_stride_bytes, hipStream_t stream) {
  using namespace dsi;
  if (n < 0 || k_ld < kDim || block_size < 1 || num_blocks < 0 ||
      block_stride_bytes < (int64_t)block_size * kRow)
    return DSI_EINVAL;
  if (n == 0) return DSI_OK;
  if (!k || !slot_mapping || !pool) return DSI_EINVAL;
  if ((reinterpret_cast<uintptr_t>(k) & 3) || (k_ld & 1) || (reinterpret_cast<uintptr_t>(pool) & 3) ||
      (block_stride_bytes & 3))
    return DSI_EALIGN;
  const int64_t blocks = (n + kQuantWaves - 1) / kQuantWaves;
  if (blocks > 0x7FFFFFFF) return DSI_EUNSUPPORTED;
  hipLaunchKernelGGL(k_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, k, n, k_ld, slot_mapping, pool,
                     num_blocks * block_size, block_size, block_stride_bytes);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}

extern "C" int dsi_k_quant_and_cache_mxfp4(const uint16_t* k, int64_t n, int64_t k_ld, const int64_t* slot_mapping,
                                           uint8_t* pool, int64_t num_blocks, int32_t block_size,
                                           int64_t block_stride_bytes, hipStream_t stream) {
  using namespace dsi;
  if (n < 0 || k_ld < kDim || block_size < 1 || num_blocks < 0 ||
      block_stride_bytes < (int64_t)block_size * kRow4)
    return DSI_EINVAL;
  if (n == 0) return DSI_OK;
  if (!k || !slot_mapping || !pool) return DSI_EINVAL;
  if ((reinterpret_cast<uintptr_t>(k) & 3) || (k_ld & 1) || (reinterpret_cast<uintptr_t>(pool) & 3) ||
      (block_stride_bytes & 3))
    return DSI_EALIGN;
  const int64_t blocks = (n + kQuantWaves - 1) / kQuantWaves;
  if (blocks > 0x7FFFFFFF) return DSI_EUNSUPPORTED;
  hipLaunchKernelGGL(k_quant_mxfp4_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, k, n, k_ld, slot_mapping,
                     pool, num_blocks * block_size, block_size, block_stride_bytes);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}
