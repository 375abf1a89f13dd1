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
