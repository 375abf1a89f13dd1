// Whole-range runs of the device converters the indexer kernels use (include/dsi_probe.h), for the tests that
// compare them with the CPU oracle.  Every probe calls the kernels' own inline functions from common.h.
#include "common.h"
#include "dsi_probe.h"

namespace dsi {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocks = 4096;

// Thread t takes a contiguous part of [0, n): its first pattern's code is compared with the code of the pattern
// before it, then every next pattern's with its predecessor's.
__global__ __launch_bounds__(kProbeThreads) void e4m3_changes_kernel(uint32_t u0, int64_t n, uint32_t* trans,
                                                                     uint32_t cap, uint32_t* ntrans,
                                                                     uint32_t* first) {
  const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (n + nthreads - 1) / nthreads;
  const int64_t lo = t * per, hi = min(lo + per, n);
  if (lo >= hi) return;
  auto code = [](uint32_t u) {
    const float x = __uint_as_float(u);
    return e4m3x4_hw(x, x, x, x) & 0xFFu;
  };
  uint32_t prev = code(u0 + (uint32_t)(lo > 0 ? lo - 1 : 0));
  if (lo == 0) *first = prev;
  for (int64_t i = lo; i < hi; i++) {
    const uint32_t u = u0 + (uint32_t)i;
    const uint32_t c = code(u);
    if (c != prev) {
      const uint32_t slot = atomicAdd(ntrans, 1u);
      if (slot < cap) {
        trans[2 * slot] = u;
        trans[2 * slot + 1] = c;
      }
    }
    prev = c;
  }
}

__global__ void e4m3_decode_kernel(uint16_t* f16_out, uint16_t* bf16_out) {
  const uint32_t c = threadIdx.x;  // 256 threads, one code each
  const uint32_t word = c * 0x01010101u;
  const uint2 h = e4m3x4_to_f16x4(word);
  f16_out[c] = (uint16_t)(h.x & 0xFFFFu);
  const bf16x8 b = e4m3x8_to_bf16x8(word, word);
  bf16_out[c] = __builtin_bit_cast(uint16_t, b[0]);
}

__global__ void fp4_decode_kernel(uint16_t* out) {
  const uint32_t e = blockIdx.x, code = threadIdx.x;  // 256 x 16
  const uint32_t word = code * 0x11111111u;           // the code in every nibble
  const bf16x8 b = fp4x8_to_bf16x8(word, e8m0_to_f32(e));
  out[e * 16 + code] = __builtin_bit_cast(uint16_t, b[0]);
}

}  // namespace
}  // namespace dsi

extern "C" int dsip_e4m3_encode_changes(uint32_t u0, int64_t n, uint32_t* trans, uint32_t cap, uint32_t* ntrans,
                                        uint32_t* first, hipStream_t stream) {
  if (!trans || !ntrans || !first || n < 1 || (int64_t)u0 + n > ((int64_t)1 << 32)) return DSI_EINVAL;
  hipLaunchKernelGGL(dsi::e4m3_changes_kernel, dim3(dsi::kProbeBlocks), dim3(dsi::kProbeThreads), 0, stream, u0, n,
                     trans, cap, ntrans, first);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}

extern "C" int dsip_e4m3_decode_all(uint16_t* f16_out, uint16_t* bf16_out, hipStream_t stream) {
  if (!f16_out || !bf16_out) return DSI_EINVAL;
  hipLaunchKernelGGL(dsi::e4m3_decode_kernel, dim3(1), dim3(256), 0, stream, f16_out, bf16_out);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}

extern "C" int dsip_fp4_decode_all(uint16_t* out, hipStream_t stream) {
  if (!out) return DSI_EINVAL;
  hipLaunchKernelGGL(dsi::fp4_decode_kernel, dim3(256), dim3(16), 0, stream, out);
  return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH;
}
