// Measured ceilings for the indexer rooflines: register-only matrix-core loops
// and HBM streaming read / copy.  Built into its own library; the indexer path
// does not use it.
#include <hip/hip_runtime.h>

#include "dsi.h"
#include "dsi_ceiling.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChains = 16;

// A 16-byte load, with the non-temporal hint (streaming data: the loads set the "nt" bit) or
// without it.
template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

// Eight pseudo-random E4M3 codes with exponent field 8..15 (magnitudes 2 to 448, random sign and mantissa; the NaN
// codes become the largest finite ones), decoded exactly to f16 by the hardware converter: operands whose bits switch
// like the indexer's FP8 data, so that the loop runs at the clock the chip's power limit allows on such data.
__device__ __forceinline__ f16x8 random_f16x8(uint32_t seed) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 h[4];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    uint32_t x = seed * 0x9E3779B1u + (uint32_t)i * 0x85EBCA77u;
    x ^= x >> 15;
    x *= 0x2C1B3C6Du;
    x ^= x >> 12;
    x *= 0x297A2D39u;
    x ^= x >> 15;
    x |= 0x40404040u;                                              // exponent field >= 8
    x -= (((x & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u) >> 7;  // 0x7F / 0xFF -> 0x7E / 0xFE
    h[2 * i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false);
    h[2 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true);
  }
  return f16x8{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
}

template <int KIND, bool RANDOM>
__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(float* __restrict__ sink, int iters) {
  f32x4 c[kChains];
#pragma unroll
  for (int j = 0; j < kChains; j++) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Operands depend on the thread id so the compiler cannot fold the loop; their
  // values are small and finite (f16 halves, FP8 codes 0x30..0x37 = 0.5..0.9375), or
  // random FP8 codes decoded to f16.
  f16x8 a16, b16;
  i32x8 a8, b8;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    a16[j] = (_Float16)((threadIdx.x & 7) * 0.125f + j * 0.0625f);
    b16[j] = (_Float16)(0.5f + j * 0.03125f);
    a8[j] = 0x30303030 | ((threadIdx.x + j) & 7);
    b8[j] = 0x30303030 | (j & 7);
  }
  if constexpr (RANDOM) {
    a16 = random_f16x8(blockIdx.x * kThreads + threadIdx.x);
    b16 = random_f16x8(0x10000u + threadIdx.x);
  }
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int j = 0; j < kChains; j++) {
      if constexpr (KIND == 0)
        c[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a16, b16, c[j], 0, 0, 0);
      else
        c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c[j], 0, 0, 0, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; j++) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// The 32x32x16 f16 form (32,768 flop per instruction) with 8 independent chains; the
// accumulators (128 registers) live in the accumulation registers.
constexpr int kChains32 = 8;

template <bool RANDOM>
__global__ __launch_bounds__(kThreads) void mfma32_loop_kernel(float* __restrict__ sink, int iters) {
  f32x16 c[kChains32];
#pragma unroll
  for (int j = 0; j < kChains32; j++) c[j] = f32x16{};
  f16x8 a16, b16;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    a16[j] = (_Float16)((threadIdx.x & 7) * 0.125f + j * 0.0625f);
    b16[j] = (_Float16)(0.5f + j * 0.03125f);
  }
  if constexpr (RANDOM) {
    a16 = random_f16x8(blockIdx.x * kThreads + threadIdx.x);
    b16 = random_f16x8(0x10000u + threadIdx.x);
  }
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int j = 0; j < kChains32; j++) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a16, b16, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains32; j++) s += c[j][0] + c[j][5] + c[j][10] + c[j][15];
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                               uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  // four independent loads in flight per thread
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 x0 = load16<NT>(src + i), x1 = load16<NT>(src + i + stride), x2 = load16<NT>(src + i + 2 * stride),
                x3 = load16<NT>(src + i + 3 * stride);
    acc ^= x0 ^ x1 ^ x2 ^ x3;
  }
  for (; i < n16; i += stride) acc ^= load16<NT>(src + i);
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        size_t n16) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// Whole pages of page_bytes at pool + pages[i] * block_stride, P pages per workgroup round, each
// page read by the workgroup's 256 threads in up to three 16-byte loads each (all 3P in flight).
// A page id outside [0, n_blocks) is read as nothing.
constexpr int kPageRounds = 3;  // pages of at most 3 * 256 * 16 = 12 KB
template <int P, bool NT>
__global__ __launch_bounds__(kThreads) void paged_read_kernel(const uint8_t* __restrict__ pool, int64_t block_stride,
                                                              int64_t n_blocks, const int* __restrict__ pages,
                                                              int n_pages, int page_bytes, uint32_t* __restrict__ sink) {
  const int n16 = page_bytes / 16, t = threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int p0 = blockIdx.x * P; p0 < n_pages; p0 += gridDim.x * P) {
    u32x4 x[P][kPageRounds];
#pragma unroll
    for (int q = 0; q < P; q++) {
      const int p = p0 + q;
      const int id = pages[min(p, n_pages - 1)];
      const bool ok = p < n_pages && id >= 0 && id < n_blocks;
      const u32x4* base = reinterpret_cast<const u32x4*>(pool + (ok ? (int64_t)id * block_stride : 0));
#pragma unroll
      for (int r = 0; r < kPageRounds; r++) {
        const int j = r * kThreads + t;
        x[q][r] = u32x4{0u, 0u, 0u, 0u};
        if (ok && j < n16) x[q][r] = load16<NT>(base + j);
      }
    }
#pragma unroll
    for (int q = 0; q < P; q++)
#pragma unroll
      for (int r = 0; r < kPageRounds; r++) acc ^= x[q][r];
  }
  sink[(size_t)blockIdx.x * kThreads + t] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

int launched() { return hipGetLastError() == hipSuccess ? DSI_OK : DSI_ELAUNCH; }

}  // namespace

extern "C" int dsic_mfma_loop(int32_t kind, int32_t workgroups, int32_t iters, float* sink, hipStream_t stream) {
  if (kind < 0 || kind > 4 || workgroups < 1 || iters < 1 || !sink) return DSI_EINVAL;
  const dim3 grid(workgroups), block(kThreads);
  switch (kind) {
    case 0: hipLaunchKernelGGL((mfma_loop_kernel<0, false>), grid, block, 0, stream, sink, iters); break;
    case 1: hipLaunchKernelGGL((mfma_loop_kernel<1, false>), grid, block, 0, stream, sink, iters); break;
    case 2: hipLaunchKernelGGL(mfma32_loop_kernel<false>, grid, block, 0, stream, sink, iters); break;
    case 3: hipLaunchKernelGGL((mfma_loop_kernel<0, true>), grid, block, 0, stream, sink, iters); break;
    default: hipLaunchKernelGGL(mfma32_loop_kernel<true>, grid, block, 0, stream, sink, iters); break;
  }
  return launched();
}

extern "C" int dsic_stream_read(const void* src, size_t bytes, int32_t workgroups, int32_t nontemporal,
                                uint32_t* sink, hipStream_t stream) {
  if (!src || !sink || bytes == 0 || (bytes & 15) || workgroups < 1 || workgroups > 4096) return DSI_EINVAL;
  if (nontemporal != 0 && nontemporal != 1) return DSI_EINVAL;
  if (reinterpret_cast<uintptr_t>(src) & 15) return DSI_EALIGN;
  auto k = nontemporal ? stream_read_kernel<true> : stream_read_kernel<false>;
  hipLaunchKernelGGL(k, dim3(workgroups), dim3(kThreads), 0, stream, static_cast<const u32x4*>(src), bytes / 16,
                     sink);
  return launched();
}

extern "C" int dsic_copy(const void* src, void* dst, size_t bytes, int32_t workgroups, hipStream_t stream) {
  if (!src || !dst || bytes == 0 || (bytes & 15) || workgroups < 1) return DSI_EINVAL;
  if ((reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(dst) & 15)) return DSI_EALIGN;
  hipLaunchKernelGGL(copy_kernel, dim3(workgroups), dim3(kThreads), 0, stream, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), bytes / 16);
  return launched();
}

extern "C" int dsic_paged_read(const void* pool, int64_t pool_bytes, int64_t block_stride, const int32_t* pages,
                               int32_t n_pages, int32_t page_bytes, int32_t pages_per_round, int32_t nontemporal,
                               int32_t workgroups, uint32_t* sink, hipStream_t stream) {
  if (!pool || !pages || !sink || n_pages < 1 || workgroups < 1 || workgroups > 4096) return DSI_EINVAL;
  if (pages_per_round != 4 && pages_per_round != 8) return DSI_EINVAL;
  if (nontemporal != 0 && nontemporal != 1) return DSI_EINVAL;
  if (page_bytes < 16 || (page_bytes & 15) || page_bytes > kPageRounds * kThreads * 16) return DSI_EINVAL;
  if (block_stride < page_bytes || (block_stride & 15) || pool_bytes < page_bytes) return DSI_EINVAL;
  if (reinterpret_cast<uintptr_t>(pool) & 15) return DSI_EALIGN;
  // blocks whose whole page lies in the pool
  const int64_t n_blocks = (pool_bytes - page_bytes) / block_stride + 1;
  auto k = pages_per_round == 8 ? (nontemporal ? paged_read_kernel<8, true> : paged_read_kernel<8, false>)
                                : (nontemporal ? paged_read_kernel<4, true> : paged_read_kernel<4, false>);
  hipLaunchKernelGGL(k, dim3(workgroups), dim3(kThreads), 0, stream, static_cast<const uint8_t*>(pool), block_stride,
                     n_blocks, pages, n_pages, page_bytes, sink);
  return launched();
}
