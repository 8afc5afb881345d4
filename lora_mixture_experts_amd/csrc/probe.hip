// Measurement probes (include/moelora_probe.h): a streaming read of HBM and a loop of
// independent bf16 MFMAs, the on-box ceilings the layer's throughput is compared with.
#include "common.h"
#include "moelora.h"
#include "moelora_probe.h"
#include "tile_pipeline.h"

namespace moelora {
namespace {

constexpr int kReadGrid = 2048;

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = tid;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(src + i + j * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  sink[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

__device__ __forceinline__ uint32_t probe_hash(uint32_t v) {
  v ^= v >> 16;
  v *= 0x7feb352du;
  v ^= v >> 15;
  v *= 0x846ca68bu;
  return v ^ (v >> 16);
}

// bf16 pair of random sign and mantissa, exponent 126 or 127 (|value| in [0.5, 2))
__device__ __forceinline__ uint32_t probe_bf16x2(uint32_t h) {
  return (h & 0x80ff80ffu) | 0x3f003f00u;
}

__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float* __restrict__ sink) {
  const uint32_t gid = blockIdx.x * 256 + threadIdx.x;
  u32x4 a, b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] = probe_bf16x2(probe_hash(2 * (4 * gid + j) + 1));
    b[j] = probe_bf16x2(probe_hash(2 * (4 * gid + j) + 2));
  }
  f32x16 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = mfma32(a, b, acc[t]);
  }
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[t][v];
  sink[gid] = s;
}

}  // namespace
}  // namespace moelora

using namespace moelora;

extern "C" {

int moe_lora_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0 || bytes % 16 != 0) return MOELORA_EINVAL_DIMS;
  if (!src || !sink) return MOELORA_ENULL;
  if (((uintptr_t)src & 15u) != 0 || ((uintptr_t)sink & 3u) != 0) return MOELORA_EALIGN;
  hipLaunchKernelGGL(probe_read_kernel, dim3(kReadGrid), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? MOELORA_OK : MOELORA_EHIP;
}

int moe_lora_probe_mfma(int32_t iters, int32_t n_workgroups, float* sink, void* stream) {
  if (iters < 1 || n_workgroups < 1) return MOELORA_EINVAL_DIMS;
  if (!sink) return MOELORA_ENULL;
  if (((uintptr_t)sink & 3u) != 0) return MOELORA_EALIGN;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(n_workgroups), dim3(256), 0, (hipStream_t)stream,
                     iters, sink);
  return hipGetLastError() == hipSuccess ? MOELORA_OK : MOELORA_EHIP;
}

}  // extern "C"
