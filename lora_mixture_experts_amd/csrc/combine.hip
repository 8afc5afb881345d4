// Weighted top-k combine: y[t] = sum_j w[t][j] * D[row(t*k + j)], summed in slot order in fp32,
// then rounded once to bf16 (round-to-nearest-even). D holds the down GEMM's output rows in the
// sorted (expert, adapter) order; pair_row maps a pair to its row. D may arrive as ksplit partial
// buffers (split-K of the down GEMM); they are added in split order first.
//
// Page "vLLM MoE LoRA SageMaker Bedrock", section "Entendendo os Modelos MoE": the outputs of
// the experts a token was sent to are aggregated. Each thread owns four consecutive features of
// one token, so every load and store is a full 16-byte (D) or 8-byte (y) access.
#include "common.h"
#include "kernels.h"

namespace moelora {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ D, int ksplit,
                                                      int64_t split_stride,
                                                      const int* __restrict__ pair_row,
                                                      const float* __restrict__ topk_w, int T,
                                                      int k, int h, uint16_t* __restrict__ y) {
  const int h4 = h >> 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)T * h4) return;
  const int t = (int)(idx / h4);
  const int c = (int)(idx - (int64_t)t * h4) * 4;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const float w = topk_w[(size_t)t * k + j];
    const size_t row = (size_t)pair_row[(size_t)t * k + j];
    f32x4 d = *reinterpret_cast<const f32x4*>(D + row * h + c);
    for (int z = 1; z < ksplit; ++z)
      d += *reinterpret_cast<const f32x4*>(D + z * split_stride + row * h + c);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(w, d[v], acc[v]);
  }
  u32x2 packed = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  *reinterpret_cast<u32x2*>(y + (size_t)t * h + c) = packed;
}

hipError_t launch_combine(const float* D, int ksplit, int64_t split_stride, const int* pair_row,
                          const float* topk_w, int T, int k, int h, uint16_t* y,
                          hipStream_t stream) {
  const int64_t n = (int64_t)T * (h / 4);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, D,
                     ksplit, split_stride, pair_row, topk_w, T, k, h, y);
  return hipGetLastError();
}

}  // namespace moelora
