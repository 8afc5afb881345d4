// Weighted top-k combine: y[t] = sum_j w[t][j] * D[row(t*k + j)], summed in slot order in fp32,
// then rounded once to bf16 (round-to-nearest-even). D holds the down GEMM's output rows in the
// sorted (expert, adapter) order; pair_row maps a pair to its row. D may arrive as two partial
// buffers (split-K of the down GEMM, ksplit = 2); they are added in split order first.
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
  // the pair rows and weights of all slots are loaded first, then the D rows of four slots at a
  // time (both split parts), so the slots cost a few memory round trips instead of two each
  int rows[kMaxTopk];
  float wts[kMaxTopk];
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j) {
    if (j < k) {
      wts[j] = topk_w[(size_t)t * k + j];
      rows[j] = pair_row[(size_t)t * k + j];
    }
  }
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j0 = 0; j0 < kMaxTopk; j0 += 4) {
    if (j0 >= k) break;
    f32x4 d0[4], d1[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = j0 + jj;
      d0[jj] = zero;
      d1[jj] = zero;
      if (j < k) {
        const size_t off = (size_t)rows[j] * h + c;
        d0[jj] = *reinterpret_cast<const f32x4*>(D + off);
        if (ksplit > 1) d1[jj] = *reinterpret_cast<const f32x4*>(D + split_stride + off);
      }
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = j0 + jj;
      if (j < k) {
        f32x4 d = d0[jj];
        if (ksplit > 1) d += d1[jj];  // split order
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(wts[j], d[v], acc[v]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // (keeps the next slots' loads, and registers, apart)
  }
  u32x2 packed = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  *reinterpret_cast<u32x2*>(y + (size_t)t * h + c) = packed;
}

hipError_t launch_combine(const float* D, int ksplit, int64_t split_stride, const int* pair_row,
                          const float* topk_w, int T, int k, int h, uint16_t* y,
                          hipStream_t stream) {
  const int64_t n = (int64_t)T * (h / 4);
  if (n <= 0) return hipSuccess;
  if (ksplit < 1 || ksplit > 2 || k < 1 || k > kMaxTopk) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, D,
                     ksplit, split_stride, pair_row, topk_w, T, k, h, y);
  return hipGetLastError();
}

}  // namespace moelora
