// Weighted top-k combine: y[t] = sum_j w[t][j] * D[row(t*k + j)], summed in slot order in fp32,
// then rounded once to bf16 (round-to-nearest-even). D holds the down GEMM's output rows in the
// sorted (expert, adapter) order; pair_row maps a pair to its row. D may arrive as two partial
// buffers (split-K of the down GEMM: every tile in ksplit parts, or, per tile as d_parts says,
// 1 to 4 parts); a row's parts are added in part order first.
//
// Page "vLLM MoE LoRA SageMaker Bedrock", section "Entendendo os Modelos MoE": the outputs of
// the experts a token was sent to are aggregated. Each thread owns sixteen consecutive features
// of one token, so every load and store is a full 16-byte access.
#include "common.h"
#include "kernels.h"

namespace moelora {

// MAXP: the most parts a row can have (1 or 2: every row has ksplit; 4: d_parts says).
// Each thread owns 16 consecutive features of one token: a slot's D row is read as four 16-byte
// pieces per part, so the chain of dependent loads (pair row, part count, D) is paid once per
// 64 bytes of each row.
template <int MAXP>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  constexpr int CH = 4;  // 4-feature chunks per thread
  const int h = a.h, k = a.k;
  const int hq = h / (4 * CH);
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.T * hq) return;
  const int t = (int)(idx / hq);
  const int c = (int)(idx - (int64_t)t * hq) * 4 * CH;
  f32x4 acc[CH];
#pragma unroll
  for (int q = 0; q < CH; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the pair rows and weights of all slots are loaded first, then the D rows of two slots at a
  // time (every part), so the slots cost a few memory round trips instead of two each
  int rows[kMaxTopk], np[kMaxTopk];
  float wts[kMaxTopk];
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j) {
    if (j < k) {
      wts[j] = a.topk_w[(size_t)t * k + j];
      rows[j] = a.pair_row[(size_t)t * k + j];
    }
  }
  const bool per_tile = MAXP > 2;
  const int ct = per_tile ? c / a.part_cols : 0;
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j)
    if (j < k)
      np[j] = per_tile ? a.d_parts[(size_t)(rows[j] / a.part_rows) * a.part_ncol + ct] : a.ksplit;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  constexpr int JS = 2;  // slots per batch of loads
#pragma unroll
  for (int j0 = 0; j0 < kMaxTopk; j0 += JS) {
    if (j0 >= k) break;
    f32x4 d[JS][MAXP][CH];
#pragma unroll
    for (int jj = 0; jj < JS; ++jj) {
      const int j = j0 + jj;
      const size_t off = j < k ? (size_t)rows[j] * h + c : 0;
#pragma unroll
      for (int p = 0; p < MAXP; ++p)
#pragma unroll
        for (int q = 0; q < CH; ++q) {
          d[jj][p][q] = zero;
          if (j < k && p < np[j])
            d[jj][p][q] = *reinterpret_cast<const f32x4*>(a.D + p * a.split_stride + off + 4 * q);
        }
    }
#pragma unroll
    for (int jj = 0; jj < JS; ++jj) {
      const int j = j0 + jj;
      if (j < k) {
#pragma unroll
        for (int q = 0; q < CH; ++q) {
          f32x4 dv = d[jj][0][q];
#pragma unroll
          for (int p = 1; p < MAXP; ++p)
            if (p < np[j]) dv += d[jj][p][q];  // part order
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[q][v] = __builtin_fmaf(wts[j], dv[v], acc[q][v]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // (keeps the next slots' loads, and registers, apart)
  }
  const u32x4 lo = {pack_bf16x2(acc[0][0], acc[0][1]), pack_bf16x2(acc[0][2], acc[0][3]),
                    pack_bf16x2(acc[1][0], acc[1][1]), pack_bf16x2(acc[1][2], acc[1][3])};
  const u32x4 hi = {pack_bf16x2(acc[2][0], acc[2][1]), pack_bf16x2(acc[2][2], acc[2][3]),
                    pack_bf16x2(acc[3][0], acc[3][1]), pack_bf16x2(acc[3][2], acc[3][3])};
  u32x4* yp = reinterpret_cast<u32x4*>(a.y + (size_t)t * h + c);
  yp[0] = lo;
  yp[1] = hi;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  const int64_t n = (int64_t)a.T * (a.h / 16);
  if (n <= 0) return hipSuccess;
  if (a.h % 16 != 0) return hipErrorInvalidValue;
  if (a.ksplit < 1 || a.ksplit > kMaxParts || a.k < 1 || a.k > kMaxTopk) return hipErrorInvalidValue;
  if (a.d_parts && (a.part_rows <= 0 || a.part_cols <= 0 || a.part_cols % 16 != 0))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (a.d_parts)
    hipLaunchKernelGGL(combine_kernel<kMaxParts>, grid, dim3(256), 0, stream, a);
  else if (a.ksplit == 1)
    hipLaunchKernelGGL(combine_kernel<1>, grid, dim3(256), 0, stream, a);
  else if (a.ksplit == 2)
    hipLaunchKernelGGL(combine_kernel<2>, grid, dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moelora
