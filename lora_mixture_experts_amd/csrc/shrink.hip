// LoRA shrink z = x A for the rows of the sorted layout.
//
// Page "vLLM MoE LoRA SageMaker Bedrock", section "O Papel da Multi-LoRA": the shrink computes
// z = xA, reducing h_in inputs to r outputs. Section "Otimizações em Nível de Kernel": with r
// in the tens and h_in in the thousands there are few outputs and long sums, so the sum over
// K is split across thread groups that produce partial sums (split-K). Page "Punica:
// Multi-Tenant LoRA Serving": rows that share an adapter form a segment and are computed
// together against that adapter's weights.
//
// Work decomposition: one workgroup per (16-row tile of the sorted layout, K split). Rows of a
// tile belong to one expert and are sorted by adapter, so the adapters of a tile form
// contiguous runs; each run is one 16 x r x K MFMA product against A[adapter][expert]
// (rows of the tile outside the run are computed and dropped). The four wavefronts of the
// workgroup take interleaved 128-wide K steps of the split and are summed through LDS. The
// partial sums of split s go to zpart[s]; consumers add the S parts in order, so the result
// does not depend on scheduling.
#include "common.h"
#include "kernels.h"

namespace moelora {

template <bool GATHER>
__global__ __launch_bounds__(256) void lora_shrink_kernel(ShrinkArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row0 = blockIdx.x * 16;
  const int s = blockIdx.y;
  const int nblk = *a.n_blocks;
  if (row0 >= nblk * a.bm) return;
  const int e = a.block_expert[row0 / a.bm];

  __shared__ int s_pair[16], s_ad[16];
  __shared__ float red[4][16][65];
  if (tid < 16) {
    const int p = a.sorted_pairs[row0 + tid];
    s_pair[tid] = p;
    s_ad[tid] = p >= 0 ? sanitize_adapter(a.adapter_ids[p / a.k], a.nA) : -1;
  }
  __syncthreads();

  const int K = a.K, r = a.r;
  const int nks = K / 128;
  const int per = (nks + a.S - 1) / a.S;
  const int ks0 = s * per, ks1 = min(nks, ks0 + per);
  const int m = lane & 15, kq = lane >> 4;
  const int n_ct = r < 16 ? 1 : r / 16;

  // Token rows through buffer loads: a padding row gets an out-of-range offset and reads zeros
  // without touching memory (its outputs are never stored). Unconditional loads keep the
  // compiler's outstanding-load count exact.
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, a.x_bytes);
  uint32_t xo;
  {
    const int p = s_pair[m];
    xo = p < 0 ? kOutOfRange
               : (uint32_t)((GATHER ? (size_t)(p / a.k) : (size_t)(row0 + m)) * K * 2);
  }

  int i = 0;
  while (i < 16) {
    const int ad = s_ad[i];
    if (ad < 0) {
      ++i;
      continue;
    }
    int j = i + 1;
    while (j < 16 && s_ad[j] == ad) ++j;

    f32x4 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* Abase = a.Aw + ((size_t)ad * a.E + e) * (size_t)r * K;
    for (int ks = ks0 + wave; ks < ks1; ks += 4) {
      const int kb = ks * 128 + kq * 32;
      u32x4 xa[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        xa[jj] = bufld16(xr, xo + 2u * (uint32_t)(kb + 8 * jj));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c < n_ct) {
          const int q = min(c * 16 + m, r - 1);  // columns q >= r (rank 8) are never stored
          u32x4 bw[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) bw[jj] = ldg16(Abase + (size_t)q * K + kb + 8 * jj);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc[c] = mfma16(xa[jj], bw[jj], acc[c]);
        }
      }
    }
    // acc[c] holds rows 4*(lane/16)+v of column q = 16c + lane%16
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c < n_ct) {
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave][4 * kq + v][c * 16 + m] = acc[c][v];
      }
    }
    __syncthreads();
    for (int idx = tid; idx < 16 * r; idx += 256) {
      const int row = idx / r, q = idx - row * r;
      if (row >= i && row < j) {
        const float z = (red[0][row][q] + red[1][row][q]) + (red[2][row][q] + red[3][row][q]);
        a.zpart[((size_t)s * a.cap + row0 + row) * r + q] = z;
      }
    }
    __syncthreads();
    i = j;
  }
}

hipError_t launch_shrink(bool gather, const ShrinkArgs& a, int tiles, hipStream_t stream) {
  if (tiles <= 0) return hipSuccess;
  dim3 grid(tiles, a.S);
  if (gather)
    hipLaunchKernelGGL(lora_shrink_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(lora_shrink_kernel<false>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moelora
