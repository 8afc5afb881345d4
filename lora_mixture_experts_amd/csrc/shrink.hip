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
// workgroup take different runs, each over the split's whole K range. The partial sums of
// split s go to zpart[s]; consumers add the S parts in order, so the result does not depend
// on scheduling.
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

  // adapter runs of the tile: run_lo[i]..run_hi[i] share adapter run_ad[i]
  __shared__ int s_pair[16], s_ad[16], s_nrun, s_lo[16], s_hi[16], s_rad[16];
  if (tid < 16) {
    const int p = a.sorted_pairs[row0 + tid];
    s_pair[tid] = p;
    s_ad[tid] = p >= 0 ? sanitize_adapter(a.adapter_ids[p / a.k], a.nA) : -1;
  }
  __syncthreads();
  if (tid == 0) {
    int n = 0;
    for (int i = 0; i < 16;) {
      const int ad = s_ad[i];
      int j = i + 1;
      while (j < 16 && s_ad[j] == ad) ++j;
      if (ad >= 0) {
        s_lo[n] = i;
        s_hi[n] = j;
        s_rad[n] = ad;
        ++n;
      }
      i = j;
    }
    s_nrun = n;
  }
  __syncthreads();

  const int K = a.K, r = a.r;
  const int nks = K / 128;
  const int per = (nks + a.S - 1) / a.S;
  const int ks0 = min(nks, s * per), ks1 = min(nks, ks0 + per);
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

  // Each wavefront owns whole runs (run index = wave, wave + 4, ...) over this split's K range;
  // no cross-wave reduction is needed.
  for (int run = wave; run < s_nrun; run += 4) {
    const int lo = s_lo[run], hi = s_hi[run], ad = s_rad[run];
    const uint16_t* Abase = a.Aw + ((size_t)ad * a.E + e) * (size_t)r * K;
    f32x4 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int ks = ks0; ks < ks1; ++ks) {
      const int kb = ks * 128 + kq * 32;
      u32x4 xa[4], bw[4][4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) xa[jj] = bufld16(xr, xo + 2u * (uint32_t)(kb + 8 * jj));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // columns q >= r (rank 8) re-read row r-1; they are never stored
        const int q = min(c * 16 + m, r - 1);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          bw[c][jj] = c < n_ct ? ldg16(Abase + (size_t)q * K + kb + 8 * jj) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c < n_ct) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc[c] = mfma16(xa[jj], bw[c][jj], acc[c]);
        }
      }
    }
    // acc[c] holds rows 4*(lane/16)+v of column q = 16c + lane%16
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int q = c * 16 + m;
      if (c < n_ct && q < r) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = 4 * kq + v;
          if (row >= lo && row < hi) a.zpart[((size_t)s * a.cap + row0 + row) * r + q] = acc[c][v];
        }
      }
    }
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
