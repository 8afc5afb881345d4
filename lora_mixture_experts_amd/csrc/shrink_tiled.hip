// LoRA shrink z = x A for the rows of the sorted layout, for batches with many rows per expert.
//
// Page "vLLM MoE LoRA SageMaker Bedrock", section "O Papel da Multi-LoRA": the shrink reduces
// h_in inputs to r outputs; section "Otimizações em Nível de Kernel": with few outputs and long
// sums the sum over K is split across thread groups (split-K). Page "Punica: Multi-Tenant LoRA
// Serving": rows that share an adapter form a segment computed against that adapter's weights.
//
// With hundreds of rows per expert the adapter runs (segments) are long, and the 16-row shrink
// would fetch a run's A slab once per 16 rows. Here a workgroup takes 64 rows of the sorted
// layout and one K split, and for each adapter run overlapping its rows it runs the LDS-staged
// MFMA main loop of the expert GEMMs on a 64 x 64 tile: token rows outside the run and A rows
// past r load zeros through out-of-range buffer offsets (no traffic), so the A slab of the split
// is fetched once per 64 rows and shared by the four wavefronts through LDS. The runs are the
// segments of the segment table that overlap the rows, found from the row block's first segment.
// A sub-block with more than a few runs (short runs, e.g. one token per adapter) is left to the
// 16-row shrink, launched after this one over the same rows.
// Split s writes its partial sums to zpart[s] for the run's rows; the parts are added later.
#include "common.h"
#include "kernels.h"
#include "segments.h"
#include "tile_pipeline.h"

namespace moelora {

namespace {
constexpr int kSubRows = 64;  // rows of the sorted layout per workgroup
using ShrinkPipe = TilePipe<kSubRows, 64, 32, 32, 64, 3, false, 4>;
}  // namespace

template <bool GATHER>
__global__ __launch_bounds__(256) void lora_shrink_tiled_kernel(ShrinkArgs a) {
  using Pipe = ShrinkPipe;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // Pipe::LDS_BYTES
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / Pipe::WAVES_N, wn = wave % Pipe::WAVES_N;
  const int fr = lane & 31, fg = lane >> 5;

  // (64-row sub-block, split) items, split by split; each XCD takes an equal contiguous range
  // (neighbouring sub-blocks of one run and split share their A slab in its L2)
  const int live_sub = *a.n_blocks * a.bm / kSubRows;
  const int live = live_sub * a.S;
  const int per_xcd = (live + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  const int item = (blockIdx.x & 7) * per_xcd + slot;
  if (slot >= per_xcd || item >= live) return;
  const int s = item / live_sub;
  const int row0 = (item - s * live_sub) * kSubRows;
  const int blk = row0 / a.bm;
  const int e = a.block_expert[blk];
  const int first = a.block_seg[blk];
  if (first < 0) return;
  const int nseg = *a.n_seg;
  // sub-blocks of many short runs are left to the 16-row shrink
  if (count_runs64(a.block_seg, a.seg_table, nseg, a.nA, blk, row0, kShrink64MaxRuns) >
      kShrink64MaxRuns)
    return;
  const int K = a.K, r = a.r;
  // split s: the same 128-wide K steps as the 16-row shrink's split s
  const int nks = K / 128;
  const int per = (nks + a.S - 1) / a.S;
  const int ks0 = min(nks, s * per), ks1 = min(nks, ks0 + per);
  const int kspan = (ks1 - ks0) * 128;
  const uint32_t kbyte0 = (uint32_t)ks0 * 256;

  // per-lane token-row offsets of the A-operand loads (before run masking) and A-slab row
  // offsets of the B-operand loads
  uint32_t xrow[Pipe::NA], ao[Pipe::NB];
  int trow[Pipe::NA];
#pragma unroll
  for (int i = 0; i < Pipe::NA; ++i) {
    const int row = Pipe::load_row(i, wave, lane);
    const int chunk = Pipe::load_chunk(row, lane);
    trow[i] = row;
    const int p = a.sorted_pairs[row0 + row];
    xrow[i] = p < 0 ? kOutOfRange
                    : (uint32_t)((GATHER ? (size_t)(p / a.k) : (size_t)(row0 + row)) * K * 2) +
                          kbyte0 + 16u * chunk;
  }
#pragma unroll
  for (int i = 0; i < Pipe::NB; ++i) {
    const int q = Pipe::load_row(i, wave, lane);
    const int chunk = Pipe::load_chunk(q, lane);
    ao[i] = q < r ? (uint32_t)(q * K * 2) + kbyte0 + 16u * chunk : kOutOfRange;
  }
  const u32x4 xr = buffer_desc(a.X, a.x_bytes);

  for (int c0 = first;; c0 += 64) {
    // lane j: segment c0 + j clipped to the sub-block (segments from the block's first one on
    // start in order; those that end before the sub-block are skipped)
    const int sj = c0 + lane;
    int lo = 0, hi = 0, ad = -1;
    bool before_end = false;
    if (sj < nseg) {
      const u32x4 sg = *reinterpret_cast<const u32x4*>(a.seg_table + 4 * (size_t)sj);
      const int st = (int)sg[2], cnt = (int)sg[3];
      before_end = st < row0 + kSubRows;
      lo = max(st - row0, 0);
      hi = min(st + cnt - row0, kSubRows);
      ad = sanitize_adapter((int)sg[1], a.nA);
    }
    const uint64_t more = __ballot(before_end);
    uint64_t runs = __ballot(before_end && hi > lo && ad >= 0);
    while (runs) {
      const int j = __builtin_ctzll(runs);
      runs &= runs - 1;
      const int rlo = __builtin_amdgcn_readlane(lo, j), rhi = __builtin_amdgcn_readlane(hi, j);
      const int rad = __builtin_amdgcn_readlane(ad, j);
      uint32_t xo[Pipe::NA];
#pragma unroll
      for (int i = 0; i < Pipe::NA; ++i)
        xo[i] = (trow[i] >= rlo && trow[i] < rhi) ? xrow[i] : kOutOfRange;
      const u32x4 ar = buffer_desc(a.Aw + ((size_t)rad * a.E + e) * (size_t)r * K,
                                   (uint32_t)((size_t)r * K * 2));
      f32x16 acc[1][1];
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[0][0][v] = 0.f;
      __syncthreads();  // every wavefront is done with the previous run's LDS stages
      if (kspan > 0) Pipe::run(acc, xr, xo, ar, ao, lds, kspan, wave, lane);
      // lane: rows wm*32 + 8*(v/4) + 4*fg + (v%4), rank column wn*32 + fr
      const int q = wn * 32 + fr;
      if (q < r) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * 32 + 8 * (v / 4) + 4 * fg + (v % 4);
          if (row >= rlo && row < rhi)
            a.zpart[((size_t)s * a.cap + row0 + row) * r + q] = acc[0][0][v];
        }
      }
    }
    if (!(more >> 63)) break;
  }
}

hipError_t launch_shrink_tiled(bool gather, const ShrinkArgs& a, int n_sub_max,
                               hipStream_t stream) {
  if (n_sub_max <= 0) return hipSuccess;
  if (a.r > 64 || a.bm % kSubRows != 0 || a.K % 128 != 0) return hipErrorInvalidValue;
  constexpr int lds_bytes = ShrinkPipe::LDS_BYTES;
  dim3 grid((unsigned)(((int64_t)n_sub_max * a.S + 7) / 8 * 8));
  if (gather)
    hipLaunchKernelGGL(lora_shrink_tiled_kernel<true>, grid, dim3(256), lds_bytes, stream, a);
  else
    hipLaunchKernelGGL(lora_shrink_tiled_kernel<false>, grid, dim3(256), lds_bytes, stream, a);
  return hipGetLastError();
}

}  // namespace moelora
