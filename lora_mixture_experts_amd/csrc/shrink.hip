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
// contiguous runs; each run is one 16 x r x K MFMA product against A[adapter][expert] in which
// only the run's rows load x (the other rows read zeros through out-of-range buffer offsets,
// at no memory traffic, and their outputs are dropped). The shrink streams A (r x K per run).
// With one or two runs the four wavefronts share each run, splitting the split's K range;
// with more they take whole runs in parallel. A wavefront keeps the loads of its next 128-wide
// K step in flight while the current one is multiplied; the partial products of wavefronts
// sharing a run are added in LDS in wavefront order. The partial sums of split s go to
// zpart[s]; consumers add the S parts in order, so the result does not depend on scheduling.
#include "common.h"
#include "kernels.h"
#include "segments.h"

namespace moelora {

// NCT: 16-column tiles of z (rank 8 and 16: 1, 32: 2, 64: 4).
template <bool GATHER, int NCT>
__global__ __launch_bounds__(256) void lora_shrink_kernel(ShrinkArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Work order. With long adapter runs (xcd_ranges) the live (16-row tile, split) items are
  // numbered split by split, tile by tile, and each XCD (hardware workgroup ids go round-robin
  // over the 8) is given an equal contiguous range, so that neighbouring tiles of one run and
  // split run on one XCD and share the A slab of their K range in its L2. Otherwise the S splits
  // of a tile take consecutive ids: the tile follows from the id alone, so the tile's rows are
  // fetched together with the live row count instead of after it.
  int s, row0;
  if (a.xcd_ranges) {
    const int live16 = *a.n_blocks * a.bm / 16;
    const int live = live16 * a.S;
    const int per_xcd = (live + 7) >> 3;
    const int slot = blockIdx.x >> 3;
    if (slot >= per_xcd) return;
    const int item = (blockIdx.x & 7) * per_xcd + slot;
    if (item >= live) return;
    s = item / live16;
    row0 = (item - s * live16) * 16;
  } else {
    const int tile = blockIdx.x / a.S;
    s = blockIdx.x - tile * a.S;
    row0 = tile * 16;
    if (row0 + 16 > a.cap) return;  // (ids of the grid's round-up to the 8 XCDs)
  }
  // rows, adapters and expert of the tile (a tile past the live rows reads stale entries of the
  // sorted layout, inside its capacity, and leaves)
  __shared__ int s_pair[16], s_ad[16], s_nrun, s_lo[16], s_hi[16], s_rad[16];
  if (tid < 16) {
    s_pair[tid] = a.sorted_pairs[row0 + tid];
    s_ad[tid] = a.sorted_ad[row0 + tid];
  }
  const int e = a.block_expert[row0 / a.bm];
  if (!a.xcd_ranges && row0 >= *a.n_blocks * a.bm) return;
  // with the 64-row shrink, only the tiles of sub-blocks it leaves (many short runs)
  if (a.after64 && count_runs64(a.block_seg, a.seg_table, *a.n_seg, a.nA, row0 / a.bm,
                                row0 & ~63, kShrink64MaxRuns) <= kShrink64MaxRuns)
    return;
  __syncthreads();
  // adapter runs of the tile: rows s_lo[i] .. s_hi[i] - 1 share adapter s_rad[i] (rows without
  // an adapter belong to no run). A run starts where the adapter changes; lanes 0-15 of the
  // first wavefront hold the rows.
  if (wave == 0) {
    const int ad = lane < 16 ? s_ad[lane] : -2;
    const int prev = (lane >= 1 && lane < 16) ? s_ad[lane - 1] : -2;
    const bool change = lane < 16 && (lane == 0 || ad != prev);
    const uint64_t chg = __ballot(change);
    const uint64_t starts = __ballot(change && ad >= 0);
    if (change && ad >= 0) {
      const int idx = (int)__popcll(starts & lanemask_lt());
      const uint64_t later = chg & ~((2ull << lane) - 1ull);  // lane < 16
      s_lo[idx] = lane;
      s_hi[idx] = later ? (int)__ffsll((unsigned long long)later) - 1 : 16;
      s_rad[idx] = ad;
    }
    if (lane == 0) s_nrun = (int)__popcll(starts);
  }
  __syncthreads();

  const int nrun = s_nrun;
  if (nrun == 0) return;
  // ng groups of gs wavefronts (ng: the smallest power of two >= min(nrun, 4)); a group takes
  // every ng-th run and its members split the run's K range of this split
  const int ng = nrun >= 3 ? 4 : nrun;
  const int gs = 4 / ng;
  const int grp = wave / gs, mem = wave % gs;

  const int K = a.K, r = a.r;
  const int nks = K / 128;
  const int per = (nks + a.S - 1) / a.S;
  const int ks0 = min(nks, s * per), ks1 = min(nks, ks0 + per);
  // this wavefront's share of the split (contiguous 128-wide steps)
  const int wper = (ks1 - ks0 + gs - 1) / gs;
  const int w0 = min(ks1, ks0 + mem * wper), w1 = min(ks1, w0 + wper);
  const int m = lane & 15, kq = lane >> 4;

  __shared__ f32x4 s_part[4][NCT][64];  // [wave][column tile][lane]

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, a.x_bytes);
  const int p_m = s_pair[m];
  const uint32_t x_row_off =
      p_m < 0 ? kOutOfRange
              : (uint32_t)((GATHER ? (size_t)(p_m / a.k) : (size_t)(row0 + m)) * K * 2);

  // every group runs the same number of rounds, so the barriers below are uniform
  const int rounds = (nrun + ng - 1) / ng;
  for (int round = 0; round < rounds; ++round) {
    const int run = round * ng + grp;
    const bool active = run < nrun;
    const int lo = active ? s_lo[run] : 0, hi = active ? s_hi[run] : 0;
    // uniform: the A descriptor must live in scalar registers (from a value the compiler cannot
    // prove uniform it would build a per-lane loop around every load)
    const int ad = __builtin_amdgcn_readfirstlane(active ? s_rad[run] : 0);
    // rows outside the run (all rows, for an idle group) read zeros without touching memory
    const uint32_t xo = (m >= lo && m < hi) ? x_row_off : kOutOfRange;
    const __amdgpu_buffer_rsrc_t ar =
        make_rsrc(a.Aw + ((size_t)ad * a.E + e) * (size_t)r * K, (uint32_t)((size_t)r * K * 2));
    // A rows q >= r (rank 8) read zeros as well; they are never stored
    uint32_t ao[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int q = c * 16 + m;
      ao[c] = (active && q < r) ? (uint32_t)((size_t)q * K * 2) : kOutOfRange;
    }
    f32x4 acc[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 xa0[4], bw0[NCT][4], xa1[4], bw1[NCT][4];
    // step ks covers k in [128 ks, 128 ks + 128); MFMA jj takes k = 32 jj + 8 kq .. + 8 from lane
    // (m, kq), so each load instruction reads 64 contiguous bytes of every row it touches
    auto load = [&](int ks, u32x4* xa, u32x4 (*bw)[4]) {
      const uint32_t kb = (uint32_t)(ks * 128 + kq * 8) * 2;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) xa[jj] = bufld16(xr, xo + kb + 64u * jj);
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) bw[c][jj] = bufld16(ar, ao[c] + kb + 64u * jj);
    };
    auto mma = [&](const u32x4* xa, const u32x4 (*bw)[4]) {
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[c] = mfma16(xa[jj], bw[c][jj], acc[c]);
    };
    // Steps in pairs with ping-pong register sets (the loads of the next step are in flight
    // while the current one is multiplied), then an odd last step. Every load is
    // unconditional (past the end it re-reads the last step), and no branch encloses an MFMA.
    const int n = w1 - w0;
    if (n > 0) {
      load(w0, xa0, bw0);
      int i = 0;
      for (; i + 2 <= n; i += 2) {
        load(w0 + i + 1, xa1, bw1);
        __builtin_amdgcn_sched_barrier(0);
        mma(xa0, bw0);
        __builtin_amdgcn_sched_barrier(0);
        load(min(w0 + i + 2, w1 - 1), xa0, bw0);
        __builtin_amdgcn_sched_barrier(0);
        mma(xa1, bw1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i < n) mma(xa0, bw0);
    }
    // acc[c] holds rows 4*(lane/16)+v of column q = 16c + lane%16
    auto store = [&](int c, f32x4 t) {
      const int q = c * 16 + m;
      if (q < r) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = 4 * kq + v;
          if (row >= lo && row < hi) a.zpart[((size_t)s * a.cap + row0 + row) * r + q] = t[v];
        }
      }
    };
    if (gs == 1) {
      if (active) {
#pragma unroll
        for (int c = 0; c < NCT; ++c) store(c, acc[c]);
      }
      continue;
    }
    // partials of the group's wavefronts -> LDS; its first wavefront adds them in order
#pragma unroll
    for (int c = 0; c < NCT; ++c) s_part[wave][c][lane] = acc[c];
    __syncthreads();
    if (active && mem == 0) {
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        f32x4 t = s_part[wave][c][lane];
        for (int j = 1; j < gs; ++j) t += s_part[wave + j][c][lane];
        store(c, t);
      }
    }
    __syncthreads();  // s_part is reused by the next round
  }
}

// Segment shrink, for layouts whose adapter runs are short (a few rows per expert, many
// adapters): one wavefront per (adapter segment, K split), where the 16-row shrink walks the
// runs of a tile one after another. The segment table gives the run (expert, adapter, first
// row, rows), so the A loads of the split are issued as soon as the table entry has arrived,
// next to the row ids; a run's rows are taken 16 at a time (one 16 x r x K product each, rows
// past the run load zeros). Each wavefront keeps two 128-wide K steps of loads in flight (the
// same step order and split boundaries as the 16-row shrink) and writes the run's rows of
// zpart[s]; the wavefronts of a workgroup are independent (no LDS, no barrier). After the
// 64-row shrink (after64) it takes only the rows of the 64-row sub-blocks that one leaves (more
// than kShrink64MaxRuns runs), so every row is written by one of the two.
template <bool GATHER, int NCT>
__global__ __launch_bounds__(256) void lora_shrink_seg_kernel(ShrinkArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int task = blockIdx.x * 4 + wave;
  const int j = task / a.S, s = task - j * a.S;  // the S splits of a segment on neighbours
  if (j >= *a.n_seg) return;
  const u32x4 sg = *reinterpret_cast<const u32x4*>(a.seg_table + 4 * (size_t)j);
  const int e = __builtin_amdgcn_readfirstlane((int)sg[0]);
  const int ad = __builtin_amdgcn_readfirstlane(sanitize_adapter((int)sg[1], a.nA));
  const int st = __builtin_amdgcn_readfirstlane((int)sg[2]);
  const int cnt = __builtin_amdgcn_readfirstlane((int)sg[3]);
  if (ad < 0 || cnt <= 0) return;
  const int K = a.K, r = a.r;
  const int nks = K / 128;
  const int per = (nks + a.S - 1) / a.S;
  const int ks0 = min(nks, s * per), ks1 = min(nks, ks0 + per);
  const int n = ks1 - ks0;
  if (n <= 0) return;
  const int m = lane & 15, kq = lane >> 4;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, a.x_bytes);
  const __amdgpu_buffer_rsrc_t ar =
      make_rsrc(a.Aw + ((size_t)ad * a.E + e) * (size_t)r * K, (uint32_t)((size_t)r * K * 2));
  uint32_t ao[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int q = c * 16 + m;
    ao[c] = q < r ? (uint32_t)((size_t)q * K * 2) : kOutOfRange;
  }
  const int nseg = *a.n_seg;
  for (int c0 = 0; c0 < cnt; c0 += 16) {
    // take: bit i for row st + c0 + i. After the 64-row shrink, the rows of the 64-row
    // sub-blocks it took (few runs) are not this kernel's.
    uint32_t take = 0xffffu;
    if (a.after64) {
      const int r0 = st + c0, r1 = st + min(cnt, c0 + 16) - 1;
      const int sb0 = r0 & ~63, sb1 = r1 & ~63;
      const bool many0 = count_runs64(a.block_seg, a.seg_table, nseg, a.nA, sb0 / a.bm, sb0,
                                      kShrink64MaxRuns) > kShrink64MaxRuns;
      const bool many1 = sb1 == sb0 ? many0
                                    : count_runs64(a.block_seg, a.seg_table, nseg, a.nA,
                                                   sb1 / a.bm, sb1, kShrink64MaxRuns) >
                                          kShrink64MaxRuns;
      const int in0 = min(16, sb0 + 64 - r0);  // rows of the chunk in sub-block sb0
      const uint32_t m0 = (1u << in0) - 1u;
      take = (many0 ? m0 : 0u) | (many1 ? (0xffffu & ~m0) : 0u);
      if (take == 0u) continue;
    }
    const bool mine = c0 + m < cnt && ((take >> m) & 1u);
    const int p = mine ? a.sorted_pairs[st + c0 + m] : -1;
    const uint32_t xo =
        p < 0 ? kOutOfRange
              : (uint32_t)((GATHER ? (size_t)(p / a.k) : (size_t)(st + c0 + m)) * K * 2);
    f32x4 acc[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 xa0[4], bw0[NCT][4], xa1[4], bw1[NCT][4];
    // step ks covers k in [128 ks, 128 ks + 128); MFMA jj takes k = 32 jj + 8 kq .. + 8
    auto load_a = [&](int ks, u32x4 (*bw)[4]) {
      const uint32_t kb = (uint32_t)(ks * 128 + kq * 8) * 2;
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) bw[c][jj] = bufld16(ar, ao[c] + kb + 64u * jj);
    };
    auto load_x = [&](int ks, u32x4* xa) {
      const uint32_t kb = (uint32_t)(ks * 128 + kq * 8) * 2;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) xa[jj] = bufld16(xr, xo + kb + 64u * jj);
    };
    auto mma = [&](const u32x4* xa, const u32x4 (*bw)[4]) {
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[c] = mfma16(xa[jj], bw[c][jj], acc[c]);
    };
    // steps in pairs with ping-pong register sets; every load is unconditional (past the end it
    // re-reads the last step) and no branch encloses an MFMA
    load_a(ks0, bw0);
    load_x(ks0, xa0);
    int i = 0;
    for (; i + 2 <= n; i += 2) {
      load_a(ks0 + i + 1, bw1);
      load_x(ks0 + i + 1, xa1);
      __builtin_amdgcn_sched_barrier(0);
      mma(xa0, bw0);
      __builtin_amdgcn_sched_barrier(0);
      const int nx = min(ks0 + i + 2, ks1 - 1);
      load_a(nx, bw0);
      load_x(nx, xa0);
      __builtin_amdgcn_sched_barrier(0);
      mma(xa1, bw1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (i < n) mma(xa0, bw0);
    // acc[c] holds rows 4 kq + v of the chunk, column q = 16 c + m
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int q = c * 16 + m;
      if (q < r) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = c0 + 4 * kq + v;
          if (row < cnt && ((take >> (4 * kq + v)) & 1u))
            a.zpart[((size_t)s * a.cap + st + row) * r + q] = acc[c][v];
        }
      }
    }
  }
}

hipError_t launch_shrink_seg(bool gather, const ShrinkArgs& a, int max_segments,
                             hipStream_t stream) {
  if (max_segments <= 0) return hipSuccess;
  if (a.S < 1 || a.S > kMaxSplit || a.K % 128 != 0) return hipErrorInvalidValue;
  dim3 grid((unsigned)(((int64_t)max_segments * a.S + 3) / 4));
#define MOELORA_SHRINK_SEG(NCT_)                                                             \
  if (gather)                                                                                \
    hipLaunchKernelGGL((lora_shrink_seg_kernel<true, NCT_>), grid, dim3(256), 0, stream, a);  \
  else                                                                                       \
    hipLaunchKernelGGL((lora_shrink_seg_kernel<false, NCT_>), grid, dim3(256), 0, stream, a);
  if (a.r <= 16) {
    MOELORA_SHRINK_SEG(1)
  } else if (a.r == 32) {
    MOELORA_SHRINK_SEG(2)
  } else if (a.r == 64) {
    MOELORA_SHRINK_SEG(4)
  } else {
    return hipErrorInvalidValue;
  }
#undef MOELORA_SHRINK_SEG
  return hipGetLastError();
}

// z for the LDS-tiled GEMM epilogues: the S split parts of each row added in split order, once
// (every workgroup reading a row's z then loads it once instead of S times), and split into bf16
// high and low parts (hi = bf16(z), lo = bf16(z - hi)), written as two planes [cap][r] that
// their epilogue loads straight into MFMA operands. One thread per 8 consecutive values of a
// row; rows past the live row blocks are skipped. (The skinny GEMMs and the dense multi-LoRA
// expand add the parts themselves.)
__global__ __launch_bounds__(256) void zfinal_kernel(const float* __restrict__ zpart, int S,
                                                     int64_t cap, int r,
                                                     const int* __restrict__ n_blocks, int bm,
                                                     uint16_t* __restrict__ zhl) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = r / 8;
  const int64_t row = idx / per_row;
  if (row >= (int64_t)*n_blocks * bm) return;
  const int q = (int)(idx - row * per_row) * 8;
  f32x4 z0 = *reinterpret_cast<const f32x4*>(zpart + row * r + q);
  f32x4 z1 = *reinterpret_cast<const f32x4*>(zpart + row * r + q + 4);
  for (int sp = 1; sp < S; ++sp) {
    const float* src = zpart + (sp * cap + row) * r + q;
    z0 += *reinterpret_cast<const f32x4*>(src);
    z1 += *reinterpret_cast<const f32x4*>(src + 4);
  }
  uint32_t hb[8], lb[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float z = t < 4 ? z0[t] : z1[t - 4];
    hb[t] = f32_to_bf16_bits(z);
    lb[t] = f32_to_bf16_bits(z - __uint_as_float(hb[t] << 16));
  }
  *reinterpret_cast<u32x4*>(zhl + row * r + q) =
      u32x4{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16), hb[6] | (hb[7] << 16)};
  *reinterpret_cast<u32x4*>(zhl + (cap + row) * r + q) =
      u32x4{lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16), lb[4] | (lb[5] << 16), lb[6] | (lb[7] << 16)};
}

hipError_t launch_zfinal(const float* zpart, int S, int64_t cap, int r, const int* n_blocks,
                         int bm, int64_t max_rows, uint16_t* zhl, hipStream_t stream) {
  if (r % 8 != 0 || zhl == nullptr || S < 1 || S > kMaxSplit) return hipErrorInvalidValue;
  const int64_t n = max_rows * (r / 8);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zfinal_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, zpart,
                     S, cap, r, n_blocks, bm, zhl);
  return hipGetLastError();
}

hipError_t launch_shrink(bool gather, const ShrinkArgs& a, int tiles, hipStream_t stream) {
  if (tiles <= 0) return hipSuccess;
  // (tile, split) items for the largest row-block count, rounded up to a multiple of the 8 XCDs
  dim3 grid((unsigned)(((int64_t)tiles * a.S + 7) / 8 * 8));
#define MOELORA_SHRINK(NCT_)                                                           \
  if (gather)                                                                          \
    hipLaunchKernelGGL((lora_shrink_kernel<true, NCT_>), grid, dim3(256), 0, stream, a); \
  else                                                                                 \
    hipLaunchKernelGGL((lora_shrink_kernel<false, NCT_>), grid, dim3(256), 0, stream, a);
  if (a.r <= 16) {
    MOELORA_SHRINK(1)
  } else if (a.r == 32) {
    MOELORA_SHRINK(2)
  } else if (a.r == 64) {
    MOELORA_SHRINK(4)
  } else {
    return hipErrorInvalidValue;
  }
#undef MOELORA_SHRINK
  return hipGetLastError();
}

}  // namespace moelora
