// Expert GEMMs for many rows per expert (prefill): MFMA-bound, so weight and token tiles are
// staged through LDS and reused across a 2-D workgroup tile.
//
// Page "vLLM MoE LoRA SageMaker Bedrock", section "Entendendo os Modelos MoE" (gate_up expands
// the hidden state, down compresses it back); section "O Papel da Multi-LoRA" (y = xW + xAB,
// the expand z B added to the base output); section "Otimizações em Nível de Kernel" (the LoRA
// add fused into the kernel producing the base output, no masks when K divides the block, and
// workgroup ordering so neighbouring tiles reuse L2). Page "Punica: Multi-Tenant LoRA Serving",
// proposed-method section: tokens of one adapter form a segment that is multiplied by that
// adapter's weights in one batched operation.
//
// C[m][n] = sum_k X[m][k] W[n][k] for the BM token rows of one row block of the sorted layout
// (all of one expert) and BN output features, on 32x32x16 bf16 MFMAs (the 16x16x32 form runs at
// half their rate on CDNA4). Both operands are K-contiguous, so every fragment (32 rows x 8
// consecutive k per lane) is one 16-byte LDS read. Tiles live row-major in LDS, 64 k per row,
// with the 16-byte chunk index XOR-swizzled by the row; LDS is double-buffered with one barrier
// per 64-wide K step, global tiles are prefetched DEPTH steps ahead in registers, and the
// fragments of the next 16-wide sub-step are read while the current sub-step's MFMAs run.
//
// gate_up: the weight rows of each wave's column range are [gate i .. | up i ..] for the same
// intermediate columns i, so each lane holds gate and up of the same act element and
// SiLU-and-mul runs in registers, after the LoRA expand is added.
//
// LoRA expand (both projections): rows are sorted by adapter inside an expert, so each 32-row
// MFMA group holds a few contiguous adapter runs. For every run the group's z rows (other rows
// zero) multiply B[adapter][expert] as extra MFMAs over K = r: the segment's adapter weights are
// read once per group, not per token. z is split into bf16 high and low parts (two MFMAs) so
// the term keeps ~16 mantissa bits.
#include "common.h"
#include "kernels.h"

namespace moelora {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// D += A(32x16) * B(16x32). Lane l supplies row (l % 32) of A and column (l % 32) of B, 8
// reduction elements each, in the same slot order; lane l receives D rows
// 8*(v/4) + 4*(l/32) + (v%4), v < 16, of column (l % 32).
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

template <bool GATEUP, int BM, int BN, int WM, int WN, int DEPTH, int OCC>
__global__ __launch_bounds__(256, OCC) void tiled_gemm_kernel(GemmArgs a, int n_tiles_n,
                                                              int grid_total) {
  constexpr int BK = 64;
  constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static_assert(WAVES_M * WAVES_N == 4, "four wavefronts per workgroup");
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int CPR = BK / 8;                  // 16-byte chunks per tile row
  constexpr int CA = BM * CPR / 256;           // chunks of the token tile per thread
  constexpr int CB = BN * CPR / 256;           // chunks of the weight tile per thread
  static_assert(CA * 256 == BM * CPR && CB * 256 == BN * CPR, "tile must split over 256 threads");
  static_assert(!GATEUP || FN % 2 == 0, "gate_up needs gate and up halves per wave");
  // a sub-step's reads are all complete before its first MFMA and the next sub-step's reads are
  // interleaved after it, so at most FM + FN reads are outstanding (the LDS counter holds 15)
  static_assert(FM + FN <= 15, "one sub-step of fragment reads must fit the LDS counter");

  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // 2 * (BM + BN) * BK

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // Tile order. Hardware workgroup ids go round-robin over the 8 XCDs, so each XCD is given a
  // contiguous range of logical tiles; the ~64 workgroups an XCD runs at once then cover a
  // group of GROUP_M row blocks x GROUP_N column tiles, and every token tile and weight tile
  // fetched into that XCD's L2 serves GROUP_N resp. GROUP_M workgroups (instead of streaming
  // every token tile once per column tile).
  constexpr int GROUP_M = 8, GROUP_N = 8;
  const int hw = blockIdx.x;
  const int logical = (hw & 7) * (grid_total >> 3) + (hw >> 3);
  const int groups_m = (a.n_blocks_max + GROUP_M - 1) / GROUP_M;
  const int grp = logical / (GROUP_M * GROUP_N), within = logical % (GROUP_M * GROUP_N);
  const int blk = (grp % groups_m) * GROUP_M + within % GROUP_M;
  const int ntile = (grp / groups_m) * GROUP_N + within / GROUP_M;
  if (ntile >= n_tiles_n || blk >= a.n_blocks_max || blk >= *a.n_blocks) return;
  const int e = a.block_expert[blk];
  const int K = a.K;
  const size_t N = (size_t)a.N;  // gate_up: I; down: h
  const int row0 = blk * BM;

  // ---- per-thread global load plan (fixed over K) ----
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, a.x_bytes);
  uint32_t xo[CA];
  int a_lds[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int q = tid + 256 * i;
    const int row = q / CPR, chk = q % CPR;
    a_lds[i] = row * BK + 8 * (chk ^ (row & 7));
    const int srow = row0 + row;
    const int p = a.sorted_pairs[srow];
    xo[i] = p < 0 ? kOutOfRange
                  : (uint32_t)((GATEUP ? (size_t)(p / a.k) : (size_t)srow) * K * 2) + 16u * chk;
  }
  const uint16_t* wsrc[CB];
  int b_lds[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int q = tid + 256 * i;
    const int row = q / CPR, chk = q % CPR;
    b_lds[i] = row * BK + 8 * (chk ^ (row & 7));
    size_t wrow;
    if (GATEUP) {
      const int g = row / WN, rr = row % WN;
      const size_t col = (size_t)ntile * (BN / 2) + g * (WN / 2) + (rr % (WN / 2));
      wrow = (size_t)e * 2 * N + (rr < WN / 2 ? col : N + col);
    } else {
      wrow = (size_t)e * N + (size_t)ntile * BN + row;
    }
    wsrc[i] = a.W + wrow * K + 8 * chk;
  }

  auto lds_a = [&](int buf) { return lds + buf * (BM + BN) * BK; };
  auto lds_b = [&](int buf) { return lds + buf * (BM + BN) * BK + BM * BK; };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nks = K / BK;
  u32x4 sa0[CA], sb0[CB], sa1[CA], sb1[CB];
  // Loads are unconditional (past the end they re-read the last step), which keeps the
  // compiler's outstanding-load count exact.
#define MOELORA_GLOAD(SA, SB, KS)                                                         \
  do {                                                                                    \
    const int ks_ = min((KS), nks - 1);                                                   \
    _Pragma("unroll") for (int i = 0; i < CA; ++i) SA[i] =                                \
        bufld16(xr, xo[i] + 2u * (uint32_t)(ks_ * BK));                                   \
    _Pragma("unroll") for (int i = 0; i < CB; ++i) SB[i] = ldg16(wsrc[i] + (size_t)ks_ * BK); \
  } while (0)
#define MOELORA_LSTORE(SA, SB, BUF)                                                       \
  do {                                                                                    \
    uint16_t* A_ = lds_a(BUF);                                                            \
    uint16_t* B_ = lds_b(BUF);                                                            \
    _Pragma("unroll") for (int i = 0; i < CA; ++i)                                        \
        *reinterpret_cast<u32x4*>(A_ + a_lds[i]) = SA[i];                                 \
    _Pragma("unroll") for (int i = 0; i < CB; ++i)                                        \
        *reinterpret_cast<u32x4*>(B_ + b_lds[i]) = SB[i];                                 \
  } while (0)

  const int fr = lane & 31, fg = lane >> 5;
  // Fragments of 16-wide sub-step j of a 64-wide K step: chunk 2j + (lane / 32).
  auto read_frags = [&](const uint16_t* A, const uint16_t* B, int j, u32x4* af, u32x4* bf) {
    const int chunk = 2 * j + fg;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WM + i * 32 + fr;
      af[i] = *reinterpret_cast<const u32x4*>(A + r * BK + 8 * (chunk ^ (r & 7)));
    }
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int r = wn * WN + i * 32 + fr;
      bf[i] = *reinterpret_cast<const u32x4*>(B + r * BK + 8 * (chunk ^ (r & 7)));
    }
  };
  auto mfmas = [&](const u32x4* af, const u32x4* bf) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jn = 0; jn < FN; ++jn) acc[i][jn] = mfma32(af[i], bf[jn], acc[i][jn]);
  };
  // Four sub-steps; sub-step j+1's reads are issued between sub-step j's MFMAs.
  auto compute = [&](int buf) {
    const uint16_t* A = lds_a(buf);
    const uint16_t* B = lds_b(buf);
    u32x4 af0[FM], bf0[FN], af1[FM], bf1[FN];
    read_frags(A, B, 0, af0, bf0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4* an = (j & 1) ? af0 : af1;
      u32x4* bn = (j & 1) ? bf0 : bf1;
      const u32x4* ac = (j & 1) ? af1 : af0;
      const u32x4* bc = (j & 1) ? bf1 : bf0;
      if (j < 3) read_frags(A, B, j + 1, an, bn);
      mfmas(ac, bc);
      if (j < 3) {
        constexpr int NR = FM + FN;
        constexpr int NM = FM * FN;
        constexpr int PAIRS = NR < NM ? NR : NM;
#pragma unroll
        for (int t = 0; t < PAIRS; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        if (NR > NM) __builtin_amdgcn_sched_group_barrier(0x100, NR - NM, 0);
        if (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  MOELORA_GLOAD(sa0, sb0, 0);
  if (DEPTH == 2) MOELORA_GLOAD(sa1, sb1, 1);
  MOELORA_LSTORE(sa0, sb0, 0);
  __syncthreads();
  // sched_barrier(0) pins the phase order (the compiler would otherwise sink the prefetch below
  // the MFMAs). The LDS stores are unconditional as well (past the end they fill a buffer nobody
  // reads), so the in-flight load count stays exact.
  if (DEPTH == 2) {
    // K is a multiple of 128, so the number of 64-wide steps is even
    for (int ks = 0; ks < nks; ks += 2) {
      MOELORA_GLOAD(sa0, sb0, ks + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(0);
      __builtin_amdgcn_sched_barrier(0);
      MOELORA_LSTORE(sa1, sb1, 1);
      __syncthreads();
      MOELORA_GLOAD(sa1, sb1, ks + 3);
      __builtin_amdgcn_sched_barrier(0);
      compute(1);
      __builtin_amdgcn_sched_barrier(0);
      MOELORA_LSTORE(sa0, sb0, 0);
      __syncthreads();
    }
  } else {
    for (int ks = 0; ks < nks; ++ks) {
      const int buf = ks & 1;
      MOELORA_GLOAD(sa1, sb1, ks + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(buf);
      __builtin_amdgcn_sched_barrier(0);
      MOELORA_LSTORE(sa1, sb1, buf ^ 1);
      __syncthreads();
    }
  }
#undef MOELORA_GLOAD
#undef MOELORA_LSTORE

  // ---- epilogue ----
  // Weight row (within W1 or W2 of expert e) of column fragment jn for this lane's column.
  auto wrow_of = [&](int jn) -> size_t {
    if (GATEUP) {
      const int half = FN / 2;
      const size_t col = (size_t)ntile * (BN / 2) + wn * (WN / 2) + (jn % half) * 32 + fr;
      return jn < half ? col : N + col;
    }
    return (size_t)ntile * BN + wn * WN + jn * 32 + fr;
  };

  const int r = a.r;
  const int64_t zstride = a.cap * r;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int grow0 = row0 + wm * WM + i * 32;  // first sorted row of this 32-row group
    int ad = -1;
    {
      const int p = a.sorted_pairs[grow0 + fr];
      if (p >= 0) ad = sanitize_adapter(a.adapter_ids[p / a.k], a.nA);
    }
    uint64_t pending = __ballot(lane < 32 && ad >= 0);
    while (pending) {
      const int first = __ffsll((unsigned long long)pending) - 1;
      const int acur = __shfl(ad, first);
      const uint64_t run = __ballot(lane < 32 && ad == acur);
      pending &= ~run;
      const bool mine = (run >> fr) & 1ull;
      const uint16_t* Bad = a.Bw + ((size_t)acur * a.E + e) * (GATEUP ? 2 * N : N) * r;
      for (int q0 = 0; q0 < r; q0 += 16) {
        const int q = q0 + 8 * fg;  // this lane's 8 reduction slots
        float z[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) z[t] = 0.f;
        if (mine && q < r) {
          const float* zr = a.zpart + (size_t)(grow0 + fr) * r + q;
          for (int s = 0; s < a.S; ++s) {
            const f32x4 lo = *reinterpret_cast<const f32x4*>(zr + s * zstride);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(zr + s * zstride + 4);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              z[t] += lo[t];
              z[4 + t] += hi[t];
            }
          }
        }
        u32x4 zh, zl;
        {
          uint32_t hb[8], lb[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            hb[t] = f32_to_bf16_bits(z[t]);
            lb[t] = f32_to_bf16_bits(z[t] - __uint_as_float(hb[t] << 16));
          }
          zh = u32x4{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16),
                     hb[6] | (hb[7] << 16)};
          zl = u32x4{lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16), lb[4] | (lb[5] << 16),
                     lb[6] | (lb[7] << 16)};
        }
#pragma unroll
        for (int jn = 0; jn < FN; ++jn) {
          const u32x4 bv = q < r ? ldg16(Bad + wrow_of(jn) * r + q) : u32x4{0u, 0u, 0u, 0u};
          acc[i][jn] = mfma32(zh, bv, acc[i][jn]);
          acc[i][jn] = mfma32(zl, bv, acc[i][jn]);
        }
      }
    }
    // store: lane holds rows grow0 + 8*(v/4) + 4*(lane/32) + (v%4) of column (lane % 32)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int srow = grow0 + 8 * (v / 4) + 4 * fg + (v % 4);
      const int p = a.sorted_pairs[srow];
      if (p < 0) continue;
      if (GATEUP) {
#pragma unroll
        for (int jn = 0; jn < FN / 2; ++jn) {
          const float g = acc[i][jn][v], u = acc[i][jn + FN / 2][v];
          const float hv = g / (1.f + __expf(-g)) * u;
          a.act_out[(size_t)srow * N + wrow_of(jn)] = (uint16_t)f32_to_bf16_bits(hv);
        }
      } else {
#pragma unroll
        for (int jn = 0; jn < FN; ++jn) a.d_out[(size_t)p * N + wrow_of(jn)] = acc[i][jn][v];
      }
    }
  }
}

template <bool GATEUP, int BM, int BN, int WM, int WN, int DEPTH, int OCC>
hipError_t launch_tiled_t(const GemmArgs& a, int n_tiles_n, int total, hipStream_t stream) {
  constexpr int lds_bytes = 2 * (BM + BN) * 64 * 2;
  auto kern = tiled_gemm_kernel<GATEUP, BM, BN, WM, WN, DEPTH, OCC>;
  static bool attr_set[64] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                              lds_bytes);
    if (err != hipSuccess) return err;
    attr_set[dev] = true;
  }
  hipLaunchKernelGGL(kern, dim3(total), dim3(256), lds_bytes, stream, a, n_tiles_n, total);
  return hipGetLastError();
}

hipError_t launch_tiled(const TiledConfig& c, bool gateup, const GemmArgs& a, hipStream_t stream) {
  const int cols = gateup ? 2 * a.N : a.N;
  if (cols % c.bn != 0) return hipErrorInvalidValue;
  const int n_tiles_n = cols / c.bn;
  // grouped order (8 x 8 tiles per group, see the kernel), padded to whole groups and to a
  // multiple of the 8 XCDs
  const int gm = (a.n_blocks_max + 7) / 8, gn = (n_tiles_n + 7) / 8;
  int total = gm * gn * 64;
  total = (total + 7) / 8 * 8;
  if (total <= 0) return hipSuccess;
#define MOELORA_TILED(BM_, BN_, WM_, WN_, DEPTH_, OCC_)                                       \
  if (c.bm == BM_ && c.bn == BN_ && c.wm == WM_ && c.wn == WN_ && c.depth == DEPTH_)          \
    return gateup                                                                             \
        ? launch_tiled_t<true, BM_, BN_, WM_, WN_, DEPTH_, OCC_>(a, n_tiles_n, total, stream) \
        : launch_tiled_t<false, BM_, BN_, WM_, WN_, DEPTH_, OCC_>(a, n_tiles_n, total, stream);
  MOELORA_TILED(128, 128, 64, 64, 2, 2)
  MOELORA_TILED(128, 128, 64, 64, 1, 2)
  MOELORA_TILED(64, 128, 32, 64, 2, 2)
  MOELORA_TILED(256, 128, 128, 64, 2, 1)
  MOELORA_TILED(256, 128, 128, 64, 1, 1)
  MOELORA_TILED(128, 256, 64, 128, 2, 1)
  MOELORA_TILED(128, 256, 64, 128, 1, 1)
  MOELORA_TILED(256, 256, 128, 128, 1, 1)
  MOELORA_TILED(256, 256, 128, 128, 2, 1)
  MOELORA_TILED(128, 512, 64, 256, 1, 1)
#undef MOELORA_TILED
  return hipErrorInvalidValue;
}

}  // namespace moelora
