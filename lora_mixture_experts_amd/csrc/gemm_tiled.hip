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
// (all of one expert) and BN output features. Both operands are K-contiguous, so every MFMA
// fragment (16 rows x 8 consecutive k per lane) is one 16-byte LDS read. Tiles are stored
// row-major in LDS with the 16-byte chunk index XOR-swizzled by the row, double-buffered, one
// barrier per K step; the next K step's global loads are issued before the current MFMAs.
//
// gate_up: the BN weight rows of a tile are arranged per wave column as [gate i .. | up i ..] for
// the same intermediate columns i, so each lane holds gate and up of the same act element and
// SiLU-and-mul runs in registers. The LoRA expand is added before it.
//
// LoRA expand (both projections): rows are sorted by adapter inside an expert, so each 16-row
// MFMA group holds a few contiguous adapter runs. For every run the group's z rows (other rows
// zeroed) multiply B[adapter][expert] as one more MFMA pass over K = r: the segment's adapter
// weights are read once per group, not per token. z is split into bf16 high and low parts
// (two MFMAs) so the term keeps ~16 mantissa bits.
#include "common.h"
#include "kernels.h"

namespace moelora {

// DEPTH: K steps of global prefetch (1: one register staging set, 2: two). Tiles up to 128x128
// keep two wavefronts per SIMD; 256-row tiles run one.
template <bool GATEUP, int BM, int BN, int BK, int WM, int WN, int DEPTH>
__global__ __launch_bounds__(256, (BM * BN > 128 * 128) ? 1 : 2) void tiled_gemm_kernel(
    GemmArgs a, int n_tiles_n, int grid_total) {
  constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static_assert(WAVES_M * WAVES_N == 4, "four wavefronts per workgroup");
  static_assert(BK == 64, "8 chunks of 16 bytes per LDS row");
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int CPR = BK / 8;                  // 16-byte chunks per tile row
  constexpr int CA = BM * CPR / 256;           // chunks of the token tile per thread
  constexpr int CB = BN * CPR / 256;           // chunks of the weight tile per thread
  static_assert(CA * 256 == BM * CPR && CB * 256 == BN * CPR, "tile must split over 256 threads");
  static_assert(!GATEUP || FN % 2 == 0, "gate_up needs gate and up halves per wave");

  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // 2 * (BM + BN) * BK

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // XCD-aware order: hardware workgroup ids go round-robin over the 8 XCDs; consecutive logical
  // tiles (same weight tile, neighbouring row blocks) are placed on the same XCD.
  const int hw = blockIdx.x;
  const int logical = (hw & 7) * (grid_total >> 3) + (hw >> 3);
  const int blk = logical % a.n_blocks_max;
  const int ntile = logical / a.n_blocks_max;
  if (ntile >= n_tiles_n || blk >= *a.n_blocks) return;
  const int e = a.block_expert[blk];
  const int K = a.K;
  const size_t N = (size_t)a.N;          // gate_up: I; down: h
  const int row0 = blk * BM;

  // ---- per-thread global load plan (fixed over K) ----
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, a.x_bytes);
  uint32_t xo[CA];
  int a_row[CA], a_chk[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int q = tid + 256 * i;
    a_row[i] = q / CPR;
    a_chk[i] = q % CPR;
    const int srow = row0 + a_row[i];
    const int p = a.sorted_pairs[srow];
    xo[i] = p < 0 ? kOutOfRange
                  : (uint32_t)((GATEUP ? (size_t)(p / a.k) : (size_t)srow) * K * 2) + 16u * a_chk[i];
  }
  const uint16_t* wsrc[CB];
  int b_row[CB], b_chk[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int q = tid + 256 * i;
    b_row[i] = q / CPR;
    b_chk[i] = q % CPR;
    size_t wrow;
    if (GATEUP) {
      const int g = b_row[i] / WN, rr = b_row[i] % WN;
      const size_t col = (size_t)ntile * (BN / 2) + g * (WN / 2) + (rr % (WN / 2));
      wrow = (size_t)e * 2 * N + (rr < WN / 2 ? col : N + col);
    } else {
      wrow = (size_t)e * N + (size_t)ntile * BN + b_row[i];
    }
    wsrc[i] = a.W + wrow * K + 8 * b_chk[i];
  }

  auto lds_a = [&](int buf) { return lds + buf * (BM + BN) * BK; };
  auto lds_b = [&](int buf) { return lds + buf * (BM + BN) * BK + BM * BK; };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nks = K / BK;
  // Global tiles are prefetched two K steps ahead into two register staging sets (s0, s1), so a
  // load has two compute phases to land before it is written to LDS. Loads are unconditional
  // (past the end they re-read the last step), which keeps the compiler's outstanding-load
  // count exact; LDS is double-buffered with one barrier per K step.
  u32x4 sa0[CA], sb0[CB], sa1[CA], sb1[CB];
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
    _Pragma("unroll") for (int i = 0; i < CA; ++i) *reinterpret_cast<u32x4*>(            \
        A_ + a_row[i] * BK + 8 * (a_chk[i] ^ (a_row[i] & 7))) = SA[i];                    \
    _Pragma("unroll") for (int i = 0; i < CB; ++i) *reinterpret_cast<u32x4*>(            \
        B_ + b_row[i] * BK + 8 * (b_chk[i] ^ (b_row[i] & 7))) = SB[i];                    \
  } while (0)

  const int fr = lane & 15, fg = lane >> 4;
  // MFMA fragments of the two 32-wide halves of a K step are read from LDS together into two
  // register sets; the second half's reads land while the first half's MFMAs run.
  auto read_frags = [&](const uint16_t* A, const uint16_t* B, int j, u32x4* af, u32x4* bf) {
    const int chunk = fg + 4 * j;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WM + i * 16 + fr;
      af[i] = *reinterpret_cast<const u32x4*>(A + r * BK + 8 * (chunk ^ (r & 7)));
    }
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int r = wn * WN + i * 16 + fr;
      bf[i] = *reinterpret_cast<const u32x4*>(B + r * BK + 8 * (chunk ^ (r & 7)));
    }
  };
  auto mfmas = [&](const u32x4* af, const u32x4* bf) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jn = 0; jn < FN; ++jn) acc[i][jn] = mfma16(af[i], bf[jn], acc[i][jn]);
  };
  auto compute = [&](int buf) {
    static_assert(BK == 64, "two 32-wide halves per K step");
    const uint16_t* A = lds_a(buf);
    const uint16_t* B = lds_b(buf);
    u32x4 af0[FM], bf0[FN], af1[FM], bf1[FN];
    read_frags(A, B, 0, af0, bf0);
    __builtin_amdgcn_sched_barrier(0);
    // the second half's reads are interleaved one per MFMA of the first half (the LDS counter
    // holds at most 15 outstanding reads, so issuing all 16 up front would force a full wait)
    read_frags(A, B, 1, af1, bf1);
    mfmas(af0, bf0);
#pragma unroll
    for (int t = 0; t < FM + FN; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN), 0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(af1, bf1);
  };

  MOELORA_GLOAD(sa0, sb0, 0);
  if (DEPTH == 2) MOELORA_GLOAD(sa1, sb1, 1);
  MOELORA_LSTORE(sa0, sb0, 0);
  __syncthreads();
  // sched_barrier(0) pins the phase order: without it the compiler sinks the prefetch below
  // the MFMAs, which shortens the time the loads have to land. The LDS stores are
  // unconditional as well (past the end they fill a buffer nobody reads), so the compiler can
  // count exactly which loads are still in flight.
  if (DEPTH == 2) {
    for (int ks = 0; ks < nks; ks += 2) {
      // even step: compute buffer 0, stage step ks+1 (set 1) into buffer 1
      MOELORA_GLOAD(sa0, sb0, ks + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(0);
      __builtin_amdgcn_sched_barrier(0);
      MOELORA_LSTORE(sa1, sb1, 1);
      __syncthreads();
      // odd step (K is a multiple of 128, so the number of 64-wide steps is even): compute buffer 1, stage step ks+2 (set 0) into buffer 0
      MOELORA_GLOAD(sa1, sb1, ks + 3);
      __builtin_amdgcn_sched_barrier(0);
      compute(1);
      __builtin_amdgcn_sched_barrier(0);
      MOELORA_LSTORE(sa0, sb0, 0);
      __syncthreads();
    }
  } else {
    // one staging set: the next step's loads are issued before the current MFMAs
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
      const size_t col = (size_t)ntile * (BN / 2) + wn * (WN / 2) + (jn % half) * 16 + fr;
      return jn < half ? col : N + col;
    }
    return (size_t)ntile * BN + wn * WN + jn * 16 + fr;
  };

  const int r = a.r;
  const int64_t zstride = a.cap * r;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int grow0 = row0 + wm * WM + i * 16;  // first sorted row of this 16-row group
    int ad = -1;
    {
      const int p = a.sorted_pairs[grow0 + fr];
      if (p >= 0) ad = sanitize_adapter(a.adapter_ids[p / a.k], a.nA);
    }
    uint64_t pending = __ballot(lane < 16 && ad >= 0);
    while (pending) {
      const int first = __ffsll((unsigned long long)pending) - 1;
      const int acur = __shfl(ad, first);
      const uint64_t run = __ballot(lane < 16 && ad == acur);
      pending &= ~run;
      const bool mine = (run >> fr) & 1ull;
      const uint16_t* Bad = a.Bw + ((size_t)acur * a.E + e) * (GATEUP ? 2 * N : N) * r;
      for (int q0 = 0; q0 < r; q0 += 32) {
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
          uint32_t h[8], l[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            h[t] = f32_to_bf16_bits(z[t]);
            l[t] = f32_to_bf16_bits(z[t] - __uint_as_float(h[t] << 16));
          }
          zh = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
          zl = u32x4{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16)};
        }
#pragma unroll
        for (int jn = 0; jn < FN; ++jn) {
          const u32x4 bv = q < r ? ldg16(Bad + wrow_of(jn) * r + q) : u32x4{0u, 0u, 0u, 0u};
          acc[i][jn] = mfma16(zh, bv, acc[i][jn]);
          acc[i][jn] = mfma16(zl, bv, acc[i][jn]);
        }
      }
    }
    // store: lane holds rows grow0 + 4*fg + v of column fragment jn, column (lane % 16)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int srow = grow0 + 4 * fg + v;
      const int p = a.sorted_pairs[srow];
      if (p < 0) continue;
      if (GATEUP) {
#pragma unroll
        for (int jn = 0; jn < FN / 2; ++jn) {
          const float g = acc[i][jn][v], u = acc[i][jn + FN / 2][v];
          const float hv = g / (1.f + __expf(-g)) * u;
          const size_t col = wrow_of(jn);
          a.act_out[(size_t)srow * N + col] = (uint16_t)f32_to_bf16_bits(hv);
        }
      } else {
#pragma unroll
        for (int jn = 0; jn < FN; ++jn) a.d_out[(size_t)p * N + wrow_of(jn)] = acc[i][jn][v];
      }
    }
  }
}

template <bool GATEUP, int BM, int BN, int WM, int WN>
hipError_t launch_tiled_t(const GemmArgs& a, int n_tiles_n, int total, hipStream_t stream) {
  constexpr int DEPTH = BM * BN > 128 * 128 ? 1 : 2;
  constexpr int lds_bytes = 2 * (BM + BN) * 64 * 2;
  static bool attr_set[64] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    err = hipFuncSetAttribute((const void*)tiled_gemm_kernel<GATEUP, BM, BN, 64, WM, WN, DEPTH>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (err != hipSuccess) return err;
    attr_set[dev] = true;
  }
  hipLaunchKernelGGL((tiled_gemm_kernel<GATEUP, BM, BN, 64, WM, WN, DEPTH>), dim3(total), dim3(256),
                     lds_bytes, stream, a, n_tiles_n, total);
  return hipGetLastError();
}

hipError_t launch_tiled(const TiledConfig& c, bool gateup, const GemmArgs& a, hipStream_t stream) {
  const int cols = gateup ? 2 * a.N : a.N;
  const int n_tiles_n = cols / c.bn;
  int total = n_tiles_n * a.n_blocks_max;
  total = (total + 7) / 8 * 8;
  if (total <= 0) return hipSuccess;
#define MOELORA_TILED(BM_, BN_, WM_, WN_)                                              \
  if (c.bm == BM_ && c.bn == BN_ && c.wm == WM_ && c.wn == WN_)                        \
    return gateup ? launch_tiled_t<true, BM_, BN_, WM_, WN_>(a, n_tiles_n, total, stream) \
                  : launch_tiled_t<false, BM_, BN_, WM_, WN_>(a, n_tiles_n, total, stream);
  MOELORA_TILED(128, 128, 64, 64)
  MOELORA_TILED(64, 128, 32, 64)
  MOELORA_TILED(256, 256, 128, 128)
  MOELORA_TILED(256, 128, 128, 64)
#undef MOELORA_TILED
  return hipErrorInvalidValue;
}

}  // namespace moelora
