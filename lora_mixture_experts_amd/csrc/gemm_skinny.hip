// Expert GEMMs for few rows per expert (decode): the layer is bound by streaming the frozen
// expert weights from HBM, so every weight byte is read once per row block and the few token
// rows ride along.
//
// Page "vLLM MoE LoRA SageMaker Bedrock", section "Entendendo os Modelos MoE": gate_up expands
// the hidden state to the intermediate size, down compresses it back. Section "O Papel da
// Multi-LoRA": each projection adds the LoRA expand z B to the base output. Section
// "Otimizações em Nível de Kernel": the LoRA add is fused into the kernel that produces the
// base output rather than launched separately, and loads need no masks when K divides the
// block (K is a multiple of 128 here). Page "AWS SageMaker MoE kernel optimizations" (aib.vote),
// second paragraph: with M = 1 decode, the matrix unit's fixed M dimension is filled by
// swapping operands so the large weight dimension sits on it.
//
// Mapping on CDNA4: a 16x16x32 bf16 MFMA takes 16 weight rows as its A operand and 16 token
// rows (one row block of the sorted layout, NT blocks of 16 per workgroup) as its B operand:
// the swapped-operand form. Each wavefront owns one 16-wide output tile; per 128-wide K step a
// lane loads 64 contiguous bytes of its weight row(s) and of its token row, and the four MFMAs
// of the step consume them in a lane-local order that both operands share (the sum over K does
// not depend on the order). The next step's loads are issued before the current MFMAs.
//
// gate_up: a wave owns act columns [n0, n0+16): gate rows n0.. and up rows I+n0..; the
//   epilogue adds z1 B1 to both, applies SiLU-and-mul and stores act (bf16) at the sorted row.
// down:    a wave owns output features [n0, n0+16) of W2; the epilogue adds z2 B2 and stores
//   the fp32 expert output at the sorted row of D (the combine finds a pair's row).
#include "common.h"
#include "kernels.h"
#include "lora_mfma.h"

namespace moelora {

// NT: 16-row token tiles per row block (BM = 16*NT). P: 16-byte loads per lane per weight row
// and K step (K step = 32*P). RT: 16-row output tiles per wave (per projection for gate_up).
// Down may split K over gridDim.z: split z writes its partial sums to its own D buffer and only
// split 0 adds the LoRA term; the combine adds the splits in order.
// PIPE: two register sets alternate so the next step's loads overlap the current MFMAs;
// otherwise each step loads then computes and latency is hidden by other wavefronts only.
// SPLIT (gate_up only, RT = 1): waves 0-1 stream gate rows and waves 2-3 the matching up rows,
// one weight tile per wave; the up accumulators reach the gate waves through LDS.
// FP8: the weights are E4M3 codes (a.W8) with one float32 scale per output row (a.wscale).
// Each 16-byte load of a row brings the codes of two of the token rows' 8-element K chunks;
// they become bf16 in registers just before their MFMAs (exact: every E4M3 value is a bf16),
// and each accumulator row is multiplied by its row's scale after the main loop, before the
// LoRA term (bf16 weights, unscaled) is added.
template <int NT, bool GATEUP, int P, int RT, bool PIPE, bool SPLIT, bool FP8 = false>
__global__ __launch_bounds__(256) void skinny_gemm_kernel(GemmArgs a) {
  static_assert(!SPLIT || (GATEUP && RT == 1), "SPLIT is a gate_up mode with one tile per wave");
  static_assert(!FP8 || (P % 2 == 0 && !SPLIT), "FP8 rows come in 16-byte pairs of K chunks");
  constexpr int PW = FP8 ? P / 2 : P;  // weight loads per lane, row and K step
  constexpr int NW = SPLIT ? 1 : (GATEUP ? 2 : 1) * RT;
  constexpr int BM = 16 * NT;
  constexpr int KS = 32 * P;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Work order: the live (row block, column tile) items are numbered column tile by column
  // tile within each row block, and every XCD (hardware workgroup ids go round-robin over the
  // 8) gets an equal contiguous share: it takes whole row blocks, whose token rows stay in its
  // L2 while the column tiles pass, and streams consecutive weight rows of one expert.
  const int ncol = a.n_col_tiles;
  const int nblk = *a.n_blocks;
  const int live = nblk * ncol;
  const int per_xcd = (live + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  const int t = (blockIdx.x & 7) * per_xcd + slot;
  if (slot >= per_xcd || t >= live) return;
  const int blk = t / ncol;
  const int ctile = t - blk * ncol;
  // The block's expert and token rows (pair ids, adapters); the pair and adapter serve the
  // epilogue too, so their latency hides behind the main loop. Token rows are read with buffer loads: a padding row (pair -1) gets an out-of-range
  // offset and loads zeros without touching memory. Every load stays unconditional, which keeps
  // the compiler's count of outstanding loads exact, so the prefetch below overlaps the MFMAs.
  const int m = lane & 15, kq = lane >> 4;
  const int K = a.K;
  const int e = a.block_expert[blk];
  uint32_t xo[NT];
  int pair[NT], adap[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = blk * BM + nt * 16 + m;
    const int p = a.sorted_pairs[row];
    pair[nt] = p;
    adap[nt] = a.sorted_ad[row];
    xo[nt] = p < 0 ? kOutOfRange : (uint32_t)((GATEUP ? (size_t)(p / a.k) : (size_t)row) * K * 2);
  }
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, a.x_bytes);

  const int n0 = SPLIT ? (ctile * 2 + (wave & 1)) * 16 : (ctile * 4 + wave) * 16 * RT;
  const bool up_wave = SPLIT && wave >= 2;
  __shared__ f32x4 s_up[SPLIT ? 2 * 64 * NT : 1];
  const int zsplit = blockIdx.z;
  constexpr int BMZ = 16 * NT;

  // The block's z rows go into LDS for the epilogue (rows without an adapter hold values nobody
  // reads): the sum of the shrink's K-split parts, added here in split order. Only K split 0 of
  // down adds the LoRA term. Run after the first
  // weight loads are issued, so the two latencies overlap. (The grid covers N exactly: every
  // wavefront has columns.)
  __shared__ __attribute__((aligned(16))) float s_z[BMZ * 64];
  auto z_prologue = [&]() {
    if (zsplit != 0) return;
    const int nz = BMZ * a.r;
    const size_t off = (size_t)blk * BMZ * a.r;
    {
      // every part's load is issued before the first add (parts past zsplits re-read the last
      // one and are not added), so the sum costs one memory round trip
      const size_t part = (size_t)a.cap * a.r;
      for (int i = threadIdx.x * 4; i < nz; i += 256 * 4) {
        f32x4 zz[kMaxSplit];
#pragma unroll
        for (int sp = 0; sp < kMaxSplit; ++sp)
          zz[sp] = *reinterpret_cast<const f32x4*>(a.zpart + min(sp, a.zsplits - 1) * part + off + i);
        f32x4 z = zz[0];
#pragma unroll
        for (int sp = 1; sp < kMaxSplit; ++sp)
          if (sp < a.zsplits) z += zz[sp];
        *reinterpret_cast<f32x4*>(s_z + i) = z;
      }
    }
    __syncthreads();
  };
  const size_t N = (size_t)a.N;
  const int nks = K / KS;
  const int ks0 = (nks * zsplit) / a.ksplit, ks1 = (nks * (zsplit + 1)) / a.ksplit;

  // weight row of tile w for this lane's MFMA row (m), and the first of the 4 accumulator rows
  // it holds (4 kq)
  size_t wrow[NW];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if (SPLIT) {
      wrow[0] = (size_t)e * 2 * N + (up_wave ? N : 0) + n0;
    } else if (GATEUP) {
      wrow[rt] = (size_t)e * 2 * N + n0 + 16 * rt;
      wrow[NW - RT + rt] = (size_t)e * 2 * N + N + n0 + 16 * rt;
    } else {
      wrow[rt] = (size_t)e * N + n0 + 16 * rt;
    }
  }
  // (bf16 rows: K elements of 2 bytes; E4M3 rows: K bytes)
  const uint8_t* wp[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w)
    wp[w] = FP8 ? a.W8 + (wrow[w] + m) * K : reinterpret_cast<const uint8_t*>(a.W + (wrow[w] + m) * K);
  // FP8: the scales of the 4 accumulator rows of each tile, fetched ahead of the main loop
  float wsc[NW][4];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int v = 0; v < 4; ++v) wsc[w][v] = FP8 ? a.wscale[wrow[w] + 4 * kq + v] : 1.f;

  f32x4 acc[NW][NT];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[w][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Two register sets alternate (ping-pong): while one step's MFMAs run, the next step's loads
  // are in flight. Loads are never conditional: past the last step they re-read the last step
  // (L2 hits, results unused), so the compiler's outstanding-load count stays exact and its
  // wait before each compute covers only the older set.
  u32x4 wa[NW][PW], xa[NT][P], wb[NW][PW], xb[NT][P];
#define MOELORA_LOAD(W_, X_, KB_)                                              \
  do {                                                                         \
    _Pragma("unroll") for (int w = 0; w < NW; ++w)                             \
      _Pragma("unroll") for (int j = 0; j < PW; ++j)                           \
        W_[w][j] = ldg16(wp[w] + (FP8 ? 1 : 2) * ((KB_) + (FP8 ? 16 : 8) * j)); \
    _Pragma("unroll") for (int nt = 0; nt < NT; ++nt)                          \
      _Pragma("unroll") for (int j = 0; j < P; ++j)                            \
        X_[nt][j] = bufld16(xr, xo[nt] + 2u * (uint32_t)((KB_) + 8 * j));      \
  } while (0)
#define MOELORA_COMPUTE(W_, X_)                                                \
  do {                                                                         \
    _Pragma("unroll") for (int j = 0; j < P; ++j)                              \
      _Pragma("unroll") for (int w = 0; w < NW; ++w) {                         \
        const u32x4 wv = FP8 ? e4m3x8_to_bf16(W_[w][j / 2], j % 2) : W_[w][j % PW]; \
        _Pragma("unroll") for (int nt = 0; nt < NT; ++nt)                      \
          acc[w][nt] = mfma16(wv, X_[nt][j], acc[w][nt]);                      \
      }                                                                        \
  } while (0)
  const int nsteps = ks1 - ks0;
  if (!PIPE || nsteps == 0) z_prologue();
  if (!PIPE) {
    for (int i = 0; i < nsteps; ++i) {
      const int kb = (ks0 + i) * KS + kq * (8 * P);
      MOELORA_LOAD(wa, xa, kb);
      MOELORA_COMPUTE(wa, xa);
    }
  } else if (nsteps > 0) {
    const int kb0 = ks0 * KS + kq * (8 * P);
    MOELORA_LOAD(wa, xa, kb0);
    z_prologue();
    for (int i = 0; i < nsteps; i += 2) {
      // sched_barrier(0) keeps the compiler from interleaving the phases (which would bring
      // the waits for the in-flight set back in front of the MFMAs)
      MOELORA_LOAD(wb, xb, kb0 + min(i + 1, nsteps - 1) * KS);
      __builtin_amdgcn_sched_barrier(0);
      MOELORA_COMPUTE(wa, xa);
      __builtin_amdgcn_sched_barrier(0);
      MOELORA_LOAD(wa, xa, kb0 + min(i + 2, nsteps - 1) * KS);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < nsteps) MOELORA_COMPUTE(wb, xb);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#undef MOELORA_LOAD
#undef MOELORA_COMPUTE

  // Epilogue: lane holds weight rows n0 + 16*rt + 4*kq + v (v < 4) for token row (lane % 16).
  if (FP8) {
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[w][nt][v] *= wsc[w][v];
  }
  // The LoRA term (down: K split 0 only), onto the accumulators.
  if (zsplit == 0) {
    int brow[NW];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (SPLIT) {
        brow[0] = (up_wave ? (int)N : 0) + n0;
      } else if (GATEUP) {
        brow[rt] = n0 + 16 * rt;
        brow[NW - RT + rt] = (int)N + n0 + 16 * rt;
      } else {
        brow[rt] = n0 + 16 * rt;
      }
    }
    const size_t rows_e = (GATEUP ? 2 : 1) * N;
    // runs per batch of B loads: fewer for down, whose register count sets its occupancy
    constexpr int RB = (GATEUP ? 8 : 4) / NW > 0 ? (GATEUP ? 8 : 4) / NW : 1;
    lora_mfma<NT, NW, RB>(acc, brow, a.Bw + (size_t)e * rows_e * a.r, (size_t)a.E * rows_e * a.r,
                          a.r, s_z, adap, lane);
  }
  if (SPLIT) {
    if (up_wave) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) s_up[((wave & 1) * NT + nt) * 64 + lane] = acc[0][nt];
    }
    __syncthreads();
    if (up_wave) return;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = blk * BM + nt * 16 + m;
    if (pair[nt] < 0) continue;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int nb = n0 + 16 * rt + 4 * kq;
      if (GATEUP) {
        float gu[2][4];  // gate, up
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          gu[0][v] = acc[rt][nt][v];
          gu[1][v] = SPLIT ? s_up[((wave & 1) * NT + nt) * 64 + lane][v] : acc[NW - RT + rt][nt][v];
        }
        float hv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) hv[v] = gu[0][v] / (1.f + __expf(-gu[0][v])) * gu[1][v];
        u32x2 packed = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
        *reinterpret_cast<u32x2*>(a.act_out + (size_t)row * N + nb) = packed;
      } else {
        float d[1][4];
#pragma unroll
        for (int v = 0; v < 4; ++v) d[0][v] = acc[rt][nt][v];
        *reinterpret_cast<f32x4*>(a.d_out + zsplit * a.d_split_stride + (size_t)row * N + nb) =
            f32x4{d[0][0], d[0][1], d[0][2], d[0][3]};
      }
    }
  }
}

hipError_t launch_skinny(const SkinnyConfig& c, bool gateup, const GemmArgs& a, int grid_y,
                         hipStream_t stream, bool fp8) {
  const bool split = gateup && c.split;
  const int cols_per_wg = split ? 32 : 4 * 16 * c.rt;
  if (a.N % cols_per_wg != 0) return hipErrorInvalidValue;  // every wavefront has columns
  const int ncol = a.N / cols_per_wg;
  if (ncol <= 0 || grid_y <= 0) return hipSuccess;
  if (a.zsplits < 1 || a.zsplits > kMaxSplit) return hipErrorInvalidValue;  // z parts to add
  if (ncol != a.n_col_tiles) return hipErrorInvalidValue;
  // one workgroup per (row block, column tile) for the largest block count, in a 1-D grid
  // rounded up to the 8 XCDs (the kernel maps its id onto the live items)
  const int total = ((grid_y * ncol) + 7) / 8 * 8;
  dim3 grid(total, 1, gateup ? 1 : a.ksplit), block(256);
#define MOELORA_SKINNY_FP8(NT_, P_, RT_)                                                          \
  if (c.nt == NT_ && c.p == P_ && c.rt == RT_ && c.pipe == 1 && !split && fp8) {                  \
    if (gateup)                                                                                   \
      hipLaunchKernelGGL((skinny_gemm_kernel<NT_, true, P_, RT_, true, false, true>), grid, block, \
                         0, stream, a);                                                           \
    else                                                                                          \
      hipLaunchKernelGGL((skinny_gemm_kernel<NT_, false, P_, RT_, true, false, true>), grid,      \
                         block, 0, stream, a);                                                    \
    return hipGetLastError();                                                                     \
  }
  // E4M3 weights (16- and 32-row blocks; 64- and 128-wide K steps)
  MOELORA_SKINNY_FP8(1, 2, 1)
  MOELORA_SKINNY_FP8(1, 2, 2)
  MOELORA_SKINNY_FP8(2, 2, 1)
  MOELORA_SKINNY_FP8(2, 2, 2)
  MOELORA_SKINNY_FP8(1, 4, 1)
  MOELORA_SKINNY_FP8(1, 4, 2)
  MOELORA_SKINNY_FP8(2, 4, 1)
  MOELORA_SKINNY_FP8(2, 4, 2)
  if (fp8) return hipErrorInvalidValue;
#undef MOELORA_SKINNY_FP8
#define MOELORA_SKINNY(NT_, P_, RT_, PIPE_)                                                       \
  if (c.nt == NT_ && c.p == P_ && c.rt == RT_ && c.pipe == PIPE_ && !split) {                     \
    if (gateup)                                                                                   \
      hipLaunchKernelGGL((skinny_gemm_kernel<NT_, true, P_, RT_, PIPE_, false>), grid, block, 0,  \
                         stream, a);                                                              \
    else                                                                                          \
      hipLaunchKernelGGL((skinny_gemm_kernel<NT_, false, P_, RT_, PIPE_, false>), grid, block, 0, \
                         stream, a);                                                              \
    return hipGetLastError();                                                                     \
  }
#define MOELORA_SKINNY_SPLIT(NT_, P_, PIPE_)                                                      \
  if (c.nt == NT_ && c.p == P_ && c.rt == 1 && c.pipe == PIPE_ && split) {                        \
    hipLaunchKernelGGL((skinny_gemm_kernel<NT_, true, P_, 1, PIPE_, true>), grid, block, 0,       \
                       stream, a);                                                                \
    return hipGetLastError();                                                                     \
  }
  MOELORA_SKINNY(1, 2, 1, true)
  MOELORA_SKINNY(1, 2, 2, true)
  MOELORA_SKINNY(1, 4, 1, true)
  MOELORA_SKINNY(1, 4, 1, false)
  MOELORA_SKINNY(1, 4, 2, true)
  MOELORA_SKINNY(1, 4, 2, false)
  MOELORA_SKINNY(1, 8, 1, true)
  MOELORA_SKINNY(1, 8, 1, false)
  MOELORA_SKINNY(2, 2, 1, true)
  MOELORA_SKINNY(2, 2, 2, true)
  MOELORA_SKINNY(2, 4, 1, true)
  MOELORA_SKINNY(2, 4, 2, true)
  MOELORA_SKINNY(2, 8, 1, true)
  MOELORA_SKINNY(4, 4, 1, true)
  MOELORA_SKINNY_SPLIT(1, 4, true)
  MOELORA_SKINNY_SPLIT(1, 4, false)
  MOELORA_SKINNY_SPLIT(1, 8, true)
  MOELORA_SKINNY_SPLIT(1, 8, false)
#undef MOELORA_SKINNY
#undef MOELORA_SKINNY_SPLIT
  return hipErrorInvalidValue;
}

}  // namespace moelora
