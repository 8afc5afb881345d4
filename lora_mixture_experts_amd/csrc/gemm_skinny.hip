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
//   the fp32 expert output at the pair's row of D (pair order t*k + j).
#include "common.h"
#include "kernels.h"

namespace moelora {

__device__ __forceinline__ float dot8_bf16(const float* z, u32x4 v) {
  float s = z[0] * bf16_lo(v.x);
  s += z[1] * bf16_hi(v.x);
  s += z[2] * bf16_lo(v.y);
  s += z[3] * bf16_hi(v.y);
  s += z[4] * bf16_lo(v.z);
  s += z[5] * bf16_hi(v.z);
  s += z[6] * bf16_lo(v.w);
  s += z[7] * bf16_hi(v.w);
  return s;
}

// out[v] += sum_q z[q] * Brow_v[q] for the 4 rows at Bbase + v*r (r multiple of 8).
__device__ __forceinline__ void lora_expand4(const float* __restrict__ zrow, int64_t zstride, int S,
                                             const uint16_t* __restrict__ Bbase, int r, float* out) {
  for (int q0 = 0; q0 < r; q0 += 8) {
    float z[8];
#pragma unroll
    for (int qq = 0; qq < 8; ++qq) z[qq] = 0.f;
    for (int s = 0; s < S; ++s) {
#pragma unroll
      for (int qq = 0; qq < 8; ++qq) z[qq] += zrow[s * zstride + q0 + qq];
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) out[v] += dot8_bf16(z, ldg16(Bbase + (size_t)v * r + q0));
  }
}

template <int NT, bool GATEUP>
__global__ __launch_bounds__(256) void skinny_gemm_kernel(GemmArgs a) {
  constexpr int NW = GATEUP ? 2 : 1;
  constexpr int BM = 16 * NT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * 4 + wave) * 16;
  if (n0 >= a.N) return;
  const int blk = blockIdx.y;
  if (blk >= *a.n_blocks) return;
  const int e = a.block_expert[blk];
  const int m = lane & 15, kq = lane >> 4;
  const int K = a.K;
  const size_t N = (size_t)a.N;

  const uint16_t* wp[NW];
  if (GATEUP) {
    wp[0] = a.W + ((size_t)e * 2 * N + n0 + m) * K;
    wp[NW - 1] = a.W + ((size_t)e * 2 * N + N + n0 + m) * K;
  } else {
    wp[0] = a.W + ((size_t)e * N + n0 + m) * K;
  }
  const uint16_t* xp[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = blk * BM + nt * 16 + m;
    const int p = a.sorted_pairs[row];
    xp[nt] = p < 0 ? nullptr : (GATEUP ? a.X + (size_t)(p / a.k) * K : a.X + (size_t)row * K);
  }

  f32x4 acc[NW][NT];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[w][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nks = K / 128;
  int kb = kq * 32;
  u32x4 wc[NW][4], xc[NT][4];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int j = 0; j < 4; ++j) wc[w][j] = ldg16(wp[w] + kb + 8 * j);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int j = 0; j < 4; ++j) xc[nt][j] = xp[nt] ? ldg16(xp[nt] + kb + 8 * j) : u32x4{0u, 0u, 0u, 0u};

  for (int ks = 0; ks < nks; ++ks) {
    const bool more = ks + 1 < nks;
    const int kn = kb + 128;
    u32x4 wn[NW][4], xn[NT][4];
    if (more) {
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int j = 0; j < 4; ++j) wn[w][j] = ldg16(wp[w] + kn + 8 * j);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xn[nt][j] = xp[nt] ? ldg16(xp[nt] + kn + 8 * j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[w][nt] = mfma16(wc[w][j], xc[nt][j], acc[w][nt]);
    if (more) {
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int j = 0; j < 4; ++j) wc[w][j] = wn[w][j];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) xc[nt][j] = xn[nt][j];
    }
    kb = kn;
  }

  // Epilogue: lane holds weight rows n0 + 4*kq + v (v < 4) for token row (lane % 16).
  const int64_t zstride = a.cap * a.r;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = blk * BM + nt * 16 + m;
    const int p = a.sorted_pairs[row];
    if (p < 0) continue;
    const int ad = sanitize_adapter(a.adapter_ids[p / a.k], a.nA);
    const int nb = n0 + 4 * kq;
    if (GATEUP) {
      float g[4], u[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        g[v] = acc[0][nt][v];
        u[v] = acc[NW - 1][nt][v];
      }
      if (ad >= 0) {
        const float* zrow = a.zpart + (size_t)row * a.r;
        const uint16_t* bg = a.Bw + (((size_t)ad * a.E + e) * 2 * N + nb) * a.r;
        lora_expand4(zrow, zstride, a.S, bg, a.r, g);
        lora_expand4(zrow, zstride, a.S, bg + N * a.r, a.r, u);
      }
      float h[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) h[v] = g[v] / (1.f + __expf(-g[v])) * u[v];
      u32x2 packed = {pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
      *reinterpret_cast<u32x2*>(a.act_out + (size_t)row * N + nb) = packed;
    } else {
      float d[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) d[v] = acc[0][nt][v];
      if (ad >= 0) {
        const float* zrow = a.zpart + (size_t)row * a.r;
        const uint16_t* bd = a.Bw + (((size_t)ad * a.E + e) * N + nb) * a.r;
        lora_expand4(zrow, zstride, a.S, bd, a.r, d);
      }
      *reinterpret_cast<f32x4*>(a.d_out + (size_t)p * N + nb) = f32x4{d[0], d[1], d[2], d[3]};
    }
  }
}

hipError_t launch_skinny(int nt, bool gateup, const GemmArgs& a, int grid_x, int grid_y,
                         hipStream_t stream) {
  if (grid_x <= 0 || grid_y <= 0) return hipSuccess;
  dim3 grid(grid_x, grid_y), block(256);
#define MOELORA_SKINNY(NT_)                                                               \
  if (nt == NT_) {                                                                        \
    if (gateup)                                                                           \
      hipLaunchKernelGGL((skinny_gemm_kernel<NT_, true>), grid, block, 0, stream, a);     \
    else                                                                                  \
      hipLaunchKernelGGL((skinny_gemm_kernel<NT_, false>), grid, block, 0, stream, a);    \
    return hipGetLastError();                                                             \
  }
  MOELORA_SKINNY(1)
  MOELORA_SKINNY(2)
  MOELORA_SKINNY(4)
#undef MOELORA_SKINNY
  return hipErrorInvalidValue;
}

}  // namespace moelora
