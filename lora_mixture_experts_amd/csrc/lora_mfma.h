// LoRA expand of a block of token rows as MFMAs, per adapter run (internal to libmoelora;
// used by the skinny expert GEMMs and by the dense multi-LoRA expand).
#pragma once

#include "common.h"

namespace moelora {

// LoRA expand of the block, as MFMAs added onto the base accumulators: for every adapter run
// (the distinct adapters of the block's live rows; the sorted layout keeps one expert's rows of
// one adapter contiguous), acc[t][nt] += B_t z^T, where B_t holds the 16 weight rows of output
// tile t (rows brow[t] .. +15 of the expert's B for the run's adapter, r ranks each) and z the
// shrink output of the rows of token tile nt, zero outside the run. B_t is the A operand (lane:
// row m, ranks 8*kq ..), z the B operand (lane: token row m, the same ranks), so the result lands
// in the accumulator layout of the base product. z (fp32) enters as two bf16 parts, z = hi + lo
// with lo = bf16(z - hi), which keeps about 16 of its mantissa bits. Up to RB runs' B fragments
// are loaded before any of their MFMAs, so a block's runs cost a few memory round trips rather
// than one per run.
template <int NT, int NW, int RB>
__device__ __forceinline__ void lora_mfma(f32x4 (&acc)[NW][NT], const int (&brow)[NW],
                                          const uint16_t* __restrict__ bexp, size_t ad_stride,
                                          int r, const float* s_z, const int (&adap)[NT],
                                          int lane) {
  const int m = lane & 15, kq = lane >> 4;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int c0 = 0; c0 < r; c0 += 32) {
    const int q = c0 + 8 * kq;  // this lane's 8 ranks
    u32x4 zh[NT], zl[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      zh[nt] = zero;
      zl[nt] = zero;
      if (q < r) {
        const float* zr = s_z + (nt * 16 + m) * r + q;
        const f32x4 z0 = *reinterpret_cast<const f32x4*>(zr);
        const f32x4 z1 = *reinterpret_cast<const f32x4*>(zr + 4);
        const float z[8] = {z0[0], z0[1], z0[2], z0[3], z1[0], z1[1], z1[2], z1[3]};
        float hi[8], lo[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          hi[i] = __uint_as_float(f32_to_bf16_bits(z[i]) << 16);
          lo[i] = z[i] - hi[i];
        }
        zh[nt] = u32x4{pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3]),
                       pack_bf16x2(hi[4], hi[5]), pack_bf16x2(hi[6], hi[7])};
        zl[nt] = u32x4{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                       pack_bf16x2(lo[4], lo[5]), pack_bf16x2(lo[6], lo[7])};
      }
    }
    // rows of each token tile still to do (lanes 0-15 carry rows 0-15; the masks are uniform)
    uint32_t todo[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) todo[nt] = (uint32_t)__ballot(adap[nt] >= 0) & 0xffffu;
    while (true) {
      int rad[RB];
      uint32_t rmask[RB][NT];
      int nr = 0;
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        int nt0 = -1;
#pragma unroll
        for (int nt = NT - 1; nt >= 0; --nt)
          if (todo[nt]) nt0 = nt;
        if (nt0 < 0) break;
        int adv = adap[0];
#pragma unroll
        for (int nt = 1; nt < NT; ++nt)
          if (nt == nt0) adv = adap[nt];
        const int ad = __builtin_amdgcn_readlane(adv, __builtin_ctz(todo[nt0]));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint32_t mk = (uint32_t)__ballot(adap[nt] == ad) & todo[nt];
          rmask[i][nt] = mk;
          todo[nt] &= ~mk;
        }
        rad[i] = ad;
        nr = i + 1;
      }
      if (nr == 0) break;
      u32x4 bl[RB][NW];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        if (i < nr) {
          const uint16_t* ba = bexp + (size_t)rad[i] * ad_stride;
#pragma unroll
          for (int t = 0; t < NW; ++t)
            bl[i][t] = q < r ? ldg16(ba + (size_t)(brow[t] + m) * r + q) : zero;
        }
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        if (i < nr) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            if (rmask[i][nt]) {
              const bool in = (rmask[i][nt] >> m) & 1u;
              const u32x4 a_hi = in ? zh[nt] : zero, a_lo = in ? zl[nt] : zero;
#pragma unroll
              for (int t = 0; t < NW; ++t) {
                acc[t][nt] = mfma16(bl[i][t], a_hi, acc[t][nt]);
                acc[t][nt] = mfma16(bl[i][t], a_lo, acc[t][nt]);
              }
            }
          }
        }
      }
    }
  }
}

}  // namespace moelora
