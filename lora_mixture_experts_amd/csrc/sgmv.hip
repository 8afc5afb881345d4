// Dense multi-LoRA (segmented gather matrix-vector, SGMV): the expand that adds z B_a^T to the
// token rows of y in place. Page "Punica: Multi-Tenant LoRA Serving", sections on the proposed
// method: one base model serves a batch whose tokens carry different adapters, and the LoRA add
// runs per segment of tokens that share an adapter (here: the align kernel's segments with a
// single expert). Page "vLLM MoE LoRA SageMaker Bedrock", section "O Papel da Multi-LoRA": the
// expand multiplies the shrink output z by B.
//
// One workgroup per (16-row block of the sorted layout, 64 output columns): each wavefront owns
// 16 columns, computes the block's LoRA term with MFMAs per adapter run (the run's B rows on
// the A side, z as bf16 high + low parts on the B side) and adds it to y (bf16, read, added in
// fp32, rounded once) at each token's row. Tokens without an adapter are not touched.
#include "common.h"
#include "kernels.h"
#include "lora_mfma.h"

namespace moelora {

__global__ __launch_bounds__(256) void sgmv_expand_kernel(SgmvArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // work order as the skinny GEMMs: whole row blocks, an equal contiguous share per XCD
  const int ncol = a.N / 64;
  const int live = *a.n_blocks * ncol;
  const int per_xcd = (live + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  const int t = (blockIdx.x & 7) * per_xcd + slot;
  if (slot >= per_xcd || t >= live) return;
  const int blk = t / ncol;
  const int ctile = t - blk * ncol;
  const int m = lane & 15, kq = lane >> 4;
  const int row = blk * 16 + m;
  const int tok = a.sorted_pairs[row];  // one pair per token: the pair id is the token
  const int adap[1] = {a.sorted_ad[row]};

  // the block's z rows into LDS: the shrink's split parts added in split order, every part's
  // load issued before the first add (parts past zsplits re-read the last one, unused)
  __shared__ __attribute__((aligned(16))) float s_z[16 * 64];
  const int nz = 16 * a.r;
  const size_t off = (size_t)blk * 16 * a.r, part = (size_t)a.cap * a.r;
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
  __syncthreads();

  f32x4 acc[1][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}};
  const int n0 = (ctile * 4 + wave) * 16;
  const int brow[1] = {n0};
  lora_mfma<1, 1, 8>(acc, brow, a.B, (size_t)a.N * a.r, a.r, s_z, adap, lane);

  // lane: output columns n0 + 4 kq + v of token row m
  if (tok >= 0 && adap[0] >= 0) {
    uint16_t* yp = a.y + (size_t)tok * a.N + n0 + 4 * kq;
    const u32x2 old = *reinterpret_cast<const u32x2*>(yp);
    const float y0 = bf16_lo(old.x) + acc[0][0][0], y1 = bf16_hi(old.x) + acc[0][0][1];
    const float y2 = bf16_lo(old.y) + acc[0][0][2], y3 = bf16_hi(old.y) + acc[0][0][3];
    *reinterpret_cast<u32x2*>(yp) = u32x2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
  }
}

hipError_t launch_sgmv_expand(const SgmvArgs& a, int max_blocks, hipStream_t stream) {
  if (a.N % 64 != 0 || a.zsplits < 1 || a.zsplits > kMaxSplit) return hipErrorInvalidValue;
  const int64_t items = (int64_t)max_blocks * (a.N / 64);
  if (items <= 0) return hipSuccess;
  hipLaunchKernelGGL(sgmv_expand_kernel, dim3((unsigned)((items + 7) / 8 * 8)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace moelora
