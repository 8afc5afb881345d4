// Internal helpers shared by the HIP kernels and the host entry points of libmoelora.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moelora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxTopk = 16;
constexpr int kMaxExperts = 1024;
constexpr int kMaxSplit = 8;  // split-K parts of the LoRA shrink
constexpr int kMaxParts = 4;  // K parts of the down GEMM's output D

// ------------------------------------------------------------------------------------------
// bf16 <-> f32. A bf16 is the upper half of an IEEE binary32.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Round-to-nearest-even to bf16; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate. Lane l supplies row (l % 16) of A
// and column (l % 16) of B, 8 reduction elements each, in the same reduction-slot order; lane
// l receives D rows 4*(l/16) .. 4*(l/16)+3 of column (l % 16).
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Eight E4M3 codes (half `hi` of the 16 in v, bytes in K order) as one bf16 MFMA operand. The
// hardware conversion decodes the OCP E4M3 format into float32; the bf16 is its upper half
// (exact, as E4M3 has 3 mantissa bits and a narrower exponent range).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(u32x4 v, int hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const uint32_t d0 = hi ? v.z : v.x, d1 = hi ? v.w : v.y;
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)d0, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)d0, true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)d1, false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)d1, true);
  auto pack = [](f32x2 f) {
    return __builtin_amdgcn_perm(__float_as_uint(f.y), __float_as_uint(f.x), 0x07060302u);
  };
  return u32x4{pack(a), pack(b), pack(c), pack(d)};
}

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Raw buffer loads: a load whose byte offset is at or past the buffer's size returns zeros
// and touches no memory, so padding lanes can take part in a load without a branch.
constexpr uint32_t kOutOfRange = 0x80000000u;  // offsets of padding lanes (buffers < 2 GiB)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 bufld16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  return (1ull << (threadIdx.x & 63)) - 1ull;
}

// The sorted-row layout every GEMM pass shares: rows are token-expert pairs sorted by
// (expert, adapter, token), each expert block padded to a multiple of the row-block size;
// padding rows hold pair id -1.
struct RowInfo {
  int pair;     // t * topk + j, or -1 for padding
  int token;    // pair / topk
  int adapter;  // adapter of the token, -1 for none or padding
};

__device__ __forceinline__ int sanitize_adapter(int a, int nA) {
  return (a >= 0 && a < nA) ? a : -1;
}

}  // namespace moelora

// ------------------------------------------------------------------------------------------
// Workspace layout (host side). Every region starts on a 256-byte boundary.
// ------------------------------------------------------------------------------------------
struct MoeLoraLayout {
  size_t topk_ids, topk_w, tok_flags, flags, sorted, expert_off, n_blocks, block_expert, block_seg,
      pair_row, sorted_ad, seg_table, n_seg, z1, z2, zhl, act, dpair, d_parts,
      align_lists, logits;
  size_t total;
  int64_t cap;     // rows of the sorted layout at the largest row-block size
  int max_bm;      // largest row-block size any path uses
};

bool moelora_make_layout(int T, int h, int I, int E, int nA, int r, int topk, int bm, int dsplit,
                         MoeLoraLayout* L);
