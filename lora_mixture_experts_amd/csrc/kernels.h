// Kernel argument blocks and kernel declarations of libmoelora (internal).
#pragma once

#include "common.h"

namespace moelora {

constexpr int kAlignThreads = 1024;
constexpr int kAlignStaticLds = 17 * 1024;  // >= the align kernel's static LDS (16.7 KB)
constexpr int kLdsBytes = 160 * 1024;

struct AlignArgs {
  const int* topk_ids;     // [T*k], or nullptr: expert 0 for every pair (no routing)
  const int* adapter_ids;  // [T]
  const int* tok_flags;    // [T] or nullptr
  int T, k, E, nA, seg_pad, block_m;
  int* sorted_pairs;    // [>= padded total]
  int* expert_offsets;  // [E+1]
  int* seg_table;       // [T*k][4]
  int* n_seg;           // [1]
  int* flags;           // [1]
  int* block_expert;    // [padded total / block_m] or nullptr
  int* block_seg;       // [padded total / block_m]: segment holding the block's first row, or -1
                        // (a block of padding rows); written when block_expert is
  int* pair_row;        // [T*k]: sorted row of each pair, or nullptr
  int* sorted_ad;       // [>= padded total]: adapter of each sorted row (-1: none or padding),
                        // or nullptr
  int* n_blocks;        // [1] or nullptr
  int* g_lists;         // workspace for the arrays when they do not fit in LDS
  int lists_in_lds;
  int digit_bits;  // radix digit width D (1..10)
  int passes;      // digits of the bucket key (passes * D >= its bit width)
  int seg_cap;     // min(T*k, E*(nA+1)) + 1: room for the segment starts (and deltas)
};

// Radix digits of the align kernel for E*(nA+1) buckets: as few passes of at most 10 bits as
// the key width needs, the width spread evenly over them.
inline void align_digits(int E, int nA, int* digit_bits, int* passes) {
  const uint32_t nb = (uint32_t)E * (uint32_t)(nA + 1);
  int bits = 0;
  while (bits < 31 && (1u << bits) < nb) ++bits;
  if (bits < 1) bits = 1;
  *passes = (bits + 9) / 10;
  *digit_bits = (bits + *passes - 1) / *passes;
}

inline int align_seg_cap(int T, int k, int E, int nA) {
  const int64_t P = (int64_t)T * k, nb = (int64_t)E * (nA + 1);
  return (int)((P < nb ? P : nb) + 1);
}

// ints of the align kernel's arrays: keys and two pair-id buffers [T*k] each, segment starts and
// deltas [seg_cap] each
inline size_t align_list_ints(int T, int k, int E, int nA) {
  return 3 * (size_t)T * k + 2 * (size_t)align_seg_cap(T, k, E, nA);
}

// Adapter segments of a dense multi-LoRA batch (sgmv_sort_kernel): the sorted layout of the
// tokens that carry an adapter, by (adapter, token), in 16-row blocks.
constexpr int kSgmvSortMaxTokens = 1024;
constexpr int kSgmvSortMaxAdapters = 1024;
struct SgmvSortArgs {
  const int* adapter_ids;  // [T]
  int T, nA;
  int* sorted_pairs;  // [>= round_up(T, 16)]: token of each row, -1 for padding
  int* sorted_ad;     // its adapter, -1 for padding
  int* block_expert;  // [blocks]: 0
  int* n_blocks;      // [1]
  int* flags;         // [1]: MOELORA_FLAG_ADAPTER_RANGE when an id is out of range
};

// LoRA shrink z = X A^T for the rows of the sorted layout.
struct ShrinkArgs {
  const uint16_t* X;  // gather: x [T][K]; otherwise act [cap][K]
  uint32_t x_bytes;   // size of X (< 2 GiB)
  const int* sorted_pairs;
  const int* sorted_ad;  // adapter of each sorted row, -1 for none or padding
  const int* block_expert;
  const int* block_seg;  // (64-row shrink) first segment of each row block, or -1
  const int* seg_table;  // (64-row shrink) [n_seg][4]
  const int* n_seg;
  const int* n_blocks;
  int bm;
  const int* adapter_ids;
  int k, nA, E, r, K;
  const uint16_t* Aw;  // [nA][E][r][K]
  int S;               // K splits over workgroups
  float* zpart;        // [S][cap][r]; written for the rows that carry an adapter
  int64_t cap;
  int xcd_ranges;      // 1: split-major order, each XCD a contiguous range of it (long runs);
                       // 0: tile-major, the S splits of a 16-row tile on consecutive ids
  int after64;         // 16-row shrink: only the sub-blocks the 64-row shrink leaves
};

// Base GEMM of one projection for the rows of the sorted layout, with the LoRA expand (and
// for gate_up the SiLU-and-mul) in the epilogue.
struct GemmArgs {
  const uint16_t* X;   // gate_up: x [T][K]; down: act [cap][K]
  uint32_t x_bytes;    // size of X (< 2 GiB)
  const uint16_t* W;   // gate_up: W1 [E][2I][h]; down: W2 [E][h][I]
  const uint8_t* W8;   // skinny FP8 entry: the same weights as E4M3 codes (W unused)
  const float* wscale; // with W8: one scale per weight row ([E][2I] or [E][h])
  const uint16_t* Bw;  // gate_up: B1 [nA][E][2I][r]; down: B2 [nA][E][h][r]
  const float* zpart;   // skinny: [zsplits][cap][r] the LoRA shrink's split parts, added in
  int zsplits;          //   the prologue in split order
  const uint16_t* zhl;  // tiled: [2][cap][r] the same as bf16 high and low planes
  int64_t cap;
  const int* sorted_pairs;
  const int* sorted_ad;  // adapter of each sorted row, -1 for none or padding
  const int* block_expert;
  const int* block_seg;  // first segment of each row block (or -1), see AlignArgs
  const int* seg_table;  // [n_seg][4]: expert, adapter, first sorted row, rows
  const int* n_seg;
  const int* n_blocks;
  const int* adapter_ids;
  int k, nA, E, r;
  int K;  // reduction length
  int N;  // gate_up: I (act columns); down: h
  uint16_t* act_out;  // gate_up: [cap][I]
  float* d_out;       // down: [parts][cap][h] partial sums, rows in sorted order
  int ksplit;         // down: K splits of every tile; gate_up: 1
  int64_t d_split_stride;
  int tail_split;     // tiled down, > 1: the tiles of the last partial round of n_cu workgroups
                      // split K in tail_split parts (the others none); 0: ksplit for all
  int n_cu;           // workgroups resident at once (one tiled tile per CU), a multiple of 8
  int* d_parts;       // tiled down: [row tile][column tile] K parts written (combine reads it)
  int n_blocks_max;   // row blocks the grid is sized for (>= *n_blocks)
  int layout_bm;      // tiled: row-block size of the sorted layout (a multiple of the tile's BM;
                      // a larger one is walked in BM-row sub-tiles)
  int n_col_tiles;    // skinny: column tiles of one row block (N / columns per workgroup)
  int lora_ext;       // tiled: 1 lets tiles with few adapter runs add the LoRA expand as extra K
                      // steps of the main loop (0: always in the epilogue)
};

// Dense multi-LoRA expand: y[t] += z[t] B_a^T over the sorted layout of T tokens (k = 1, E = 1).
struct SgmvArgs {
  const int* sorted_pairs;  // [cap]: token of each sorted row, -1 for padding
  const int* sorted_ad;     // [cap]: its adapter, -1 for none or padding
  const int* n_blocks;      // live 16-row blocks
  const float* zpart;       // [zsplits][cap][r] the shrink's split parts, added in split order
  int zsplits;
  int64_t cap;
  const uint16_t* B;        // [nA][N][r]
  uint16_t* y;              // [T][N], updated in place
  int N, r;
};

// Tile shape of the LDS-staged GEMM: nw wavefronts of WM x WN each; NST LDS stages of BK k.
struct TiledConfig {
  int bm, bn, wm, wn;
  int bk, nst;
  int nw = 4;
};

// Tile shape of the skinny (few rows per expert) GEMM.
struct SkinnyConfig {
  int nt;  // 16-row token tiles per row block
  int p;   // 16-byte loads per lane per weight row and K step (K step = 32 * p)
  int rt;  // 16-row output tiles per wavefront
  int pipe;   // 1: ping-pong register sets (loads of step k+1 overlap MFMAs of step k)
  int split;  // gate_up: gate and up rows streamed by different wavefronts
};

// Host launchers (each defined next to its kernel). They return the launch status.
hipError_t launch_route(const float* logits, int T, int E, int k, int* topk_ids, float* topk_w,
                        int* tok_flags, hipStream_t stream);
hipError_t launch_align(const AlignArgs& a, size_t dyn_lds, hipStream_t stream);
hipError_t launch_sgmv_sort(const SgmvSortArgs& a, hipStream_t stream);
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* W, int T, int K, int E,
                                float* logits, hipStream_t stream);
hipError_t launch_shrink(bool gather, const ShrinkArgs& a, int tiles, hipStream_t stream);
// one wavefront per (adapter segment, K split), for up to max_segments segments (short runs)
hipError_t launch_shrink_seg(bool gather, const ShrinkArgs& a, int max_segments,
                             hipStream_t stream);
hipError_t launch_shrink_tiled(bool gather, const ShrinkArgs& a, int n_sub_max,
                               hipStream_t stream);
hipError_t launch_zfinal(const float* zpart, int S, int64_t cap, int r, const int* n_blocks,
                         int bm, int64_t max_rows, uint16_t* zhl, hipStream_t stream);
hipError_t launch_skinny(const SkinnyConfig& c, bool gateup, const GemmArgs& a, int grid_y,
                         hipStream_t stream, bool fp8 = false);
hipError_t launch_tiled(const TiledConfig& c, bool gateup, const GemmArgs& a, hipStream_t stream,
                        bool fp8 = false);
hipError_t launch_sgmv_expand(const SgmvArgs& a, int max_blocks, hipStream_t stream);
// D parts: d_parts == nullptr: ksplit parts for every row; else d_parts[(row / part_rows) *
// part_ncol + col / part_cols] parts (1 to 4) for the tile holding (row, col).
struct CombineArgs {
  const float* D;
  int ksplit;
  int64_t split_stride;
  const int* d_parts;
  int part_rows, part_cols, part_ncol;
  const int* pair_row;
  const float* topk_w;
  int T, k, h;
  uint16_t* y;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

}  // namespace moelora
