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
// (all of one expert) and BN output features. The main loop (TilePipe) loads both operand
// tiles straight from HBM into a ring of LDS stages and runs 32x32x16 bf16 MFMAs on them.
//
// gate_up: the weight rows of each wave's column range are [gate i .. | up i ..] for the same
// intermediate columns i, so each lane holds gate and up of the same act element and
// SiLU-and-mul runs in registers, after the LoRA expand is added.
//
// LoRA expand (both projections): rows are sorted by adapter inside an expert, so the rows of a
// tile form a few contiguous adapter runs. For every run, the tile's columns of
// B[adapter][expert] are loaded into LDS once and every 32-row MFMA group the run overlaps adds
// (z restricted to the run's rows) x B as extra MFMAs over K = r: a segment's adapter weights
// are read once per tile, not per token. z is split into bf16 high and low parts (two MFMAs)
// so the term keeps ~16 mantissa bits.
#include "common.h"
#include "kernels.h"
#include "tile_pipeline.h"

namespace moelora {

// Store of a finished tile at its rows of the sorted layout: SiLU-and-mul (gate_up, into act) or
// the plain store (down, into the K split's part of D). Padding rows hold zeros (their token rows
// were loaded as zeros and carry no adapter) and are stored like the others, so the store needs
// no per-row lookup. Lane l holds rows 8*(v/4) + 4*(l/32) + (v%4) of each 32-row group and column
// (l % 32) of each 32-column fragment.
template <bool GATEUP, int BN, int WM, int WN, int FM, int FN>
__device__ __forceinline__ void tiled_store(const GemmArgs& a, f32x16 (&acc)[FM][FN], int row0,
                                            int wm, int wn, int ntile, int ks, int lane) {
  const size_t N = (size_t)a.N;
  const int fr = lane & 31, fg = lane >> 5;
  // column of fragment jn: gate_up act column (gate and up halves share it); down output column
  auto col_of = [&](int jn) -> size_t {
    if (GATEUP) return (size_t)ntile * (BN / 2) + wn * (WN / 2) + (jn % (FN / 2)) * 32 + fr;
    return (size_t)ntile * BN + wn * WN + jn * 32 + fr;
  };
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const size_t srow = (size_t)row0 + wm * WM + i * 32 + 8 * (v / 4) + 4 * fg + (v % 4);
      if (GATEUP) {
#pragma unroll
        for (int jn = 0; jn < FN / 2; ++jn) {
          const float g = acc[i][jn][v], u = acc[i][jn + FN / 2][v];
          const float hv = g / (1.f + __expf(-g)) * u;
          a.act_out[srow * N + col_of(jn)] = (uint16_t)f32_to_bf16_bits(hv);
        }
      } else {
#pragma unroll
        for (int jn = 0; jn < FN; ++jn)
          a.d_out[ks * a.d_split_stride + srow * N + col_of(jn)] = acc[i][jn][v];
      }
    }
  }
}

// Lane of the n-th set bit of a wavefront-uniform mask.
__device__ __forceinline__ int nth_set_bit(uint64_t m, int n) {
  for (int i = 0; i < n; ++i) m &= m - 1;
  return __builtin_ctzll(m);
}

// LoRA expand of a whole tile, after the main loop (its LDS stages are free by then). The rows of
// a tile are sorted by adapter, so the segments of the segment table that overlap it are runs of
// one adapter; they start at the block's first segment, and lane j of every wavefront takes
// segment first + j clipped to the tile (64 at a time), so no table is built. For each run with
// an adapter the tile's columns of B[adapter][expert] (BN rows x r, r-contiguous) are loaded
// straight into LDS, up to as many runs at once as fit, with one wait per batch, and every 32-row
// group the run overlaps adds (z restricted to the run's rows) x B over K = r. z (the sum of the
// shrink's split parts as bf16 high and low planes) is loaded while the first batch is in
// flight.
template <bool GATEUP, int BM, int BN, int WM, int WN, int FM, int FN, uint32_t LDS_BYTES,
          int NWAVES>
__device__ __forceinline__ void lora_expand_segs(const GemmArgs& a, f32x16 (&acc)[FM][FN],
                                                 uint16_t* lds, int blk, int row0, int wm, int wn,
                                                 int ntile, int e, int wave, int lane) {
  constexpr int MAXSL = 4;  // 16-wide slices of r (r <= 64)
  static_assert(LDS_BYTES >= BN * 64 * 2, "the B tile of one run must fit");
  const int first = a.block_seg[blk];
  if (first < 0) return;
  const int nseg = *a.n_seg;
  const int r = a.r;
  const size_t N = (size_t)a.N;
  const size_t w_rows = GATEUP ? 2 * N : N;
  const int fr = lane & 31, fg = lane >> 5;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;

  // B tile of one run in LDS: BN rows (the tile's weight rows) x r, the 16-byte chunk index
  // XOR-swizzled by the row (rows of r/8 chunks; 1 KB load blocks of 512/r rows). A fragment
  // read takes 16 consecutive rows at one chunk per 256-byte pass of the 64 LDS banks, so rows
  // 16/cpr apart must land in different slots.
  const int cpr = r / 8, rpb = 512 / r;
  const int rsh = 16 / cpr;  // rows per swizzle step
  auto swz = [&](int row, int c) { return c ^ ((row / rsh) & (cpr - 1)); };
  const uint32_t run_bytes = (uint32_t)BN * r * 2;
  const int rb = (int)(LDS_BYTES / run_bytes);  // runs per batch (>= 2)
  const int bpr = BN / rpb;                     // load blocks per run
  auto wrow_of_tile_row = [&](int row) -> size_t {
    if (GATEUP) {
      const int g = row / WN, rr = row % WN;
      const size_t col = (size_t)ntile * (BN / 2) + g * (WN / 2) + (rr % (WN / 2));
      return rr < WN / 2 ? col : N + col;
    }
    return (size_t)ntile * BN + row;
  };

  // z of this wavefront's rows as bf16 high and low parts (one load each per 32-row group and
  // 16-wide slice of r)
  u32x4 zh[FM][MAXSL], zl[FM][MAXSL];
  auto load_z = [&]() {
    const uint16_t* zhp = a.zhl;
    const uint16_t* zlp = a.zhl + (size_t)a.cap * r;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const size_t zrow = (size_t)(row0 + wm * WM + i * 32 + fr) * r;
#pragma unroll
      for (int sl = 0; sl < MAXSL; ++sl) {
        const int q = 16 * sl + 8 * fg;
        const u32x4 zero{0u, 0u, 0u, 0u};
        zh[i][sl] = q < r ? *reinterpret_cast<const u32x4*>(zhp + zrow + q) : zero;
        zl[i][sl] = q < r ? *reinterpret_cast<const u32x4*>(zlp + zrow + q) : zero;
      }
    }
  };

  // lane j: segment c0 + j, clipped to the tile (segments from the block's first one on start
  // inside the tile until one starts past it)
  int c0 = first, lo = 0, hi = 0, ad = -1;
  uint64_t in_mask = 0, runs = 0, batch = 0;
  int nb = 0;
  auto chunk = [&]() {
    const int sj = c0 + lane;
    bool in = false;
    lo = hi = 0;
    ad = -1;
    if (sj < nseg) {
      const u32x4 sg = *reinterpret_cast<const u32x4*>(a.seg_table + 4 * (size_t)sj);
      const int st = (int)sg[2], cnt = (int)sg[3];
      in = st < row0 + BM;
      lo = max(st - row0, 0);
      hi = min(st + cnt - row0, BM);
      ad = sanitize_adapter((int)sg[1], a.nA);
    }
    in_mask = __ballot(in);
    runs = __ballot(in && ad >= 0);
  };
  // the next chunk with runs with an adapter, if any
  auto next_runs = [&]() {
    while (!runs && (in_mask >> 63)) {
      c0 += 64;
      chunk();
    }
  };
  // the next batch (the lowest rb runs left), its B tiles loaded into LDS
  auto issue_batch = [&]() {
    batch = 0;
    nb = 0;
    while (runs && nb < rb) {
      batch |= runs & (~runs + 1);
      runs &= runs - 1;
      ++nb;
    }
    for (int bl = wave; bl < nb * bpr; bl += NWAVES) {
      const int kk = bl / bpr, bi = bl % bpr;
      const int adk = __builtin_amdgcn_readlane(ad, nth_set_bit(batch, kk));
      const int row = bi * rpb + lane / cpr;
      const int ch = swz(row, lane % cpr);
      const u32x4 br = buffer_desc(a.Bw + ((size_t)adk * a.E + e) * w_rows * r,
                                   (uint32_t)(w_rows * r * 2));
      lds_dma16(br, (uint32_t)(wrow_of_tile_row(row) * r * 2) + 16u * ch, 0u,
                lds0 + kk * run_bytes + bi * 1024);
    }
  };

  chunk();
  next_runs();
  if (!runs) return;
  issue_batch();
  load_z();  // while the first batch is in flight
  while (true) {
    wait_vmcnt<0>();
    __syncthreads();
    for (int kk = 0; kk < nb; ++kk) {
      const int j = nth_set_bit(batch, kk);
      const int rlo = __builtin_amdgcn_readlane(lo, j), rhi = __builtin_amdgcn_readlane(hi, j);
      const uint16_t* bt = lds + kk * (run_bytes / 2);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int g0 = wm * WM + i * 32;
        if (rlo >= g0 + 32 || rhi <= g0) continue;
        const bool inr = g0 + fr >= rlo && g0 + fr < rhi;
#pragma unroll
        for (int sl = 0; sl < MAXSL; ++sl) {
          if (16 * sl >= r) continue;
          const int c = 2 * sl + fg;
          const u32x4 zero{0u, 0u, 0u, 0u};
          const u32x4 za = inr ? zh[i][sl] : zero, zb = inr ? zl[i][sl] : zero;
#pragma unroll
          for (int jn = 0; jn < FN; ++jn) {
            const int n = wn * WN + jn * 32 + fr;
            const u32x4 bv =
                8 * c < r ? *reinterpret_cast<const u32x4*>(bt + n * r + 8 * swz(n, c)) : zero;
            acc[i][jn] = mfma32(za, bv, acc[i][jn]);
            acc[i][jn] = mfma32(zb, bv, acc[i][jn]);
          }
        }
      }
    }
    __syncthreads();  // the next batch overwrites the B tiles
    next_runs();
    if (!runs) break;
    issue_batch();
  }
}

template <bool GATEUP, int BM, int BN, int WM, int WN, int BK, int NST, int NW>
__global__ __launch_bounds__(64 * NW, 1) void tiled_gemm_kernel(GemmArgs a, int n_tiles_n,
                                                            int /*grid_total*/) {
  using Pipe = TilePipe<BM, BN, WM, WN, BK, NST, true, NW>;
  constexpr int FM = Pipe::FM, FN = Pipe::FN, NA = Pipe::NA, NB = Pipe::NB;
  static_assert(!GATEUP || FN % 2 == 0, "gate_up needs gate and up halves per wave");

  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // Pipe::LDS_BYTES

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / Pipe::WAVES_N, wn = wave % Pipe::WAVES_N;

  // Tile order. The live tiles (n_blocks row blocks x n_tiles_n column tiles; the grid is
  // sized for the largest n_blocks) are numbered column group by column group, row group by row
  // group, in groups of up to 4 row blocks x 4 column tiles (measured best of the shapes from
  // 2x8 to 16x8 on prefill and both adapter-stress batches). Hardware workgroup ids go
  // round-robin over the 8 XCDs, so each XCD is given an equal contiguous range of that
  // numbering: the workgroups it runs at once cover a few groups, every token tile and weight
  // tile fetched into its L2 serves several of them, and no XCD gets more tiles than another.
  // (down may also split K: split ks of every tile comes after all tiles of split ks - 1)
  const int nblk = *a.n_blocks;
  const int tiles = nblk * n_tiles_n;
  const int live = tiles * (GATEUP ? 1 : a.ksplit);
  const int per_xcd = (live + 7) >> 3;
  const int hw = blockIdx.x;
  const int slot = hw >> 3;
  const int tk = (hw & 7) * per_xcd + slot;
  if (slot >= per_xcd || tk >= live) return;
  const int ks = GATEUP ? 0 : tk / tiles;        // K split
  const int t = tk - ks * tiles;
  constexpr int GR = 4, GC = 4;                   // row blocks and column tiles per group
  const int cg = t / (nblk * GC);                 // column group (all but the last GC wide)
  const int cols = min(GC, n_tiles_n - cg * GC);
  const int u = t - cg * nblk * GC;
  const int rg = u / (GR * cols);                 // row group (all but the last GR tall)
  const int rows = min(GR, nblk - rg * GR);
  const int w = u - rg * GR * cols;
  const int blk = rg * GR + w % rows;
  const int ntile = cg * GC + w / rows;
  const int e = a.block_expert[blk];
  const int K = a.K;
  const int kspan = GATEUP ? K : K / a.ksplit;  // this split's K range: [ks * kspan, +kspan)
  const uint32_t kbyte0 = (uint32_t)ks * kspan * 2;
  const size_t N = (size_t)a.N;
  const int row0 = blk * BM;
  const size_t w_rows = GATEUP ? 2 * N : N;  // weight rows of one expert

  // byte offsets of the chunk each lane loads at K step 0 (padding rows: out of range, zeros)
  uint32_t xo[NA], wo[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int row = Pipe::load_row(i, wave, lane);
    const int chunk = Pipe::load_chunk(row, lane);
    const int srow = row0 + row;
    const int p = a.sorted_pairs[srow];
    xo[i] = p < 0 ? kOutOfRange
                  : (uint32_t)((GATEUP ? (size_t)(p / a.k) : (size_t)srow) * K * 2) + kbyte0 +
                        16u * chunk;
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int row = Pipe::load_row(i, wave, lane);
    const int chunk = Pipe::load_chunk(row, lane);
    size_t wrow;
    if (GATEUP) {
      const int g = row / WN, rr = row % WN;
      const size_t col = (size_t)ntile * (BN / 2) + g * (WN / 2) + (rr % (WN / 2));
      wrow = rr < WN / 2 ? col : N + col;
    } else {
      wrow = (size_t)ntile * BN + row;
    }
    wo[i] = (uint32_t)(wrow * K * 2) + kbyte0 + 16u * chunk;
  }
  const u32x4 xr = buffer_desc(a.X, a.x_bytes);
  const u32x4 wr = buffer_desc(a.W + (size_t)e * w_rows * K, (uint32_t)(w_rows * K * 2));

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  Pipe::run(acc, xr, xo, wr, wo, lds, kspan, wave, lane);

  __syncthreads();  // every wavefront is done with the main loop's LDS stages

  // the LoRA term goes into K split 0 only (the combine adds the splits)
  if (ks == 0)
    lora_expand_segs<GATEUP, BM, BN, WM, WN, FM, FN, Pipe::LDS_BYTES, NW>(a, acc, lds, blk, row0,
                                                                           wm, wn, ntile, e, wave,
                                                                           lane);
  tiled_store<GATEUP, BN, WM, WN, FM, FN>(a, acc, row0, wm, wn, ntile, ks, lane);
}

template <bool GATEUP, int BM, int BN, int WM, int WN, int BK, int NST, int NW>
hipError_t launch_tiled_t(const GemmArgs& a, int n_tiles_n, int total, hipStream_t stream) {
  constexpr int lds_bytes = TilePipe<BM, BN, WM, WN, BK, NST, true, NW>::LDS_BYTES;
  static_assert(lds_bytes <= kLdsBytes, "LDS stages must fit");
  auto kern = tiled_gemm_kernel<GATEUP, BM, BN, WM, WN, BK, NST, NW>;
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
  hipLaunchKernelGGL(kern, dim3(total), dim3(64 * NW), lds_bytes, stream, a, n_tiles_n, total);
  return hipGetLastError();
}

hipError_t launch_tiled(const TiledConfig& c, bool gateup, const GemmArgs& a, hipStream_t stream) {
  const int cols = gateup ? 2 * a.N : a.N;
  if (cols % c.bn != 0) return hipErrorInvalidValue;
  const int splits = gateup ? 1 : a.ksplit;
  if (splits < 1 || (a.K / splits) % c.bk != 0 || a.K % splits != 0) return hipErrorInvalidValue;
  const int n_tiles_n = cols / c.bn;
  // one workgroup per (row block, column tile, K split) for the largest row-block count,
  // rounded up to a multiple of the 8 XCDs
  int total = a.n_blocks_max * n_tiles_n * splits;
  total = (total + 7) / 8 * 8;
  if (total <= 0) return hipSuccess;
#define MOELORA_TILED(BM_, BN_, WM_, WN_, BK_, NST_, NW_)                                   \
  if (c.bm == BM_ && c.bn == BN_ && c.wm == WM_ && c.wn == WN_ && c.bk == BK_ && c.nst == NST_ && \
      c.nw == NW_)                                                                              \
    return gateup                                                                               \
        ? launch_tiled_t<true, BM_, BN_, WM_, WN_, BK_, NST_, NW_>(a, n_tiles_n, total, stream) \
        : launch_tiled_t<false, BM_, BN_, WM_, WN_, BK_, NST_, NW_>(a, n_tiles_n, total, stream);
  MOELORA_TILED(64, 128, 32, 64, 64, 2, 4)
  MOELORA_TILED(128, 128, 32, 64, 64, 2, 8)
  MOELORA_TILED(256, 256, 64, 128, 64, 2, 8)
  MOELORA_TILED(64, 256, 32, 64, 64, 2, 8)
#undef MOELORA_TILED
  return hipErrorInvalidValue;
}

}  // namespace moelora
