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

// Store of a finished tile at its rows of the sorted layout: SiLU-and-mul (gate_up, into act as
// bf16) or the plain fp32 store (down, into the K split's part of D), real rows only. Lane l holds rows 8*(v/4) + 4*(l/32) + (v%4) of each
// 32-row group and column (l % 32) of each 32-column fragment, so it goes through LDS (the main
// loop's stages are free by then): 16 rows at a time, each wavefront writes its values into its
// own region, row-major (rows padded so that the two lane halves, 4 rows apart, hit different
// banks), then reads whole 16-byte pieces of rows back and stores them: one global store per
// 1 KB rather than one per element column and row.
template <bool GATEUP, int BN, int WM, int WN, int FM, int FN, int NW, uint32_t LDS_BYTES>
__device__ __forceinline__ void tiled_store(const GemmArgs& a, f32x16 (&acc)[FM][FN],
                                            uint16_t* lds, int row0, int wm, int wn, int ntile,
                                            int ks, int wave, int lane) {
  constexpr int EB = GATEUP ? 2 : 4;          // bytes per stored element
  constexpr int COLS = GATEUP ? WN / 2 : WN;  // stored columns of the wavefront
  constexpr int STRIDE = COLS * EB + 32;      // LDS bytes per row
  constexpr int PR = 16;                      // rows per pass
  constexpr int CPRW = COLS * EB / 16;        // 16-byte pieces per row
  static_assert(NW * PR * STRIDE <= (int)LDS_BYTES, "store staging must fit the LDS stages");
  static_assert((PR * CPRW) % 64 == 0, "whole pieces per lane");
  const int fr = lane & 31, fg = lane >> 5;
  char* base = reinterpret_cast<char*>(lds) + wave * (PR * STRIDE);
  const size_t N = (size_t)a.N;
  // rows of this wavefront past the expert's last real row are padding: nothing reads them (the
  // down GEMM, the shrink and the combine take real rows only), so they are not stored. The
  // padding of an expert's block is a suffix: its start is the count of real rows.
  int wave_real = 0;
#pragma unroll
  for (int i = 0; i < (WM + 63) / 64; ++i) {
    const int rr = i * 64 + lane;
    const bool real = rr < WM && a.sorted_pairs[(size_t)row0 + wm * WM + rr] >= 0;
    wave_real += (int)__popcll(__ballot(real));
  }
  const size_t col0 =
      GATEUP ? (size_t)ntile * (BN / 2) + wn * (WN / 2) : (size_t)ntile * BN + wn * WN;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __syncthreads();  // the previous pass's pieces are read
#pragma unroll
      for (int vv = 0; vv < 8; ++vv) {
        const int v = 8 * h + vv;
        const int r = 8 * (vv / 4) + 4 * fg + (vv % 4);  // row within the pass
        if (GATEUP) {
#pragma unroll
          for (int jn = 0; jn < FN / 2; ++jn) {
            const float g = acc[i][jn][v], u = acc[i][jn + FN / 2][v];
            const float hv = g / (1.f + __expf(-g)) * u;
            *reinterpret_cast<uint16_t*>(base + r * STRIDE + (jn * 32 + fr) * 2) =
                (uint16_t)f32_to_bf16_bits(hv);
          }
        } else {
#pragma unroll
          for (int jn = 0; jn < FN; ++jn)
            *reinterpret_cast<float*>(base + r * STRIDE + (jn * 32 + fr) * 4) = acc[i][jn][v];
        }
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < PR * CPRW / 64; ++it) {
        const int idx = it * 64 + lane;
        const int r = idx / CPRW, c = idx % CPRW;
        const u32x4 val = *reinterpret_cast<const u32x4*>(base + r * STRIDE + c * 16);
        const size_t srow = (size_t)row0 + wm * WM + i * 32 + 16 * h + r;
        if (i * 32 + 16 * h + r >= wave_real) continue;
        if (GATEUP)
          *reinterpret_cast<u32x4*>(a.act_out + srow * N + col0 + c * 8) = val;
        else
          *reinterpret_cast<u32x4*>(a.d_out + ks * a.d_split_stride + srow * N + col0 + c * 4) =
              val;
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
    runs = __ballot(in && ad >= 0 && hi > lo);
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

// 16 zero bytes: the B-side source of extension-step slices that hold no run.
__device__ __align__(16) uint32_t g_zero16[4] = {0u, 0u, 0u, 0u};

// Loads of the tiled GEMM: the main K steps read the token rows (X) and the expert's weight rows
// (W) through buffer descriptors; the extension steps that follow (the LoRA expand as extra K,
// see tiled_gemm_kernel) read z (bf16, one plane [cap][r]) for the rows of each run, zeros for
// the other rows, and the runs' B rows through 64-bit addresses (B spans all adapters).
// STREAM_W: the weight tiles are loaded with the non-temporal hint (bf16 down, whose weight
// tiles no other tile of the same expert reads at the same time, each step a whole 128-byte line
// of every row; gate_up's are shared by the row tiles of a group and must stay in L2).
template <class Pipe, bool STREAM_W = false>
struct LoraExtLoader {
  static constexpr int NA = Pipe::NA, NB = Pipe::NB, BKS = Pipe::SUB * 16;
  // 64-run chunks of the run tables: one run per row of the 192-row tiles of the adapter-stress
  // layouts (down, many one-row runs: 0.45 -> 0.39 ms with one adapter per token); one chunk
  // for the others, where more runs than fit the quarter-of-the-loop rule never occur (prefill's
  // 256-row tiles: at most 16 runs of rank 64) and the extra search costs the main loop 3%
  static constexpr int RC = Pipe::TILE_M == 192 ? 3 : 1;
  u32x4 xr, wr, zr;
  uint32_t xo[NA], wo[NB];  // main steps: offsets at step 0
  int nks;                  // main steps
  int jrow[NA];             // run holding the A row of load block i (-1: none)
  uint32_t zo[NA];          // byte offset of that row's chunk in the z plane
  int slot_a[NA], slot_b[NB];  // run slot (within a step) of the chunk each lane loads
  uint32_t bo[NB];          // byte offset of the B chunk inside one (adapter, expert) slice
  const char* bexp;         // B slice of (adapter 0, this expert)
  size_t a_stride;          // bytes between adapters' slices of one expert
  int run_ad[RC];           // lane j of chunk c: adapter of run 64 c + j
  int nr, rps;              // runs; runs per extension step
  uint32_t xe[NA];          // prepared extension step: A offsets
  const void* be[NB];       // and B addresses

  __device__ __forceinline__ int main_steps() const { return nks; }
  __device__ __forceinline__ void load_main(int d, int ks, uint32_t lds_addr) {
    if (d < NA) lds_dma16(xr, xo[d], (uint32_t)ks * BKS * 2, lds_addr);
    else if (STREAM_W) lds_dma16_nt(wr, wo[d - NA], (uint32_t)ks * Pipe::BROW, lds_addr);
    else lds_dma16(wr, wo[d - NA], (uint32_t)ks * Pipe::BROW, lds_addr);
  }
  __device__ __forceinline__ void prep(int ks) {
    if (ks < nks) return;
    const int x = ks - nks;
#pragma unroll
    for (int i = 0; i < NA; ++i) xe[i] = (x * rps + slot_a[i] == jrow[i]) ? zo[i] : kOutOfRange;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int j = x * rps + slot_b[i];
      const int jj = j < nr ? j : 0;
      int adj = __shfl(run_ad[0], jj & 63);
#pragma unroll
      for (int c = 1; c < RC; ++c) {
        const int v = __shfl(run_ad[c], jj & 63);
        adj = (jj >> 6) == c ? v : adj;
      }
      be[i] = j < nr ? (const void*)(bexp + (size_t)adj * a_stride + bo[i]) : (const void*)g_zero16;
    }
  }
  __device__ __forceinline__ void load(int d, int ks, uint32_t lds_addr) {
    if (ks < nks) {
      load_main(d, ks, lds_addr);
    } else {
      if (d < NA) lds_dma16(zr, xe[d], 0u, lds_addr);
      else lds_dma16_global(be[d - NA], lds_addr);
    }
  }
};

// FP8: the weights are E4M3 codes (a.W8) with one float32 scale per weight row (a.wscale):
// staged in LDS as bytes, converted to bf16 fragments after the LDS read, and each accumulator
// column multiplied by its row's scale after the main loop, before the LoRA term (bf16 weights,
// unscaled, always in the epilogue) is added.
template <bool GATEUP, int BM, int BN, int WM, int WN, int BK, int NST, int NW, bool FP8 = false>
__global__ __launch_bounds__(64 * NW, 1) void tiled_gemm_kernel(GemmArgs a, int n_tiles_n,
                                                            int /*grid_total*/) {
  // (192-row tiles interleave the fragment reads with the MFMAs: measured faster there, slower
  // on the 256-row tiles)
  using Pipe = TilePipe<BM, BN, WM, WN, BK, NST, BM == 192, NW, FP8>;
  constexpr int FM = Pipe::FM, FN = Pipe::FN, NA = Pipe::NA, NB = Pipe::NB;
  static_assert(!GATEUP || FN % 2 == 0, "gate_up needs gate and up halves per wave");

  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // Pipe::LDS_BYTES

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / Pipe::WAVES_N, wn = wave % Pipe::WAVES_N;

  // Tile order. The live tiles (n_blocks row blocks x n_tiles_n column tiles; the grid is
  // sized for the largest n_blocks) are numbered column group by column group, row group by row
  // group, in groups of up to 4 row blocks x 4 column tiles (measured best of the shapes from
  // 2x8 to 16x8 on prefill and both adapter-stress batches; sub-tiles: below). Hardware workgroup ids go
  // round-robin over the 8 XCDs, so each XCD is given an equal contiguous range of that
  // numbering: the workgroups it runs at once cover a few groups, every token tile and weight
  // tile fetched into its L2 serves several of them, and no XCD gets more tiles than another.
  // (down may also split K: split ks of every tile comes after all tiles of split ks - 1)
  // Row tiles: the layout's row blocks, or (tiles smaller than the layout's blocks) every
  // BM-row sub-tile of them, a row group then being the sub-tiles of one block: they read the
  // same weight tiles at the same time, so each weight tile leaves HBM once per block (measured
  // on 192-row blocks in 64-row tiles against groups of four sub-tiles that straddle blocks:
  // gate_up fetches 11% less with one adapter, one adapter per token 3-8% faster). A sub-tile of
  // padding rows only returns at once.
  const int sub = a.layout_bm / BM;
  const int nblk = *a.n_blocks * sub;
  const int tiles = nblk * n_tiles_n;
  const int hw = blockIdx.x;
  const int slot = hw >> 3;
  int ks, t, nparts;  // K part of this workgroup, its tile, the tile's parts
  if (!GATEUP && a.tail_split > 1) {
    // Tail split: the tiles that fill whole rounds of n_cu resident workgroups run undivided
    // (each XCD an equal contiguous range, as below); the tiles of the last, partial round split
    // K in tail_split parts, dealt to the XCDs in turn, so that round is as full as the others.
    const int full = tiles / a.n_cu * a.n_cu, tail = tiles - full;
    const int fpx = full >> 3;
    if (slot < fpx) {
      t = (hw & 7) * fpx + slot;
      ks = 0;
      nparts = 1;
    } else {
      const int v = (slot - fpx) * 8 + (hw & 7);
      if (v >= tail * a.tail_split) return;
      t = full + v / a.tail_split;
      ks = v % a.tail_split;
      nparts = a.tail_split;
    }
  } else {
    const int live = tiles * (GATEUP ? 1 : a.ksplit);
    const int per_xcd = (live + 7) >> 3;
    const int tk = (hw & 7) * per_xcd + slot;
    if (slot >= per_xcd || tk >= live) return;
    ks = GATEUP ? 0 : tk / tiles;  // K split
    t = tk - ks * tiles;
    nparts = GATEUP ? 1 : a.ksplit;
  }
  const int GR = sub > 1 ? sub : 4;                // row tiles per group
  const int GC = sub > 1 ? 8 : 4;                  // column tiles per group (8 with sub-tiles:
                                                   // their token rows re-read half as often, -2%)
  const int cg = t / (nblk * GC);                 // column group (all but the last GC wide)
  const int cols = min(GC, n_tiles_n - cg * GC);
  const int u = t - cg * nblk * GC;
  const int rg = u / (GR * cols);                 // row group (all but the last GR tall)
  const int rows = min(GR, nblk - rg * GR);
  const int w = u - rg * GR * cols;
  const int rt = rg * GR + w % rows;  // row tile
  const int ntile = cg * GC + w / rows;
  const int row0 = rt * BM;
  // (an expert's padding is a suffix of its block: a sub-tile that starts on it holds no row)
  if (sub > 1 && a.sorted_pairs[row0] < 0) return;
  const int blk = row0 / a.layout_bm;  // its row block of the layout
  const int e = a.block_expert[blk];
  const int K = a.K;
  const int kspan = K / nparts;  // this part's K range: [ks * kspan, +kspan)
  // the combine learns from d_parts how many parts of D hold this tile
  if (!GATEUP && ks == 0 && a.d_parts) a.d_parts[(size_t)rt * n_tiles_n + ntile] = nparts;
  const uint32_t kbyte0 = (uint32_t)ks * kspan * 2;
  const size_t N = (size_t)a.N;
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
  // weight row of tile row n (gate_up: the wave's column range is [gate .. | up ..] of the same
  // act columns)
  auto wrow_of = [&](int n) -> size_t {
    if (GATEUP) {
      const int g = n / WN, rr = n % WN;
      const size_t col = (size_t)ntile * (BN / 2) + g * (WN / 2) + (rr % (WN / 2));
      return rr < WN / 2 ? col : N + col;
    }
    return (size_t)ntile * BN + n;
  };
  constexpr int WB = FP8 ? 1 : 2;  // bytes per weight
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int row = Pipe::load_row_b(i, wave, lane);
    const int chunk = Pipe::load_chunk_b(row, lane);
    wo[i] = (uint32_t)(wrow_of(row) * K * WB) + (uint32_t)ks * kspan * WB + 16u * chunk;
  }
  const u32x4 xr = buffer_desc(a.X, a.x_bytes);
  const u32x4 wr =
      FP8 ? buffer_desc(a.W8 + (size_t)e * w_rows * K, (uint32_t)(w_rows * K))
          : buffer_desc(a.W + (size_t)e * w_rows * K, (uint32_t)(w_rows * K * 2));

  // (measured: the bf16 down weight tiles streamed non-temporally, one-adapter stress down -8%;
  // gate_up's the same way, stress gate_up +25%; E4M3 rows of 64 bytes per step, half a cache
  // line, +24%: the hint drops the line before its second half is read)
  LoraExtLoader<Pipe, !GATEUP && !FP8> ld;
  ld.xr = xr;
  ld.wr = wr;
  ld.zr = buffer_desc(a.zhl, (uint32_t)((size_t)a.cap * a.r * 2));
  ld.nks = kspan / BK;
#pragma unroll
  for (int i = 0; i < NA; ++i) ld.xo[i] = xo[i];
#pragma unroll
  for (int i = 0; i < NB; ++i) ld.wo[i] = wo[i];
  ld.nr = 0;
  const int r = a.r;
  ld.rps = BK / r;
  const int cpr_r = r / 8;  // 16-byte chunks per run in an extension step
  bool use_ext = false;
  int nsteps = kspan / BK;

  // The LoRA expand as extra K steps when the tile's runs are few (the adapter segments clipped
  // to its rows, adapter >= 0): step x multiplies z of the rows of runs x*rps .. x*rps+rps-1,
  // each run in its own r-wide slice of the step's BK, zeros elsewhere, by the same slices of
  // the runs' B rows, so the expand streams through the main loop's pipeline. Every wavefront
  // finds the runs itself (lane j of register c holds run 64 c + j; 192-row tiles: one run per
  // row, others up to 64) while the first K steps' loads are in flight. Tiles with more extension steps than a
  // quarter of the main loop take the epilogue instead (lora_expand_segs).
  auto build_runs = [&]() {
    const int first = a.block_seg[blk];
    if (FP8 || ks != 0 || first < 0 || !a.lora_ext) return;
    // up to RC chunks of 64 segments from the block's first; lane j of chunk c holds the chunk's
    // j-th run (compacted), whose index among the tile's runs is base[c] + j
    constexpr int RC = decltype(ld)::RC;
    int run_ad[RC], run_lo[RC], run_hi[RC], base[RC + 1];
    base[0] = 0;
    bool more = true;  // the last segment looked at starts inside the tile: the next one may too
#pragma unroll
    for (int c = 0; c < RC; ++c) {
      run_ad[c] = 0;
      run_lo[c] = 0;
      run_hi[c] = 0;
      base[c + 1] = base[c];
      if (!more) continue;
      const int sj = first + 64 * c + lane;
      bool in = false, run = false;
      int lo = 0, hi = 0, ad = -1;
      if (sj < *a.n_seg) {
        const u32x4 sg = *reinterpret_cast<const u32x4*>(a.seg_table + 4 * (size_t)sj);
        const int st = (int)sg[2], cnt = (int)sg[3];
        in = st < row0 + BM;
        lo = max(st - row0, 0);
        hi = min(st + cnt - row0, BM);
        ad = sanitize_adapter((int)sg[1], a.nA);
        run = in && ad >= 0 && hi > lo;
      }
      const uint64_t m = __ballot(run);
      more = (__ballot(in) >> 63) != 0;
      // lane j <- run j (lanes without a run send theirs to lane 63, unused past the count)
      const int tgt = run ? __popcll(m & lanemask_lt()) : 63;
      run_ad[c] = __builtin_amdgcn_ds_permute(tgt * 4, ad);
      run_lo[c] = __builtin_amdgcn_ds_permute(tgt * 4, lo);
      run_hi[c] = __builtin_amdgcn_ds_permute(tgt * 4, hi);
      base[c + 1] = base[c] + __popcll(m);
    }
    if (more) {
      const int sn = first + 64 * RC;
      more = sn < *a.n_seg && a.seg_table[4 * (size_t)sn + 2] < row0 + BM;
    }
    const int nr = base[RC];
    const int n_ext = (nr + ld.rps - 1) / ld.rps;
    if (more || n_ext == 0 || 4 * n_ext > ld.nks) return;
    use_ext = true;
    ld.nr = nr;
#pragma unroll
    for (int c = 0; c < RC; ++c) ld.run_ad[c] = run_ad[c];
    nsteps = ld.nks + n_ext;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int row = Pipe::load_row(i, wave, lane);
      const int chunk = Pipe::load_chunk(row, lane);
      // the last run starting at or before the row (runs are disjoint and in row order): in
      // each chunk, the count of its runs that start at or before it; every lane takes part in
      // every shuffle
      int j = -1, hi_j = 0;
#pragma unroll
      for (int c = 0; c < RC; ++c) {
        const int nc = base[c + 1] - base[c];
        if (nc == 0) continue;  // (wavefront-uniform)
        int b = 0;
#pragma unroll
        for (int step = 64; step > 0; step >>= 1) {
          const int cand = b + step;
          const int lo_c = __shfl(run_lo[c], max(min(cand, nc) - 1, 0));
          if (cand <= nc && lo_c <= row) b = cand;
        }
        const int h = __shfl(run_hi[c], b > 0 ? b - 1 : 0);
        if (b > 0) {
          j = base[c] + b - 1;
          hi_j = h;
        }
      }
      ld.jrow[i] = (j >= 0 && row < hi_j) ? j : -1;
      ld.slot_a[i] = chunk / cpr_r;
      ld.zo[i] = (uint32_t)(((size_t)(row0 + row) * r + (chunk % cpr_r) * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int row = Pipe::load_row_b(i, wave, lane);
      const int chunk = Pipe::load_chunk_b(row, lane);
      const size_t wrow = wrow_of(row);
      ld.slot_b[i] = chunk / cpr_r;
      ld.bo[i] = (uint32_t)((wrow * r + (chunk % cpr_r) * 8) * 2);
    }
    ld.bexp = reinterpret_cast<const char*>(a.Bw + (size_t)e * w_rows * r);
    ld.a_stride = (size_t)a.E * w_rows * r * 2;
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  Pipe::run_steps(acc, ld, lds, nsteps, wave, lane, build_runs);

  __syncthreads();  // every wavefront is done with the main loop's LDS stages

  if (FP8) {  // per-row scales of the E4M3 weights (lane: column fr of each 32-column fragment)
    const float* sc = a.wscale + (size_t)e * w_rows;
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) {
      const float s = sc[wrow_of(wn * WN + jn * 32 + (lane & 31))];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][jn][v] *= s;
    }
  }

  // the LoRA term goes into K split 0 only (the combine adds the splits); tiles with many runs
  // add it here, after the main loop
  if (ks == 0 && !use_ext)
    lora_expand_segs<GATEUP, BM, BN, WM, WN, FM, FN, Pipe::LDS_BYTES, NW>(a, acc, lds, blk, row0,
                                                                           wm, wn, ntile, e, wave,
                                                                           lane);
  tiled_store<GATEUP, BN, WM, WN, FM, FN, NW, Pipe::LDS_BYTES>(a, acc, lds, row0, wm, wn, ntile, ks,
                                                                wave, lane);
}

template <bool GATEUP, int BM, int BN, int WM, int WN, int BK, int NST, int NW, bool FP8 = false>
hipError_t launch_tiled_t(const GemmArgs& a, int n_tiles_n, int total, hipStream_t stream) {
  constexpr int lds_bytes = TilePipe<BM, BN, WM, WN, BK, NST, BM == 192, NW, FP8>::LDS_BYTES;
  static_assert(lds_bytes <= kLdsBytes, "LDS stages must fit");
  auto kern = tiled_gemm_kernel<GATEUP, BM, BN, WM, WN, BK, NST, NW, FP8>;
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

hipError_t launch_tiled(const TiledConfig& c, bool gateup, const GemmArgs& a, hipStream_t stream,
                        bool fp8) {
  const int cols = gateup ? 2 * a.N : a.N;
  if (cols % c.bn != 0) return hipErrorInvalidValue;
  const int splits = gateup ? 1 : (a.tail_split > 1 ? a.tail_split : a.ksplit);
  if (splits < 1 || splits > kMaxParts || (a.K / splits) % c.bk != 0 || a.K % splits != 0)
    return hipErrorInvalidValue;
  if (!gateup && a.tail_split > 1 && (a.n_cu <= 0 || a.n_cu % 8 != 0 || !a.d_parts))
    return hipErrorInvalidValue;
  const int n_tiles_n = cols / c.bn;
  // one workgroup per (row block, column tile, K split) for the largest row-block count,
  // rounded up to a multiple of the 8 XCDs
  if (a.layout_bm % c.bm != 0 || (a.layout_bm != c.bm && c.bm != 64))
    return hipErrorInvalidValue;
  int total = a.n_blocks_max * (a.layout_bm / c.bm) * n_tiles_n * splits;
  total = (total + 7) / 8 * 8;
  if (total <= 0) return hipSuccess;
  // E4M3 weights: the tiles the path picks by default
#define MOELORA_TILED8(BM_, BN_, WM_, WN_, GU_)                                                  \
  if (fp8 && gateup == GU_ && c.bm == BM_ && c.bn == BN_ && c.wm == WM_ && c.wn == WN_ &&        \
      c.bk == 64 && c.nst == 2 && c.nw == (BM_ * BN_ / (WM_ * WN_)))                            \
    return launch_tiled_t<GU_, BM_, BN_, WM_, WN_, 64, 2, BM_ * BN_ / (WM_ * WN_), true>(         \
        a, n_tiles_n, total, stream);
  MOELORA_TILED8(64, 256, 32, 64, true)
  MOELORA_TILED8(64, 128, 32, 64, false)
  MOELORA_TILED8(128, 128, 32, 64, true)
  MOELORA_TILED8(128, 128, 32, 64, false)
  MOELORA_TILED8(256, 256, 64, 128, true)
  MOELORA_TILED8(256, 256, 64, 128, false)
  MOELORA_TILED8(192, 256, 96, 64, false)
#undef MOELORA_TILED8
  if (fp8) return hipErrorInvalidValue;
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
  MOELORA_TILED(192, 256, 96, 64, 64, 2, 8)
  MOELORA_TILED(128, 256, 64, 64, 64, 2, 8)
  MOELORA_TILED(256, 256, 128, 128, 64, 2, 4)
  // down only (one 32-column fragment per wave: no gate/up halves)
  if (!gateup && c.bm == 192 && c.bn == 128 && c.wm == 96 && c.wn == 32 && c.bk == 64 &&
      c.nst == 2 && c.nw == 8)
    return launch_tiled_t<false, 192, 128, 96, 32, 64, 2, 8>(a, n_tiles_n, total, stream);
#undef MOELORA_TILED
  return hipErrorInvalidValue;
}

}  // namespace moelora
