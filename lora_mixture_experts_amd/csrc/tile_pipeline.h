// Main loop of the LDS-tiled expert GEMM: operand tiles are loaded from HBM straight into a
// ring of LDS stages and multiplied on 32x32x16 bf16 MFMAs. Internal to libmoelora.
//
// C[m][n] += sum_k A[m][k] B[n][k] for a BM x BN tile, NWAVES wavefronts of WM x WN each.
// Both operands are K-contiguous, so every MFMA fragment (32 rows x 8 consecutive k per lane)
// is one 16-byte LDS read. A stage holds BK k of both tiles, row-major, BK k per row, with the
// 16-byte chunk index XOR-swizzled by the row so that fragment reads are free of bank
// conflicts. K step s lives in stage s % NST. The barrier of step s sits before its last
// 16-wide sub-step: by then every wavefront has read all of step s (its last fragments are in
// registers) and step s + 1 has landed; right after it the loads of step s + NST refill the
// stage of step s, and the MFMAs of the last sub-step run while the first fragments of step
// s + 1 are read. A load thus has NST - 1 steps of MFMAs to land.
#pragma once

#include "common.h"

namespace moelora {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// D += A(32x16) * B(16x32). Lane l supplies row (l % 32) of A and column (l % 32) of B, 8
// reduction elements each, in the same slot order; lane l receives D rows
// 8*(v/4) + 4*(l/32) + (v%4), v < 16, of column (l % 32).
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// One 16-byte load per lane straight into LDS (no register receives the data): the 64 lanes of
// the wavefront fill the 1 KB at lds_addr (lane l at lds_addr + 16 l) from the buffer at byte
// offset voff + soff. The LDS address goes through M0 and must be wavefront-uniform. Written
// as inline assembly because the compiler, unable to tell which LDS stage such a load fills,
// would otherwise wait for every one of them before any LDS read; the caller waits (vmcnt) and
// synchronises before the data is read.
__device__ __forceinline__ void lds_dma16(u32x4 rsrc, uint32_t voff, uint32_t soff,
                                          uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_addr), "s"(soff)
               : "memory", "m0");
}

// As lds_dma16 with the non-temporal hint: for operands streamed through once (read by one
// tile), so that they do not evict from L2 what other tiles of the same wave of workgroups
// read again.
__device__ __forceinline__ void lds_dma16_nt(u32x4 rsrc, uint32_t voff, uint32_t soff,
                                             uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen nt lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_addr), "s"(soff)
               : "memory", "m0");
}

// As lds_dma16 from a 64-bit global address per lane (any buffer size; no zero fill).
__device__ __forceinline__ void lds_dma16_global(const void* addr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(addr), "s"(lds_addr)
               : "memory", "m0");
}

// Buffer descriptor of [base, base + bytes): loads at offsets >= bytes return zeros.
__device__ __forceinline__ u32x4 buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  return u32x4{(uint32_t)b, (uint32_t)(b >> 32) & 0xffffu, bytes, 0x00020000u};
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// W8: the B tile holds one-byte E4M3 codes (BK bytes per row) instead of bf16; its fragments are
// converted to bf16 after the LDS read. The k order inside a stage then differs from the bf16
// tile's (lane group fg takes k 32 fg + 8 j .. + 7 in sub-step j, on both operands), so that one
// 16-byte read of a code row serves two sub-steps.
//
// ILV: the fragment reads of the next sub-step are issued between the MFMAs of the current one
// (one read after each MFMA) instead of ahead of them.
template <int BM, int BN, int WM, int WN, int BK, int NST, bool ILV = false, int NWAVES = 4,
          bool W8 = false>
struct TilePipe {
  static_assert(BK == 32 || BK == 64, "K step of 32 or 64");
  static_assert(!W8 || BK == 64, "E4M3 tiles take 64-wide K steps");
  static_assert(NST >= 2, "at least two LDS stages");
  static constexpr int TILE_M = BM;
  static constexpr int WAVES_N = BN / WN;
  static_assert((BM / WM) * WAVES_N == NWAVES, "WM x WN wavefront tiles cover the tile");
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int CPR = BK / 8;               // 16-byte chunks per A tile row
  static constexpr int RPB = 64 / CPR;             // A tile rows per 1 KB load block
  static constexpr int BROW = W8 ? BK : 2 * BK;    // bytes per B tile row
  static constexpr int CPRB = BROW / 16;           // 16-byte chunks per B tile row
  static constexpr int RPBB = 64 / CPRB;           // B tile rows per 1 KB load block
  static constexpr int NA = BM / RPB / NWAVES;     // load blocks per wavefront and stage (A)
  static constexpr int NB = BN / RPBB / NWAVES;    // (B)
  static constexpr int PER = NA + NB;              // loads per wavefront and stage
  static constexpr int SUB = BK / 16;              // MFMA sub-steps per stage
  static constexpr uint32_t A_BYTES = BM * BK * 2;
  static constexpr uint32_t STAGE_BYTES = A_BYTES + BN * BROW;
  static constexpr uint32_t LDS_BYTES = NST * STAGE_BYTES;
  static_assert(NA * RPB * NWAVES == BM && NB * RPBB * NWAVES == BN,
                "tiles must split into load blocks");
  static_assert(FM + FN <= 15, "one sub-step of fragment reads must fit the LDS counter");
  static_assert((NST - 1) * PER < 64, "in-flight loads must fit vmcnt");

  // Slot of chunk c in tile row r (XOR swizzle). The LDS has 64 banks of 4 bytes and serves a
  // 16-byte-per-lane read 16 lanes (256 bytes) at a time; the 16 lanes of a fragment read hold
  // 16 consecutive rows at one chunk, so rows that share their 256-byte bank alignment
  // (every 2nd row at 128 bytes per row, every 4th at 64) must land in different slots.
  __device__ static __forceinline__ int swz(int r, int c) {
    return BK == 64 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 2) & 3));
  }
  __device__ static __forceinline__ int swz_b(int r, int c) {
    return W8 ? (c ^ ((r >> 2) & 3)) : swz(r, c);
  }
  // Tile row and K chunk that lane `lane` of wavefront `wave` loads in its i-th block of A
  // (load_row_b / load_chunk_b: of B): the lane fills slot lane % CPR of row lane / CPR of the
  // block, so it fetches the chunk that the swizzle puts in that slot of that (tile) row.
  __device__ static __forceinline__ int load_row(int i, int wave, int lane) {
    return (i * NWAVES + wave) * RPB + lane / CPR;
  }
  __device__ static __forceinline__ int load_chunk(int row, int lane) {
    return swz(row, lane % CPR);
  }
  __device__ static __forceinline__ int load_row_b(int i, int wave, int lane) {
    return (i * NWAVES + wave) * RPBB + lane / CPRB;
  }
  __device__ static __forceinline__ int load_chunk_b(int row, int lane) {
    return swz_b(row, lane % CPRB);
  }

  // The loads of a K step: PER 1 KB blocks per wavefront, block d (< NA: the A tile, else the B
  // tile) going to LDS byte address lds_addr. A loader provides prep(ks) (called once before the
  // loads of step ks are issued), load(d, ks, lds_addr), and main_steps(): steps below it may
  // also be loaded with load_main(d, ks, lds_addr), which has no step-dependent branch.
  //
  // Loader of plain operand tiles: xo[NA], wo[NB] are the byte offsets (in xr, wr) of the chunk
  // each lane loads at K step 0; step ks adds ks * BK * 2 bytes.
  struct BufferLoader {
    u32x4 xr, wr;
    const uint32_t* xo;
    const uint32_t* wo;
    __device__ __forceinline__ int main_steps() const { return 1 << 30; }
    __device__ __forceinline__ void prep(int) {}
    __device__ __forceinline__ void load_main(int d, int ks, uint32_t lds_addr) {
      if (d < NA) lds_dma16(xr, xo[d], (uint32_t)ks * BK * 2, lds_addr);
      else lds_dma16(wr, wo[d - NA], (uint32_t)ks * BROW, lds_addr);
    }
    __device__ __forceinline__ void load(int d, int ks, uint32_t lds_addr) {
      load_main(d, ks, lds_addr);
    }
  };

  __device__ static __forceinline__ void run(f32x16 (&acc)[FM][FN], u32x4 xr, const uint32_t* xo,
                                             u32x4 wr, const uint32_t* wo, uint16_t* lds, int K,
                                             int wave, int lane) {
    BufferLoader ld{xr, wr, xo, wo};
    int nks = K / BK;
    run_steps(acc, ld, lds, nks, wave, lane, [] {});
  }

  // nks K steps of loads from `ld`; `mid` runs once the first NST steps' loads are in flight,
  // before the first wait (work that can overlap their latency), and may raise nks (steps past
  // the first NST only).
  template <class Loader, class Mid>
  __device__ static __forceinline__ void run_steps(f32x16 (&acc)[FM][FN], Loader& ld,
                                                   uint16_t* lds, int& nks, int wave, int lane,
                                                   Mid mid) {
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
    auto block_addr = [&](int d, int stage) {
      const uint32_t sa = lds0 + stage * STAGE_BYTES + wave * 1024;
      return d < NA ? sa + d * NWAVES * 1024 : sa + A_BYTES + (d - NA) * NWAVES * 1024;
    };
    auto issue = [&](int ks, int stage) {
      ld.prep(ks);
#pragma unroll
      for (int d = 0; d < PER; ++d) ld.load(d, ks, block_addr(d, stage));
    };
    const int fr = lane & 31, fg = lane >> 5;
    u32x4 bq[FN];  // W8: the 16 codes of each B fragment row that serve sub-steps j, j + 1
    auto read_frags = [&](int stage, int j, u32x4* af, u32x4* bf) {
      const uint16_t* A = lds + stage * (STAGE_BYTES / 2);
      const char* B = reinterpret_cast<const char*>(A) + A_BYTES;
      const int c = W8 ? 4 * fg + j : 2 * j + fg;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WM + i * 32 + fr;
        af[i] = *reinterpret_cast<const u32x4*>(A + r * BK + 8 * swz(r, c));
      }
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int r = wn * WN + i * 32 + fr;
        if (W8) {
          if ((j & 1) == 0)
            bq[i] = *reinterpret_cast<const u32x4*>(B + r * BROW + 16 * swz_b(r, 2 * fg + j / 2));
          bf[i] = e4m3x8_to_bf16(bq[i], j & 1);
        } else {
          bf[i] = *reinterpret_cast<const u32x4*>(B + r * BROW + 16 * swz_b(r, c));
        }
      }
    };
    auto mfmas_interleaved = [&](const u32x4* af, const u32x4* bf, bool reads_pending) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jn = 0; jn < FN; ++jn) acc[i][jn] = mfma32(af[i], bf[jn], acc[i][jn]);
      if (reads_pending) {
        constexpr int NR = FM + FN, NM = FM * FN, PAIRS = NR < NM ? NR : NM;
#pragma unroll
        for (int t = 0; t < PAIRS; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        if (NR > NM) __builtin_amdgcn_sched_group_barrier(0x100, NR - NM, 0);
        if (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
      }
    };

    // The last sub-step's MFMAs with the refill loads of step ks_load spread between them (one
    // load after MFMA floor(d * NM / PER)), so that issuing them does not stall the MFMA pipe.
    auto mfmas_with_loads = [&](const u32x4* af, const u32x4* bf, int ks_load, int st,
                                auto&& load_fn) {
      constexpr int NM = FM * FN;
#pragma unroll
      for (int t = 0; t < NM; ++t) {
        acc[t / FN][t % FN] = mfma32(af[t / FN], bf[t % FN], acc[t / FN][t % FN]);
#pragma unroll
        for (int d = 0; d < PER; ++d) {
          if ((d * NM) / PER != t) continue;
          load_fn(d, ks_load, block_addr(d, st));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // prologue: steps 0 .. NST-1 in flight, wait for step 0
#pragma unroll
    for (int s = 0; s < NST; ++s)
      if (s < nks) issue(s, s);
    mid();
    if (nks >= NST) wait_vmcnt<(NST - 1) * PER>();
    else wait_vmcnt<0>();
    __syncthreads();

    u32x4 af0[FM], bf0[FN], af1[FM], bf1[FN];
    read_frags(0, 0, af0, bf0);
    __builtin_amdgcn_sched_barrier(0);
    // All steps but the last end with the barrier and the refill. No branch encloses an MFMA
    // (the compiler would keep a second copy of the accumulators): near the end the refill
    // re-loads the last step into the stage just consumed, which no later step reads. While
    // the refills are main K steps (ld.main_steps()) the loop takes the loader's branch-free
    // main-step loads.
    int stage = 0;
    auto step = [&](int ks, auto&& load_fn, auto&& prep_fn) {
      const int next = stage + 1 == NST ? 0 : stage + 1;
#pragma unroll
      for (int j = 0; j < SUB; ++j) {
        u32x4* an = (j & 1) ? af0 : af1;
        u32x4* bn = (j & 1) ? bf0 : bf1;
        const u32x4* ac = (j & 1) ? af1 : af0;
        const u32x4* bc = (j & 1) ? bf1 : bf0;
        if (j < SUB - 1) {
          read_frags(stage, j + 1, an, bn);
          if (!ILV) __builtin_amdgcn_sched_barrier(0);
          mfmas_interleaved(ac, bc, true);
          __builtin_amdgcn_sched_barrier(0);
          continue;
        }
        // Step ks + 1 has landed once only the loads of steps ks + 2 .. ks + NST - 1 are
        // outstanding (everything, near the end, where the refills re-load the last step).
        if (ks + NST - 1 < nks) wait_vmcnt<(NST - 2) * PER>();
        else wait_vmcnt<0>();
        __syncthreads();
        const int ks_load = ks + NST < nks ? ks + NST : nks - 1;
        prep_fn(ks_load);
        read_frags(next, 0, an, bn);
        __builtin_amdgcn_sched_barrier(0);
        mfmas_with_loads(ac, bc, ks_load, stage, load_fn);
      }
      stage = next;
    };
    const int main_end = ld.main_steps() - NST;  // refills of steps < main_end + NST are main
    int ks = 0;
    for (; ks + 1 < nks && ks < main_end; ++ks)
      step(ks, [&](int d, int k, uint32_t a) { ld.load_main(d, k, a); }, [](int) {});
    for (; ks + 1 < nks; ++ks)
      step(ks, [&](int d, int k, uint32_t a) { ld.load(d, k, a); }, [&](int k) { ld.prep(k); });
    // last step: no barrier, no refill
#pragma unroll
    for (int j = 0; j < SUB; ++j) {
      u32x4* an = (j & 1) ? af0 : af1;
      u32x4* bn = (j & 1) ? bf0 : bf1;
      const u32x4* ac = (j & 1) ? af1 : af0;
      const u32x4* bc = (j & 1) ? bf1 : bf0;
      if (j < SUB - 1) read_frags(stage, j + 1, an, bn);
      __builtin_amdgcn_sched_barrier(0);
      mfmas_interleaved(ac, bc, j < SUB - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the refills of the last steps are still in flight: let them land before LDS is released
    wait_vmcnt<0>();
  }
};

}  // namespace moelora
