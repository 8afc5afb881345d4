// C ABI of libmoelora: argument validation, workspace carve-up and the launch sequence of the
// fused MoE + multi-LoRA layer (declared in include/moelora.h).
#include <algorithm>
#include <mutex>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "kernels.h"
#include "moelora.h"

using namespace moelora;

namespace {

constexpr int kMaxBM = 256;      // largest row block any GEMM path uses
constexpr int kMaxDownSplit = 2;  // K splits of the down GEMM
constexpr size_t kScratchBytes = (size_t)128 << 20;  // static scratch of the no-alloc entry

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
int64_t round_up64(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

int validate_dims(const moe_lora_dims* d, int32_t topk) {
  if (!d) return MOELORA_ENULL;
  if (d->T < 0 || d->hidden <= 0 || d->inter <= 0 || d->n_experts <= 0 || d->n_adapters <= 0)
    return MOELORA_EINVAL_DIMS;
  if (d->hidden % 128 != 0 || d->inter % 128 != 0) return MOELORA_EINVAL_DIMS;
  if (d->n_experts > kMaxExperts) return MOELORA_EINVAL_DIMS;
  if (!(d->rank == 8 || d->rank == 16 || d->rank == 32 || d->rank == 64)) return MOELORA_EINVAL_DIMS;
  if (topk < 1 || topk > d->n_experts || topk > kMaxTopk) return MOELORA_EINVAL_DIMS;
  // every index the kernels form in 32 bits must fit
  const int64_t P = (int64_t)d->T * topk;
  if (P + (int64_t)d->n_experts * kMaxBM >= ((int64_t)1 << 30)) return MOELORA_EINVAL_DIMS;
  if ((int64_t)d->n_experts * (d->n_adapters + 1) >= ((int64_t)1 << 28)) return MOELORA_EINVAL_DIMS;
  // x and the intermediate activations are read with 32-bit buffer offsets (< 2 GiB each)
  // (the activations are checked against the capacity of the path a call takes, once planned)
  if ((int64_t)d->T * d->hidden * 2 >= ((int64_t)1 << 31)) return MOELORA_EINVAL_DIMS;
  // so is one expert's slice of W1 (2I x h, the larger of the two projections)
  if ((int64_t)2 * d->inter * d->hidden * 2 >= ((int64_t)1 << 31)) return MOELORA_EINVAL_DIMS;
  return MOELORA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_device() {
  static int known[64];  // 0 unknown, 1 gfx950, -1 other
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOELORA_EHIP;
  if (dev < 0 || dev >= 64) return MOELORA_EDEVICE;
  if (known[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOELORA_EHIP;
    known[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  return known[dev] == 1 ? MOELORA_OK : MOELORA_EDEVICE;
}

// Workgroups of the 256-row tiled GEMM resident at once: one per CU, rounded down to the 8 XCDs
// (per device, looked up once); 0 on error.
int resident_tiles() {
  static int known[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (known[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    known[dev] = n / 8 * 8;
  }
  return known[dev];
}

// Align kernel's LDS: its arrays (keys, two pair-id buffers, segment starts and deltas, with the
// radix digit counts overlaying the segment region) when they fit, else the digit counts only
// and the arrays go to the workspace. Returns the dynamic LDS bytes and fills the kernel's sizes.
size_t align_lds_plan(int T, int k, int E, int nA, AlignArgs* a) {
  const size_t budget = (size_t)(kLdsBytes - kAlignStaticLds);
  align_digits(E, nA, &a->digit_bits, &a->passes);
  a->seg_cap = align_seg_cap(T, k, E, nA);
  const size_t P = (size_t)T * k;
  const size_t counts = (size_t)(kAlignThreads / 64) << a->digit_bits;
  const size_t seg_region = std::max(2 * (size_t)a->seg_cap, counts);
  const size_t in_lds = sizeof(int) * (3 * P + seg_region);
  a->lists_in_lds = in_lds <= budget ? 1 : 0;
  return a->lists_in_lds ? in_lds : sizeof(int) * counts;
}

// GEMM path from the mean rows per expert (known on the host; per-expert counts are not):
// the skinny path streams weights once per 16/32-row block, the tiled path stages tiles in LDS
// for MFMA-bound row counts. MOELORA_PATH=skinny|skinny1|skinny2|skinny4 forces the skinny path (and
// its row-block size) for experiments.
struct PathPlan {
  bool tiled;
  int nt;  // skinny: 16-row token tiles per row block
  TiledConfig tc;     // gate_up tile
  TiledConfig tc_dn;  // down tile (same bm)
  int bm;  // row-block size of the sorted layout
};

PathPlan pick_path(int64_t P, int E, int h, int I) {
  const double mean = (double)P / E;
  PathPlan pl;
  pl.tiled = mean > 24.0;
  pl.nt = mean <= 12.0 ? 1 : (mean <= 24.0 ? 2 : 4);
  // Row-block size against padding: an expert wastes up to bm - 1 rows, so the 256-row tile
  // (most MFMA work per loaded byte) only pays once experts hold several hundred rows.
  // 128- and 256-row tiles run eight wavefronts (two per SIMD): one wavefront's LDS waits and
  // barriers are covered by the other's MFMAs
  const TiledConfig t64{64, 128, 32, 64, 64, 2, 4}, t64w{64, 256, 32, 64, 64, 2, 8},
      t128{128, 128, 32, 64, 64, 2, 8}, t192{192, 256, 96, 64, 64, 2, 8},
      t256{256, 256, 64, 128, 64, 2, 8};
  const bool fits256 = (2 * I) % 256 == 0 && h % 256 == 0;
  pl.tc = mean < 192.0 ? t64 : (mean < 768.0 || !fits256 ? t128 : t256);
  pl.tc_dn = pl.tc;
  // 64-row blocks: gate_up (2I wide) takes 256 columns per tile with eight wavefronts
  if (mean < 192.0) pl.tc = t64w;
  // About 100 to 160 rows per expert (weight-streaming bound): the layout pads each expert to
  // 192 rows, so that down reads every expert's W2 once, in 192-row tiles; gate_up walks the
  // same layout in 64-row tiles (tiles of padding only are skipped), which keeps two workgroups
  // per CU and its LoRA epilogue short when many adapters share a tile (measured on the
  // adapter-stress batches, ~128 rows per expert: down 0.44 -> 0.35 ms with one adapter)
  if (mean >= 96.0 && mean <= 160.0 && fits256) pl.tc_dn = t192;
  // MOELORA_TILED="bm,bn,wm,wn,bk,nst[,nw][;...]" forces the tiles of gate_up (and of
  // down when a second set follows) for experiments
  static int forced = -1;  // -1 unread, 0 none, 1 skinny, 2 tiled, 3/4 skinny with 1/2 tiles
  static TiledConfig ft, ftd;
  if (forced < 0) {
    forced = 0;
    const char* env = getenv("MOELORA_PATH");
    if (env && !strcmp(env, "skinny")) forced = 1;
    if (env && !strcmp(env, "skinny1")) forced = 3;
    if (env && !strcmp(env, "skinny2")) forced = 4;
    if (env && !strcmp(env, "skinny4")) forced = 5;
    const char* tenv = getenv("MOELORA_TILED");
    if (tenv) {
      auto parse = [](const char* str, TiledConfig* c) {
        int v[7] = {0, 0, 0, 0, 64, 2, 4};
        const int n = sscanf(str, "%d,%d,%d,%d,%d,%d,%d", &v[0], &v[1], &v[2], &v[3], &v[4], &v[5],
                             &v[6]);
        *c = TiledConfig{v[0], v[1], v[2], v[3], v[4], v[5], v[6]};
        return n >= 4;
      };
      if (parse(tenv, &ft)) {
        ftd = ft;
        const char* semi = strchr(tenv, ';');
        TiledConfig d2;
        if (semi && parse(semi + 1, &d2)) ftd = d2;
        forced = 2;
      }
    }
  }
  if (forced == 1) pl.tiled = false;
  if (forced >= 3 && forced <= 5) {
    pl.tiled = false;
    pl.nt = forced == 3 ? 1 : (forced == 4 ? 2 : 4);
  }
  if (forced == 2) {
    pl.tiled = true;
    pl.tc = ft;
    pl.tc_dn = ftd;
  }
  // column tiles must divide the GEMM widths (2I for gate_up, h for down; 128 always does), and
  // the smaller row tile must divide the larger (the layout's row block)
  const int bmax = std::max(pl.tc.bm, pl.tc_dn.bm), bmin = std::min(pl.tc.bm, pl.tc_dn.bm);
  if ((2 * I) % pl.tc.bn != 0 || h % pl.tc_dn.bn != 0 || bmin <= 0 || bmax % bmin != 0) {
    pl.tc = mean < 192.0 ? t64 : t128;
    pl.tc_dn = pl.tc;
  }
  pl.bm = pl.tiled ? std::max(pl.tc.bm, pl.tc_dn.bm) : 16 * pl.nt;
  return pl;
}

bool skinny_instantiated(const SkinnyConfig& c, bool gateup) {
  static const int have[][5] = {{1, 2, 1, 1, 0}, {1, 2, 2, 1, 0}, {1, 4, 1, 1, 0}, {1, 4, 1, 0, 0}, {1, 4, 2, 1, 0}, {1, 4, 2, 0, 0},
                                {1, 8, 1, 1, 0}, {1, 8, 1, 0, 0}, {2, 2, 1, 1, 0}, {2, 2, 2, 1, 0}, {2, 4, 1, 1, 0}, {2, 4, 2, 1, 0},
                                {2, 8, 1, 1, 0},
                                {4, 4, 1, 1, 0}, {1, 4, 1, 1, 1}, {1, 4, 1, 0, 1}, {1, 8, 1, 1, 1},
                                {1, 8, 1, 0, 1}};
  if (c.split && !gateup) return false;
  for (const auto& h : have)
    if (h[0] == c.nt && h[1] == c.p && h[2] == c.rt && h[3] == c.pipe && h[4] == c.split) return true;
  return false;
}

// Tile shapes of the two skinny GEMMs and the down split. MOELORA_SKINNY_CFG=
// "pg,rg,pipe_g,split_g,pd,rd,pipe_d,ks" overrides them for experiments (ignored when the
// combination is not compiled or not valid for the sizes).
struct SkinnyPlan {
  SkinnyConfig gu, dn;
  int ksplit;
};

SkinnyPlan pick_skinny(int nt, int h, int I) {
  SkinnyPlan pl;
  // measured on decode (16 experts, ~8 rows each) and FG (128 experts, 16 rows each): gate_up
  // keeps gate and up rows in one wavefront; down streams two row tiles per wavefront (and on
  // 16-row blocks splits K in two). 64-wide K steps (two 16-byte loads per lane and row) leave
  // registers for more workgroups per CU than 128-wide ones; on 32-row blocks (short K loops,
  // many experts) gate_up also streams two row tiles per wavefront.
  pl.gu = nt == 1 ? SkinnyConfig{nt, 2, 1, 1, 0}
                  : (nt == 2 ? SkinnyConfig{nt, 2, 2, 1, 0} : SkinnyConfig{nt, 4, 1, 1, 0});
  pl.dn = SkinnyConfig{nt, nt <= 2 ? 2 : 4, nt <= 2 ? 2 : 1, 1, 0};
  pl.ksplit = nt == 1 ? 2 : 1;
  static int ov[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  static bool parsed = false;
  if (!parsed) {
    const char* env = getenv("MOELORA_SKINNY_CFG");
    if (env)
      sscanf(env, "%d,%d,%d,%d,%d,%d,%d,%d", &ov[0], &ov[1], &ov[2], &ov[3], &ov[4], &ov[5], &ov[6],
             &ov[7]);
    parsed = true;
  }
  if (ov[0]) {
    const SkinnyConfig gu{nt, ov[0], ov[1], ov[2], ov[3]}, dn{nt, ov[4], ov[5], ov[6], 0};
    const bool ok = skinny_instantiated(gu, true) && skinny_instantiated(dn, false) &&
                    h % (32 * gu.p) == 0 && I % (32 * dn.p) == 0 && I % (32 * gu.rt) == 0 &&
                    h % (16 * dn.rt) == 0 && ov[7] >= 1 && ov[7] <= kMaxDownSplit;
    if (ok) {
      pl.gu = gu;
      pl.dn = dn;
      pl.ksplit = ov[7];
    }
  }
  return pl;
}

// K splits of the LoRA shrink: enough (tile, split) workgroups to fill the chip, at most
// kMaxSplit and at least one 128-wide step each.
int pick_splits(int64_t tiles, int K) {
  int s = (int)((1024 + tiles - 1) / (tiles > 0 ? tiles : 1));
  s = s < 1 ? 1 : (s > kMaxSplit ? kMaxSplit : s);
  const int nks = K / 128;
  s = s > nks ? nks : s;
  // the kernels give split j the 128-wide steps [j * per, (j + 1) * per), per = ceil(nks / s);
  // fewer splits with the same per leave none of them empty
  const int per = (nks + s - 1) / s;
  return (nks + per - 1) / per;
}

// Everything about a layer call that follows from the sizes alone: the GEMM path and its row-block
// size, the skinny tiles, the K splits of down and of the two LoRA shrinks, the launch grids.
struct ForwardPlan {
  PathPlan path;
  SkinnyPlan sk;  // skinny tiles; sk.ksplit is the down GEMM's K splits on either path
  int bm;
  int64_t P;
  int max_blocks;  // row blocks of the largest padded layout
  int tiles16;     // 16-row tiles of it
  int n_sub_max;   // 64-row sub-blocks of it
  int s1, s2;      // K splits of the gate_up and down shrinks
  bool shrink64;   // 64-row shrink on the tiled path
  int tail_split;  // tiled down: K parts of the last round's tiles (0: sk.ksplit for every tile)
  int d_parts() const { return tail_split > 1 ? tail_split : sk.ksplit; }
};

ForwardPlan make_plan(const moe_lora_dims* d, int topk, bool fp8) {
  ForwardPlan pl;
  const int h = d->hidden, I = d->inter, E = d->n_experts, r = d->rank;
  pl.P = (int64_t)d->T * topk;
  pl.tail_split = 0;
  pl.path = pick_path(pl.P, E, h, I);
  pl.bm = pl.path.bm;
  pl.sk = pick_skinny(pl.path.nt, h, I);
  if (fp8) {
    // E4M3 rows carry half the bytes per K element: 128-wide K steps keep the bf16 kernels'
    // bytes in flight per load (measured: decode gate_up 0.35 -> 0.31 ms); down on 32-row
    // blocks (short K loops of many experts) keeps 64-wide steps
    pl.sk.gu.p = 4;
    pl.sk.dn.p = pl.path.nt == 1 ? 4 : 2;
  }
  if (pl.path.tiled) {
    // tiled down: split K in two when the tiles would fill the chip fewer than four times (the
    // last, partial round of 256x256 tiles then costs a large share of the time)
    const int64_t est_tiles =
        (int64_t)((pl.P + pl.bm - 1) / pl.bm + E) * (h / pl.path.tc_dn.bn);
    pl.sk.ksplit = est_tiles < 4 * 256 && pl.path.tc_dn.bm != 192 ? kMaxDownSplit : 1;
    // 256-row tiles (one per CU): only the last, partial round splits K, in four parts
    // (MOELORA_DOWN_TAIL=0 keeps the split of every tile, for experiments)
    static int down_tail = -1;
    if (down_tail < 0) {
      const char* env = getenv("MOELORA_DOWN_TAIL");
      down_tail = env ? atoi(env) : 1;
    }
    if (down_tail && pl.sk.ksplit > 1 && pl.path.tc_dn.bm == 256 && (I / 64) % 4 == 0) {
      pl.tail_split = 4;
      pl.sk.ksplit = 1;
    }
    // MOELORA_DOWN_SPLIT=1|2 overrides it (experiments)
    static int down_split = -1;
    if (down_split < 0) {
      const char* env = getenv("MOELORA_DOWN_SPLIT");
      down_split = env ? atoi(env) : 0;
    }
    if (down_split == 1 || down_split == 2) {
      pl.sk.ksplit = down_split;
      pl.tail_split = 0;
    }
  }
  const int64_t max_rows = pl.P + (int64_t)E * (pl.bm - 1);
  pl.max_blocks = (int)((max_rows + pl.bm - 1) / pl.bm);
  pl.tiles16 = pl.max_blocks * (pl.bm / 16);
  // Split the shrink's K by the tiles that can hold pairs (at most P/16 plus one partial tile per
  // expert), not by the padded grid: padding tiles exit at once.
  const int64_t live_tiles = std::min<int64_t>(pl.tiles16, (pl.P + 15) / 16 + E);
  pl.s1 = pick_splits(live_tiles, h);
  pl.s2 = pick_splits(live_tiles, I);
  // a short K (a few 128-wide steps, e.g. the down shrink of small experts) takes one step per
  // split: more workgroups, each with one load round trip per adapter run (measured: the
  // fine-grained batch's down shrink, 6 steps, 33.5 -> 24.5 us at 6 splits against 3)
  if (h / 128 <= kMaxSplit) pl.s1 = h / 128;
  if (I / 128 <= kMaxSplit) pl.s2 = I / 128;
  // On the tiled path (row blocks of >= 64 rows) the shrink takes 64 rows per workgroup where a
  // sub-block holds few adapter runs, so that a run's A slab is fetched once per 64 rows; the
  // 16-row shrink then takes the rest. Both use the same K splits, as many as either needs to
  // fill the chip (MOELORA_SHRINK64=0 turns the 64-row shrink off, for experiments).
  static int shrink64_env = -1;
  if (shrink64_env < 0) {
    const char* env = getenv("MOELORA_SHRINK64");
    shrink64_env = env ? atoi(env) : 1;
  }
  pl.shrink64 = shrink64_env != 0 && pl.path.tiled && r <= 64 && pl.bm % 64 == 0;
  pl.n_sub_max = pl.max_blocks * pl.bm / 64;
  if (pl.shrink64) {
    const int64_t live_sub = std::min<int64_t>(pl.n_sub_max, (pl.P + 63) / 64 + E);
    pl.s1 = std::max(pl.s1, pick_splits(live_sub, h));
    pl.s2 = std::max(pl.s2, pick_splits(live_sub, I));
  }
  return pl;
}

}  // namespace

// Workspace regions for a call with row blocks of bm rows and dsplit K splits of down: only what
// that path uses (decode: ~30 MB; 256-row prefill blocks: ~0.6 GB).
bool moelora_make_layout(int T, int h, int I, int E, int nA, int r, int topk, int bm, int dsplit,
                         MoeLoraLayout* L) {
  const int64_t P = (int64_t)T * topk;
  L->max_bm = bm;
  L->cap = round_up64(P + (int64_t)E * (bm - 1), 256);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + (bytes ? bytes : 1));
    return o;
  };
  L->flags = take(16);  // first, so moe_lora_debug_status can find it without the sizes
  L->topk_ids = take(4 * (size_t)P);
  L->topk_w = take(4 * (size_t)P);
  L->tok_flags = take(4 * (size_t)T);
  L->sorted = take(4 * (size_t)L->cap);
  L->expert_off = take(4 * (size_t)(E + 1));
  L->n_blocks = take(4);
  L->block_expert = take(4 * (size_t)(L->cap / 16 + 1));
  L->block_seg = take(4 * (size_t)(L->cap / 16 + 1));
  L->pair_row = take(4 * (size_t)P);
  L->sorted_ad = take(4 * (size_t)L->cap);
  L->seg_table = take(16 * (size_t)P);
  L->n_seg = take(4);
  L->z1 = take(4 * (size_t)kMaxSplit * L->cap * r);
  L->z2 = take(4 * (size_t)kMaxSplit * L->cap * r);
  L->zhl = take(2 * 2 * (size_t)L->cap * r);
  L->act = take(2 * (size_t)L->cap * I);
  L->dpair = take(4 * (size_t)dsplit * L->cap * h);
  L->d_parts = take(4 * (size_t)(L->cap / 64 + 1) * (size_t)(h / 64 + 1));
  L->align_lists = take(4 * align_list_ints(T, topk, E, nA));
  L->logits = take(4 * (size_t)T * E);
  L->total = off;
  return true;
}

namespace {

// The plan and workspace layout of a forward call; MOELORA_EINVAL_DIMS when a buffer the kernels
// address with 32-bit offsets would reach 2 GiB (the activations at this path's capacity).
int plan_and_layout(const moe_lora_dims* d, int32_t topk, bool fp8, ForwardPlan* pl,
                    MoeLoraLayout* L) {
  const int rc = validate_dims(d, topk);
  if (rc != MOELORA_OK) return rc;
  *pl = make_plan(d, topk, fp8);
  moelora_make_layout(d->T, d->hidden, d->inter, d->n_experts, d->n_adapters, d->rank, topk, pl->bm,
                      pl->d_parts(), L);
  // act [cap][I] bf16 is read with 32-bit buffer offsets, and padding lanes use offset 2^31
  if (L->cap * (int64_t)d->inter * 2 >= ((int64_t)1 << 31)) return MOELORA_EINVAL_DIMS;
  return MOELORA_OK;
}

}  // namespace

extern "C" {

size_t moe_lora_workspace_size(const moe_lora_dims* d, int32_t topk) {
  ForwardPlan pl;
  MoeLoraLayout L;
  if (plan_and_layout(d, topk, false, &pl, &L) != MOELORA_OK) return 0;
  return L.total;
}

int moe_lora_workspace_layout(const moe_lora_dims* d, int32_t topk, moe_lora_layout_info* out) {
  if (!out) return MOELORA_ENULL;
  ForwardPlan pl;
  MoeLoraLayout L;
  const int rc = plan_and_layout(d, topk, false, &pl, &L);
  if (rc != MOELORA_OK) return rc;
  out->tiled = pl.path.tiled ? 1 : 0;
  out->block_m = pl.bm;
  out->capacity = L.cap;
  out->workspace_bytes = (int64_t)L.total;
  out->topk_ids = (int64_t)L.topk_ids;
  out->topk_w = (int64_t)L.topk_w;
  out->sorted_pairs = (int64_t)L.sorted;
  out->expert_offsets = (int64_t)L.expert_off;
  out->seg_table = (int64_t)L.seg_table;
  out->n_seg = (int64_t)L.n_seg;
  out->n_blocks = (int64_t)L.n_blocks;
  out->block_expert = (int64_t)L.block_expert;
  out->block_seg = (int64_t)L.block_seg;
  out->pair_row = (int64_t)L.pair_row;
  out->sorted_ad = (int64_t)L.sorted_ad;
  return MOELORA_OK;
}

int64_t moe_lora_sorted_capacity(const moe_lora_dims* d, int32_t topk, int32_t seg_pad,
                                 int32_t block_m) {
  if (validate_dims(d, topk) != MOELORA_OK) return -1;
  if (seg_pad < 1 || seg_pad > 256 || block_m < 1 || block_m > 256) return -1;
  return (int64_t)d->T * topk * seg_pad + (int64_t)d->n_experts * (block_m - 1);
}

const char* moe_lora_strerror(int code) {
  switch (code) {
    case MOELORA_OK: return "ok";
    case MOELORA_EINVAL_DIMS: return "sizes out of the supported range";
    case MOELORA_ENULL: return "a required pointer is NULL";
    case MOELORA_EALIGN: return "a tensor pointer is not 16-byte aligned";
    case MOELORA_EWORKSPACE: return "workspace too small or not 256-byte aligned";
    case MOELORA_EHIP: return "HIP launch or runtime error";
    case MOELORA_EDEVICE: return "current device is not gfx950";
    case MOELORA_EUNSUPPORTED: return "this combination of arguments is not supported";
    case MOELORA_ESCRATCH:
      return "the call needs more workspace than the static scratch of moe_lora_forward_noalloc "
             "(128 MiB)";
    default: return "unknown error code";
  }
}

}  // extern "C"

namespace {

// Records stage boundary i on the stream when the caller asked for timing events.
bool mark(void* const* ev, int i, hipStream_t s) {
  return !ev || !ev[i] || hipEventRecord((hipEvent_t)ev[i], s) == hipSuccess;
}

// The launch sequence of one layer call (arguments already checked, T > 0).
int enqueue_forward(const ForwardPlan& pl, const MoeLoraLayout& L, const void* x,
                    const float* router_logits, const void* W_router, const void* W1,
                    const void* W2, const void* A1, const void* B1, const void* A2, const void* B2,
                    const int32_t* adapter_ids, int32_t topk, const moe_lora_dims* d, void* y,
                    char* ws, hipStream_t stream, void* const* ev, const float* w1_scale,
                    const float* w2_scale) {
  const bool fp8 = w1_scale != nullptr;
  const int T = d->T, h = d->hidden, I = d->inter, E = d->n_experts, nA = d->n_adapters, r = d->rank;
  int* topk_ids = (int*)(ws + L.topk_ids);
  float* topk_w = (float*)(ws + L.topk_w);
  int* tok_flags = (int*)(ws + L.tok_flags);
  int* sorted = (int*)(ws + L.sorted);
  int* n_blocks = (int*)(ws + L.n_blocks);
  int* block_expert = (int*)(ws + L.block_expert);
  int* block_seg = (int*)(ws + L.block_seg);
  int* pair_row = (int*)(ws + L.pair_row);
  int* sorted_ad = (int*)(ws + L.sorted_ad);
  float* z1 = (float*)(ws + L.z1);
  float* z2 = (float*)(ws + L.z2);
  uint16_t* act = (uint16_t*)(ws + L.act);
  float* dpair = (float*)(ws + L.dpair);

  if (W_router) {  // router GEMM: logits into the workspace
    float* logits = (float*)(ws + L.logits);
    if (launch_router_logits((const uint16_t*)x, (const uint16_t*)W_router, T, h, E, logits,
                             stream) != hipSuccess)
      return MOELORA_EHIP;
    router_logits = logits;
  }

  if (!mark(ev, 0, stream)) return MOELORA_EHIP;
  if (launch_route(router_logits, T, E, topk, topk_ids, topk_w, tok_flags, stream) != hipSuccess)
    return MOELORA_EHIP;
  if (!mark(ev, 1, stream)) return MOELORA_EHIP;

  const PathPlan& path = pl.path;
  const int bm = pl.bm;
  AlignArgs al;
  al.topk_ids = topk_ids;
  al.adapter_ids = adapter_ids;
  al.tok_flags = tok_flags;
  al.T = T;
  al.k = topk;
  al.E = E;
  al.nA = nA;
  al.seg_pad = 1;
  al.block_m = bm;
  al.sorted_pairs = sorted;
  al.expert_offsets = (int*)(ws + L.expert_off);
  al.seg_table = (int*)(ws + L.seg_table);
  al.n_seg = (int*)(ws + L.n_seg);
  al.flags = (int*)(ws + L.flags);
  al.block_expert = block_expert;
  al.block_seg = block_seg;
  al.pair_row = pair_row;
  al.sorted_ad = sorted_ad;
  al.n_blocks = n_blocks;
  al.g_lists = (int*)(ws + L.align_lists);
  const size_t lds = align_lds_plan(T, topk, E, nA, &al);
  if (launch_align(al, lds, stream) != hipSuccess) return MOELORA_EHIP;
  if (!mark(ev, 2, stream)) return MOELORA_EHIP;

  ShrinkArgs sh;
  sh.sorted_pairs = sorted;
  sh.sorted_ad = sorted_ad;
  sh.block_expert = block_expert;
  sh.n_blocks = n_blocks;
  sh.bm = bm;
  sh.adapter_ids = adapter_ids;
  sh.k = topk;
  sh.nA = nA;
  sh.E = E;
  sh.r = r;
  sh.xcd_ranges = path.tiled ? 1 : 0;
  sh.block_seg = block_seg;
  sh.seg_table = al.seg_table;
  sh.n_seg = al.n_seg;

  GemmArgs g;
  g.cap = L.cap;
  g.tail_split = 0;
  g.n_cu = 0;
  g.d_parts = nullptr;
  g.sorted_pairs = sorted;
  g.sorted_ad = sorted_ad;
  g.block_expert = block_expert;
  g.block_seg = block_seg;
  g.seg_table = al.seg_table;
  g.n_seg = al.n_seg;
  g.n_blocks = n_blocks;
  g.adapter_ids = adapter_ids;
  g.k = topk;
  g.nA = nA;
  g.E = E;
  g.r = r;
  g.act_out = act;
  g.d_out = dpair;
  g.n_blocks_max = pl.max_blocks;
  g.layout_bm = bm;
  // MOELORA_LORA_EXT=0 keeps every tiled LoRA expand in the epilogue (experiments)
  static int lora_ext_env = -1;
  if (lora_ext_env < 0) {
    const char* env = getenv("MOELORA_LORA_EXT");
    lora_ext_env = env ? atoi(env) : 1;
  }
  g.lora_ext = lora_ext_env != 0 ? 1 : 0;

  // gate_up: shrink z1 = x A1, then W1 GEMM + z1 B1 + SiLU-and-mul -> act
  sh.X = (const uint16_t*)x;
  sh.x_bytes = (uint32_t)((size_t)T * h * 2);
  sh.Aw = (const uint16_t*)A1;
  sh.K = h;
  sh.S = pl.s1;
  sh.zpart = z1;
  sh.cap = L.cap;
  sh.after64 = pl.shrink64 ? 1 : 0;
  // rows the 64-row shrink leaves (all rows on the weight-streaming path, where runs are a row
  // or two): one wavefront per adapter segment and K split (MOELORA_SEGSHRINK=0: the 16-row
  // shrink, for experiments; measured: fine-grained layer 0.483 -> 0.453 ms, one adapter per
  // token 1.85 -> 1.81 ms)
  static int seg_env = -1;
  if (seg_env < 0) {
    const char* env = getenv("MOELORA_SEGSHRINK");
    seg_env = env ? atoi(env) : 1;
  }
  const bool seg_shrink = seg_env != 0;
  auto shrink = [&](bool gather) {
    if (pl.shrink64 && launch_shrink_tiled(gather, sh, pl.n_sub_max, stream) != hipSuccess)
      return false;
    return (seg_shrink ? launch_shrink_seg(gather, sh, (int)pl.P, stream)
                       : launch_shrink(gather, sh, pl.tiles16, stream)) == hipSuccess;
  };
  if (!shrink(true)) return MOELORA_EHIP;
  uint16_t* zhl = path.tiled ? (uint16_t*)(ws + L.zhl) : nullptr;
  // the skinny GEMMs add the split parts themselves (one launch fewer per projection); the
  // tiled GEMMs take z as bf16 high and low planes, made by zfinal
  const int64_t max_rows = (int64_t)pl.max_blocks * bm;
  if (path.tiled &&
      launch_zfinal(z1, pl.s1, L.cap, r, n_blocks, bm, max_rows, zhl, stream) != hipSuccess)
    return MOELORA_EHIP;
  if (!mark(ev, 3, stream)) return MOELORA_EHIP;
  g.X = (const uint16_t*)x;
  g.x_bytes = (uint32_t)((size_t)T * h * 2);
  g.W = (const uint16_t*)W1;
  g.W8 = (const uint8_t*)W1;
  g.wscale = w1_scale;
  g.Bw = (const uint16_t*)B1;
  g.zhl = zhl;
  g.zpart = z1;
  g.zsplits = path.tiled ? 0 : pl.s1;
  g.K = h;
  g.N = I;
  g.ksplit = 1;
  g.d_split_stride = L.cap * (int64_t)h;
  g.n_col_tiles = g.N / (pl.sk.gu.split ? 32 : 64 * pl.sk.gu.rt);
  const hipError_t gu_err = path.tiled
                                ? launch_tiled(path.tc, true, g, stream, fp8)
                                : launch_skinny(pl.sk.gu, true, g, pl.max_blocks, stream, fp8);
  if (gu_err != hipSuccess) return MOELORA_EHIP;
  if (!mark(ev, 4, stream)) return MOELORA_EHIP;

  // down: shrink z2 = act A2, then W2 GEMM + z2 B2 -> D (fp32, sorted rows)
  sh.X = act;
  sh.x_bytes = (uint32_t)((size_t)L.cap * I * 2);
  sh.Aw = (const uint16_t*)A2;
  sh.K = I;
  sh.S = pl.s2;
  sh.zpart = z2;
  if (!shrink(false)) return MOELORA_EHIP;
  if (path.tiled &&
      launch_zfinal(z2, pl.s2, L.cap, r, n_blocks, bm, max_rows, zhl, stream) != hipSuccess)
    return MOELORA_EHIP;
  g.zpart = z2;
  g.zsplits = path.tiled ? 0 : pl.s2;
  if (!mark(ev, 5, stream)) return MOELORA_EHIP;
  g.X = act;
  g.x_bytes = (uint32_t)((size_t)L.cap * I * 2);
  g.W = (const uint16_t*)W2;
  g.W8 = (const uint8_t*)W2;
  g.wscale = w2_scale;
  g.Bw = (const uint16_t*)B2;
  g.K = I;
  g.N = h;
  g.ksplit = pl.sk.ksplit;
  g.tail_split = path.tiled ? pl.tail_split : 0;
  g.n_cu = 0;
  g.d_parts = nullptr;
  if (g.tail_split > 1) {
    g.n_cu = resident_tiles();
    if (g.n_cu <= 0) return MOELORA_EHIP;
    g.d_parts = (int*)(ws + L.d_parts);
  }
  g.n_col_tiles = g.N / (64 * pl.sk.dn.rt);
  const hipError_t dn_err = path.tiled
                                ? launch_tiled(path.tc_dn, false, g, stream, fp8)
                                : launch_skinny(pl.sk.dn, false, g, pl.max_blocks, stream, fp8);
  if (dn_err != hipSuccess) return MOELORA_EHIP;
  if (!mark(ev, 6, stream)) return MOELORA_EHIP;

  // weighted top-k combine -> y (bf16)
  CombineArgs cb;
  cb.D = dpair;
  cb.ksplit = pl.sk.ksplit;
  cb.split_stride = L.cap * (int64_t)h;
  cb.d_parts = g.d_parts;
  cb.part_rows = path.tc_dn.bm;
  cb.part_cols = path.tc_dn.bn;
  cb.part_ncol = h / path.tc_dn.bn;
  cb.pair_row = pair_row;
  cb.topk_w = topk_w;
  cb.T = T;
  cb.k = topk;
  cb.h = h;
  cb.y = (uint16_t*)y;
  if (launch_combine(cb, stream) != hipSuccess) return MOELORA_EHIP;
  if (!mark(ev, 7, stream)) return MOELORA_EHIP;
  return MOELORA_OK;
}

// Host checks of a layer call, before anything is enqueued: sizes, the FP8 path's range,
// pointers (NULL, 16-byte alignment; W_router and the scales when given), the workspace and the
// device. logits may be NULL when W_router is given (the router GEMM writes them into the
// workspace). Fills the plan and layout.
int check_forward(const void* x, const float* router_logits, const void* W_router, const void* W1,
                  const void* W2, const void* A1, const void* B1, const void* A2, const void* B2,
                  const int32_t* adapter_ids, int32_t topk, const moe_lora_dims* d, const void* y,
                  const void* workspace, size_t workspace_bytes, const float* w1_scale,
                  const float* w2_scale, bool fp8, ForwardPlan* pl, MoeLoraLayout* L,
                  bool in_scratch = false) {
  int rc = plan_and_layout(d, topk, fp8, pl, L);
  if (rc != MOELORA_OK) return rc;
  if (in_scratch && L->total > kScratchBytes) return MOELORA_ESCRATCH;
  if (d->T == 0) return MOELORA_OK;  // empty batch: nothing to do, pointers may be NULL
  const void* logits_or_router = W_router ? W_router : (const void*)router_logits;
  // (the workspace last: the no-alloc entry has none)
  const void* ptrs[] = {x, logits_or_router, W1, W2, A1, B1, A2, B2, adapter_ids, y, workspace};
  const int n_ptrs = in_scratch ? 10 : 11;
  for (int i = 0; i < n_ptrs; ++i)
    if (!ptrs[i]) return MOELORA_ENULL;
  for (int i = 0; i < n_ptrs; ++i)
    if (!aligned16(ptrs[i])) return MOELORA_EALIGN;
  if (fp8 && (!w1_scale || !w2_scale)) return MOELORA_ENULL;
  if (fp8 && ((((uintptr_t)w1_scale) | ((uintptr_t)w2_scale)) & 3u) != 0) return MOELORA_EALIGN;
  if (!in_scratch && ((uintptr_t)workspace & 255u) != 0) return MOELORA_EWORKSPACE;
  if (!in_scratch && workspace_bytes < L->total) return MOELORA_EWORKSPACE;
  return check_device();
}

// The layer. W_router != nullptr: the router GEMM first writes the logits into the workspace
// (router_logits unused). w1_scale/w2_scale != nullptr: W1/W2 are E4M3 codes with per-row
// scales (skinny path only).
int forward_impl(const void* x, const float* router_logits, const void* W_router, const void* W1,
                 const void* W2, const void* A1, const void* B1, const void* A2, const void* B2,
                 const int32_t* adapter_ids, int32_t topk, const moe_lora_dims* d, void* y,
                 void* workspace, size_t workspace_bytes, void* stream_, void* const* ev,
                 const float* w1_scale = nullptr, const float* w2_scale = nullptr) {
  const bool fp8 = w1_scale != nullptr || w2_scale != nullptr;
  ForwardPlan pl;
  MoeLoraLayout L;
  const int rc = check_forward(x, router_logits, W_router, W1, W2, A1, B1, A2, B2, adapter_ids, topk,
                               d, y, workspace, workspace_bytes, w1_scale, w2_scale, fp8, &pl, &L);
  if (rc != MOELORA_OK || d->T == 0) return rc;
  return enqueue_forward(pl, L, x, router_logits, W_router, W1, W2, A1, B1, A2, B2, adapter_ids,
                         topk, d, y, (char*)workspace, (hipStream_t)stream_, ev, w1_scale, w2_scale);
}

}  // namespace

extern "C" {

int moe_lora_forward(const void* x, const float* router_logits, const void* W1, const void* W2,
                     const void* A1, const void* B1, const void* A2, const void* B2,
                     const int32_t* adapter_ids, int32_t topk, const moe_lora_dims* d, void* y,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(x, router_logits, nullptr, W1, W2, A1, B1, A2, B2, adapter_ids, topk, d, y,
                      workspace, workspace_bytes, stream, nullptr);
}

int moe_lora_forward_timed(const void* x, const float* router_logits, const void* W1,
                           const void* W2, const void* A1, const void* B1, const void* A2,
                           const void* B2, const int32_t* adapter_ids, int32_t topk,
                           const moe_lora_dims* d, void* y, void* workspace,
                           size_t workspace_bytes, void* stream, void* const* stage_events) {
  if (!stage_events) return MOELORA_ENULL;
  return forward_impl(x, router_logits, nullptr, W1, W2, A1, B1, A2, B2, adapter_ids, topk, d, y,
                      workspace, workspace_bytes, stream, stage_events);
}

int moe_lora_router_logits(const void* x, const void* W_router, int32_t T, int32_t hidden,
                           int32_t n_experts, float* logits, void* stream) {
  if (T < 0 || hidden <= 0 || hidden % 128 != 0 || n_experts < 1 || n_experts > kMaxExperts)
    return MOELORA_EINVAL_DIMS;
  if ((int64_t)T * hidden * 2 >= ((int64_t)1 << 31) ||
      (int64_t)n_experts * hidden * 2 >= ((int64_t)1 << 31))
    return MOELORA_EINVAL_DIMS;
  if (T == 0) return MOELORA_OK;
  if (!x || !W_router || !logits) return MOELORA_ENULL;
  if (!aligned16(x) || !aligned16(W_router) || ((uintptr_t)logits & 3u) != 0) return MOELORA_EALIGN;
  const int rc = check_device();
  if (rc != MOELORA_OK) return rc;
  return launch_router_logits((const uint16_t*)x, (const uint16_t*)W_router, T, hidden, n_experts,
                              logits, (hipStream_t)stream) == hipSuccess
             ? MOELORA_OK
             : MOELORA_EHIP;
}

int moe_lora_forward_routed(const void* x, const void* W_router, const void* W1, const void* W2,
                            const void* A1, const void* B1, const void* A2, const void* B2,
                            const int32_t* adapter_ids, int32_t topk, const moe_lora_dims* d,
                            void* y, void* workspace, size_t workspace_bytes, void* stream) {
  if (d && d->T > 0 && !W_router) {  // (forward_impl takes a NULL W_router as "logits given")
    const int rc = validate_dims(d, topk);
    return rc != MOELORA_OK ? rc : MOELORA_ENULL;
  }
  return forward_impl(x, nullptr, W_router, W1, W2, A1, B1, A2, B2, adapter_ids, topk, d, y,
                      workspace, workspace_bytes, stream, nullptr);
}

int moe_lora_forward_fp8(const void* x, const float* router_logits, const void* W1q,
                         const float* W1_scale, const void* W2q, const float* W2_scale,
                         const void* A1, const void* B1, const void* A2, const void* B2,
                         const int32_t* adapter_ids, int32_t topk, const moe_lora_dims* d,
                         void* y, void* workspace, size_t workspace_bytes, void* stream,
                         void* const* stage_events) {
  if (!W1_scale || !W2_scale) {
    const int rc = validate_dims(d, topk);
    return rc != MOELORA_OK ? rc : MOELORA_ENULL;
  }
  return forward_impl(x, router_logits, nullptr, W1q, W2q, A1, B1, A2, B2, adapter_ids, topk, d, y,
                      workspace, workspace_bytes, stream, stage_events, W1_scale, W2_scale);
}

}  // extern "C"

namespace {

// Static scratch of moe_lora_forward_noalloc: the workspace of a layer call for callers that
// cannot allocate. One copy per GPU, alive until the process ends. In host code `scratch` is a
// host-side stand-in for the symbol, never a device address: kernels and copies get the
// per-device address that hipGetSymbolAddress returns.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // device address of `scratch` on each device, once looked up

// The address of this device's copy of `scratch` (looked up on the device's first call, with
// that device current), or nullptr on error.
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int moe_lora_forward_noalloc(const void* x, const float* router_logits, const void* W1,
                             const void* W2, const void* A1, const void* B1, const void* A2,
                             const void* B2, const int32_t* adapter_ids, int32_t topk,
                             const moe_lora_dims* d, void* y, void* stream) {
  ForwardPlan pl;
  MoeLoraLayout L;
  const int rc = check_forward(x, router_logits, nullptr, W1, W2, A1, B1, A2, B2, adapter_ids,
                               topk, d, y, nullptr, 0, nullptr, nullptr, false, &pl, &L, true);
  if (rc != MOELORA_OK || d->T == 0) return rc;
  // The layer needs no zeroed workspace: every region a kernel reads was written earlier in the
  // same call, so nothing is cleared between calls.
  char* ws = (char*)scratch_on_current_device();
  if (!ws) return MOELORA_EHIP;
  return enqueue_forward(pl, L, x, router_logits, nullptr, W1, W2, A1, B1, A2, B2, adapter_ids, topk,
                         d, y, ws, (hipStream_t)stream, nullptr, nullptr, nullptr);
}

namespace {

// Workspace of moe_lora_sgmv: flags first (moe_lora_debug_status), then the sorted layout of T
// single-expert pairs in 16-row blocks, the shrink's split parts, align scratch.
struct SgmvLayout {
  size_t flags, sorted, sorted_ad, expert_off, n_blocks, block_expert, block_seg, seg_table, n_seg,
      zpart, align_lists, total;
  int64_t cap;
};

int sgmv_validate(const moe_lora_sgmv_dims* d) {
  if (!d) return MOELORA_ENULL;
  if (d->T < 0 || d->in_features <= 0 || d->out_features <= 0 || d->n_adapters <= 0)
    return MOELORA_EINVAL_DIMS;
  if (d->in_features % 128 != 0 || d->out_features % 64 != 0) return MOELORA_EINVAL_DIMS;
  if (!(d->rank == 8 || d->rank == 16 || d->rank == 32 || d->rank == 64)) return MOELORA_EINVAL_DIMS;
  if ((int64_t)d->T * d->in_features * 2 >= ((int64_t)1 << 31)) return MOELORA_EINVAL_DIMS;
  if ((int64_t)d->T + 256 >= ((int64_t)1 << 30) || (int64_t)d->n_adapters + 1 >= ((int64_t)1 << 28))
    return MOELORA_EINVAL_DIMS;
  return MOELORA_OK;
}

void sgmv_layout(const moe_lora_sgmv_dims* d, SgmvLayout* L) {
  const int64_t T = d->T, r = d->rank;
  L->cap = round_up64(T + 15, 256);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + (bytes ? bytes : 1));
    return o;
  };
  L->flags = take(16);
  L->sorted = take(4 * (size_t)L->cap);
  L->sorted_ad = take(4 * (size_t)L->cap);
  L->expert_off = take(8);
  L->n_blocks = take(4);
  L->block_expert = take(4 * (size_t)(L->cap / 16 + 1));
  L->block_seg = take(4 * (size_t)(L->cap / 16 + 1));
  L->seg_table = take(16 * (size_t)T);
  L->n_seg = take(4);
  L->zpart = take(4 * (size_t)kMaxSplit * L->cap * r);
  L->align_lists = take(4 * align_list_ints((int)T, 1, 1, d->n_adapters));
  L->total = off;
}

}  // namespace

size_t moe_lora_sgmv_workspace_size(const moe_lora_sgmv_dims* d) {
  if (sgmv_validate(d) != MOELORA_OK) return 0;
  SgmvLayout L;
  sgmv_layout(d, &L);
  return L.total;
}

int moe_lora_sgmv(const void* x, const void* A, const void* B, const int32_t* adapter_ids,
                  const moe_lora_sgmv_dims* d, void* y, void* workspace, size_t workspace_bytes,
                  void* stream_) {
  int rc = sgmv_validate(d);
  if (rc != MOELORA_OK) return rc;
  if (d->T == 0) return MOELORA_OK;
  const void* ptrs[] = {x, A, B, adapter_ids, y, workspace};
  for (const void* p : ptrs)
    if (!p) return MOELORA_ENULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOELORA_EALIGN;
  if (((uintptr_t)workspace & 255u) != 0) return MOELORA_EWORKSPACE;
  SgmvLayout L;
  sgmv_layout(d, &L);
  if (workspace_bytes < L.total) return MOELORA_EWORKSPACE;
  rc = check_device();
  if (rc != MOELORA_OK) return rc;

  hipStream_t stream = (hipStream_t)stream_;
  char* ws = (char*)workspace;
  const int T = d->T, K = d->in_features, N = d->out_features, nA = d->n_adapters, r = d->rank;
  const int bm = 16;
  const int max_blocks = (T + bm - 1 + 15) / bm;  // T rows plus at most 15 padding rows

  // align: one expert, one pair per token; segments by adapter
  AlignArgs al;
  al.topk_ids = nullptr;
  al.adapter_ids = adapter_ids;
  al.tok_flags = nullptr;
  al.T = T;
  al.k = 1;
  al.E = 1;
  al.nA = nA;
  al.seg_pad = 1;
  al.block_m = bm;
  al.sorted_pairs = (int*)(ws + L.sorted);
  al.expert_offsets = (int*)(ws + L.expert_off);
  al.seg_table = (int*)(ws + L.seg_table);
  al.n_seg = (int*)(ws + L.n_seg);
  al.flags = (int*)(ws + L.flags);
  al.block_expert = (int*)(ws + L.block_expert);
  al.block_seg = (int*)(ws + L.block_seg);
  al.pair_row = nullptr;
  al.sorted_ad = (int*)(ws + L.sorted_ad);
  al.n_blocks = (int*)(ws + L.n_blocks);
  al.g_lists = (int*)(ws + L.align_lists);
  if (T <= kSgmvSortMaxTokens && nA <= kSgmvSortMaxAdapters) {
    // up to 1024 tokens and adapters: one pass of a one-workgroup sort of the tokens with an
    // adapter (the shrink and expand read the rows, their adapters and the block count only)
    SgmvSortArgs so;
    so.adapter_ids = adapter_ids;
    so.T = T;
    so.nA = nA;
    so.sorted_pairs = al.sorted_pairs;
    so.sorted_ad = al.sorted_ad;
    so.block_expert = al.block_expert;
    so.n_blocks = al.n_blocks;
    so.flags = al.flags;
    if (launch_sgmv_sort(so, stream) != hipSuccess) return MOELORA_EHIP;
  } else {
    const size_t lds = align_lds_plan(T, 1, 1, nA, &al);
    if (launch_align(al, lds, stream) != hipSuccess) return MOELORA_EHIP;
  }

  // shrink z = x A_a^T over 16-row tiles, split over K
  ShrinkArgs sh;
  sh.X = (const uint16_t*)x;
  sh.x_bytes = (uint32_t)((size_t)T * K * 2);
  sh.sorted_pairs = al.sorted_pairs;
  sh.sorted_ad = al.sorted_ad;
  sh.block_expert = al.block_expert;
  sh.block_seg = al.block_seg;
  sh.seg_table = al.seg_table;
  sh.n_seg = al.n_seg;
  sh.n_blocks = al.n_blocks;
  sh.bm = bm;
  sh.adapter_ids = adapter_ids;
  sh.k = 1;
  sh.nA = nA;
  sh.E = 1;
  sh.r = r;
  sh.K = K;
  sh.Aw = (const uint16_t*)A;
  sh.S = pick_splits(std::min<int64_t>(max_blocks, (T + 15) / 16 + 1), K);
  sh.zpart = (float*)(ws + L.zpart);
  sh.cap = L.cap;
  sh.xcd_ranges = 0;
  sh.after64 = 0;
  if (launch_shrink(true, sh, max_blocks, stream) != hipSuccess) return MOELORA_EHIP;

  // expand y += z B_a^T
  SgmvArgs sa;
  sa.sorted_pairs = al.sorted_pairs;
  sa.sorted_ad = al.sorted_ad;
  sa.n_blocks = al.n_blocks;
  sa.zpart = sh.zpart;  // the expand adds the split parts itself
  sa.zsplits = sh.S;
  sa.cap = L.cap;
  sa.B = (const uint16_t*)B;
  sa.y = (uint16_t*)y;
  sa.N = N;
  sa.r = r;
  if (launch_sgmv_expand(sa, max_blocks, stream) != hipSuccess) return MOELORA_EHIP;
  return MOELORA_OK;
}

int moe_lora_route_align(const float* router_logits, const int32_t* adapter_ids, int32_t topk,
                         const moe_lora_dims* d, int32_t seg_pad, int32_t block_m,
                         int32_t* topk_ids, float* topk_w, int32_t* sorted_pairs,
                         int64_t sorted_cap, int32_t* expert_offsets, int32_t* seg_table,
                         int32_t* n_seg, void* workspace, size_t workspace_bytes, void* stream_) {
  int rc = validate_dims(d, topk);
  if (rc != MOELORA_OK) return rc;
  const int64_t need = moe_lora_sorted_capacity(d, topk, seg_pad, block_m);
  if (need < 0 || sorted_cap < need) return MOELORA_EINVAL_DIMS;
  const void* ptrs[] = {router_logits, adapter_ids, topk_ids, topk_w, sorted_pairs,
                        expert_offsets, seg_table, n_seg, workspace};
  for (int i = 0; i < 9; ++i)  // the [T]-sized tensors may be NULL when T == 0
    if (!ptrs[i] && !(d->T == 0 && i < 4)) return MOELORA_ENULL;
  for (const void* p : ptrs)
    if (((uintptr_t)p & 3u) != 0) return MOELORA_EALIGN;
  if (((uintptr_t)workspace & 255u) != 0) return MOELORA_EWORKSPACE;
  ForwardPlan pl;
  MoeLoraLayout L;
  rc = plan_and_layout(d, topk, false, &pl, &L);
  if (rc != MOELORA_OK) return rc;
  if (workspace_bytes < L.total) return MOELORA_EWORKSPACE;
  rc = check_device();
  if (rc != MOELORA_OK) return rc;

  hipStream_t stream = (hipStream_t)stream_;
  char* ws = (char*)workspace;
  int* tok_flags = (int*)(ws + L.tok_flags);
  if (launch_route(router_logits, d->T, d->n_experts, topk, topk_ids, topk_w, tok_flags, stream) !=
      hipSuccess)
    return MOELORA_EHIP;
  AlignArgs al;
  al.topk_ids = topk_ids;
  al.adapter_ids = adapter_ids;
  al.tok_flags = tok_flags;
  al.T = d->T;
  al.k = topk;
  al.E = d->n_experts;
  al.nA = d->n_adapters;
  al.seg_pad = seg_pad;
  al.block_m = block_m;
  al.sorted_pairs = sorted_pairs;
  al.expert_offsets = expert_offsets;
  al.seg_table = seg_table;
  al.n_seg = n_seg;
  al.flags = (int*)(ws + L.flags);
  al.block_expert = nullptr;
  al.block_seg = nullptr;
  al.pair_row = nullptr;
  al.sorted_ad = nullptr;
  al.n_blocks = nullptr;
  al.g_lists = (int*)(ws + L.align_lists);
  const size_t lds = align_lds_plan(d->T, topk, d->n_experts, d->n_adapters, &al);
  if (launch_align(al, lds, stream) != hipSuccess) return MOELORA_EHIP;
  return MOELORA_OK;
}

int moe_lora_debug_status(const void* workspace, size_t workspace_bytes, void* stream_,
                          uint32_t* flags) {
  if (!workspace || !flags) return MOELORA_ENULL;
  if (((uintptr_t)workspace & 255u) != 0 || workspace_bytes < 16) return MOELORA_EWORKSPACE;
  hipStream_t stream = (hipStream_t)stream_;
  if (hipStreamSynchronize(stream) != hipSuccess) return MOELORA_EHIP;
  int32_t v = 0;
  if (hipMemcpy(&v, workspace, sizeof v, hipMemcpyDeviceToHost) != hipSuccess) return MOELORA_EHIP;
  *flags = (uint32_t)v;
  return MOELORA_OK;
}

}  // extern "C"
