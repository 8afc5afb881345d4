// Routing (top-k softmax) and align (token-expert pairs sorted by expert, segmented by
// adapter) for the fused MoE + multi-LoRA layer.
//
// Routing follows page "vLLM MoE LoRA SageMaker Bedrock", section "Entendendo os Modelos MoE"
// (a router sends each token to its most relevant experts, whose outputs are then
// aggregated). The sort by (expert, adapter) answers the same page's section "Implementação
// Técnica no vLLM" (expert routing and adapter selection are two sources of sparsity that need
// a dedicated design) and page "Punica: Multi-Tenant LoRA Serving" (segmented gather: a batch
// is cut into segments that share one adapter).
#include "common.h"
#include "kernels.h"

namespace moelora {

// ------------------------------------------------------------------------------------------
// Route: one wavefront per token. Each lane holds up to 16 logits (E <= 1024). Selection runs
// k rounds of a wave-wide arg-max under the order "larger logit, then lower expert id", so
// slot j holds the expert that exactly j others beat. Non-finite logits are flagged and take
// part as -infinity. Weights: softmax over the selected logits, in fp32.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int* __restrict__ topk_ids,
                                                         float* __restrict__ topk_w,
                                                         int* __restrict__ tok_flags) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float v[16];
  bool live[16];
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    live[i] = e < E;
    float f = -INFINITY;
    if (live[i]) {
      f = row[e];
      if (!__builtin_isfinite(f)) {
        bad = true;
        f = -INFINITY;
      }
    }
    v[i] = f;
  }
  float sel_v[kMaxTopk];
  int sel_e[kMaxTopk];
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j) {
    if (j >= k) continue;
    float bv = -INFINITY;
    int be = 0x7fffffff;  // "none"
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane + 64 * i;
      if (live[i] && (be == 0x7fffffff || v[i] > bv || (v[i] == bv && e < be))) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (oe != 0x7fffffff && (be == 0x7fffffff || ov > bv || (ov == bv && oe < be))) {
        bv = ov;
        be = oe;
      }
    }
    sel_v[j] = bv;
    sel_e[j] = be;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (lane + 64 * i == be) live[i] = false;
  }
  const uint64_t anybad = __ballot(bad);
  if (lane == 0) {
    const float top = sel_v[0];
    float ex[kMaxTopk];
    float den = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) {
      ex[j] = 0.f;
      if (j >= k) continue;
      ex[j] = (top == -INFINITY) ? 1.f : __expf(sel_v[j] - top);
      den += ex[j];
    }
    const float inv = 1.f / den;
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) {
      if (j >= k) continue;
      topk_ids[(size_t)t * k + j] = sel_e[j];
      topk_w[(size_t)t * k + j] = ex[j] * inv;
    }
    tok_flags[t] = anybad ? 1 : 0;
  }
}

// Route for up to 256 experts: the rank of each logit, the number of logits that beat it
// (larger, or equal with a lower expert id), is its slot when it is below k, which is the same
// selection as k rounds of arg-max. The token's logits are staged in LDS and every lane counts,
// for its (up to VPL) logits, how many of the E staged ones beat it: broadcast reads, no
// cross-lane reductions. Up to 64 experts a wavefront takes one token (four per workgroup);
// above, the four wavefronts of a workgroup share one token and each counts against a quarter
// of the logits (the counts are added through LDS), which keeps the serial compare chain per
// wavefront at E/4. Non-finite logits are flagged and take part as -infinity.
template <int VPL>
__global__ __launch_bounds__(256) void route_rank_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int* __restrict__ topk_ids,
                                                         float* __restrict__ topk_w,
                                                         int* __restrict__ tok_flags) {
  constexpr int TPB = VPL == 1 ? 4 : 1;  // tokens per workgroup
  constexpr int WPT = 4 / TPB;           // wavefronts per token
  __shared__ __attribute__((aligned(16))) float s_l[TPB][64 * VPL];
  __shared__ int s_rank[WPT][64 * VPL];
  __shared__ float s_sel[TPB][kMaxTopk];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int w = wv / WPT, part = wv % WPT;  // token slot, quarter of the comparisons
  const int t = blockIdx.x * TPB + w;
  const bool active = t < T;  // (no early exit: every wavefront reaches the barriers)
  const float* row = logits + (size_t)(active ? t : 0) * E;
  float v[VPL];
  bool bad = false;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    float f = -INFINITY;
    if (active && e < E) {
      f = row[e];
      if (!__builtin_isfinite(f)) {
        bad = true;
        f = -INFINITY;
      }
    }
    v[i] = f;
    if (part == 0) s_l[w][e] = f;  // (slots past E hold -infinity and are never counted)
  }
  __syncthreads();
  int rank[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) rank[i] = 0;
  // this wavefront's compare range [c0, c1): quarters rounded to whole 16-byte LDS reads
  const int eq = WPT == 1 ? E : ((E + 4 * WPT - 1) / (4 * WPT)) * 4;
  const int c0 = part * eq, c1 = min(E, c0 + eq);
  for (int c = c0; c < c1; c += 4) {
    const f32x4 o = *reinterpret_cast<const f32x4*>(&s_l[w][c]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int eo = c + j;
      if (eo >= c1) break;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = lane + 64 * i;
        rank[i] += (o[j] > v[i] || (o[j] == v[i] && eo < e)) ? 1 : 0;
      }
    }
  }
  if (WPT > 1) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) s_rank[part][lane + 64 * i] = rank[i];
    __syncthreads();
    if (part == 0) {
#pragma unroll
      for (int i = 0; i < VPL; ++i)
#pragma unroll
        for (int q = 1; q < WPT; ++q) rank[i] += s_rank[q][lane + 64 * i];
    }
  }
  const uint64_t anybad = __ballot(bad);
  if (part == 0) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      if (active && e < E && rank[i] < k) {
        topk_ids[(size_t)t * k + rank[i]] = e;
        s_sel[w][rank[i]] = v[i];
      }
    }
  }
  __syncthreads();
  if (active && part == 0 && lane == 0) {
    const float top = s_sel[w][0];
    float ex[kMaxTopk];
    float den = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) {
      ex[j] = 0.f;
      if (j >= k) continue;
      ex[j] = (top == -INFINITY) ? 1.f : __expf(s_sel[w][j] - top);
      den += ex[j];
    }
    const float inv = 1.f / den;
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) {
      if (j >= k) continue;
      topk_w[(size_t)t * k + j] = ex[j] * inv;
    }
    tok_flags[t] = anybad ? 1 : 0;
  }
}

// ------------------------------------------------------------------------------------------
// Align: one workgroup of 1024 threads. Each pair p = t*k + j gets the bucket key
// b = e*(nA+1) + (a+1) (e its expert, a its token's adapter, -1 for none), and the pairs are
// sorted by key, stable in pair (= token) order, by least-significant-digit radix passes of D
// bits (D <= 10, as few passes as the key width allows). A segment is a run of equal keys.
//   phase 0  keys (adapter ids validated: out of range -> flag, treated as -1), flags
//   passes   count digits per wavefront slice, exclusive scan in (digit, wavefront) order,
//            then rank and scatter; the rank of a pair among the equal digits of earlier lanes
//            of its 64-pair chunk is an exact popcount of a ballot match
//   phase 1  segment starts (key changes) -> segment id of every sorted position
//   phase 2  padded segment sizes scanned; each expert's region (the sum over its segments)
//            padded to block_m; segment table, expert offsets, row block -> segment table
//   phase 3  padding slots (-1), row block -> expert table; pair ids (and their adapters)
//            into their padded rows
// Every step is a flat loop over pairs, segments or experts: the work is O(T*k + E) whatever
// the number of adapters. The arrays live in LDS when they fit and in the workspace otherwise.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ uint64_t match_key(bool member, int key, int nbits) {
  uint64_t eq = __ballot(member);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool one = (key >> bit) & 1;
    const uint64_t b = __ballot(member && one);
    eq &= one ? b : ~b;
  }
  return member ? eq : 0ull;
}

__device__ __forceinline__ int round_up_i(int v, int m) { return (v + m - 1) / m * m; }

// Inclusive scan over the 64 lanes with DPP moves: shifts by 1, 2, 4 and 8 within each row of
// 16 lanes, then the last lane of row 0 (2) is added to row 1 (3) and that of row 1 to rows 2
// and 3. A lane whose DPP source is missing or masked off adds 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Exclusive scan of (v0, v1) over the workgroup; red needs 2*32+2 ints.
__device__ void block_excl_scan2(int v0, int v1, int& ex0, int& ex1, int& tot0, int& tot1,
                                 int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int i0 = wave_incl_scan(v0), i1 = wave_incl_scan(v1);
  if (lane == 63) {
    red[wave] = i0;
    red[32 + wave] = i1;
  }
  __syncthreads();
  if (wave == 0) {
    const int w0 = lane < nw ? red[lane] : 0;
    const int w1 = lane < nw ? red[32 + lane] : 0;
    const int s0 = wave_incl_scan(w0), s1 = wave_incl_scan(w1);
    if (lane < nw) {
      red[lane] = s0 - w0;
      red[32 + lane] = s1 - w1;
    }
    if (lane == 63) {
      red[64] = s0;
      red[65] = s1;
    }
  }
  __syncthreads();
  ex0 = red[wave] + i0 - v0;
  ex1 = red[32 + wave] + i1 - v1;
  tot0 = red[64];
  tot1 = red[65];
  __syncthreads();
}

__global__ __launch_bounds__(1024) void align_kernel(AlignArgs a) {
  extern __shared__ int smem[];
  __shared__ int s_g0[kMaxExperts];    // padded-size scan at the expert's first segment
  __shared__ int s_sexp[kMaxExperts];  // padded rows of the expert's segments
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_red[72];

  constexpr int nwaves = kAlignThreads / 64, bd = kAlignThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, k = a.k, E = a.E, nA = a.nA, P = T * k;
  const int nb1 = nA + 1;
  const int seg_pad = a.seg_pad, block_m = a.block_m;
  // p / k as a multiply by ceil(2^32 / k) and a shift: exact for p * k < 2^32
  const uint64_t k_magic = ((1ull << 32) + k - 1) / k;
  auto token_of = [&](int p) { return (int)(((uint64_t)(uint32_t)p * k_magic) >> 32); };
  auto pad_to = [&](int c) { return seg_pad == 1 ? c : round_up_i(c, seg_pad); };

  // key [P], v0 [P], v1 [P] (pair ids between passes), then the segment region: starts
  // [seg_cap] and row deltas [seg_cap]. The digit counts [nwaves << D] overlay the segment
  // region (unused until the passes are done) in LDS, or take LDS of their own when the arrays
  // are in the workspace.
  int* key = a.lists_in_lds ? smem : a.g_lists;
  int* v0 = key + P;
  int* v1 = v0 + P;
  int* seg_lo = v1 + P;
  int* delta = seg_lo + a.seg_cap;
  int* cnt = a.lists_in_lds ? seg_lo : smem;

  // phase 0
  // (loads in batches of 8 per thread, issued before any is used)
  int fl_nonfinite = 0, fl_range = 0;
  for (int t0 = 0; a.tok_flags && t0 < T; t0 += 8 * bd) {
    int f[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 + u * bd + tid;
      f[u] = t < T ? a.tok_flags[t] : 0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) fl_nonfinite |= f[u] != 0;
  }
  for (int q0 = 0; q0 < P; q0 += 8 * bd) {
    int ex[8], av[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = q0 + u * bd + tid;
      ex[u] = (p < P && a.topk_ids) ? a.topk_ids[p] : 0;
      av[u] = p < P ? a.adapter_ids[token_of(p)] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = q0 + u * bd + tid;
      if (av[u] < -1 || av[u] >= nA) {
        fl_range = 1;
        av[u] = -1;
      }
      if (p < P) key[p] = ex[u] * nb1 + av[u] + 1;
    }
  }
  for (int e = tid; e < E; e += bd) {
    s_g0[e] = 0;
    s_sexp[e] = 0;
  }
  fl_nonfinite = __syncthreads_or(fl_nonfinite);
  fl_range = __syncthreads_or(fl_range);

  // radix passes, least significant digit first; pass 0 reads the pairs in pair order
  const int D = a.digit_bits, dmask = (1 << D) - 1, ncnt = nwaves << D;
  const int PP = (P + nwaves - 1) / nwaves;
  const int p0 = min(P, wave * PP), p1 = min(P, p0 + PP);
  const int* src = nullptr;
  int* dst = v0;
  for (int pass = 0; pass < a.passes; ++pass) {
    const int shift = pass * D;
    for (int i = tid; i < ncnt; i += bd) cnt[i] = 0;
    __syncthreads();
    // digits of the wavefront's slice (only this wavefront touches row cnt[wave]; the adds
    // need no returned value, so they do not wait for each other)
    for (int base = p0; base < p1; base += 64) {
      const int i = base + lane;
      const bool valid = i < p1;
      const int p = valid ? (src ? src[i] : i) : 0;
      const int dig = valid ? (key[p] >> shift) & dmask : 0;
      const uint64_t eq = match_key(valid, dig, D);
      if (valid && (eq & lanemask_lt()) == 0ull) atomicAdd(&cnt[(wave << D) + dig], (int)__popcll(eq));
    }
    __syncthreads();
    {
      const int per_t = (ncnt + bd - 1) / bd;
      const int lo = min(ncnt, tid * per_t), hi = min(ncnt, lo + per_t);
      int sv = 0;
      for (int j = lo; j < hi; ++j) sv += cnt[((j % nwaves) << D) + j / nwaves];
      int ex, d0, tot, d1;
      block_excl_scan2(sv, 0, ex, d0, tot, d1, s_red);
      int run = ex;
      for (int j = lo; j < hi; ++j) {
        const int idx = ((j % nwaves) << D) + j / nwaves;
        const int c = cnt[idx];
        cnt[idx] = run;
        run += c;
      }
    }
    __syncthreads();
    for (int base = p0; base < p1; base += 64) {
      const int i = base + lane;
      const bool valid = i < p1;
      const int p = valid ? (src ? src[i] : i) : 0;
      const int dig = valid ? (key[p] >> shift) & dmask : 0;
      const uint64_t eq = match_key(valid, dig, D);
      int c = 0;
      if (valid && (eq & lanemask_lt()) == 0ull) c = atomicAdd(&cnt[(wave << D) + dig], (int)__popcll(eq));
      c = __shfl(c, valid ? (__ffsll((unsigned long long)eq) - 1) : lane);
      if (valid) dst[c + (int)__popcll(eq & lanemask_lt())] = p;
    }
    __syncthreads();
    src = dst;
    dst = dst == v0 ? v1 : v0;
  }
  const int* sorted = src ? src : v0;  // (no pass runs only when P == 0)
  int* sid = dst;                      // the other buffer: segment of each sorted position

  // phase 1: contiguous ranges of sorted positions per thread
  int nseg;
  {
    const int per_t = (P + bd - 1) / bd;
    const int lo = min(P, tid * per_t), hi = min(P, lo + per_t);
    const int prev0 = lo > 0 ? key[sorted[lo - 1]] : -1;
    int prev = prev0, ns = 0;
    for (int i = lo; i < hi; ++i) {
      const int kk = key[sorted[i]];
      ns += kk != prev;
      prev = kk;
    }
    int ex, d0, d1;
    block_excl_scan2(ns, 0, ex, d0, nseg, d1, s_red);
    int sg = ex - 1;
    prev = prev0;
    for (int i = lo; i < hi; ++i) {
      const int kk = key[sorted[i]];
      if (kk != prev) seg_lo[++sg] = i;
      prev = kk;
      sid[i] = sg;
    }
    if (tid == 0) seg_lo[nseg] = P;
  }
  __syncthreads();

  // phase 2: contiguous ranges of segments per thread
  const int per_s = (nseg + bd - 1) / bd;
  const int slo = min(nseg, tid * per_s), shi = min(nseg, slo + per_s);
  int gex;
  {
    int sum = 0;
    for (int sg = slo; sg < shi; ++sg) sum += pad_to(seg_lo[sg + 1] - seg_lo[sg]);
    int d0, gtot, d1;
    block_excl_scan2(sum, 0, gex, d0, gtot, d1, s_red);
    int g = gex;
    int e_prev = slo > 0 ? key[sorted[seg_lo[slo - 1]]] / nb1 : -1;
    for (int sg = slo; sg < shi; ++sg) {
      const int e = key[sorted[seg_lo[sg]]] / nb1;
      if (e != e_prev) s_g0[e] = g;
      g += pad_to(seg_lo[sg + 1] - seg_lo[sg]);
      const int e_next = sg + 1 < nseg ? key[sorted[seg_lo[sg + 1]]] / nb1 : -1;
      if (e_next != e) s_sexp[e] = g;  // the end; the start is subtracted below
      e_prev = e;
    }
  }
  __syncthreads();
  {
    // padded length of each expert's region
    int len = 0;
    if (tid < E) {
      s_sexp[tid] -= s_g0[tid];
      len = round_up_i(s_sexp[tid], block_m);
    }
    int eo, d0, tot, d1;
    block_excl_scan2(len, 0, eo, d0, tot, d1, s_red);
    if (tid < E) s_off[tid] = eo;
    if (tid == 0) s_off[E] = tot;
  }
  __syncthreads();
  {
    int g = gex;
    for (int sg = slo; sg < shi; ++sg) {
      const int i0 = seg_lo[sg], c = seg_lo[sg + 1] - i0;
      const int kk = key[sorted[i0]];
      const int e = kk / nb1;
      const int st = s_off[e] + g - s_g0[e];
      int* row = a.seg_table + 4 * sg;
      row[0] = e;
      row[1] = kk - e * nb1 - 1;
      row[2] = st;
      row[3] = c;
      // row blocks whose first row lies in this segment (with its padding) start at it
      if (a.block_seg)
        for (int bb = (st + block_m - 1) / block_m; bb * block_m < st + pad_to(c); ++bb)
          a.block_seg[bb] = sg;
      delta[sg] = st - i0;
      g += pad_to(c);
    }
  }
  for (int e = tid; e <= E; e += bd) a.expert_offsets[e] = s_off[e];
  if (tid == 0) {
    *a.n_seg = nseg;
    *a.flags = (fl_nonfinite ? 1 : 0) | (fl_range ? 2 : 0);
    if (a.n_blocks) *a.n_blocks = s_off[E] / block_m;
  }
  __syncthreads();

  // phase 3
  if (seg_pad > 1)
    for (int sg = tid; sg < nseg; sg += bd) {
      const int i0 = seg_lo[sg], c = seg_lo[sg + 1] - i0;
      const int st = i0 + delta[sg];
      for (int q = st + c; q < st + pad_to(c); ++q) {
        a.sorted_pairs[q] = -1;
        if (a.sorted_ad) a.sorted_ad[q] = -1;
      }
    }
  for (int e = wave; e < E; e += nwaves) {
    for (int q = s_off[e] + s_sexp[e] + lane; q < s_off[e + 1]; q += 64) {
      a.sorted_pairs[q] = -1;
      if (a.sorted_ad) a.sorted_ad[q] = -1;
    }
    if (a.block_expert)
      for (int bb = s_off[e] / block_m + lane; bb < s_off[e + 1] / block_m; bb += 64) {
        a.block_expert[bb] = e;
        // a block that starts on a padding row holds padding rows only
        if (a.block_seg && bb * block_m >= s_off[e] + s_sexp[e]) a.block_seg[bb] = -1;
      }
  }
  for (int i = tid; i < P; i += bd) {
    const int p = sorted[i];
    const int pos = i + delta[sid[i]];
    a.sorted_pairs[pos] = p;
    if (a.pair_row) a.pair_row[p] = pos;
    if (a.sorted_ad) a.sorted_ad[pos] = key[p] % nb1 - 1;
  }
}

// ------------------------------------------------------------------------------------------
// Router logits, logits[t][e] = sum_c x[t][c] W_router[e][c] in fp32 (page "vLLM MoE LoRA
// SageMaker Bedrock", section "Entendendo os Modelos MoE": the router scores every expert for
// each token). One workgroup per (16 tokens, 16 experts): 16x16x32 bf16 MFMAs with the router
// rows on the A side and the token rows on the B side. The product is latency-bound (a decode
// batch is a handful of tiles), so the workgroup's sixteen wavefronts take the 32-wide K chunks
// in turn (chunk c to wavefront c % 16) and each issues the loads of up to eight of its chunks
// before their MFMAs: K = 4096 costs one memory round trip. The sixteen partial tiles are added
// in wavefront order through LDS. Token rows past T and expert rows past E load zeros and are
// not stored.
// ------------------------------------------------------------------------------------------
constexpr int kRouterWaves = 16;

__global__ __launch_bounds__(64 * kRouterWaves) void router_logits_kernel(
    const uint16_t* __restrict__ x, uint32_t x_bytes, const uint16_t* __restrict__ W,
    uint32_t w_bytes, int T, int K, int E, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, kq = lane >> 4;
  const int tok = blockIdx.x * 16 + m, erow = blockIdx.y * 16 + m;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, x_bytes), wr = make_rsrc(W, w_bytes);
  const uint32_t xo = tok < T ? (uint32_t)((size_t)tok * K * 2) : kOutOfRange;
  const uint32_t wo = erow < E ? (uint32_t)((size_t)erow * K * 2) : kOutOfRange;
  const int nch = K / 32;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int c = wave;
  for (; c + kRouterWaves * 7 < nch; c += kRouterWaves * 8) {
    u32x4 xa[8], wa[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t kk = (uint32_t)((c + kRouterWaves * j) * 32 + 8 * kq) * 2;
      xa[j] = bufld16(xr, xo + kk);
      wa[j] = bufld16(wr, wo + kk);
    }
    __builtin_amdgcn_sched_barrier(0);  // all sixteen loads in flight before the first MFMA
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = mfma16(wa[j], xa[j], acc);
  }
  for (; c < nch; c += kRouterWaves) {
    const uint32_t kk = (uint32_t)(c * 32 + 8 * kq) * 2;
    acc = mfma16(bufld16(wr, wo + kk), bufld16(xr, xo + kk), acc);
  }
  // acc[v]: expert blockIdx.y*16 + 4 kq + v, token blockIdx.x*16 + m
  __shared__ f32x4 s_part[kRouterWaves][64];
  s_part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 t = s_part[0][lane];
#pragma unroll
    for (int w = 1; w < kRouterWaves; ++w) t += s_part[w][lane];
    if (tok < T) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int e = blockIdx.y * 16 + 4 * kq + v;
        if (e < E) logits[(size_t)tok * E + e] = t[v];
      }
    }
  }
}

}  // namespace moelora

namespace moelora {

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* W, int T, int K, int E,
                                float* logits, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  if (K % 128 != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((T + 15) / 16), (unsigned)((E + 15) / 16));
  hipLaunchKernelGGL(router_logits_kernel, grid, dim3(64 * kRouterWaves), 0, stream, x,
                     (uint32_t)((size_t)T * K * 2), W, (uint32_t)((size_t)E * K * 2), T, K, E,
                     logits);
  return hipGetLastError();
}

hipError_t launch_route(const float* logits, int T, int E, int k, int* topk_ids, float* topk_w,
                        int* tok_flags, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const dim3 grid((T + 3) / 4), block(256);
  const dim3 grid1((unsigned)T);  // above 64 experts: one token per workgroup
  if (E <= 64)
    hipLaunchKernelGGL(route_rank_kernel<1>, grid, block, 0, stream, logits, T, E, k, topk_ids,
                       topk_w, tok_flags);
  else if (E <= 128)
    hipLaunchKernelGGL(route_rank_kernel<2>, grid1, block, 0, stream, logits, T, E, k, topk_ids,
                       topk_w, tok_flags);
  else if (E <= 256)
    hipLaunchKernelGGL(route_rank_kernel<4>, grid1, block, 0, stream, logits, T, E, k, topk_ids,
                       topk_w, tok_flags);
  else
    hipLaunchKernelGGL(route_topk_kernel, grid, block, 0, stream, logits, T, E, k, topk_ids,
                       topk_w, tok_flags);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Adapter segments of a dense multi-LoRA batch (one projection, no experts) for up to 1024 tokens
// and 1024 adapters: one workgroup, one token per thread. The tokens that carry an adapter are
// sorted by (adapter, token): a token's rank among the equal adapters of earlier lanes of its
// wavefront comes from a ballot match, the per-(adapter, wavefront) counts are scanned in
// adapter-major order, and each token lands at its adapter's offset plus its rank. The layout
// is padded to 16-row blocks with -1 (block -> expert 0). Tokens without an adapter, or with one
// out of range (flagged), are left out: nothing of the multi-LoRA add applies to them.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void sgmv_sort_kernel(SgmvSortArgs a) {
  extern __shared__ int cnt[];  // [nA][16]: count, then offset, of adapter x wavefront
  __shared__ int s_red[72];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nA = a.nA, n_ent = nA * 16;
  for (int i = tid; i < n_ent; i += 1024) cnt[i] = 0;
  int ad = -1;
  bool bad = false;
  if (tid < a.T) {
    ad = a.adapter_ids[tid];
    if (ad < -1 || ad >= nA) {
      bad = true;
      ad = -1;
    }
  }
  const bool member = ad >= 0;
  int nbits = 1;
  while ((1 << nbits) < nA) ++nbits;
  const uint64_t eq = match_key(member, member ? ad : 0, nbits);
  const int rank = (int)__popcll(eq & lanemask_lt());
  const int any_bad = __syncthreads_or(bad);
  if (member && rank == 0) cnt[ad * 16 + wave] = (int)__popcll(eq);
  __syncthreads();
  // exclusive scan of the entries in (adapter, wavefront) order, per = entries per thread
  const int per = (n_ent + 1023) / 1024;
  const int e0 = tid * per;
  int local = 0;
  for (int j = 0; j < per; ++j)
    if (e0 + j < n_ent) local += cnt[e0 + j];
  int ex, d0, total, d1;
  block_excl_scan2(local, 0, ex, d0, total, d1, s_red);
  for (int j = 0; j < per; ++j)
    if (e0 + j < n_ent) {
      const int v = cnt[e0 + j];
      cnt[e0 + j] = ex;
      ex += v;
    }
  __syncthreads();
  if (member) {
    const int pos = cnt[ad * 16 + wave] + rank;
    a.sorted_pairs[pos] = tid;
    a.sorted_ad[pos] = ad;
  }
  const int padded = round_up_i(total, 16);
  for (int q = total + tid; q < padded; q += 1024) {
    a.sorted_pairs[q] = -1;
    a.sorted_ad[q] = -1;
  }
  for (int b = tid; b < padded / 16; b += 1024) a.block_expert[b] = 0;
  if (tid == 0) {
    *a.n_blocks = padded / 16;
    *a.flags = any_bad ? 2 : 0;
  }
}

hipError_t launch_sgmv_sort(const SgmvSortArgs& a, hipStream_t stream) {
  if (a.T < 0 || a.T > kSgmvSortMaxTokens || a.nA < 1 || a.nA > kSgmvSortMaxAdapters)
    return hipErrorInvalidValue;
  static bool attr_set[64] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    err = hipFuncSetAttribute((const void*)sgmv_sort_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)sizeof(int) * 16 * kSgmvSortMaxAdapters);
    if (err != hipSuccess) return err;
    attr_set[dev] = true;
  }
  hipLaunchKernelGGL(sgmv_sort_kernel, dim3(1), dim3(1024), sizeof(int) * 16 * a.nA, stream, a);
  return hipGetLastError();
}

hipError_t launch_align(const AlignArgs& a, size_t dyn_lds, hipStream_t stream) {
  static bool attr_set[64] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    err = hipFuncSetAttribute((const void*)align_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              kLdsBytes - kAlignStaticLds);
    if (err != hipSuccess) return err;
    attr_set[dev] = true;
  }
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kAlignThreads), dyn_lds, stream, a);
  return hipGetLastError();
}

}  // namespace moelora
