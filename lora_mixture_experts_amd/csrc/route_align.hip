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
// selection as k rounds of arg-max. The wavefront stages the token's logits in LDS and every lane
// counts, for its (up to VPL) logits, how many of the E staged ones beat it: broadcast reads, no
// cross-lane reductions. Non-finite logits are flagged and take part as -infinity.
template <int VPL>
__global__ __launch_bounds__(256) void route_rank_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int* __restrict__ topk_ids,
                                                         float* __restrict__ topk_w,
                                                         int* __restrict__ tok_flags) {
  __shared__ __attribute__((aligned(16))) float s_l[4][64 * VPL];
  __shared__ float s_sel[4][kMaxTopk];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + w;
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
    s_l[w][e] = f;  // (slots past E hold -infinity and are never counted)
  }
  __syncthreads();
  int rank[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) rank[i] = 0;
  const int e4 = (E + 3) & ~3;
  for (int c = 0; c < e4; c += 4) {
    const f32x4 o = *reinterpret_cast<const f32x4*>(&s_l[w][c]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int eo = c + j;
      if (eo >= E) break;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = lane + 64 * i;
        rank[i] += (o[j] > v[i] || (o[j] == v[i] && eo < e)) ? 1 : 0;
      }
    }
  }
  const uint64_t anybad = __ballot(bad);
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    if (active && e < E && rank[i] < k) {
      topk_ids[(size_t)t * k + rank[i]] = e;
      s_sel[w][rank[i]] = v[i];
    }
  }
  __syncthreads();
  if (active && lane == 0) {
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
// Align: one workgroup of 1024 threads.
//   phase 0  validate adapter ids (out of range -> flag, treated as -1), collect flags, stage
//   phase A  per-expert pair lists in token order: each wavefront ranks its slice of pairs by
//            expert (stable), an (expert, wavefront) scan turns the ranks into positions
//   phase D  count pairs per bucket b = e*(nA+1) + (a+1), one wavefront per expert list
//   phase 2  exclusive scans: padded segment starts, expert offsets, segment table
//   phase 3  padding slots (-1) and the row-block -> expert (and first segment) tables
//   phase 4  scatter pair ids (and each pair's row); inside a bucket pairs keep token order
// Within a wavefront, lanes with equal key are found by one ballot per key bit, so the rank of
// a pair among equal-key pairs of earlier lanes is an exact popcount. Every table lives in LDS
// when it fits and in the workspace otherwise.
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

// Exclusive scan of (v0, v1) over the workgroup; red needs 2*32+2 ints.
__device__ void block_excl_scan2(int v0, int v1, int& ex0, int& ex1, int& tot0, int& tot1,
                                 int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int i0 = v0, i1 = v1;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int a0 = __shfl_up(i0, off);
    const int a1 = __shfl_up(i1, off);
    if (lane >= off) {
      i0 += a0;
      i1 += a1;
    }
  }
  if (lane == 63) {
    red[wave] = i0;
    red[32 + wave] = i1;
  }
  __syncthreads();
  if (wave == 0) {
    const int w0 = lane < nw ? red[lane] : 0;
    const int w1 = lane < nw ? red[32 + lane] : 0;
    int s0 = w0, s1 = w1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int a0 = __shfl_up(s0, off);
      const int a1 = __shfl_up(s1, off);
      if (lane >= off) {
        s0 += a0;
        s1 += a1;
      }
    }
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
  __shared__ int s_ebase[kMaxExperts];
  __shared__ int s_sexp[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_estart[kMaxExperts + 1];
  __shared__ int s_red[72];

  constexpr int nwaves = kAlignThreads / 64, bd = kAlignThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, k = a.k, E = a.E, nA = a.nA, P = T * k;
  const int nb1 = nA + 1, nb = E * nb1;
  const int seg_pad = a.seg_pad, block_m = a.block_m;
  // p / k as a multiply by ceil(2^32 / k) and a shift: exact for p * k < 2^32
  const uint64_t k_magic = ((1ull << 32) + k - 1) / k;
  auto token_of = [&](int p) { return (int)(((uint64_t)(uint32_t)p * k_magic) >> 32); };
  auto pad_to = [&](int c) { return seg_pad == 1 ? c : round_up_i(c, seg_pad); };

  // carve LDS (or the workspace): lists elist [P] and ad [T]; the rank scratch tk [P],
  // rank [P], cnt_we [nwaves][E]; tables cnt/start [nb]. With everything in LDS the tables
  // overlay the rank scratch, which is dead once the expert lists are built.
  int *elist, *adl, *tk, *rank, *cnt_we, *cnt, *start;
  {
    int* dyn = smem;
    if (a.tables_in_lds && a.lists_in_lds) {
      elist = dyn;
      adl = elist + P;
      tk = adl + T;
      cnt = tk;
    } else {
      if (a.tables_in_lds) {
        cnt = dyn;
        dyn += 2 * nb;
      } else {
        cnt = a.g_cnt;
      }
      elist = a.lists_in_lds ? dyn : a.g_lists;
      adl = elist + P;
      tk = adl + T;
    }
    rank = tk + P;
    cnt_we = rank + P;
    start = a.tables_in_lds ? cnt + nb : a.g_start;
  }

  // phase 0
  int fl_nonfinite = 0, fl_range = 0;
  for (int i = tid; i < nwaves * E; i += bd) cnt_we[i] = 0;
  for (int i = tid; i < P; i += bd) tk[i] = a.topk_ids[i];
  for (int t = tid; t < T; t += bd) {
    int av = a.adapter_ids[t];
    if (av < -1 || av >= nA) {
      fl_range = 1;
      av = -1;
    }
    if (a.tok_flags[t]) fl_nonfinite = 1;
    adl[t] = av;
  }
  fl_nonfinite = __syncthreads_or(fl_nonfinite);
  fl_range = __syncthreads_or(fl_range);

  // phase A: stable rank of each pair among the pairs of its expert in this wavefront's slice
  const int ebits = E > 1 ? 32 - __clz(E - 1) : 0;
  const int PP = (P + nwaves - 1) / nwaves;
  {
    const int p0 = wave * PP, p1 = min(P, p0 + PP);
    for (int base = p0; base < p1; base += 64) {
      const int p = base + lane;
      const bool valid = p < p1;
      const int e = valid ? tk[p] : 0;
      const uint64_t eq = match_key(valid, e, ebits);
      int c = 0;
      if (valid && (eq & lanemask_lt()) == 0ull) c = atomicAdd(&cnt_we[wave * E + e], (int)__popcll(eq));
      const int src = valid ? (__ffsll((unsigned long long)eq) - 1) : lane;
      c = __shfl(c, src);
      if (valid) rank[p] = c + (int)__popcll(eq & lanemask_lt());
    }
  }
  __syncthreads();
  // exclusive scan of cnt_we in (expert, wavefront) order; expert e's list starts at s_estart[e]
  {
    const int n = nwaves * E;
    const int per_t = (n + bd - 1) / bd;
    const int lo = min(n, tid * per_t), hi = min(n, lo + per_t);
    int sv = 0;
    for (int i = lo; i < hi; ++i) sv += cnt_we[(i % nwaves) * E + i / nwaves];
    int ex, d0, tot, d1;
    block_excl_scan2(sv, 0, ex, d0, tot, d1, s_red);
    int run = ex;
    for (int i = lo; i < hi; ++i) {
      const int idx = (i % nwaves) * E + i / nwaves;
      const int c = cnt_we[idx];
      if (i % nwaves == 0) s_estart[i / nwaves] = run;
      cnt_we[idx] = run;
      run += c;
    }
    if (tid == 0) s_estart[E] = P;
  }
  __syncthreads();
  {
    const int p0 = wave * PP, p1 = min(P, p0 + PP);
    for (int p = p0 + lane; p < p1; p += 64) elist[cnt_we[wave * E + tk[p]] + rank[p]] = p;
  }
  __syncthreads();
  // (the rank scratch is dead from here on; the tables may overlay it)
  for (int i = tid; i < nb; i += bd) cnt[i] = 0;
  __syncthreads();

  const int nbits = 32 - __clz(nA);  // bits of a key in [0, nA]

  // phase D: counts per (expert, adapter) bucket over each expert's list
  for (int e = wave; e < E; e += nwaves) {
    const int i1 = s_estart[e + 1];
    for (int base = s_estart[e]; base < i1; base += 64) {
      const int i = base + lane;
      const bool valid = i < i1;
      const int key = valid ? adl[token_of(elist[i])] + 1 : 0;
      const uint64_t eq = match_key(valid, key, nbits);
      if (valid && (eq & lanemask_lt()) == 0ull) atomicAdd(&cnt[e * nb1 + key], (int)__popcll(eq));
    }
  }
  __syncthreads();

  // phase 2
  const int per = (nb + bd - 1) / bd;
  const int lo = min(nb, tid * per), hi = min(nb, lo + per);
  int sv = 0, sn = 0;
  for (int b = lo; b < hi; ++b) {
    const int c = cnt[b];
    sv += pad_to(c);
    sn += c > 0;
  }
  int ev, en, totv, totn;
  block_excl_scan2(sv, sn, ev, en, totv, totn, s_red);
  {
    int run = ev;
    for (int b = lo; b < hi; ++b) {
      start[b] = run;
      run += pad_to(cnt[b]);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += bd) {
    const int s0 = start[e * nb1];
    const int s1 = (e + 1 < E) ? start[(e + 1) * nb1] : totv;
    s_ebase[e] = s0;
    s_sexp[e] = s1 - s0;
  }
  __syncthreads();
  {
    const int len = (tid < E) ? round_up_i(s_sexp[tid], block_m) : 0;
    int eo, dummy_ex, tot, dummy_tot;
    block_excl_scan2(len, 0, eo, dummy_ex, tot, dummy_tot, s_red);
    if (tid < E) s_off[tid] = eo;
    if (tid == 0) s_off[E] = tot;
  }
  __syncthreads();
  {
    int nz = en;
    for (int b = lo; b < hi; ++b) {
      const int e = b / nb1;
      const int c = cnt[b];
      const int st = s_off[e] + start[b] - s_ebase[e];
      start[b] = st;
      if (c > 0) {
        int* row = a.seg_table + 4 * nz;
        row[0] = e;
        row[1] = (b - e * nb1) - 1;
        row[2] = st;
        row[3] = c;
        // row blocks whose first row lies in this segment (with its padding) start at it
        if (a.block_seg)
          for (int bb = (st + block_m - 1) / block_m; bb * block_m < st + round_up_i(c, seg_pad);
               ++bb)
            a.block_seg[bb] = nz;
        ++nz;
      }
    }
  }
  for (int e = tid; e <= E; e += bd) a.expert_offsets[e] = s_off[e];
  if (tid == 0) {
    *a.n_seg = totn;
    *a.flags = (fl_nonfinite ? 1 : 0) | (fl_range ? 2 : 0);
    if (a.n_blocks) *a.n_blocks = s_off[E] / block_m;
  }
  __syncthreads();

  // phase 3
  for (int e = wave; e < E; e += nwaves) {
    const int b0 = e * nb1;
    if (seg_pad > 1) {
      for (int q = lane; q < nb1; q += 64) {
        const int c = cnt[b0 + q];
        if (c > 0) {
          const int st = start[b0 + q];
          for (int s = st + c; s < st + round_up_i(c, seg_pad); ++s) a.sorted_pairs[s] = -1;
        }
      }
    }
    for (int s = s_off[e] + s_sexp[e] + lane; s < s_off[e + 1]; s += 64) a.sorted_pairs[s] = -1;
    if (a.block_expert)
      for (int bb = s_off[e] / block_m + lane; bb < s_off[e + 1] / block_m; bb += 64) {
        a.block_expert[bb] = e;
        // a block that starts on a padding row holds padding rows only
        if (a.block_seg && bb * block_m >= s_off[e] + s_sexp[e]) a.block_seg[bb] = -1;
      }
  }
  __syncthreads();
  for (int i = tid; i < nb; i += bd) cnt[i] = 0;
  __syncthreads();

  // phase 4
  for (int e = wave; e < E; e += nwaves) {
    const int i1 = s_estart[e + 1];
    for (int base = s_estart[e]; base < i1; base += 64) {
      const int i = base + lane;
      const bool valid = i < i1;
      const int p = valid ? elist[i] : 0;
      const int key = valid ? adl[token_of(p)] + 1 : 0;
      const uint64_t eq = match_key(valid, key, nbits);
      int cur = 0;
      if (valid && (eq & lanemask_lt()) == 0ull) cur = atomicAdd(&cnt[e * nb1 + key], (int)__popcll(eq));
      const int src = valid ? (__ffsll((unsigned long long)eq) - 1) : lane;
      cur = __shfl(cur, src);
      if (valid) {
        const int pos = start[e * nb1 + key] + cur + (int)__popcll(eq & lanemask_lt());
        a.sorted_pairs[pos] = p;
        if (a.pair_row) a.pair_row[p] = pos;
      }
    }
  }
}

}  // namespace moelora

namespace moelora {

hipError_t launch_route(const float* logits, int T, int E, int k, int* topk_ids, float* topk_w,
                        int* tok_flags, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(route_rank_kernel<1>, grid, block, 0, stream, logits, T, E, k, topk_ids,
                       topk_w, tok_flags);
  else if (E <= 128)
    hipLaunchKernelGGL(route_rank_kernel<2>, grid, block, 0, stream, logits, T, E, k, topk_ids,
                       topk_w, tok_flags);
  else if (E <= 256)
    hipLaunchKernelGGL(route_rank_kernel<4>, grid, block, 0, stream, logits, T, E, k, topk_ids,
                       topk_w, tok_flags);
  else
    hipLaunchKernelGGL(route_topk_kernel, grid, block, 0, stream, logits, T, E, k, topk_ids,
                       topk_w, tok_flags);
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
