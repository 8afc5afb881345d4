/*
 * CPU oracle for the fused MoE + multi-LoRA layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load this file:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg use it. It shares no
 * code with the HIP library.
 *
 * What it computes is the plain definition, in float64, with no intermediate rounding.
 * Inputs are read as stored (bf16, f32 or f64) and widened exactly to float64.
 *
 * Sources (the web pages the method is described on):
 *  - "vLLM MoE LoRA SageMaker Bedrock" (cloudtroop), section "Entendendo os Modelos MoE":
 *    a router sends each token to its most relevant experts and their outputs are
 *    aggregated; each expert is a gate_up projection h -> intermediate followed by a down
 *    projection back to h.
 *  - same page, section "O Papel da Multi-LoRA": for base weights W (h_in x h_out), LoRA adds
 *    A (h_in x r) and B (r x h_out), y = xW + xAB; the shrink computes z = xA, the expand
 *    multiplies z by B; four such operations per expert, adapter and request.
 *  - "Punica: Multi-Tenant LoRA Serving" (nubint review), sections on the proposed method:
 *    one copy of the base model serves a batch whose tokens carry different adapters.
 *
 * Conventions where the pages are silent (each is a reading, not a page fact):
 *  - routing weights are the softmax over the k selected logits; ties go to the lower expert
 *    id; slots are in descending logit order;
 *  - W1 stores [gate; up] (rows 0..I-1 gate, I..2I-1 up); act = silu(gate) * up with the exact
 *    logistic function;
 *  - LoRA scale 1; one (A1, B1) pair per (adapter, expert) for gate_up and one (A2, B2) for
 *    down; the down LoRA acts on act; adapter id -1 means "no adapter";
 *  - no capacity limit, biases or shared experts.
 *
 * Stored layouts (out x in, K contiguous; the pages' math matrices are the transposes):
 *  x[T][h], logits[T][E] f32, W1[E][2I][h], W2[E][h][I], A1[nA][E][r][h], B1[nA][E][2I][r],
 *  A2[nA][E][r][I], B2[nA][E][h][r], adapter_ids[T].
 *
 * FP8 expert weights (page "AWS SageMaker MoE kernel optimizations", third paragraph: FP8
 * expert weights whose scales are applied between the routing and the expert GEMMs): W1 and
 * W2 may be stored as 8-bit E4M3 codes (the OCP 8-bit floating point format: 1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN) with one
 * float32 scale per output row (channel): W[e][n][c] = decode(code[e][n][c]) * scale[e][n]
 * (a reading: the page names FP8 and scales, not their granularity).
 *
 * Pins (tests/test_oracle_pins.py): brute-force top-k against Python's sort, the full softmax
 * at k = E, the merged-weight form x(W + AB), B = 0 reducing to plain MoE, one adapter for all
 * tokens matching per-token evaluation, E = 1 against numpy matmul, a hand-worked example
 * (tests/golden/), and exact properties of the align layout.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BF16 0
#define ORC_F32 1
#define ORC_F64 2
#define ORC_FP8E4M3 3 /* uint8 E4M3 codes; weights only, with per-row scales */

#define ORC_OK 0
#define ORC_EINVAL -1
#define ORC_ENONFINITE -2
#define ORC_EADAPTER -3
#define ORC_ENOMEM -4

typedef struct {
  int32_t T, hidden, inter, n_experts, n_adapters, rank, topk;
} orc_dims;

static double bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP E4M3: (-1)^s * 2^(e-7) * (1 + m/8) for e > 0, (-1)^s * 2^-6 * (m/8) for e = 0; NaN for
 * e = 15, m = 7 (the largest finite magnitude is 448). Exact in float64. */
static double fp8e4m3_to_f64(uint8_t b) {
  const int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m / 8.0, -6);
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* Element i of a stored tensor, widened exactly to float64. */
static double ld(const void *p, int dt, size_t i) {
  if (dt == ORC_BF16) return bf16_to_f64(((const uint16_t *)p)[i]);
  if (dt == ORC_F32) return (double)((const float *)p)[i];
  if (dt == ORC_FP8E4M3) return fp8e4m3_to_f64(((const uint8_t *)p)[i]);
  return ((const double *)p)[i];
}

/* sum_c v[c] * M[off + c], c < len, in order c = 0, 1, ... */
static double dot_row(const double *v, const void *M, int dt, size_t off, int len) {
  double s = 0.0;
  if (dt == ORC_BF16) {
    const uint16_t *m = (const uint16_t *)M + off;
    for (int c = 0; c < len; ++c) s += v[c] * bf16_to_f64(m[c]);
  } else if (dt == ORC_F32) {
    const float *m = (const float *)M + off;
    for (int c = 0; c < len; ++c) s += v[c] * (double)m[c];
  } else if (dt == ORC_FP8E4M3) {
    const uint8_t *m = (const uint8_t *)M + off;
    for (int c = 0; c < len; ++c) s += v[c] * fp8e4m3_to_f64(m[c]);
  } else {
    const double *m = (const double *)M + off;
    for (int c = 0; c < len; ++c) s += v[c] * m[c];
  }
  return s;
}

/* ------------------------------------------------------------------------------------------
 * Route. Expert e' beats e when its logit is larger, or equal with a lower id. The rank of e
 * is the number of experts that beat it; e is selected iff rank < k and takes slot = rank.
 * The weights are the softmax over the selected logits.
 * ------------------------------------------------------------------------------------------ */
static int beats(const float *row, int a, int b) {
  return row[a] > row[b] || (row[a] == row[b] && a < b);
}

int oracle_route(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *topk_ids,
                 double *topk_w) {
  if (T < 0 || E <= 0 || k <= 0 || k > E) return ORC_EINVAL;
  for (int32_t t = 0; t < T; ++t) {
    const float *row = logits + (size_t)t * E;
    for (int32_t e = 0; e < E; ++e)
      if (!isfinite(row[e])) return ORC_ENONFINITE;
    for (int32_t e = 0; e < E; ++e) {
      int32_t rank = 0;
      for (int32_t o = 0; o < E; ++o)
        if (o != e && beats(row, o, e)) ++rank;
      if (rank < k) topk_ids[(size_t)t * k + rank] = e;
    }
    if (topk_w) {
      double top = row[topk_ids[(size_t)t * k]];
      double den = 0.0;
      for (int32_t j = 0; j < k; ++j) den += exp((double)row[topk_ids[(size_t)t * k + j]] - top);
      for (int32_t j = 0; j < k; ++j)
        topk_w[(size_t)t * k + j] = exp((double)row[topk_ids[(size_t)t * k + j]] - top) / den;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------------
 * Align. Pair p = t*k + j goes to expert e_p = topk_ids[p] with the token's adapter
 * a_p = adapter_ids[t]. Pairs are sorted by the key (e_p, a_p, t), ascending (a = -1 first);
 * the key is unique because a token never holds one expert twice.
 * Segments are the maximal runs of equal (e, a). In the padded layout each segment's length
 * is rounded up to a multiple of seg_pad, then each expert's block to a multiple of block_m;
 * padding slots hold -1. expert_offsets[e] is the padded start of expert e's block and
 * expert_offsets[E] the padded total. seg_table rows are (e, a, padded start, real count).
 * ------------------------------------------------------------------------------------------ */
typedef struct {
  int32_t e, a, t, p;
} orc_key;

static int key_cmp(const void *x, const void *y) {
  const orc_key *u = (const orc_key *)x, *v = (const orc_key *)y;
  if (u->e != v->e) return u->e < v->e ? -1 : 1;
  if (u->a != v->a) return u->a < v->a ? -1 : 1;
  if (u->t != v->t) return u->t < v->t ? -1 : 1;
  return 0;
}

static int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

int oracle_align(const int32_t *topk_ids, const int32_t *adapter_ids, int32_t T, int32_t k,
                 int32_t E, int32_t nA, int32_t seg_pad, int32_t block_m, int32_t *sorted_pairs,
                 int64_t sorted_cap, int32_t *expert_offsets, int32_t *seg_table, int32_t seg_cap,
                 int32_t *n_seg) {
  if (T < 0 || k <= 0 || E <= 0 || nA <= 0 || seg_pad <= 0 || block_m <= 0) return ORC_EINVAL;
  size_t P = (size_t)T * k;
  for (size_t p = 0; p < P; ++p)
    if (topk_ids[p] < 0 || topk_ids[p] >= E) return ORC_EINVAL;
  for (int32_t t = 0; t < T; ++t)
    if (adapter_ids[t] < -1 || adapter_ids[t] >= nA) return ORC_EADAPTER;

  orc_key *keys = (orc_key *)malloc(sizeof(orc_key) * (P ? P : 1));
  if (!keys) return ORC_ENOMEM;
  for (size_t p = 0; p < P; ++p) {
    keys[p].e = topk_ids[p];
    keys[p].a = adapter_ids[p / k];
    keys[p].t = (int32_t)(p / k);
    keys[p].p = (int32_t)p;
  }
  qsort(keys, P, sizeof(orc_key), key_cmp);

  for (int64_t i = 0; i < sorted_cap; ++i) sorted_pairs[i] = -1;
  int64_t pos = 0;
  int32_t ns = 0;
  size_t i = 0;
  for (int32_t e = 0; e < E; ++e) {
    expert_offsets[e] = (int32_t)pos;
    int64_t start_e = pos;
    while (i < P && keys[i].e == e) {
      size_t j = i;
      while (j < P && keys[j].e == e && keys[j].a == keys[i].a) ++j;
      int64_t cnt = (int64_t)(j - i);
      if (pos + cnt > sorted_cap || ns >= seg_cap) {
        free(keys);
        return ORC_EINVAL;
      }
      seg_table[4 * ns + 0] = e;
      seg_table[4 * ns + 1] = keys[i].a;
      seg_table[4 * ns + 2] = (int32_t)pos;
      seg_table[4 * ns + 3] = (int32_t)cnt;
      ++ns;
      for (size_t q = i; q < j; ++q) sorted_pairs[pos + (int64_t)(q - i)] = keys[q].p;
      pos += round_up(cnt, seg_pad);
      i = j;
    }
    pos = start_e + round_up(pos - start_e, block_m);
    if (pos > sorted_cap) {
      free(keys);
      return ORC_EINVAL;
    }
  }
  expert_offsets[E] = (int32_t)pos;
  *n_seg = ns;
  free(keys);
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------------
 * Forward. For each requested token t and slot j (expert e = sel_j, adapter a = adapter_ids[t]):
 *   z1[q]  = sum_c x[t][c] A1[a][e][q][c]                         (LoRA shrink, gate_up)
 *   g[n]   = sum_c x[t][c] W1[e][n][c] + sum_q z1[q] B1[a][e][n][q] (base + LoRA expand), n < 2I
 *   act[i] = silu(g[i]) * g[I+i],  silu(v) = v / (1 + exp(-v))
 *   z2[q]  = sum_i act[i] A2[a][e][q][i]                          (LoRA shrink, down)
 *   d[m]   = sum_i act[i] W2[e][m][i] + sum_q z2[q] B2[a][e][m][q]
 *   y[t][m] = sum_j w[t][j] d_j[m], in slot order.
 * With a = -1 the z terms are zero.
 * t[] holds the tensors in the order x, W1, W2, A1, B1, A2, B2 and dt[] their dtypes.
 * oracle_forward_scaled also takes the per-row scales of W1 [E][2I] and W2 [E][h] (float32),
 * required when that weight is stored as E4M3 codes (NULL otherwise): the row's sum is the
 * sum over the decoded codes times the row's scale.
 * tokens/n_tokens select the output rows (NULL: all T tokens, in order). y is
 * [n_tokens][h]; d_pairs, when not NULL, receives the per-slot expert outputs
 * [n_tokens][k][h].
 * ------------------------------------------------------------------------------------------ */
static double silu(double v) { return v / (1.0 + exp(-v)); }

int oracle_forward_scaled(const orc_dims *d, const void *const *t, const int32_t *dt,
                          const float *w1_scale, const float *w2_scale, const float *logits,
                          const int32_t *adapter_ids, const int32_t *tokens, int32_t n_tokens,
                          double *y, double *d_pairs) {
  const int32_t T = d->T, h = d->hidden, I = d->inter, E = d->n_experts, nA = d->n_adapters,
                r = d->rank, k = d->topk;
  if (T < 0 || h <= 0 || I <= 0 || E <= 0 || nA <= 0 || r <= 0 || k <= 0 || k > E)
    return ORC_EINVAL;
  const void *x = t[0], *W1 = t[1], *W2 = t[2], *A1 = t[3], *B1 = t[4], *A2 = t[5], *B2 = t[6];
  const int dx = dt[0], dW1 = dt[1], dW2 = dt[2], dA1 = dt[3], dB1 = dt[4], dA2 = dt[5],
            dB2 = dt[6];
  for (int i = 0; i < 7; ++i)
    if (dt[i] == ORC_FP8E4M3 && i != 1 && i != 2) return ORC_EINVAL;
  if ((dW1 == ORC_FP8E4M3) != (w1_scale != NULL) || (dW2 == ORC_FP8E4M3) != (w2_scale != NULL))
    return ORC_EINVAL;
  int32_t n = tokens ? n_tokens : T;
  for (int32_t i = 0; i < n; ++i) {
    int32_t tok = tokens ? tokens[i] : i;
    if (tok < 0 || tok >= T) return ORC_EINVAL;
    if (adapter_ids[tok] < -1 || adapter_ids[tok] >= nA) return ORC_EADAPTER;
    for (int32_t e = 0; e < E; ++e)
      if (!isfinite(logits[(size_t)tok * E + e])) return ORC_ENONFINITE;
  }

  int status = ORC_OK;
#pragma omp parallel
  {
    double *xr = (double *)malloc(sizeof(double) * (size_t)h);
    double *g = (double *)malloc(sizeof(double) * 2 * (size_t)I);
    double *act = (double *)malloc(sizeof(double) * (size_t)I);
    double *z1 = (double *)malloc(sizeof(double) * (size_t)r);
    double *z2 = (double *)malloc(sizeof(double) * (size_t)r);
    double *dv = (double *)malloc(sizeof(double) * (size_t)h);
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    double *w = (double *)malloc(sizeof(double) * (size_t)k);
    if (!xr || !g || !act || !z1 || !z2 || !dv || !sel || !w) {
#pragma omp atomic write
      status = ORC_ENOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int32_t i = 0; i < n; ++i) {
        const int32_t tok = tokens ? tokens[i] : i;
        const int32_t a = adapter_ids[tok];
        oracle_route(logits + (size_t)tok * E, 1, E, k, sel, w);
        for (int32_t c = 0; c < h; ++c) xr[c] = ld(x, dx, (size_t)tok * h + c);
        double *yrow = y + (size_t)i * h;
        for (int32_t m = 0; m < h; ++m) yrow[m] = 0.0;
        for (int32_t j = 0; j < k; ++j) {
          const int32_t e = sel[j];
          /* gate_up: shrink, base, expand */
          if (a >= 0) {
            for (int32_t q = 0; q < r; ++q)
              z1[q] = dot_row(xr, A1, dA1, (((size_t)a * E + e) * r + q) * h, h);
          }
          for (int32_t nn = 0; nn < 2 * I; ++nn) {
            double v = dot_row(xr, W1, dW1, ((size_t)e * 2 * I + nn) * h, h);
            if (w1_scale) v *= (double)w1_scale[(size_t)e * 2 * I + nn];
            if (a >= 0) v += dot_row(z1, B1, dB1, (((size_t)a * E + e) * 2 * I + nn) * r, r);
            g[nn] = v;
          }
          /* SiLU-and-mul */
          for (int32_t ii = 0; ii < I; ++ii) act[ii] = silu(g[ii]) * g[I + ii];
          /* down: shrink, base, expand */
          if (a >= 0) {
            for (int32_t q = 0; q < r; ++q)
              z2[q] = dot_row(act, A2, dA2, (((size_t)a * E + e) * r + q) * I, I);
          }
          for (int32_t m = 0; m < h; ++m) {
            double v = dot_row(act, W2, dW2, ((size_t)e * h + m) * I, I);
            if (w2_scale) v *= (double)w2_scale[(size_t)e * h + m];
            if (a >= 0) v += dot_row(z2, B2, dB2, (((size_t)a * E + e) * h + m) * r, r);
            dv[m] = v;
          }
          if (d_pairs) memcpy(d_pairs + ((size_t)i * k + j) * h, dv, sizeof(double) * (size_t)h);
          /* combine in slot order */
          for (int32_t m = 0; m < h; ++m) yrow[m] += w[j] * dv[m];
        }
      }
    }
    free(xr);
    free(g);
    free(act);
    free(z1);
    free(z2);
    free(dv);
    free(sel);
    free(w);
  }
  return status;
}

int oracle_forward(const orc_dims *d, const void *const *t, const int32_t *dt,
                   const float *logits, const int32_t *adapter_ids, const int32_t *tokens,
                   int32_t n_tokens, double *y, double *d_pairs) {
  return oracle_forward_scaled(d, t, dt, NULL, NULL, logits, adapter_ids, tokens, n_tokens, y,
                               d_pairs);
}

/* ------------------------------------------------------------------------------------------
 * Dense multi-LoRA (segmented gather matrix-vector, SGMV). Page "Punica: Multi-Tenant LoRA
 * Serving", sections on the proposed method: one copy of the base model serves a batch whose
 * tokens use different adapters; the LoRA add of one projection is applied per segment of
 * tokens that share an adapter. Page "vLLM MoE LoRA SageMaker Bedrock", section "O Papel da
 * Multi-LoRA": the shrink computes z = xA, the expand adds zB.
 *   y_out[t][n] = y_in[t][n] + sum_q z[t][q] B[a][n][q],  z[t][q] = sum_c x[t][c] A[a][q][c]
 * for a = adapter_ids[t] >= 0; y_out = y_in for a = -1. Layouts: x[T][K], A[nA][r][K],
 * B[nA][N][r] (stored out x in), y[T][N]; dt[] gives the dtypes of x, A, B, y_in.
 * ------------------------------------------------------------------------------------------ */
int oracle_sgmv(const void *x, const void *A, const void *B, const void *y_in, const int32_t *dt,
                const int32_t *adapter_ids, int32_t T, int32_t K, int32_t N, int32_t nA,
                int32_t r, double *y_out) {
  if (T < 0 || K <= 0 || N <= 0 || nA <= 0 || r <= 0) return ORC_EINVAL;
  for (int32_t t = 0; t < T; ++t)
    if (adapter_ids[t] < -1 || adapter_ids[t] >= nA) return ORC_EADAPTER;
  int status = ORC_OK;
#pragma omp parallel
  {
    double *xr = (double *)malloc(sizeof(double) * (size_t)K);
    double *z = (double *)malloc(sizeof(double) * (size_t)r);
    if (!xr || !z) {
#pragma omp atomic write
      status = ORC_ENOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int32_t t = 0; t < T; ++t) {
        const int32_t a = adapter_ids[t];
        double *yr = y_out + (size_t)t * N;
        for (int32_t n = 0; n < N; ++n) yr[n] = ld(y_in, dt[3], (size_t)t * N + n);
        if (a < 0) continue;
        for (int32_t c = 0; c < K; ++c) xr[c] = ld(x, dt[0], (size_t)t * K + c);
        for (int32_t q = 0; q < r; ++q) z[q] = dot_row(xr, A, dt[1], ((size_t)a * r + q) * K, K);
        for (int32_t n = 0; n < N; ++n) yr[n] += dot_row(z, B, dt[2], ((size_t)a * N + n) * r, r);
      }
    }
    free(xr);
    free(z);
  }
  return status;
}

/* Router logits: logits[t][e] = sum_c x[t][c] W_router[e][c] (page "vLLM MoE LoRA SageMaker
 * Bedrock", section "Entendendo os Modelos MoE": a router scores every expert for each token
 * before the top-k selection). x [T][h], W_router [E][h]; dtypes in dt[0], dt[1]. */
int oracle_router_logits(const void *x, const void *W_router, const int32_t *dt, int32_t T,
                         int32_t h, int32_t E, double *logits) {
  if (T < 0 || h <= 0 || E <= 0) return ORC_EINVAL;
  int status = ORC_OK;
#pragma omp parallel
  {
    double *xr = (double *)malloc(sizeof(double) * (size_t)h);
    if (!xr) {
#pragma omp atomic write
      status = ORC_ENOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int32_t t = 0; t < T; ++t) {
        for (int32_t c = 0; c < h; ++c) xr[c] = ld(x, dt[0], (size_t)t * h + c);
        for (int32_t e = 0; e < E; ++e)
          logits[(size_t)t * E + e] = dot_row(xr, W_router, dt[1], (size_t)e * h, h);
      }
    }
    free(xr);
  }
  return status;
}

/* E4M3 codes decoded to float64, for the tests. */
int oracle_fp8e4m3_decode(const uint8_t *codes, int64_t n, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = fp8e4m3_to_f64(codes[i]);
  return ORC_OK;
}

/* Thread count the forward uses (OpenMP's default team size). */
int oracle_num_threads(void) { return omp_get_max_threads(); }
