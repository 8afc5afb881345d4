/*
 * Sanitizer run of the CPU oracle (test infrastructure): the oracle's source is compiled into
 * this driver with -fsanitize=address,undefined, and every entry point runs on a small seeded
 * case, with a few invariants checked and bad arguments rejected. Exit status 0 = clean.
 */
#include <stdio.h>

#include "../../oracle/moelora_oracle.c"

static uint64_t lcg_state = 0x9E3779B97F4A7C15ull;
static double lcg_normal(void) { /* sum of 4 uniforms, centred: enough for a smoke input */
  double s = 0.0;
  for (int i = 0; i < 4; ++i) {
    lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
    s += (double)(lcg_state >> 11) / 9007199254740992.0;
  }
  return (s - 2.0) * 1.7320508;
}
static uint16_t to_bf16(double v) { /* truncating is enough for inputs */
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      return 1;                                                   \
    }                                                             \
  } while (0)

int main(void) {
  enum { T = 7, h = 32, I = 48, E = 5, nA = 3, r = 8, k = 2 };
  float logits[T * E];
  int32_t ad[T];
  for (int i = 0; i < T * E; ++i) logits[i] = (float)lcg_normal();
  logits[3] = logits[4]; /* a tie */
  for (int t = 0; t < T; ++t) ad[t] = (t % 4) - 1;
  int32_t ids[T * k];
  double w[T * k];
  CHECK(oracle_route(logits, T, E, k, ids, w) == ORC_OK);
  for (int t = 0; t < T; ++t) CHECK(fabs(w[t * k] + w[t * k + 1] - 1.0) < 1e-12);
  CHECK(oracle_route(logits, T, E, E + 1, ids, w) == ORC_EINVAL);

  int32_t sp[T * k * 8 + E * 64], off[E + 1], seg[T * k * 4], ns = 0;
  const int pads[3][2] = {{1, 1}, {4, 16}, {1, 64}};
  for (int c = 0; c < 3; ++c) {
    CHECK(oracle_align(ids, ad, T, k, E, nA, pads[c][0], pads[c][1], sp,
                       (int64_t)(sizeof sp / sizeof sp[0]), off, seg, T * k, &ns) == ORC_OK);
    int seen[T * k];
    memset(seen, 0, sizeof seen);
    for (int i = 0; i < off[E]; ++i)
      if (sp[i] >= 0) seen[sp[i]]++;
    for (int p = 0; p < T * k; ++p) CHECK(seen[p] == 1);
  }
  CHECK(oracle_align(ids, ad, T, k, E, nA, 1, 1, sp, 2, off, seg, T * k, &ns) != ORC_OK);

  /* bf16 weights and inputs */
  const size_t nx = (size_t)T * h, nW1 = (size_t)E * 2 * I * h, nW2 = (size_t)E * h * I,
               nA1 = (size_t)nA * E * r * h, nB1 = (size_t)nA * E * 2 * I * r,
               nA2 = (size_t)nA * E * r * I, nB2 = (size_t)nA * E * h * r;
  const size_t sizes[7] = {nx, nW1, nW2, nA1, nB1, nA2, nB2};
  uint16_t *buf[7];
  for (int i = 0; i < 7; ++i) {
    buf[i] = (uint16_t *)malloc(sizes[i] * 2);
    for (size_t j = 0; j < sizes[i]; ++j) buf[i][j] = to_bf16(0.1 * lcg_normal());
  }
  const void *tens[7] = {buf[0], buf[1], buf[2], buf[3], buf[4], buf[5], buf[6]};
  const int32_t dt[7] = {ORC_BF16, ORC_BF16, ORC_BF16, ORC_BF16, ORC_BF16, ORC_BF16, ORC_BF16};
  orc_dims d = {T, h, I, E, nA, r, k};
  double y[T * h], y2[3 * h], dp[3 * k * h];
  CHECK(oracle_forward(&d, tens, dt, logits, ad, NULL, 0, y, NULL) == ORC_OK);
  const int32_t toks[3] = {6, 0, 3};
  CHECK(oracle_forward(&d, tens, dt, logits, ad, toks, 3, y2, dp) == ORC_OK);
  for (int i = 0; i < 3; ++i)
    for (int c = 0; c < h; ++c) CHECK(y2[i * h + c] == y[toks[i] * h + c]);
  int32_t bad_ad[T];
  memcpy(bad_ad, ad, sizeof ad);
  bad_ad[2] = nA;
  CHECK(oracle_forward(&d, tens, dt, logits, bad_ad, NULL, 0, y, NULL) != ORC_OK);

  /* E4M3 expert weights with per-row scales */
  uint8_t *q1 = (uint8_t *)malloc(nW1), *q2 = (uint8_t *)malloc(nW2);
  float *s1 = (float *)malloc(sizeof(float) * E * 2 * I), *s2 = (float *)malloc(sizeof(float) * E * h);
  for (size_t j = 0; j < nW1; ++j) q1[j] = (uint8_t)(lcg_state >> (j % 56)) & 0x77;
  for (size_t j = 0; j < nW2; ++j) q2[j] = (uint8_t)(lcg_state >> (j % 53)) & 0x76;
  for (int j = 0; j < E * 2 * I; ++j) s1[j] = 0.01f * (1 + j % 3);
  for (int j = 0; j < E * h; ++j) s2[j] = 0.02f;
  const void *tq[7] = {buf[0], q1, q2, buf[3], buf[4], buf[5], buf[6]};
  const int32_t dq[7] = {ORC_BF16, ORC_FP8E4M3, ORC_FP8E4M3, ORC_BF16, ORC_BF16, ORC_BF16, ORC_BF16};
  CHECK(oracle_forward_scaled(&d, tq, dq, s1, s2, logits, ad, NULL, 0, y, NULL) == ORC_OK);
  for (int i = 0; i < T * h; ++i) CHECK(isfinite(y[i]));
  CHECK(oracle_forward_scaled(&d, tq, dq, NULL, s2, logits, ad, NULL, 0, y, NULL) == ORC_EINVAL);
  double dec[256];
  uint8_t codes[256];
  for (int i = 0; i < 256; ++i) codes[i] = (uint8_t)i;
  CHECK(oracle_fp8e4m3_decode(codes, 256, dec) == ORC_OK);
  CHECK(dec[0x38] == 1.0 && dec[0x7e] == 448.0 && isnan(dec[0x7f]));

  /* dense multi-LoRA and router logits */
  const int32_t sdt[4] = {ORC_BF16, ORC_BF16, ORC_BF16, ORC_BF16};
  double ys[T * 2 * I];
  CHECK(oracle_sgmv(buf[0], buf[3], buf[4], buf[1], sdt, ad, T, h, 2 * I, nA, r, ys) == ORC_OK);
  CHECK(oracle_sgmv(buf[0], buf[3], buf[4], buf[1], sdt, bad_ad, T, h, 2 * I, nA, r, ys) != ORC_OK);
  double lg[T * E];
  const int32_t rdt[2] = {ORC_BF16, ORC_BF16};
  CHECK(oracle_router_logits(buf[0], buf[1], rdt, T, h, E, lg) == ORC_OK);

  for (int i = 0; i < 7; ++i) free(buf[i]);
  free(q1);
  free(q2);
  free(s1);
  free(s2);
  printf("oracle sanitizer run: ok\n");
  return 0;
}
