/*
 * Sanitizer run of the library's host side (test infrastructure): the C ABI's argument checks,
 * workspace sizing and layout queries, built with -fsanitize=address,undefined on the host
 * code and linked against launchers that abort if reached (every call here must be refused
 * on the host, before any device work). Exit status 0 = clean.
 */
#include <stdint.h>
#include <stdio.h>

#include "moelora.h"
#include "moelora_probe.h"

#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      return 1;                                                   \
    }                                                             \
  } while (0)

static void *fake(int i) { return (void *)(uintptr_t)(0x100000u * (unsigned)(i + 1)); }

int main(void) {
  const moe_lora_dims shapes[] = {{64, 4096, 11008, 16, 8, 16},    {4096, 4096, 14336, 8, 32, 64},
                                  {256, 2048, 768, 128, 64, 32},   {1024, 4096, 11008, 16, 1024, 16},
                                  {16, 256, 512, 8, 4, 8},         {0, 256, 512, 8, 4, 8},
                                  {1, 128, 128, 1, 1, 64},         {200000, 128, 4096, 1, 1, 8}};
  const int topks[] = {2, 2, 8, 2, 2, 2, 1, 1};
  for (unsigned i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
    const size_t n = moe_lora_workspace_size(&shapes[i], topks[i]);
    CHECK(n > 0 && n % 256 == 0);
    moe_lora_layout_info info;
    CHECK(moe_lora_workspace_layout(&shapes[i], topks[i], &info) == MOELORA_OK);
    CHECK(info.workspace_bytes == (int64_t)n && info.capacity >= (int64_t)shapes[i].T * topks[i]);
    CHECK(moe_lora_sorted_capacity(&shapes[i], topks[i], 1, info.block_m) <= info.capacity);
  }
  const moe_lora_dims bad[] = {{16, 100, 512, 8, 4, 8}, {16, 256, 192, 8, 4, 8}, {16, 256, 512, 8, 4, 12},
                               {16, 256, 512, 0, 4, 8}, {16, 256, 512, 2000, 4, 8}, {-1, 256, 512, 8, 4, 8},
                               {270000, 128, 4096, 1, 1, 8}};
  for (unsigned i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
    CHECK(moe_lora_workspace_size(&bad[i], 1) == 0);
    moe_lora_layout_info info;
    CHECK(moe_lora_workspace_layout(&bad[i], 1, &info) != MOELORA_OK);
  }
  CHECK(moe_lora_workspace_size(NULL, 2) == 0);
  CHECK(moe_lora_workspace_layout(&shapes[0], 2, NULL) == MOELORA_ENULL);

  const moe_lora_dims d = {16, 256, 512, 8, 4, 8};
  const size_t ws = moe_lora_workspace_size(&d, 2);
  void *p[13];
  for (int i = 0; i < 13; ++i) p[i] = fake(i);
  /* forward: each NULL, each misaligned pointer, a short or misaligned workspace */
  for (int i = 0; i < 11; ++i) {
    void *q[11];
    for (int j = 0; j < 11; ++j) q[j] = p[j];
    q[i] = NULL;
    CHECK(moe_lora_forward(q[0], q[1], q[2], q[3], q[4], q[5], q[6], q[7], q[8], 2, &d, q[9], q[10],
                           ws, NULL) == MOELORA_ENULL);
    CHECK(moe_lora_forward_routed(q[0], q[1], q[2], q[3], q[4], q[5], q[6], q[7], q[8], 2, &d, q[9],
                                  q[10], ws, NULL) == MOELORA_ENULL);
    if (i < 10)
      CHECK(moe_lora_forward_noalloc(q[0], q[1], q[2], q[3], q[4], q[5], q[6], q[7], q[8], 2, &d,
                                     q[9], NULL) == MOELORA_ENULL);
    q[i] = (char *)p[i] + 8;
    CHECK(moe_lora_forward(q[0], q[1], q[2], q[3], q[4], q[5], q[6], q[7], q[8], 2, &d, q[9], q[10],
                           ws, NULL) == MOELORA_EALIGN);
  }
  CHECK(moe_lora_forward(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], 2, &d, p[9],
                         (char *)p[10] + 16, ws, NULL) == MOELORA_EWORKSPACE);
  CHECK(moe_lora_forward(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], 2, &d, p[9], p[10],
                         ws - 1, NULL) == MOELORA_EWORKSPACE);
  CHECK(moe_lora_forward(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], 9, &d, p[9], p[10], ws,
                         NULL) == MOELORA_EINVAL_DIMS);
  void *const ev[MOELORA_N_STAGES + 1] = {0};
  CHECK(moe_lora_forward_timed(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], 2, &d, p[9],
                               p[10], ws, NULL, NULL) == MOELORA_ENULL);
  CHECK(moe_lora_forward_timed(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], 2, &d, p[9],
                               p[10], ws - 1, NULL, ev) == MOELORA_EWORKSPACE);
  /* FP8: missing or misaligned scales */
  CHECK(moe_lora_forward_fp8(p[0], p[1], p[2], NULL, p[4], p[5], p[6], p[7], p[8], p[9], p[10], 2,
                             &d, p[11], p[12], ws, NULL, NULL) == MOELORA_ENULL);
  CHECK(moe_lora_forward_fp8(p[0], p[1], p[2], (float *)((char *)p[3] + 2), p[4], p[5], p[6], p[7],
                             p[8], p[9], p[10], 2, &d, p[11], p[12], ws, NULL, NULL) == MOELORA_EALIGN);
  /* no-alloc: beyond its scratch */
  const moe_lora_dims big = {4096, 4096, 14336, 8, 32, 64};
  CHECK(moe_lora_forward_noalloc(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], 2, &big, p[9],
                                 NULL) == MOELORA_ESCRATCH);
  /* empty batches need nothing */
  const moe_lora_dims empty = {0, 256, 512, 8, 4, 8};
  CHECK(moe_lora_forward(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 2, &empty, NULL, NULL,
                         0, NULL) == MOELORA_OK);
  /* route/align */
  const int64_t cap = moe_lora_sorted_capacity(&d, 2, 1, 16);
  CHECK(cap == 32 + 8 * 15);
  CHECK(moe_lora_sorted_capacity(&d, 2, 0, 16) == -1);
  CHECK(moe_lora_route_align(p[0], p[1], 2, &d, 1, 16, p[2], p[3], p[4], cap - 1, p[5], p[6], p[7],
                             p[8], ws, NULL) == MOELORA_EINVAL_DIMS);
  CHECK(moe_lora_route_align(p[0], p[1], 2, &d, 1, 16, p[2], p[3], NULL, cap, p[5], p[6], p[7], p[8],
                             ws, NULL) == MOELORA_ENULL);
  /* SGMV, router, probes */
  const moe_lora_sgmv_dims sd = {50, 128, 64, 3, 8};
  CHECK(moe_lora_sgmv_workspace_size(&sd) > 0);
  const moe_lora_sgmv_dims sbad = {50, 100, 64, 3, 8};
  CHECK(moe_lora_sgmv_workspace_size(&sbad) == 0);
  CHECK(moe_lora_sgmv(p[0], p[1], NULL, p[3], &sd, p[4], p[5], moe_lora_sgmv_workspace_size(&sd),
                      NULL) == MOELORA_ENULL);
  CHECK(moe_lora_router_logits(p[0], p[1], 4, 100, 8, (float *)p[2], NULL) == MOELORA_EINVAL_DIMS);
  CHECK(moe_lora_router_logits(p[0], NULL, 4, 128, 8, (float *)p[2], NULL) == MOELORA_ENULL);
  CHECK(moe_lora_probe_read(p[0], 100, (uint32_t *)p[1], NULL) == MOELORA_EINVAL_DIMS);
  CHECK(moe_lora_probe_mfma(0, 4, (float *)p[1], NULL) == MOELORA_EINVAL_DIMS);
  for (int c = -9; c <= 1; ++c) CHECK(moe_lora_strerror(c) != NULL);
  uint32_t flags = 0;
  CHECK(moe_lora_debug_status(NULL, 16, NULL, &flags) == MOELORA_ENULL);
  printf("abi host sanitizer run: ok\n");
  return 0;
}
