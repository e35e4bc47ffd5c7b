/* Plain-C use of the libdg C ABI on device 0: device buffers from the HIP runtime, then
 * the step's sampler head, acceptance, renoise, self-conditioning and stop test, checked
 * against closed forms rather than the oracle. With an all-zero embedding table every
 * logit is 0, so p0 is uniform over the vocabulary:
 *   entropy = ln V at every position, argmax = id 0 (ties go to the lowest id);
 *   no position fits a budget b < ln V, so nothing is accepted and every token is
 *   redrawn, inside [0, V);
 *   s = p0 E = 0, so z = W2 GELU(W1 0) = 0 whatever W1 and W2 hold;
 *   the stop test at step 0 with no previous argmax gives flag 0.
 * dg_accept_renoise_stop on the same entropies must give the three calls' results, and
 * dg_selfcond_accept after a second sampler head the same acceptance, tokens, flag and z.
 * Also: a NULL pointer and tau = 0 are refused with a message and nothing enqueued.
 * Built by the package's build step next to libdg.so; prints "c_abi_check: ok" and
 * exits 0 when every check holds, else prints the first failure and exits 1. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dg.h"

#define FAIL(...)                   \
  do {                              \
    printf("c_abi_check: ");        \
    printf(__VA_ARGS__);            \
    printf("\n");                   \
    return 1;                       \
  } while (0)
#define HIP_OK(x)                                                     \
  do {                                                                \
    hipError_t e_ = (x);                                              \
    if (e_ != hipSuccess) FAIL("%s: %s", #x, hipGetErrorString(e_));  \
  } while (0)
#define DG_OK_OR_FAIL(ctx, x)                                         \
  do {                                                                \
    dg_status s_ = (x);                                               \
    if (s_ != DG_OK) FAIL("%s: status %d (%s)", #x, (int)s_, dg_last_error(ctx)); \
  } while (0)

int main(void) {
  const dg_dims m = {1000, 64, 16, 2, 1, 32, 64};
  const int V = m.V, d = m.d, C = m.C, F = m.F;
  dg_ctx ctx = NULL;
  if (dg_create(&ctx, 0, NULL) != DG_OK) FAIL("dg_create failed");

  const size_t ws_bytes = dg_workspace_bytes(&m, 0);
  if (ws_bytes == 0) FAIL("dg_workspace_bytes returned 0");
  void *ws = NULL;
  dg_bf16 *E = NULL, *H = NULL, *W1 = NULL, *W2 = NULL, *z = NULL;
  float *ent = NULL;
  int32_t *am = NULL, *tok = NULL, *nacc = NULL, *flag = NULL, *tok2 = NULL, *nacc2 = NULL, *flag2 = NULL;
  int32_t *tok3 = NULL, *nacc3 = NULL, *flag3 = NULL;
  uint8_t *acc = NULL, *acc2 = NULL, *acc3 = NULL;
  dg_bf16 *z3 = NULL;
  HIP_OK(hipMalloc(&ws, ws_bytes));
  HIP_OK(hipMalloc((void **)&E, (size_t)V * d * 2));
  HIP_OK(hipMalloc((void **)&H, (size_t)C * d * 2));
  HIP_OK(hipMalloc((void **)&W1, (size_t)F * d * 2));
  HIP_OK(hipMalloc((void **)&W2, (size_t)d * F * 2));
  HIP_OK(hipMalloc((void **)&z, (size_t)C * d * 2));
  HIP_OK(hipMalloc((void **)&ent, (size_t)C * 4));
  HIP_OK(hipMalloc((void **)&am, (size_t)C * 4));
  HIP_OK(hipMalloc((void **)&tok, (size_t)C * 4));
  HIP_OK(hipMalloc((void **)&acc, (size_t)C));
  HIP_OK(hipMalloc((void **)&nacc, 4));
  HIP_OK(hipMalloc((void **)&flag, 4));
  HIP_OK(hipMalloc((void **)&tok2, (size_t)C * 4));
  HIP_OK(hipMalloc((void **)&acc2, (size_t)C));
  HIP_OK(hipMalloc((void **)&nacc2, 4));
  HIP_OK(hipMalloc((void **)&flag2, 4));
  HIP_OK(hipMalloc((void **)&tok3, (size_t)C * 4));
  HIP_OK(hipMalloc((void **)&acc3, (size_t)C));
  HIP_OK(hipMalloc((void **)&nacc3, 4));
  HIP_OK(hipMalloc((void **)&flag3, 4));
  HIP_OK(hipMalloc((void **)&z3, (size_t)C * d * 2));

  /* E = 0; H, W1, W2 = arbitrary finite bf16 values (alternating +-0.5, +-0.25) */
  HIP_OK(hipMemset(E, 0, (size_t)V * d * 2));
  uint16_t *host = (uint16_t *)malloc((size_t)F * d * 2);
  if (!host) FAIL("host allocation");
  for (int i = 0; i < F * d; ++i) host[i] = (i & 1) ? 0xBF00u : 0x3E80u;
  HIP_OK(hipMemcpy(H, host, (size_t)C * d * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(W1, host, (size_t)F * d * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(W2, host, (size_t)d * F * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(z, 0xFF, (size_t)C * d * 2)); /* NaN bits: every z element must be written */

  /* refused calls enqueue nothing and leave a message */
  if (dg_logits_entropy(ctx, &m, NULL, E, 0.8f, ws, ent, am) != DG_ERR_NULL) FAIL("NULL H accepted");
  if (strlen(dg_last_error(ctx)) == 0) FAIL("no message for the NULL H");
  if (dg_logits_entropy(ctx, &m, H, E, 0.0f, ws, ent, am) != DG_ERR_RANGE) FAIL("tau = 0 accepted");

  DG_OK_OR_FAIL(ctx, dg_logits_entropy(ctx, &m, H, E, 0.8f, ws, ent, am));
  DG_OK_OR_FAIL(ctx, dg_entropy_accept(ctx, 1, C, ent, 0.1f, acc, nacc));
  DG_OK_OR_FAIL(ctx, dg_renoise(ctx, 1, C, V, am, acc, 7u, 0u, 0u, tok));
  DG_OK_OR_FAIL(ctx, dg_selfcond(ctx, &m, ws, E, W1, W2, z));
  DG_OK_OR_FAIL(ctx, dg_stop_test(ctx, 1, C, ent, am, NULL, 0.005f, 0, 48, flag));
  DG_OK_OR_FAIL(ctx, dg_accept_renoise_stop(ctx, 1, C, V, ent, 0.1f, am, am, NULL, 7u, 0u, 0, 0.005f, 48,
                                            acc2, nacc2, tok2, flag2));
  DG_OK_OR_FAIL(ctx, dg_logits_entropy(ctx, &m, H, E, 0.8f, ws, ent, am));
  HIP_OK(hipMemset(z3, 0xFF, (size_t)C * d * 2));
  dg_accept_args aa;
  memset(&aa, 0, sizeof aa);
  aa.B = 1;
  aa.entropy = ent;
  aa.b = 0.1f;
  aa.x0 = am;
  aa.argmax = am;
  aa.prev_argmax = NULL;
  aa.seed = 7u;
  aa.canvas_base = 0u;
  aa.step = 0;
  aa.thr = 0.005f;
  aa.N = 48;
  aa.accept = acc3;
  aa.n_accept = nacc3;
  aa.tokens = tok3;
  aa.flag = flag3;
  DG_OK_OR_FAIL(ctx, dg_selfcond_accept(ctx, &m, ws, E, W1, W2, z3, &aa));
  DG_OK_OR_FAIL(ctx, dg_sync(ctx));

  float h_ent[16];
  int32_t h_am[16], h_tok[16], h_nacc, h_flag, h_tok2[16], h_nacc2, h_flag2;
  uint8_t h_acc[16], h_acc2[16];
  HIP_OK(hipMemcpy(h_ent, ent, sizeof h_ent, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_am, am, sizeof h_am, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_tok, tok, sizeof h_tok, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_acc, acc, sizeof h_acc, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&h_nacc, nacc, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&h_flag, flag, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(host, z, (size_t)C * d * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_tok2, tok2, sizeof h_tok2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_acc2, acc2, sizeof h_acc2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&h_nacc2, nacc2, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&h_flag2, flag2, 4, hipMemcpyDeviceToHost));
  if (memcmp(h_tok2, h_tok, sizeof h_tok) || memcmp(h_acc2, h_acc, sizeof h_acc) || h_nacc2 != h_nacc ||
      h_flag2 != h_flag)
    FAIL("dg_accept_renoise_stop differs from the three calls");
  HIP_OK(hipMemcpy(h_tok2, tok3, sizeof h_tok2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_acc2, acc3, sizeof h_acc2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&h_nacc2, nacc3, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&h_flag2, flag3, 4, hipMemcpyDeviceToHost));
  if (memcmp(h_tok2, h_tok, sizeof h_tok) || memcmp(h_acc2, h_acc, sizeof h_acc) || h_nacc2 != h_nacc ||
      h_flag2 != h_flag)
    FAIL("dg_selfcond_accept's acceptance differs from the three calls");
  {
    uint16_t *z3h = (uint16_t *)malloc((size_t)C * d * 2);
    if (!z3h) FAIL("host allocation");
    HIP_OK(hipMemcpy(z3h, z3, (size_t)C * d * 2, hipMemcpyDeviceToHost));
    const int same = memcmp(z3h, host, (size_t)C * d * 2) == 0;
    free(z3h);
    if (!same) FAIL("dg_selfcond_accept's z differs from dg_selfcond's");
  }

  const double lnV = log((double)V);
  for (int c = 0; c < C; ++c) {
    if (fabs(h_ent[c] - lnV) > 1e-4) FAIL("entropy[%d] = %.7f, expected ln %d = %.7f", c, h_ent[c], V, lnV);
    if (h_am[c] != 0) FAIL("argmax[%d] = %d, expected 0", c, h_am[c]);
    if (h_acc[c] != 0) FAIL("position %d accepted", c);
    if (h_tok[c] < 0 || h_tok[c] >= V) FAIL("token[%d] = %d outside [0, %d)", c, h_tok[c], V);
  }
  if (h_nacc != 0) FAIL("n_accept = %d, expected 0", h_nacc);
  if (h_flag != 0) FAIL("stop flag = %d, expected 0", h_flag);
  for (int i = 0; i < C * d; ++i)
    if ((host[i] & 0x7FFFu) != 0) FAIL("z element %d = 0x%04x, expected 0", i, host[i]);

  free(host);
  hipFree(ws); hipFree(E); hipFree(H); hipFree(W1); hipFree(W2); hipFree(z);
  hipFree(ent); hipFree(am); hipFree(tok); hipFree(acc); hipFree(nacc); hipFree(flag);
  hipFree(tok2); hipFree(acc2); hipFree(nacc2); hipFree(flag2);
  hipFree(tok3); hipFree(acc3); hipFree(nacc3); hipFree(flag3); hipFree(z3);
  dg_destroy(ctx);
  printf("c_abi_check: ok\n");
  return 0;
}
