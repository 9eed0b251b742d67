/*
 * A plain C caller of the routing library: device buffers from the HIP
 * runtime's C API, then route -> assign -> layout -> dispatch -> stand-in ->
 * combine through include/moe_route.h, checked against invariants computed
 * on the host (no Python, no torch). Built as a shared library so a test can
 * call moe_c_abi_check() in-process; returns 0 when every check holds and
 * prints the first failure otherwise.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe_route.h"

#define FAIL(...)                       \
  do {                                  \
    fprintf(stderr, "c-abi check: ");   \
    fprintf(stderr, __VA_ARGS__);       \
    fprintf(stderr, "\n");              \
    rc = 1;                             \
    goto done;                          \
  } while (0)

#define HIP_OK(call)                                                      \
  do {                                                                    \
    hipError_t e_ = (call);                                               \
    if (e_ != hipSuccess) FAIL("%s: %s", #call, hipGetErrorString(e_));   \
  } while (0)

#define MOE_OK_OR_FAIL(call)                                                   \
  do {                                                                         \
    moe_status s_ = (call);                                                    \
    if (s_ != MOE_OK) FAIL("%s: %s (%s)", #call, moe_status_string(s_), moe_last_error()); \
  } while (0)

static uint32_t lcg(uint32_t* s) {
  *s = *s * 1664525u + 1013904223u;
  return *s;
}

/* bf16 bits of a small value v/8 (exact in bf16) */
static uint16_t bf16_bits(int v) {
  float f = (float)v / 8.0f;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

int moe_c_abi_check(void) {
  enum { T = 700, E = 16, K = 4, H = 64, R = 4 };
  const int n = T * K;
  int rc = 0;
  float* h_logits = (float*)malloc(sizeof(float) * T * E);
  uint16_t* h_x = (uint16_t*)malloc(2u * T * H);
  int32_t* h_idx = (int32_t*)malloc(4u * n);
  float* h_w = (float*)malloc(4u * n);
  int32_t* h_counts = (int32_t*)malloc(4u * E);
  int32_t* h_pos = (int32_t*)malloc(4u * n);
  int32_t* h_src = (int32_t*)malloc(4u * n);
  int32_t* h_roff = (int32_t*)malloc(4u * (R + 1));
  uint16_t* h_send = (uint16_t*)malloc(2u * n * H);
  char* seen = (char*)calloc(n, 1);
  void *d_logits = NULL, *d_x = NULL, *d_idx = NULL, *d_w = NULL, *d_counts = NULL, *d_assign = NULL,
       *d_active = NULL, *d_rank_of = NULL, *d_eoff = NULL, *d_roff = NULL, *d_pos = NULL,
       *d_src = NULL, *d_dedup = NULL, *d_send = NULL, *d_y = NULL, *d_out = NULL, *d_ws = NULL;
  size_t ws_bytes = 0;
  uint32_t seed = 12345u;
  moe_problem p;
  p.T = T; p.E = E; p.k = K; p.H = H; p.R = R; p.act_dtype = MOE_BF16; p.flags = 0;

  if (!h_logits || !h_x || !h_idx || !h_w || !h_counts || !h_pos || !h_src || !h_roff || !h_send || !seen)
    FAIL("host allocation");
  /* distinct logits per token: a random permutation of E values */
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) h_logits[t * E + e] = (float)e;
    for (int e = E - 1; e > 0; --e) {
      const int j = (int)(lcg(&seed) % (uint32_t)(e + 1));
      const float tmp = h_logits[t * E + e];
      h_logits[t * E + e] = h_logits[t * E + j];
      h_logits[t * E + j] = tmp;
    }
  }
  for (int i = 0; i < T * H; ++i) h_x[i] = bf16_bits((int)(lcg(&seed) % 33u) - 16);

  /* error path first: a NULL input is refused before anything is enqueued */
  if (moe_route(&p, NULL, NULL, NULL, NULL, NULL, 0, NULL) != MOE_ERR_INVALID_ARG)
    FAIL("moe_route accepted NULL logits");
  if (strlen(moe_last_error()) == 0) FAIL("no error text for a refused call");

  MOE_OK_OR_FAIL(moe_workspace_bytes(&p, &ws_bytes));
  HIP_OK(hipMalloc(&d_logits, sizeof(float) * T * E));
  HIP_OK(hipMalloc(&d_x, 2u * T * H));
  HIP_OK(hipMalloc(&d_idx, 4u * n));
  HIP_OK(hipMalloc(&d_w, 4u * n));
  HIP_OK(hipMalloc(&d_counts, 4u * E));
  HIP_OK(hipMalloc(&d_assign, 4u * E));
  HIP_OK(hipMalloc(&d_active, 4u * R));
  HIP_OK(hipMalloc(&d_rank_of, 4u * E));
  HIP_OK(hipMalloc(&d_eoff, 4u * E));
  HIP_OK(hipMalloc(&d_roff, 4u * (R + 1)));
  HIP_OK(hipMalloc(&d_pos, 4u * n));
  HIP_OK(hipMalloc(&d_src, 4u * n));
  HIP_OK(hipMalloc(&d_dedup, 4u * R));
  HIP_OK(hipMalloc(&d_send, 2u * n * H));
  HIP_OK(hipMalloc(&d_y, 2u * n * H));
  HIP_OK(hipMalloc(&d_out, 2u * T * H));
  HIP_OK(hipMalloc(&d_ws, ws_bytes));
  HIP_OK(hipMemcpy(d_logits, h_logits, sizeof(float) * T * E, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_x, h_x, 2u * T * H, hipMemcpyHostToDevice));

  MOE_OK_OR_FAIL(moe_route(&p, (const float*)d_logits, (int32_t*)d_idx, (float*)d_w,
                           (int32_t*)d_counts, d_ws, ws_bytes, NULL));
  MOE_OK_OR_FAIL(moe_assign_replicas(&p, (const int32_t*)d_counts, NULL, 1, (int32_t*)d_assign,
                                     (int32_t*)d_active, NULL));
  MOE_OK_OR_FAIL(moe_layout(&p, (const int32_t*)d_idx, (const int32_t*)d_assign, NULL, 1,
                            (int32_t*)d_rank_of, (int32_t*)d_eoff, (int32_t*)d_roff,
                            (int32_t*)d_pos, (int32_t*)d_src, (int32_t*)d_dedup, d_ws, ws_bytes,
                            NULL));
  MOE_OK_OR_FAIL(moe_dispatch(&p, d_x, (const int32_t*)d_pos, d_send, NULL));
  MOE_OK_OR_FAIL(moe_expert_standin(&p, d_send, (const int32_t*)d_src, (const int32_t*)d_idx, d_y,
                                    NULL));
  MOE_OK_OR_FAIL(moe_combine(&p, d_y, (const int32_t*)d_pos, (const float*)d_w, d_out, NULL));
  HIP_OK(hipDeviceSynchronize());

  HIP_OK(hipMemcpy(h_idx, d_idx, 4u * n, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_w, d_w, 4u * n, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_counts, d_counts, 4u * E, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_pos, d_pos, 4u * n, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_src, d_src, 4u * n, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_roff, d_roff, 4u * (R + 1), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_send, d_send, 2u * n * H, hipMemcpyDeviceToHost));

  /* top-k: the k largest logits in descending order; weights sum to 1 */
  for (int t = 0; t < T; ++t) {
    double wsum = 0.0;
    for (int j = 0; j < K; ++j) {
      const int e = h_idx[t * K + j];
      if (e < 0 || e >= E) FAIL("idx out of range");
      if (h_logits[t * E + e] != (float)(E - 1 - j)) FAIL("token %d slot %d is not the %d-th largest", t, j, j);
      wsum += h_w[t * K + j];
    }
    if (fabs(wsum - 1.0) > 1e-5) FAIL("weights of token %d sum to %f", t, wsum);
  }
  /* demand vector: counts match idx, and sum to T k */
  {
    int tot = 0;
    for (int e = 0; e < E; ++e) {
      int c = 0;
      for (int i = 0; i < n; ++i) c += h_idx[i] == e;
      if (c != h_counts[e]) FAIL("counts[%d] = %d, idx holds %d", e, h_counts[e], c);
      tot += c;
    }
    if (tot != n || h_roff[R] != n) FAIL("total rows");
  }
  /* layout: pos is a permutation, src its inverse, rows grouped by expert in
     token order, and every send row is a bit copy of its token's row */
  for (int i = 0; i < n; ++i) {
    const int r = h_pos[i];
    if (r < 0 || r >= n || seen[r]) FAIL("pos is not a permutation at %d", i);
    seen[r] = 1;
    if (h_src[r] != i) FAIL("src[pos[%d]] != %d", i, i);
    if (memcmp(h_send + (size_t)r * H, h_x + (size_t)(i / K) * H, 2u * H) != 0) FAIL("send row %d", r);
  }
  for (int r = 1; r < n; ++r) {
    const int a = h_src[r - 1], b = h_src[r];
    const int ea = h_idx[a], eb = h_idx[b];
    if (ea > eb || (ea == eb && a > b)) FAIL("send rows %d, %d out of (expert, token) order", r - 1, r);
  }
  /* the one-call route + assignment + layout writes the same tables */
  {
    int32_t* h_pos2 = (int32_t*)malloc(4u * n);
    int32_t* h_idx2 = (int32_t*)malloc(4u * n);
    int32_t* h_roff2 = (int32_t*)malloc(4u * (R + 1));
    int same = h_pos2 && h_idx2 && h_roff2;
    if (same) {
      HIP_OK(hipMemset(d_pos, 0xff, 4u * n));
      MOE_OK_OR_FAIL(moe_route_assign_layout(&p, (const float*)d_logits, NULL, 1, (int32_t*)d_idx,
                                             (float*)d_w, (int32_t*)d_counts, (int32_t*)d_assign,
                                             (int32_t*)d_active, (int32_t*)d_rank_of,
                                             (int32_t*)d_eoff, (int32_t*)d_roff, (int32_t*)d_pos,
                                             (int32_t*)d_src, (int32_t*)d_dedup, d_ws, ws_bytes,
                                             NULL));
      HIP_OK(hipDeviceSynchronize());
      HIP_OK(hipMemcpy(h_pos2, d_pos, 4u * n, hipMemcpyDeviceToHost));
      HIP_OK(hipMemcpy(h_idx2, d_idx, 4u * n, hipMemcpyDeviceToHost));
      HIP_OK(hipMemcpy(h_roff2, d_roff, 4u * (R + 1), hipMemcpyDeviceToHost));
      same = memcmp(h_pos2, h_pos, 4u * n) == 0 && memcmp(h_idx2, h_idx, 4u * n) == 0 &&
             memcmp(h_roff2, h_roff, 4u * (R + 1)) == 0;
    }
    free(h_pos2); free(h_idx2); free(h_roff2);
    if (!same) FAIL("moe_route_assign_layout differs from the three calls");
  }
  printf("c-abi check ok: T=%d E=%d k=%d H=%d R=%d\n", T, E, K, H, R);

done:
  hipFree(d_logits); hipFree(d_x); hipFree(d_idx); hipFree(d_w); hipFree(d_counts);
  hipFree(d_assign); hipFree(d_active); hipFree(d_rank_of); hipFree(d_eoff); hipFree(d_roff);
  hipFree(d_pos); hipFree(d_src); hipFree(d_dedup); hipFree(d_send); hipFree(d_y); hipFree(d_out);
  hipFree(d_ws);
  free(h_logits); free(h_x); free(h_idx); free(h_w); free(h_counts); free(h_pos); free(h_src);
  free(h_roff); free(h_send); free(seen);
  return rc;
}
