/*
 * A plain C caller of the routing library: device buffers from the HIP
 * runtime's C API, then every entry point of include/moe_route.h, checked
 * against invariants computed on the host (no Python, no torch). Built as a
 * shared library so a test can call it in-process:
 *   moe_c_abi_check()       route -> assign -> layout -> dispatch ->
 *                           stand-in -> combine, and the one-call plan;
 *   moe_c_abi_check_rest()  the one-call single-send plan and the
 *                           allocation-free plan against the separate calls,
 *                           the single-send layout, dispatch and fan-out,
 *                           the two backward calls, the routing statistics
 *                           and the token-balanced split.
 * Each returns 0 when every check holds and prints the first failure
 * otherwise.
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

/* the value of a bf16 bit pattern */
static double bf16_val(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* round an fp32 value to bf16, to nearest even (NaN stays a quiet NaN) */
static uint16_t bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

enum {
  B_LOGITS, B_X, B_IDX, B_W, B_COUNTS, B_ASSIGN, B_ACTIVE, B_RANK_OF, B_EOFF, B_ROFF, B_POS,
  B_SRC, B_DEDUP, B_SSOFF, B_SSROW, B_SSTOK, B_SEND, B_SEND_SS, B_SEND2, B_Y, B_DY, B_DW, B_DX,
  B_SCOUNTS, B_COSEL, B_STATS, B_GOP, B_BACT, B_BTOK, B_COUNT
};

/* the routing tables written by the plan calls, compared between them */
static const int kPlanOut[] = {B_IDX, B_W, B_COUNTS, B_ASSIGN, B_ACTIVE, B_RANK_OF, B_EOFF,
                               B_ROFF, B_POS, B_SRC, B_DEDUP};
enum { kNPlanOut = sizeof(kPlanOut) / sizeof(kPlanOut[0]) };

int moe_c_abi_check_rest(void) {
  enum { T = 700, E = 16, K = 4, H = 64, R = 4, PER = E / R };
  const int n = T * K;
  int rc = 0;
  size_t sz[B_COUNT];
  void* d[B_COUNT] = {0};
  void* h[B_COUNT] = {0};
  void* a[B_COUNT] = {0}; /* the one-call plan's outputs */
  void* ws = NULL;
  size_t ws_bytes = 0;
  uint32_t seed = 999u;
  moe_problem p;
  p.T = T; p.E = E; p.k = K; p.H = H; p.R = R; p.act_dtype = MOE_BF16; p.flags = 0;

  sz[B_LOGITS] = 4u * T * E;  sz[B_X] = 2u * T * H;
  sz[B_IDX] = sz[B_W] = sz[B_POS] = sz[B_SRC] = sz[B_SSROW] = sz[B_SSTOK] = sz[B_DW] =
      sz[B_GOP] = 4u * n;
  sz[B_COUNTS] = sz[B_ASSIGN] = sz[B_RANK_OF] = sz[B_EOFF] = 4u * E;
  sz[B_ACTIVE] = sz[B_DEDUP] = sz[B_BACT] = sz[B_BTOK] = 4u * R;
  sz[B_ROFF] = sz[B_SSOFF] = 4u * (R + 1);
  sz[B_SEND] = sz[B_SEND_SS] = sz[B_SEND2] = sz[B_Y] = sz[B_DY] = 2u * n * H;
  sz[B_DX] = 2u * T * H;
  sz[B_SCOUNTS] = 4u * R * R;
  sz[B_COSEL] = 4u * E * E;
  sz[B_STATS] = 8u * 4;
  for (int i = 0; i < B_COUNT; ++i) {
    h[i] = malloc(sz[i]);
    a[i] = malloc(sz[i]);
    if (!h[i] || !a[i]) FAIL("host allocation");
    HIP_OK(hipMalloc(&d[i], sz[i]));
  }
  MOE_OK_OR_FAIL(moe_workspace_bytes(&p, &ws_bytes));
  HIP_OK(hipMalloc(&ws, ws_bytes));

  {
    float* lg = (float*)h[B_LOGITS];
    uint16_t* x = (uint16_t*)h[B_X];
    for (int t = 0; t < T; ++t) { /* distinct logits: a random permutation of 0..E-1 */
      for (int e = 0; e < E; ++e) lg[t * E + e] = (float)e;
      for (int e = E - 1; e > 0; --e) {
        const int j = (int)(lcg(&seed) % (uint32_t)(e + 1));
        const float tmp = lg[t * E + e];
        lg[t * E + e] = lg[t * E + j];
        lg[t * E + j] = tmp;
      }
    }
    for (int i = 0; i < T * H; ++i) x[i] = bf16_bits((int)(lcg(&seed) % 33u) - 16);
  }
  HIP_OK(hipMemcpy(d[B_LOGITS], h[B_LOGITS], sz[B_LOGITS], hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d[B_X], h[B_X], sz[B_X], hipMemcpyHostToDevice));

  /* 1. the one-call single-send plan; every output pre-filled with 0xff */
  for (int i = B_IDX; i <= B_SSTOK; ++i) HIP_OK(hipMemset(d[i], 0xff, sz[i]));
  MOE_OK_OR_FAIL(moe_route_assign_layout_single_send(
      &p, (const float*)d[B_LOGITS], NULL, 1, (int32_t*)d[B_IDX], (float*)d[B_W],
      (int32_t*)d[B_COUNTS], (int32_t*)d[B_ASSIGN], (int32_t*)d[B_ACTIVE], (int32_t*)d[B_RANK_OF],
      (int32_t*)d[B_EOFF], (int32_t*)d[B_ROFF], (int32_t*)d[B_POS], (int32_t*)d[B_SRC],
      (int32_t*)d[B_DEDUP], (int32_t*)d[B_SSOFF], (int32_t*)d[B_SSROW], (int32_t*)d[B_SSTOK], ws,
      ws_bytes, NULL));
  HIP_OK(hipDeviceSynchronize());
  for (int i = B_IDX; i <= B_SSTOK; ++i) HIP_OK(hipMemcpy(a[i], d[i], sz[i], hipMemcpyDeviceToHost));

  /* 2. the three separate calls write the same tables */
  for (int i = B_IDX; i <= B_SSTOK; ++i) HIP_OK(hipMemset(d[i], 0xff, sz[i]));
  MOE_OK_OR_FAIL(moe_route(&p, (const float*)d[B_LOGITS], (int32_t*)d[B_IDX], (float*)d[B_W],
                           (int32_t*)d[B_COUNTS], ws, ws_bytes, NULL));
  MOE_OK_OR_FAIL(moe_assign_replicas(&p, (const int32_t*)d[B_COUNTS], NULL, 1,
                                     (int32_t*)d[B_ASSIGN], (int32_t*)d[B_ACTIVE], NULL));
  MOE_OK_OR_FAIL(moe_layout_single_send(
      &p, (const int32_t*)d[B_IDX], (const int32_t*)d[B_ASSIGN], NULL, 1, (int32_t*)d[B_RANK_OF],
      (int32_t*)d[B_EOFF], (int32_t*)d[B_ROFF], (int32_t*)d[B_POS], (int32_t*)d[B_SRC],
      (int32_t*)d[B_DEDUP], (int32_t*)d[B_SSOFF], (int32_t*)d[B_SSROW], (int32_t*)d[B_SSTOK], ws,
      ws_bytes, NULL));
  HIP_OK(hipDeviceSynchronize());
  for (int i = B_IDX; i <= B_SSTOK; ++i) {
    HIP_OK(hipMemcpy(h[i], d[i], sz[i], hipMemcpyDeviceToHost));
    if (memcmp(h[i], a[i], sz[i]) != 0)
      FAIL("moe_route_assign_layout_single_send differs from the three calls (buffer %d)", i);
  }

  /* 3. the allocation-free plan writes the same tables */
  for (int c = 0; c < kNPlanOut; ++c) HIP_OK(hipMemset(d[kPlanOut[c]], 0xff, sz[kPlanOut[c]]));
  MOE_OK_OR_FAIL(moe_route_assign_layout_noalloc(
      &p, (const float*)d[B_LOGITS], NULL, 1, (int32_t*)d[B_IDX], (float*)d[B_W],
      (int32_t*)d[B_COUNTS], (int32_t*)d[B_ASSIGN], (int32_t*)d[B_ACTIVE], (int32_t*)d[B_RANK_OF],
      (int32_t*)d[B_EOFF], (int32_t*)d[B_ROFF], (int32_t*)d[B_POS], (int32_t*)d[B_SRC],
      (int32_t*)d[B_DEDUP], NULL));
  HIP_OK(hipDeviceSynchronize());
  for (int c = 0; c < kNPlanOut; ++c) {
    const int i = kPlanOut[c];
    HIP_OK(hipMemcpy(a[i], d[i], sz[i], hipMemcpyDeviceToHost));
    if (memcmp(h[i], a[i], sz[i]) != 0)
      FAIL("moe_route_assign_layout_noalloc differs from the three calls (buffer %d)", i);
  }

  /* 4. the single-send layout: one row per (token, rank), the rank's rows in
     token order, every slot of a token on that rank pointing at it */
  {
    const int32_t* idx = (const int32_t*)h[B_IDX];
    const int32_t* rank_of = (const int32_t*)h[B_RANK_OF];
    const int32_t* dedup = (const int32_t*)h[B_DEDUP];
    const int32_t* off = (const int32_t*)h[B_SSOFF];
    const int32_t* row = (const int32_t*)h[B_SSROW];
    const int32_t* tok = (const int32_t*)h[B_SSTOK];
    const int32_t* pos = (const int32_t*)h[B_POS];
    int pairs = 0;
    /* every index the host checks below dereferences, in range first */
    for (int i = 0; i < n; ++i)
      if (idx[i] < 0 || idx[i] >= E || pos[i] < 0 || pos[i] >= n || row[i] < 0 || row[i] >= n)
        FAIL("pair %d: idx %d, pos %d or ss_row %d out of range", i, idx[i], pos[i], row[i]);
    for (int q = 0; q < R; ++q)
      if (off[q + 1] < off[q] || off[q + 1] > n) FAIL("ss_rank_offsets not ascending within [0, %d]", n);
    for (int e = 0; e < E; ++e)
      if (rank_of[e] != e / PER) FAIL("rank_of[%d] = %d without a replica table", e, rank_of[e]);
    if (off[0] != 0) FAIL("ss_rank_offsets[0] = %d", off[0]);
    for (int q = 0; q < R; ++q)
      if (off[q + 1] - off[q] != dedup[q]) FAIL("rank %d holds %d single-send rows, dedup %d", q,
                                                off[q + 1] - off[q], dedup[q]);
    for (int t = 0; t < T; ++t) {
      for (int j = 0; j < K; ++j) {
        const int q = rank_of[idx[t * K + j]];
        const int r = row[t * K + j];
        int first = 1;
        if (r < off[q] || r >= off[q + 1]) FAIL("ss_row of token %d slot %d outside rank %d", t, j, q);
        if (tok[r] != t) FAIL("ss_token[%d] = %d, expected %d", r, tok[r], t);
        for (int jj = 0; jj < j; ++jj) {
          if (rank_of[idx[t * K + jj]] == q) {
            first = 0;
            if (row[t * K + jj] != r) FAIL("token %d: slots %d and %d share rank %d but not a row", t, jj, j, q);
          }
        }
        pairs += first;
      }
    }
    if (pairs != off[R]) FAIL("%d (token, rank) pairs against %d single-send rows", pairs, off[R]);
    for (int q = 0; q < R; ++q)
      for (int r = off[q] + 1; r < off[q + 1]; ++r)
        if (tok[r] <= tok[r - 1]) FAIL("rank %d's single-send rows out of token order at %d", q, r);
  }

  /* 5. single-send dispatch, then the fan-out, equal the plain dispatch */
  HIP_OK(hipMemset(d[B_SEND2], 0, sz[B_SEND2]));
  MOE_OK_OR_FAIL(moe_dispatch(&p, d[B_X], (const int32_t*)d[B_POS], d[B_SEND], NULL));
  MOE_OK_OR_FAIL(moe_single_send_dispatch(&p, d[B_X], (const int32_t*)d[B_SSROW], d[B_SEND_SS], n, NULL));
  MOE_OK_OR_FAIL(moe_single_send_expand(&p, d[B_SEND_SS], (const int32_t*)d[B_SSOFF],
                                        (const int32_t*)d[B_SSTOK], (const int32_t*)d[B_SSROW],
                                        (const int32_t*)d[B_POS], n, d[B_SEND2], NULL));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(h[B_SEND], d[B_SEND], sz[B_SEND], hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h[B_SEND_SS], d[B_SEND_SS], sz[B_SEND_SS], hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h[B_SEND2], d[B_SEND2], sz[B_SEND2], hipMemcpyDeviceToHost));
  if (memcmp(h[B_SEND2], h[B_SEND], sz[B_SEND]) != 0) FAIL("the fan-out differs from moe_dispatch");
  {
    const int32_t* row = (const int32_t*)h[B_SSROW];
    const uint16_t* ss = (const uint16_t*)h[B_SEND_SS];
    const uint16_t* x = (const uint16_t*)h[B_X];
    for (int i = 0; i < n; ++i)
      if (memcmp(ss + (size_t)row[i] * H, x + (size_t)(i / K) * H, 2u * H) != 0)
        FAIL("single-send row %d is not token %d's row", row[i], i / K);
  }

  /* 6. backward: dy = round16(w dout), dw = <y, dout>, dx = sum of the
     token's dy rows; dout is x */
  MOE_OK_OR_FAIL(moe_expert_standin(&p, d[B_SEND], (const int32_t*)d[B_SRC],
                                    (const int32_t*)d[B_IDX], d[B_Y], NULL));
  MOE_OK_OR_FAIL(moe_combine_backward(&p, d[B_X], d[B_Y], (const int32_t*)d[B_POS],
                                      (const float*)d[B_W], d[B_DY], (float*)d[B_DW], NULL));
  MOE_OK_OR_FAIL(moe_dispatch_backward(&p, d[B_DY], (const int32_t*)d[B_POS], d[B_DX], NULL));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(h[B_Y], d[B_Y], sz[B_Y], hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h[B_DY], d[B_DY], sz[B_DY], hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h[B_DW], d[B_DW], sz[B_DW], hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h[B_DX], d[B_DX], sz[B_DX], hipMemcpyDeviceToHost));
  {
    const int32_t* pos = (const int32_t*)h[B_POS];
    const float* w = (const float*)h[B_W];
    const float* dw = (const float*)h[B_DW];
    const uint16_t* x = (const uint16_t*)h[B_X];
    const uint16_t* y = (const uint16_t*)h[B_Y];
    const uint16_t* dy = (const uint16_t*)h[B_DY];
    const uint16_t* dx = (const uint16_t*)h[B_DX];
    for (int i = 0; i < n; ++i) {
      const int t = i / K;
      const size_t r = (size_t)pos[i];
      double dot = 0.0, mag = 0.0;
      for (int c = 0; c < H; ++c) {
        const double g = bf16_val(x[(size_t)t * H + c]);
        /* one fp32 product, one rounding to bf16: bit for bit */
        const uint16_t want = bf16_rne(w[i] * (float)g);
        if (dy[r * H + c] != want)
          FAIL("dy row %zu chunk %d: %g against %g", r, c, bf16_val(dy[r * H + c]), bf16_val(want));
        dot += bf16_val(y[r * H + c]) * g;
        mag += fabs(bf16_val(y[r * H + c]) * g);
      }
      if (fabs((double)dw[i] - dot) > 1e-5 * mag + 1e-30) FAIL("dw[%d] = %g against %g", i, dw[i], dot);
    }
    for (int t = 0; t < T; ++t) {
      for (int c = 0; c < H; ++c) {
        double want = 0.0, mag = 0.0;
        for (int j = 0; j < K; ++j) {
          const double v = bf16_val(dy[(size_t)pos[t * K + j] * H + c]);
          want += v;
          mag += fabs(v);
        }
        /* fp32 sums of k terms, one rounding to bf16 (8 significant bits:
           half a unit in the last place is at most 2^-8 of the value) */
        if (fabs(bf16_val(dx[(size_t)t * H + c]) - want) > fabs(want) / 256 + 1e-6 * mag)
          FAIL("dx[%d][%d] = %g against %g", t, c, bf16_val(dx[(size_t)t * H + c]), want);
      }
    }
  }

  /* 7. routing statistics: counts exact, ratios from the same integers */
  MOE_OK_OR_FAIL(moe_routing_stats(&p, (const int32_t*)d[B_IDX], (const int32_t*)d[B_COUNTS],
                                   (const int32_t*)d[B_RANK_OF], (int32_t*)d[B_SCOUNTS],
                                   (int32_t*)d[B_COSEL], (double*)d[B_STATS], NULL));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(h[B_SCOUNTS], d[B_SCOUNTS], sz[B_SCOUNTS], hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h[B_COSEL], d[B_COSEL], sz[B_COSEL], hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h[B_STATS], d[B_STATS], sz[B_STATS], hipMemcpyDeviceToHost));
  {
    const int32_t* idx = (const int32_t*)h[B_IDX];
    const int32_t* counts = (const int32_t*)h[B_COUNTS];
    const int32_t* rank_of = (const int32_t*)h[B_RANK_OF];
    const int32_t* S = (const int32_t*)h[B_SCOUNTS];
    const int32_t* C = (const int32_t*)h[B_COSEL];
    const double* st = (const double*)h[B_STATS];
    int wantS[R * R], wantC[E * E], load[R];
    double gsum = 0.0, dev2 = 0.0, want[4];
    int maxc = 0, diag = 0;
    memset(wantS, 0, sizeof(wantS));
    memset(wantC, 0, sizeof(wantC));
    memset(load, 0, sizeof(load));
    for (int t = 0; t < T; ++t) {
      const int s = (int)((long)t * R / T);
      for (int j = 0; j < K; ++j) {
        ++wantS[s * R + rank_of[idx[t * K + j]]];
        for (int jj = 0; jj < K; ++jj) {
          const int ea = idx[t * K + j], eb = idx[t * K + jj];
          if (ea < eb) ++wantC[ea * E + eb];
        }
      }
    }
    if (memcmp(S, wantS, sizeof(wantS)) != 0) FAIL("send-counts matrix");
    if (memcmp(C, wantC, sizeof(wantC)) != 0) FAIL("co-selection histogram");
    for (int e = 0; e < E; ++e) maxc = counts[e] > maxc ? counts[e] : maxc;
    for (int s = 0; s < R; ++s)
      for (int q = 0; q < R; ++q) load[q] += wantS[s * R + q];
    for (int q = 0; q < R; ++q) diag += wantS[q * R + q];
    for (int i = 0; i < R; ++i)
      for (int j = 0; j < R; ++j) gsum += fabs((double)(load[i] - load[j]));
    for (int q = 0; q < R; ++q) {
      const double dq = (double)load[q] / n - 1.0 / R;
      dev2 += dq * dq;
    }
    want[0] = maxc / ((double)n / E);
    want[1] = gsum / (2.0 * R * n);
    want[2] = dev2 == 0.0 ? INFINITY : ((R - 1.0) / (R * dev2) - 1.0) / R;
    want[3] = (double)diag / n;
    for (int i = 0; i < 4; ++i)
      if (!(fabs(st[i] - want[i]) <= 1e-12 * fabs(want[i]) || st[i] == want[i]))
        FAIL("stats[%d] = %.17g against %.17g", i, st[i], want[i]);
  }

  /* 8. token-balanced split without a replica table: every pair on its
     expert's one rank */
  MOE_OK_OR_FAIL(moe_token_balanced_split(&p, (const int32_t*)d[B_IDX], (const int32_t*)d[B_COUNTS],
                                          (const int32_t*)d[B_POS], (const int32_t*)d[B_EOFF], NULL,
                                          1, (int32_t*)d[B_GOP], (int32_t*)d[B_BACT],
                                          (int32_t*)d[B_BTOK], NULL));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(h[B_GOP], d[B_GOP], sz[B_GOP], hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h[B_BACT], d[B_BACT], sz[B_BACT], hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h[B_BTOK], d[B_BTOK], sz[B_BTOK], hipMemcpyDeviceToHost));
  {
    const int32_t* idx = (const int32_t*)h[B_IDX];
    const int32_t* counts = (const int32_t*)h[B_COUNTS];
    const int32_t* gop = (const int32_t*)h[B_GOP];
    const int32_t* act = (const int32_t*)h[B_BACT];
    const int32_t* tok = (const int32_t*)h[B_BTOK];
    for (int i = 0; i < n; ++i)
      if (gop[i] != idx[i] / PER) FAIL("gpu_of_pair[%d] = %d, expert %d", i, gop[i], idx[i]);
    for (int q = 0; q < R; ++q) {
      int wt = 0, wa = 0;
      for (int e = q * PER; e < (q + 1) * PER; ++e) {
        wt += counts[e];
        wa += counts[e] > 0;
      }
      if (tok[q] != wt || act[q] != wa) FAIL("rank %d: %d pairs / %d active, expected %d / %d", q,
                                             tok[q], act[q], wt, wa);
    }
  }
  printf("c-abi check (rest) ok: T=%d E=%d k=%d H=%d R=%d\n", T, E, K, H, R);

done:
  for (int i = 0; i < B_COUNT; ++i) {
    hipFree(d[i]);
    free(h[i]);
    free(a[i]);
  }
  hipFree(ws);
  return rc;
}
