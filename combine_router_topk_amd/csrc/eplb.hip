// Token-balanced (EPLB-style) replica routing: the baseline that the METRO
// greedy assignment is compared against.
//
// "METRO AllGather vs AllToAll for MoE decode", section "Add the
// expert-weight traffic term": spreading an expert's tokens over all of its
// replicas balances tokens but activates more replicas per GPU than
// grouping them on one replica; the greedy is reported against EPLB's token
// routing.
//
// The n pairs routed to expert e, in the order of e's send segment (token
// order), are cut into contiguous shares over e's m valid replicas (entries
// in [0, R), in table order): replica j takes n / m pairs, one more when
// j < n mod m. Without a replica table an expert has one copy, on rank
// e / (E / R).
//
// Two kernels:
//  1. split_pairs: one pair per thread; the pair's place among its expert's
//     pairs is its row in the expert's segment (pos - expert_offsets[e]),
//     and the share index follows in closed form.
//  2. split_summary (one workgroup): per GPU, the activated replicas (shares
//     that are not empty) and the pairs served, from the counts alone.
#include "device.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kSplitThreads = 256;
constexpr int kSummaryThreads = 1024;

// Expert e's replica row in registers, every slot's load issued before any
// is used (the test on the slot is uniform); slots past maxrep hold -1.
__device__ __forceinline__ void rep_row(const int32_t* __restrict__ rep, int e, int maxrep,
                                        int (&x)[kMaxK]) {
  const int32_t* row = rep + (size_t)e * maxrep;
#pragma unroll
  for (int s = 0; s < kMaxK; ++s) x[s] = s < maxrep ? row[s] : -1;
}

// The j-th valid replica (entries in [0, R), table order) of a row in
// registers, -1 if there is none, and the number of valid replicas.
__device__ __forceinline__ int nth_replica(const int (&x)[kMaxK], int R, int j, int* m_out) {
  int m = 0, g_j = -1;
#pragma unroll
  for (int s = 0; s < kMaxK; ++s) {
    const bool ok = x[s] >= 0 && x[s] < R;
    if (ok && m == j) g_j = x[s];
    m += ok ? 1 : 0;
  }
  *m_out = m;
  return g_j;
}

// Replica index taking the i-th of n pairs under contiguous shares n / m
// (+1 for the first n mod m replicas); i is clamped into [0, n).
__device__ __forceinline__ int share_index(int i, int n, int m) {
  i = i < 0 ? 0 : (i >= n ? n - 1 : i);
  const int q = n / m, rem = n % m;
  const int edge = rem * (q + 1);
  return i < edge ? i / (q + 1) : rem + (i - edge) / q;
}

__global__ __launch_bounds__(kSplitThreads) void split_pairs_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ expert_offsets,
    const int32_t* __restrict__ rep, int maxrep, int n_pairs, int E, int R,
    int32_t* __restrict__ gpu_of_pair) {
  const int i = blockIdx.x * kSplitThreads + threadIdx.x;
  if (i >= n_pairs) return;
  int e = idx[i];
  int p = pos[i];
  asm volatile("" : "+v"(p));  // p's load stays beside idx's, not under the tests below
  e = e < 0 ? 0 : (e >= E ? E - 1 : e);
  const int n = counts[e];
  if (rep == nullptr) {
    gpu_of_pair[i] = e / (E / R);
    return;
  }
  int off = expert_offsets[e];
  int x[kMaxK];
  rep_row(rep, e, maxrep, x);
  asm volatile("" : "+v"(off));  // off's load stays beside counts' and the row's
  int m = 0;
  (void)nth_replica(x, R, -1, &m);
  if (m == 0 || n <= 0) {
    gpu_of_pair[i] = -1;  // no valid replica (or inconsistent counts)
    return;
  }
  const int j = share_index(p - off, n, m);
  int m2 = 0;
  gpu_of_pair[i] = nth_replica(x, R, j, &m2);
}

__global__ __launch_bounds__(kSummaryThreads) void split_summary_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ rep, int maxrep, int E, int R,
    int32_t* __restrict__ active, int32_t* __restrict__ tokens) {
  __shared__ int s_act[kMaxR];
  __shared__ int s_tok[kMaxR];
  for (int r = threadIdx.x; r < R; r += kSummaryThreads) {
    s_act[r] = 0;
    s_tok[r] = 0;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kSummaryThreads) {
    const int n = counts[e];
    if (rep == nullptr) {  // uniform
      if (n > 0) {
        const int g = e / (E / R);
        atomicAdd(&s_act[g], 1);
        atomicAdd(&s_tok[g], n);
      }
      continue;
    }
    int x[kMaxK];
    rep_row(rep, e, maxrep, x);
    int m = 0;
    (void)nth_replica(x, R, -1, &m);
    // shares over the valid replicas in table order; a slot adds 0 when it
    // is not a valid replica, its share is empty or the expert has no pairs
    // (no test on n before the row is used, so its loads stay beside n's)
    const int mm = m > 0 ? m : 1;
    const int q = n / mm, rem = n % mm;
    int j = 0;
    for (int s = 0; s < maxrep; ++s) {
      const int g = x[s < kMaxK ? s : kMaxK - 1];
      const bool ok = g >= 0 && g < R;
      const int share = q + (j < rem ? 1 : 0);
      const bool on = ok && n > 0 && share > 0;
      const int gc = ok ? g : 0;
      atomicAdd(&s_act[gc], on ? 1 : 0);
      atomicAdd(&s_tok[gc], on ? share : 0);
      j += ok ? 1 : 0;
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += kSummaryThreads) {
    active[r] = s_act[r];
    tokens[r] = s_tok[r];
  }
}

}  // namespace

hipError_t launch_token_balanced_split(const int32_t* idx, const int32_t* counts,
                                       const int32_t* pos, const int32_t* expert_offsets,
                                       const int32_t* rep, int maxrep, int T, int E, int k, int R,
                                       int32_t* gpu_of_pair, int32_t* active, int32_t* tokens,
                                       hipStream_t s) {
  const int n = T * k;
  if (n > 0 && gpu_of_pair != nullptr) {
    split_pairs_kernel<<<(n + kSplitThreads - 1) / kSplitThreads, kSplitThreads, 0, s>>>(
        idx, counts, pos, expert_offsets, rep, maxrep, n, E, R, gpu_of_pair);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  split_summary_kernel<<<1, kSummaryThreads, 0, s>>>(counts, rep, maxrep, E, R, active, tokens);
  return hipGetLastError();
}

}  // namespace moe
