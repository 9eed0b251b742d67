// Routing statistics of one batch: the send-counts matrix S, the expert
// co-selection pair histogram C, and four scalar summaries.
//
// "Diagnosing Overhead in Dispatch Operations: Cross-architecture
// Observatory", section "Methodology" (per-expert max/mean, Gini of the
// per-rank load, a fitted symmetric Dirichlet alpha, all summaries of the
// send-counts matrix); news summary of correlated expert placement and token
// shuffling, sections "Correlations in router choices" (expert pairs chosen
// together) and "Two locality techniques" (the share of assignments served on
// the token's own GPU).
//
// Token t comes from virtual rank floor(t R / T); S[s][d] counts the (token,
// slot) pairs from source rank s whose expert sits on rank d. C[a][b]
// (a < b) counts the tokens that chose both a and b.
//
// Three kernels:
//  1. stats_zero: clears S and C (a fill kernel, so a captured graph holds
//     no memset node).
//  2. stats_count: one token per thread over a grid of token chunks by row
//     slices of C; each block counts its slice of C in LDS and adds it to C
//     once; S is counted in LDS when it fits (else with atomics straight into
//     S). Integer adds commute, so the counts do not depend on the order.
//  3. stats_finalize (one workgroup): the expert maximum, the per-rank loads
//     (column sums of S), the trace, and the Gini and Dirichlet sums, all in
//     exact 64-bit integers; then a handful of fp64 operations for the four
//     ratios.
#include <algorithm>

#include "device.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kStatThreads = 256;
constexpr int kFinalThreads = 1024;
constexpr int kLdsMatrixInts = 7936;  // S up to this size is counted in LDS
constexpr int kSliceInts = 8192;      // LDS ints of one row slice of C (32 KiB) at most
constexpr int kCountLdsInts = 16384;  // the count kernel's LDS (64 KiB) at most
constexpr int kCountBlocks = 1024;    // target grid size of the count kernel

__global__ __launch_bounds__(kStatThreads) void stats_zero_kernel(int32_t* __restrict__ S, int64_t nS,
                                                                 int32_t* __restrict__ C, int64_t nC) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nS; i += stride) S[i] = 0;
  if (C != nullptr)
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nC; i += stride) C[i] = 0;
}

__device__ __forceinline__ int clamp_id(int v, int n) { return v < 0 ? 0 : (v >= n ? n - 1 : v); }

// Blocks form a grid of token chunks (x) by row slices of C (y): block
// (x, y) reads the tokens of chunk x and counts, in LDS, the pairs whose
// smaller expert a lies in slice y (a0 <= a < a0 + rows), so every slice of
// C fits in LDS whatever E is; the slice's nonzero cells are then added to
// C once per block. Blocks of slice 0 also count S (in LDS when it fits,
// else with atomics straight into S).
template <bool S_LDS>
__global__ __launch_bounds__(kStatThreads) void stats_count_kernel(
    const int32_t* __restrict__ idx, int T, int E, int k, int R, int tpb, int slice_rows,
    const int32_t* __restrict__ rank_of, int32_t* __restrict__ S, int32_t* __restrict__ C) {
  extern __shared__ int smem[];
  int* s_rank = smem;                              // [E]
  int* s_S = smem + E;                             // [R*R] when S_LDS
  int* s_C = s_S + (S_LDS ? R * R : 0);            // [slice_rows*E] when C is counted
  const bool do_s = blockIdx.y == 0;
  const bool do_c = C != nullptr;
  const int a0 = blockIdx.y * slice_rows;
  const int rows = min(slice_rows, E - a0);
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_rank[e] = clamp_id(rank_of[e], R);
  if constexpr (S_LDS)
    if (do_s)
      for (int i = threadIdx.x; i < R * R; i += blockDim.x) s_S[i] = 0;
  if (do_c)
    for (int i = threadIdx.x; i < rows * E; i += blockDim.x) s_C[i] = 0;
  __syncthreads();

  const int t0 = blockIdx.x * tpb;
  const int t1 = min(T, t0 + tpb);
  for (int t = t0 + threadIdx.x; t < t1; t += blockDim.x) {
    int e[kMaxK];
    load_slots(idx + (size_t)t * k, k, e);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) e[j] = j < k ? clamp_id(e[j], E) : 0;
    if (do_s) {
      const int src = static_cast<int>((int64_t)t * R / T);
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (j < k) {
          const int cell = src * R + s_rank[e[j]];
          if constexpr (S_LDS) atomicAdd(&s_S[cell], 1);
          else atomicAdd(&S[cell], 1);
        }
      }
    }
    if (do_c) {
#pragma unroll
      for (int i = 0; i < kMaxK; ++i) {
#pragma unroll
        for (int j = i + 1; j < kMaxK; ++j) {
          if (j < k) {
            const int a = min(e[i], e[j]) - a0, b = max(e[i], e[j]);
            // a + a0 == b only for out-of-range ids clamped to one value
            if (static_cast<unsigned>(a) < static_cast<unsigned>(rows) && a + a0 != b)
              atomicAdd(&s_C[a * E + b], 1);
          }
        }
      }
    }
  }
  __syncthreads();
  if constexpr (S_LDS)
    if (do_s)
      for (int i = threadIdx.x; i < R * R; i += blockDim.x)
        if (s_S[i] != 0) atomicAdd(&S[i], s_S[i]);
  if (do_c)
    for (int i = threadIdx.x; i < rows * E; i += blockDim.x)
      if (s_C[i] != 0) atomicAdd(&C[(size_t)a0 * E + i], s_C[i]);
}

// Block sums of three 64-bit integers at once: the three butterflies are
// independent, so their exchanges overlap, and one barrier serves all three.
__device__ __forceinline__ void block_sum3_i64(int64_t (&v)[3], int64_t (*s_red)[3]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  for (int off = kWave / 2; off > 0; off /= 2) {
#pragma unroll
    for (int i = 0; i < 3; ++i) v[i] += __shfl_xor(v[i], off);
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < 3; ++i) s_red[wave][i] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    int64_t all = 0;
    for (int w = 0; w < kFinalThreads / kWave; ++w) all += s_red[w][i];
    v[i] = all;
  }
}

__global__ __launch_bounds__(kFinalThreads) void stats_finalize_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ S, int T, int E, int k, int R,
    double* __restrict__ stats) {
  __shared__ int64_t s_load[kMaxR];
  __shared__ int64_t s_red[kFinalThreads / kWave][3];
  __shared__ int s_part[kFinalThreads];
  const int tid = threadIdx.x;  // E, R <= 1024 == blockDim.x
  const int64_t N = (int64_t)T * k;
  int64_t my_max = 0, diag = 0, load = 0;
  if (tid < E) my_max = counts[tid];
  if (tid < R) diag = S[(size_t)tid * R + tid];  // in flight with the column loads
  // column sums of S: G = 1024 / R groups of rows, each thread summing one
  // column over its group's rows with several loads in flight, then the
  // group partials added in order
  const int G = R >= kFinalThreads ? 1 : kFinalThreads / R;
  if (tid < G * R) {
    const int c = tid % R, g = tid / R;
    int part = 0;
#pragma unroll 8
    for (int s = g; s < R; s += G) part += S[(size_t)s * R + c];
    s_part[tid] = part;
  }
  __syncthreads();
  if (tid < R) {
    for (int g = 0; g < G; ++g) load += s_part[g * R + tid];
    s_load[tid] = load;
  }
  __syncthreads();
  // block maximum of the counts
  for (int off = kWave / 2; off > 0; off /= 2) {
    const int64_t o = __shfl_xor(my_max, off);
    my_max = o > my_max ? o : my_max;
  }
  __shared__ int64_t s_max[kFinalThreads / kWave];
  if ((tid & (kWave - 1)) == 0) s_max[tid / kWave] = my_max;
  __syncthreads();
  int64_t cmax = 0;
  for (int w = 0; w < kFinalThreads / kWave; ++w) cmax = s_max[w] > cmax ? s_max[w] : cmax;
  // sum over j of |L_i - L_j| for this rank i, and L_i^2
  int64_t absdiff = 0, sq = 0;
  if (tid < R) {
    for (int j = 0; j < R; ++j) {
      const int64_t d = load - s_load[j];
      absdiff += d < 0 ? -d : d;
    }
    sq = load * load;
  }
  int64_t sums[3] = {diag, absdiff, sq};
  block_sum3_i64(sums, s_red);
  const int64_t trace = sums[0], gini_num = sums[1], sum_sq = sums[2];
  if (tid == 0) {
    const double nan = __builtin_nan("");
    if (N == 0) {
      stats[0] = stats[1] = stats[2] = stats[3] = nan;
      return;
    }
    const double Nd = static_cast<double>(N);
    stats[0] = static_cast<double>(cmax * E) / Nd;
    stats[1] = static_cast<double>(gini_num) / (2.0 * static_cast<double>(R) * Nd);
    const int64_t dev = (int64_t)R * sum_sq - N * N;  // K sum L^2 - N^2, exact
    if (dev == 0) {
      stats[2] = __builtin_inf();
    } else {
      const double K = static_cast<double>(R);
      const double D = static_cast<double>(dev) / (K * Nd * Nd);
      stats[2] = (static_cast<double>(R - 1) / (K * D) - 1.0) / K;
    }
    stats[3] = static_cast<double>(trace) / Nd;
  }
}

}  // namespace

hipError_t launch_routing_stats(const int32_t* idx, const int32_t* rank_of, const int32_t* counts,
                                int T, int E, int k, int R, int32_t* S, int32_t* C, double* stats,
                                hipStream_t s) {
  const int64_t nS = (int64_t)R * R, nC = C != nullptr ? (int64_t)E * E : 0;
  const int64_t nz = nS > nC ? nS : nC;
  const int zgrid = static_cast<int>(std::min<int64_t>(1024, (nz + kStatThreads - 1) / kStatThreads));
  stats_zero_kernel<<<zgrid, kStatThreads, 0, s>>>(S, nS, C, nC);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (T > 0) {
    // C in row slices of at most kSliceInts ints (all of C in one slice when
    // it fits), within kCountLdsInts together with the rank table and S
    // (with E <= 1024 and S <= kLdsMatrixInts at least 7 rows remain); about
    // kCountBlocks blocks, token chunks whole multiples of the block size
    const bool s_lds = nS <= kLdsMatrixInts;
    const int slice_ints = std::min<int64_t>(kSliceInts, kCountLdsInts - E - (s_lds ? nS : 0));
    const int slice_rows = C != nullptr ? std::max(1, std::min(E, slice_ints / E)) : E;
    const int nslice = C != nullptr ? (E + slice_rows - 1) / slice_rows : 1;
    const int nchunk_want = std::max(1, kCountBlocks / nslice);
    int tpb = (T + nchunk_want - 1) / nchunk_want;
    tpb = ((tpb + kStatThreads - 1) / kStatThreads) * kStatThreads;
    const int nchunk = (T + tpb - 1) / tpb;
    const size_t lds = (E + (s_lds ? nS : 0) + (C != nullptr ? (int64_t)slice_rows * E : 0)) * sizeof(int);
    const dim3 grid(nchunk, nslice);
    if (s_lds)
      stats_count_kernel<true><<<grid, kStatThreads, lds, s>>>(idx, T, E, k, R, tpb, slice_rows, rank_of, S, C);
    else
      stats_count_kernel<false><<<grid, kStatThreads, lds, s>>>(idx, T, E, k, R, tpb, slice_rows, rank_of, S, C);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  stats_finalize_kernel<<<1, kFinalThreads, 0, s>>>(counts, S, T, E, k, R, stats);
  return hipGetLastError();
}

}  // namespace moe
