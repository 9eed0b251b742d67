// Dispatch layout: destination rank per expert, segment offsets, the stable
// permutation of (token, slot) pairs into send rows, and single-send dedup
// counts.
//
// "METRO AllGather vs AllToAll for MoE decode", section "Work the 8-GPU
// payload example" (an all-to-all sends each destination rank its own chunk)
// and section "Distinguish METRO from backend names" (variable-size
// all-to-all driven by per-destination counts); news summary of correlated
// expert placement and token shuffling, section "Two locality techniques"
// (a single-send dispatcher sends a token to a GPU at most once).
//
// The send buffer holds exactly T*k rows: ranks in order, inside a rank the
// experts by id, inside an expert the pairs by (token, slot).
//
// Three kernels, no global atomics:
//  1. layout_count: per block of tokens, an LDS histogram of the selected
//     experts and of the distinct destination ranks per token (dedup), each
//     written as one row of a [blocks, E] / [blocks, R] matrix.
//  2. layout_plan (one workgroup): rank of every expert; per-expert totals and
//     the exclusive scan of the expert histogram over blocks (in place);
//     expert and rank offsets in (rank, expert) order; dedup totals.
//  3. layout_permute: per block, the stable rank of each pair among the
//     block's pairs with the same expert: inside a wave by matching expert
//     ids with one ballot per id bit and counting lower lanes; across the
//     block's waves by per-wave counts in LDS; across rounds by running
//     per-expert cursors. pos = cursor + rank, src[pos] = flat pair index.
#include "device.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kCountThreads = 256;
constexpr int kPlanThreads = 1024;
constexpr int kPermThreads = 256;
constexpr int kPermWaves = kPermThreads / kWave;

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

__global__ __launch_bounds__(kCountThreads) void layout_count_kernel(
    const int32_t* __restrict__ idx, int T, int E, int k, int R, int tpb,
    const int32_t* __restrict__ assign, const int32_t* __restrict__ rep, int maxrep,
    int32_t* __restrict__ hist, int32_t* __restrict__ ded) {
  extern __shared__ int smem[];
  int* s_rank = smem;        // [E]
  int* s_hist = smem + E;    // [E]
  int* s_ded = smem + 2 * E; // [R]
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    s_rank[e] = expert_rank(e, E, R, assign, rep, maxrep);
    s_hist[e] = 0;
  }
  for (int r = threadIdx.x; r < R; r += blockDim.x) s_ded[r] = 0;
  __syncthreads();

  const int t0 = blockIdx.x * tpb;
  const int t1 = min(T, t0 + tpb);
  const size_t i0 = (size_t)t0 * k, i1 = (size_t)t1 * k;
  for (size_t i = i0 + threadIdx.x; i < i1; i += blockDim.x)
    atomicAdd(&s_hist[clamp_expert(idx[i], E)], 1);
  for (int t = t0 + threadIdx.x; t < t1; t += blockDim.x) {
    const int32_t* row = idx + (size_t)t * k;
    for (int j = 0; j < k; ++j) {
      const int r = s_rank[clamp_expert(row[j], E)];
      bool seen = false;
      for (int jj = 0; jj < j; ++jj) seen |= (s_rank[clamp_expert(row[jj], E)] == r);
      if (!seen) atomicAdd(&s_ded[r], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(size_t)blockIdx.x * E + e] = s_hist[e];
  for (int r = threadIdx.x; r < R; r += blockDim.x) ded[(size_t)blockIdx.x * R + r] = s_ded[r];
}

// Column totals of M[rows, cols] into tot[] (LDS); with `scan`, M is replaced
// by its exclusive prefix over rows, column by column. 16 waves split the rows
// into segments; lanes are columns (64 at a time).
__device__ void column_scan(int32_t* __restrict__ M, int rows, int cols, bool scan, int* tot,
                            int (*part)[kWave]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nw = kPlanThreads / kWave;
  const int seg = (rows + nw - 1) / nw;
  const int r_lo = min(rows, wave * seg), r_hi = min(rows, r_lo + seg);
  for (int c0 = 0; c0 < cols; c0 += kWave) {
    const int c = c0 + lane;
    int s = 0;
    if (c < cols)
      for (int r = r_lo; r < r_hi; ++r) s += M[(size_t)r * cols + c];
    part[wave][lane] = s;
    __syncthreads();
    int pre = 0, all = 0;
    for (int w = 0; w < nw; ++w) {
      const int v = part[w][lane];
      pre += (w < wave) ? v : 0;
      all += v;
    }
    if (c < cols) {
      if (wave == 0) tot[c] = all;
      if (scan) {
        int run = pre;
        for (int r = r_lo; r < r_hi; ++r) {
          const size_t o = (size_t)r * cols + c;
          const int v = M[o];
          M[o] = run;
          run += v;
        }
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kPlanThreads) void layout_plan_kernel(
    int T, int E, int k, int R, int nblk, int32_t* __restrict__ hist, const int32_t* __restrict__ ded,
    const int32_t* __restrict__ assign, const int32_t* __restrict__ rep, int maxrep,
    int32_t* __restrict__ rank_of, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ dedup) {
  __shared__ int s_rank[kMaxE];
  __shared__ int s_cnt[kMaxE];
  __shared__ int s_ded[kMaxR];
  __shared__ int part[kPlanThreads / kWave][kWave];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) {
    const int r = expert_rank(e, E, R, assign, rep, maxrep);
    s_rank[e] = r;
    rank_of[e] = r;
  }
  column_scan(hist, nblk, E, true, s_cnt, part);
  column_scan(const_cast<int32_t*>(ded), nblk, R, false, s_ded, part);
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    const int r = s_rank[e];
    int acc = 0;
    for (int e2 = 0; e2 < E; ++e2) {
      const int r2 = s_rank[e2];
      acc += (r2 < r || (r2 == r && e2 < e)) ? s_cnt[e2] : 0;
    }
    expert_offsets[e] = acc;
  }
  for (int r = tid; r <= R; r += blockDim.x) {
    int acc = 0;
    for (int e2 = 0; e2 < E; ++e2) acc += (s_rank[e2] < r) ? s_cnt[e2] : 0;
    rank_offsets[r] = acc;
  }
  for (int r = tid; r < R; r += blockDim.x) dedup[r] = s_ded[r];
}

__global__ __launch_bounds__(kPermThreads) void layout_permute_kernel(
    const int32_t* __restrict__ idx, int T, int E, int k, int tpb, const int32_t* __restrict__ base,
    const int32_t* __restrict__ expert_offsets, int32_t* __restrict__ pos,
    int32_t* __restrict__ src) {
  extern __shared__ int smem[];
  int* run = smem;                       // [E] next free row of each expert
  int* wcnt = smem + E;                  // [waves][E] pairs per expert in a wave
  int* wtag = smem + E + kPermWaves * E; // [waves][E] round that wrote wcnt
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    run[e] = expert_offsets[e] + base[(size_t)b * E + e];
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) wtag[w * E + e] = 0;
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nbits = E > 1 ? 32 - __builtin_clz((unsigned)(E - 1)) : 0;
  const uint64_t lt = lanemask_lt(lane);
  const int64_t i0 = (int64_t)b * tpb * k;
  const int64_t i1 = min((int64_t)T * k, i0 + (int64_t)tpb * k);
  const int n_items = T * k;
  int tag = 0;
  for (int64_t r0 = i0; r0 < i1; r0 += kPermThreads) {
    ++tag;
    const int64_t i = r0 + threadIdx.x;
    const bool valid = i < i1;
    const int e = valid ? clamp_expert(idx[i], E) : 0;
    uint64_t peers = ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool x = (e >> bit) & 1;
      const uint64_t m = ballot(x);
      peers &= x ? m : ~m;
    }
    const int rank = __popcll(peers & lt);
    const int cnt = __popcll(peers);
    const bool leader = valid && (__builtin_ctzll(peers) == lane);
    if (leader) {
      wcnt[wave * E + e] = cnt;
      wtag[wave * E + e] = tag;
    }
    __syncthreads();
    if (valid) {
      int pre = 0;
      for (int w = 0; w < wave; ++w) pre += (wtag[w * E + e] == tag) ? wcnt[w * E + e] : 0;
      const int p = run[e] + pre + rank;
      pos[i] = p;
      if (static_cast<unsigned>(p) < static_cast<unsigned>(n_items)) src[p] = static_cast<int32_t>(i);
    }
    __syncthreads();
    if (leader) atomicAdd(&run[e], cnt);
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_layout(const int32_t* idx, int T, int E, int k, int R, const int32_t* assign,
                         const int32_t* rep, int maxrep, int32_t* rank_of, int32_t* expert_offsets,
                         int32_t* rank_offsets, int32_t* pos, int32_t* src, int32_t* dedup,
                         int32_t* ws, hipStream_t s) {
  const Blocking bl = blocking_for(T, E);
  const int nblk = T > 0 ? bl.layout_nblk : 0;
  int32_t* hist = ws;                           // [nblk, E]
  int32_t* ded = ws + (size_t)bl.layout_nblk * E; // [nblk, R]
  if (nblk > 0) {
    layout_count_kernel<<<nblk, kCountThreads, (2 * E + R) * sizeof(int), s>>>(
        idx, T, E, k, R, bl.layout_tpb, assign, rep, maxrep, hist, ded);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  layout_plan_kernel<<<1, kPlanThreads, 0, s>>>(T, E, k, R, nblk, hist, ded, assign, rep, maxrep,
                                               rank_of, expert_offsets, rank_offsets, dedup);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nblk == 0) return err;
  layout_permute_kernel<<<nblk, kPermThreads, (1 + 2 * kPermWaves) * E * sizeof(int), s>>>(
      idx, T, E, k, bl.layout_tpb, hist, expert_offsets, pos, src);
  return hipGetLastError();
}

}  // namespace moe
