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
//  2. layout_plan (one workgroup): one pass over both matrices, every wave
//     loading its whole row segment in one batch: per-expert totals and the
//     exclusive scan of the expert histogram over blocks (in place), dedup
//     totals. Then the rank of every expert, per-rank row totals (LDS adds)
//     and their block scan give the rank offsets; an expert's offset is its
//     rank's offset plus the rows of lower-id experts on the same rank.
//  3. layout_permute: per block, the stable rank of each pair among the
//     block's pairs with the same expert: inside a wave by matching expert
//     ids with one ballot per id bit and counting lower lanes; across the
//     block's waves by per-wave counts in LDS; across rounds by running
//     per-expert cursors. pos = cursor + rank, src[pos] = flat pair index.
//  (3'. layout_permute_ss: the permutation and then the single-send rows,
//   in one launch, when the single-send rows are asked for.)
// A small batch (T k <= 8192 pairs) runs all of it in one workgroup instead
// (layout_small), sharing the same device functions.
#include "device.hpp"
#include "greedy.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kCountThreads = 1024;
constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kSegRegs = 48;  // rows per wave segment in the plan's column pass

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

// Counts of tokens [t0, t1) into LDS: the selected experts (s_hist) and, per
// token, its distinct destination ranks (s_ded); with lead_mask, bit j of
// lead_mask[t] marks slot j as the token's first slot on its rank. All
// threads of the block take part.
__device__ __forceinline__ void count_tokens(const int32_t* __restrict__ idx, int t0, int t1, int E, int k,
                             const int* s_rank, int* s_hist, int* s_ded,
                             int32_t* __restrict__ lead_mask) {
  const size_t i0 = (size_t)t0 * k, i1 = (size_t)t1 * k;
  for (size_t i = i0 + threadIdx.x; i < i1; i += blockDim.x)
    atomicAdd(&s_hist[clamp_expert(idx[i], E)], 1);
  for (int t = t0 + threadIdx.x; t < t1; t += blockDim.x) {
    // ranks of the token's k experts in registers, then one count per
    // distinct rank (the first slot that reaches it)
    int ids[kMaxK];
    load_slots(idx + (size_t)t * k, k, ids);
    int rk[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) rk[j] = j < k ? s_rank[clamp_expert(ids[j], E)] : -1 - j;
    int lead = 0;  // bit j: slot j is the token's first slot on its rank
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      bool seen = false;
#pragma unroll
      for (int jj = 0; jj < j; ++jj) seen |= (rk[jj] == rk[j]);
      if (j < k && !seen) {
        atomicAdd(&s_ded[rk[j]], 1);
        lead |= 1 << j;
      }
    }
    if (lead_mask != nullptr) lead_mask[t] = lead;
  }
}

__global__ __launch_bounds__(kCountThreads) void layout_count_kernel(
    const int32_t* __restrict__ idx, int T, int E, int k, int R, int tpb,
    const int32_t* __restrict__ assign, const int32_t* __restrict__ rep, int maxrep,
    int32_t* __restrict__ hist, int32_t* __restrict__ ded, int32_t* __restrict__ lead_mask) {
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
  count_tokens(idx, t0, min(T, t0 + tpb), E, k, s_rank, s_hist, s_ded, lead_mask);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(size_t)blockIdx.x * E + e] = s_hist[e];
  for (int r = threadIdx.x; r < R; r += blockDim.x) ded[(size_t)blockIdx.x * R + r] = s_ded[r];
}

// Column pass over the two per-block matrices: hist [rows, E] and ded
// [rows, R] are replaced by their exclusive prefixes over rows (column by
// column: the block's first row per expert, and per rank for single-send
// rows) and their column totals go to s_cnt and s_ded. The work is cut into
// tasks of 64 columns; the 16 waves are shared among as many tasks as fit,
// each task's waves splitting the rows into segments of at most kSegRegs
// rows (the layout blocking guarantees it), loaded in one batch and kept in
// registers: one memory round trip per group of tasks.
__device__ __forceinline__ void column_pass(int32_t* __restrict__ hist, int E, int32_t* __restrict__ ded, int R,
                            int rows, int* s_cnt, int* s_ded, int (*part)[kWave]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int ch_h = (E + kWave - 1) / kWave;
  const int tasks = ch_h + (R + kWave - 1) / kWave;
  const int S = tasks >= kPlanWaves ? 1 : kPlanWaves / tasks;  // waves per task
  const int G = kPlanWaves / S;                                 // tasks per group
  const int seg = (rows + S - 1) / S;
  const int sw = wave % S;
  const int r_lo = min(rows, sw * seg), r_hi = min(rows, r_lo + seg);
  for (int g0 = 0; g0 < tasks; g0 += G) {
    const int task = g0 + wave / S;
    const bool on = (wave / S) < G && task < tasks;
    const bool is_h = task < ch_h;
    const int cols = is_h ? E : R;
    const int c = (is_h ? task : task - ch_h) * kWave + lane;
    const bool col_ok = on && c < cols;
    int32_t* M = is_h ? hist : ded;
    int v[kSegRegs];
    int s = 0;
#pragma unroll
    for (int i = 0; i < kSegRegs; ++i) {
      const int r = r_lo + i;
      v[i] = (col_ok && r < r_hi) ? M[(size_t)r * cols + c] : 0;
      s += v[i];
    }
    part[wave][lane] = s;
    __syncthreads();
    int pre = 0, all = 0;
    if (on) {  // waves past the last task of the group own no rows of part[]
      const int w0 = (wave / S) * S;
      for (int i = 0; i < S; ++i) {
        const int x = part[w0 + i][lane];
        pre += (i < sw) ? x : 0;
        all += x;
      }
    }
    if (col_ok) {
      if (sw == 0) (is_h ? s_cnt : s_ded)[c] = all;
      int run = pre;
#pragma unroll
      for (int i = 0; i < kSegRegs; ++i) {
        const int r = r_lo + i;
        if (r < r_hi) M[(size_t)r * cols + c] = run;
        run += v[i];
      }
    }
    __syncthreads();
  }
}

// Exclusive prefix sum of one value per thread over the whole block (1024
// threads); returns the prefix and writes the block total to *total.
__device__ __forceinline__ int block_excl_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int incl = wave_incl_scan(v, lane);
  if (lane == kWave - 1) s_wave[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    const int x = s_wave[w];
    before += (w < wave) ? x : 0;
    all += x;
  }
  *total = all;
  return before + incl - v;
}

// Everything the plan derives from the per-expert totals s_cnt, the dedup
// totals s_ded and the expert ranks s_rank (each thread tid < E holds
// s_rank[tid]; s_rtok zeroed): rank_of, per-rank row totals (LDS adds) and
// their block scan (rank_offsets), dedup, each expert's offset (its rank's
// offset plus the rows of lower-id experts on the same rank), and the
// single-send rank offsets. s_rank and s_cnt must have room for E rounded up
// to 8. Optional LDS copies: s_eoff[E] of the expert offsets, s_ssoff[R] of
// the single-send offsets. All threads of the (1024-thread) block take part.
__device__ __forceinline__ void plan_finish(int E, int R, int* s_rank, int* s_cnt, const int* s_ded, int* s_rtok,
                            int* s_roff, int* s_wave, int* s_wave2, int32_t* __restrict__ rank_of,
                            int32_t* __restrict__ expert_offsets, int32_t* __restrict__ rank_offsets,
                            int32_t* __restrict__ dedup, int32_t* __restrict__ ss_rank_offsets,
                            int* s_eoff, int* s_ssoff) {
  const int tid = threadIdx.x;  // E, R <= 1024 == blockDim.x: one expert / rank per thread
  if (tid < E) {
    const int my_r = s_rank[tid];
    rank_of[tid] = my_r;
    atomicAdd(&s_rtok[my_r], s_cnt[tid]);
  } else if (tid < ((E + 7) & ~7)) {
    s_rank[tid] = 0x7fffffff;  // padding never matches a rank
    s_cnt[tid] = 0;
  }
  __syncthreads();
  int total = 0;
  const int roff = block_excl_scan(tid < R ? s_rtok[tid] : 0, s_wave, &total);
  if (tid < R) {
    s_roff[tid] = roff;
    rank_offsets[tid] = roff;
    dedup[tid] = s_ded[tid];
  }
  if (tid == 0) rank_offsets[R] = total;
  __syncthreads();
  {
    // rows of lower-id experts on the same rank: P adjacent threads per
    // expert, each scanning every P-th group of 8 LDS entries, their partial
    // sums then added with shuffles inside the wave (integer adds)
    const int P = E <= 64 ? 16 : (E <= 128 ? 8 : (E <= 256 ? 4 : (E <= 512 ? 2 : 1)));
    const int e = tid / P, q = tid % P;
    int acc = 0, er = 0;
    if (e < E) {
      er = s_rank[e];
      const int e_pad = (E + 7) & ~7;
      for (int b = q * 8; b < e_pad; b += 8 * P) {
        const int4 r0 = *reinterpret_cast<const int4*>(&s_rank[b]);
        const int4 r1 = *reinterpret_cast<const int4*>(&s_rank[b + 4]);
        const int4 c0 = *reinterpret_cast<const int4*>(&s_cnt[b]);
        const int4 c1 = *reinterpret_cast<const int4*>(&s_cnt[b + 4]);
        const int rr[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
        const int cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) acc += (rr[i] == er && b + i < e) ? cc[i] : 0;
      }
    }
    for (int off = P / 2; off > 0; off /= 2) acc += __shfl_xor(acc, off, P);
    if (e < E && q == 0) {
      expert_offsets[e] = s_roff[er] + acc;
      if (s_eoff != nullptr) s_eoff[e] = s_roff[er] + acc;
    }
  }
  if (ss_rank_offsets != nullptr) {
    // single-send rows: one per (token, rank), grouped by rank
    int ss_total = 0;
    const int ss_off = block_excl_scan(tid < R ? s_ded[tid] : 0, s_wave2, &ss_total);
    if (tid < R) {
      ss_rank_offsets[tid] = ss_off;
      if (s_ssoff != nullptr) s_ssoff[tid] = ss_off;
    }
    if (tid == 0) ss_rank_offsets[R] = ss_total;
  }
}

__global__ __launch_bounds__(kPlanThreads) void layout_plan_kernel(
    int T, int E, int k, int R, int nblk, int32_t* __restrict__ hist, int32_t* __restrict__ ded,
    const int32_t* __restrict__ assign, const int32_t* __restrict__ rep, int maxrep,
    int32_t* __restrict__ rank_of, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ dedup,
    int32_t* __restrict__ ss_rank_offsets) {
  __shared__ __align__(16) int s_rank[kMaxE + 8];
  __shared__ __align__(16) int s_cnt[kMaxE + 8];
  __shared__ int s_ded[kMaxR];
  __shared__ int s_rtok[kMaxR];
  __shared__ int s_roff[kMaxR];
  __shared__ int part[kPlanWaves][kWave];
  __shared__ int s_wave[kPlanWaves];
  __shared__ int s_wave2[kPlanWaves];
  const int tid = threadIdx.x;
  // issue the expert-rank loads now, use them after the column pass
  int my_r = 0;
  if (tid < E) my_r = expert_rank(tid, E, R, assign, rep, maxrep);
  if (tid < R) s_rtok[tid] = 0;
  column_pass(hist, E, ded, R, nblk, s_cnt, s_ded, part);  // ends with a barrier
  if (tid < E) s_rank[tid] = my_r;
  plan_finish(E, R, s_rank, s_cnt, s_ded, s_rtok, s_roff, s_wave, s_wave2, rank_of,
              expert_offsets, rank_offsets, dedup, ss_rank_offsets, nullptr, nullptr);
}

// Stable placement of the pairs [i0, i1), in order, after the running
// per-expert cursors run[e]: inside a wave by matching expert ids with one
// ballot per id bit and counting lower lanes, across the WAVES waves by
// per-wave counts tagged by round in LDS (wcnt, wtag: [WAVES][E], wtag
// zeroed), across rounds by advancing the cursors. pos = cursor + rank,
// src[pos] = flat pair index. All WAVES * 64 threads take part; ends with a
// barrier.
template <int WAVES>
__device__ __forceinline__ void permute_rounds(const int32_t* __restrict__ idx, int64_t i0, int64_t i1, int E,
                               int n_items, int* run, int* wcnt, int* wtag,
                               int32_t* __restrict__ pos, int32_t* __restrict__ src) {
  constexpr int kThreads = WAVES * kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nbits = E > 1 ? 32 - __builtin_clz((unsigned)(E - 1)) : 0;
  const uint64_t lt = lanemask_lt(lane);
  int tag = 0;
  int e_next = (i0 + threadIdx.x < i1) ? idx[i0 + threadIdx.x] : 0;  // next round's expert, prefetched
  for (int64_t r0 = i0; r0 < i1; r0 += kThreads) {
    ++tag;
    const int64_t i = r0 + threadIdx.x;
    const bool valid = i < i1;
    const int e = valid ? clamp_expert(e_next, E) : 0;
    if (i + kThreads < i1) e_next = idx[i + kThreads];
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

template <int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void layout_permute_kernel(
    const int32_t* __restrict__ idx, int T, int E, int k, int tpb, const int32_t* __restrict__ base,
    const int32_t* __restrict__ expert_offsets, int32_t* __restrict__ pos,
    int32_t* __restrict__ src) {
  extern __shared__ int smem[];
  int* run = smem;                   // [E] next free row of each expert
  int* wcnt = smem + E;              // [WAVES][E] pairs per expert in a wave
  int* wtag = smem + E + WAVES * E;  // [WAVES][E] round that wrote wcnt
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    run[e] = expert_offsets[e] + base[(size_t)b * E + e];
#pragma unroll
    for (int w = 0; w < WAVES; ++w) wtag[w * E + e] = 0;
  }
  __syncthreads();
  const int64_t i0 = (int64_t)b * tpb * k;
  const int64_t i1 = min((int64_t)T * k, i0 + (int64_t)tpb * k);
  permute_rounds<WAVES>(idx, i0, i1, E, T * k, run, wcnt, wtag, pos, src);
}

// Single-send rows: one per (token, destination rank), grouped by rank and
// inside a rank by token. A token's leader slot for a rank (its first slot
// on that rank) takes the next row of the rank; its other slots on the same
// rank reuse that row. The stable order comes from the same ballot matching
// as the expert permutation, keyed by rank and counting leaders only: a
// leader's row is the number of leaders of its rank before it; a non-leader
// sees its own leader among those before it, so its row is that count - 1.
template <int WAVES>
__device__ __forceinline__ void single_send_rounds(const int32_t* __restrict__ idx, int64_t i0, int64_t i1, int k,
                                   int E, int R, int n_items, const int* s_rank, int* run,
                                   int* wcnt, int* wtag, const int32_t* __restrict__ lead_mask,
                                   int32_t* __restrict__ ss_row, int32_t* __restrict__ ss_token) {
  constexpr int kThreads = WAVES * kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nbits = R > 1 ? 32 - __builtin_clz((unsigned)(R - 1)) : 0;
  const uint64_t lt = lanemask_lt(lane);
  int tag = 0;
  for (int64_t r0 = i0; r0 < i1; r0 += kThreads) {
    ++tag;
    const int64_t i = r0 + threadIdx.x;
    const bool valid = i < i1;
    const int ii = static_cast<int>(i);  // pair index, below 2^31
    const int t = valid ? ii / k : 0;
    const int j = valid ? ii - t * k : 0;
    const int r = valid ? s_rank[clamp_expert(idx[i], E)] : 0;
    const bool leader = valid && ((lead_mask[t] >> j) & 1);
    uint64_t peers = ballot(leader);  // leaders of the same rank
    for (int bit = 0; bit < nbits; ++bit) {
      const bool x = (r >> bit) & 1;
      const uint64_t m = ballot(x);
      peers &= x ? m : ~m;
    }
    const int before = __popcll(peers & lt);
    const int cnt = __popcll(peers);
    const bool writer = leader && (__builtin_ctzll(peers) == lane);
    if (writer) {
      wcnt[wave * R + r] = cnt;
      wtag[wave * R + r] = tag;
    }
    __syncthreads();
    if (valid) {
      int pre = 0;
      for (int w = 0; w < wave; ++w) pre += (wtag[w * R + r] == tag) ? wcnt[w * R + r] : 0;
      const int q = run[r] + pre + before - (leader ? 0 : 1);
      ss_row[i] = q;
      if (leader && static_cast<unsigned>(q) < static_cast<unsigned>(n_items)) ss_token[q] = t;
    }
    __syncthreads();
    if (writer) atomicAdd(&run[r], cnt);
    __syncthreads();
  }
}

// The permutation and the single-send rows of one block of tokens in one
// launch: the permutation rounds of layout_permute_kernel, then the
// single-send rounds, the second reusing the first's LDS tables.
// LDS: max((1 + 2 WAVES) E, E + (1 + 2 WAVES) R) ints.
template <int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void layout_permute_ss_kernel(
    const int32_t* __restrict__ idx, int T, int E, int k, int R, int tpb,
    const int32_t* __restrict__ base, const int32_t* __restrict__ expert_offsets,
    const int32_t* __restrict__ rank_of, const int32_t* __restrict__ ss_base,
    const int32_t* __restrict__ ss_rank_offsets, const int32_t* __restrict__ lead_mask,
    int32_t* __restrict__ pos, int32_t* __restrict__ src, int32_t* __restrict__ ss_row,
    int32_t* __restrict__ ss_token) {
  extern __shared__ int smem[];
  const int b = blockIdx.x;
  const int64_t i0 = (int64_t)b * tpb * k;
  const int64_t i1 = min((int64_t)T * k, i0 + (int64_t)tpb * k);
  {
    int* run = smem;                   // [E] next free row of each expert
    int* wcnt = smem + E;              // [WAVES][E]
    int* wtag = smem + E + WAVES * E;  // [WAVES][E]
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      run[e] = expert_offsets[e] + base[(size_t)b * E + e];
#pragma unroll
      for (int w = 0; w < WAVES; ++w) wtag[w * E + e] = 0;
    }
    __syncthreads();
    permute_rounds<WAVES>(idx, i0, i1, E, T * k, run, wcnt, wtag, pos, src);  // ends with a barrier
  }
  int* s_rank = smem;                       // [E]
  int* run = smem + E;                      // [R] next free single-send row of each rank
  int* wcnt = smem + E + R;                 // [WAVES][R]
  int* wtag = smem + E + R + WAVES * R;     // [WAVES][R]
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_rank[e] = rank_of[e];
  for (int r = threadIdx.x; r < R; r += blockDim.x) {
    run[r] = ss_rank_offsets[r] + ss_base[(size_t)b * R + r];
#pragma unroll
    for (int w = 0; w < WAVES; ++w) wtag[w * R + r] = 0;
  }
  __syncthreads();
  single_send_rounds<WAVES>(idx, i0, i1, k, E, R, T * k, s_rank, run, wcnt, wtag, lead_mask,
                            ss_row, ss_token);
}

// The whole layout of a small batch (T k <= kSmallPairs) in one workgroup:
// counts, plan, permutation and single-send rows, every table in LDS, with
// the same device code as the multi-block kernels. A decode batch then
// takes one launch instead of three or four. `assign` may point to global
// memory or LDS. smem holds small_layout_ints(E, R) ints.
constexpr int kSmallPairs = 8192;
constexpr int kSmallLdsInts = 16 * 1024 - 64;  // dynamic LDS under 64 KiB beside 128 static bytes

__host__ __device__ constexpr int small_layout_ints(int E, int R) {
  // s_rank, s_cnt (E rounded up for the plan's padding), four [R] tables,
  // run[M] and the two [16][M] wave tables, M = max(E, R)
  return 2 * ((E + 8) & ~7) + 4 * R + (1 + 2 * kPlanWaves) * (E > R ? E : R);
}

__device__ __forceinline__ void layout_small_block(
    const int32_t* __restrict__ idx, int T, int E, int k, int R, const int32_t* assign,
    const int32_t* __restrict__ rep, int maxrep, int32_t* __restrict__ rank_of,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ rank_offsets,
    int32_t* __restrict__ pos, int32_t* __restrict__ src, int32_t* __restrict__ dedup,
    int32_t* __restrict__ ss_rank_offsets, int32_t* __restrict__ ss_row,
    int32_t* __restrict__ ss_token, int32_t* __restrict__ lead, int* smem, int* s_wave,
    int* s_wave2) {
  const int ep = (E + 8) & ~7;  // room for the plan's padding to a multiple of 8
  const int M = E > R ? E : R;
  int* s_rank = smem;            // [ep]
  int* s_cnt = s_rank + ep;      // [ep]
  int* s_ded = s_cnt + ep;       // [R]
  int* s_rtok = s_ded + R;       // [R]
  int* s_roff = s_rtok + R;      // [R]
  int* s_ssoff = s_roff + R;     // [R]
  int* run = s_ssoff + R;        // [M]
  int* wcnt = run + M;           // [16][M]
  int* wtag = wcnt + kPlanWaves * M;  // [16][M]
  const bool ss = ss_rank_offsets != nullptr;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    s_rank[e] = expert_rank(e, E, R, assign, rep, maxrep);
    s_cnt[e] = 0;
  }
  for (int r = threadIdx.x; r < R; r += blockDim.x) {
    s_ded[r] = 0;
    s_rtok[r] = 0;
  }
  __syncthreads();
  count_tokens(idx, 0, T, E, k, s_rank, s_cnt, s_ded, ss ? lead : nullptr);
  __syncthreads();
  plan_finish(E, R, s_rank, s_cnt, s_ded, s_rtok, s_roff, s_wave, s_wave2, rank_of,
              expert_offsets, rank_offsets, dedup, ss_rank_offsets, run, s_ssoff);
  for (int i = threadIdx.x; i < kPlanWaves * E; i += blockDim.x) wtag[i] = 0;
  __syncthreads();
  permute_rounds<kPlanWaves>(idx, 0, (int64_t)T * k, E, T * k, run, wcnt, wtag, pos, src);
  if (!ss) return;  // uniform: a kernel argument
  for (int r = threadIdx.x; r < R; r += blockDim.x) run[r] = s_ssoff[r];
  for (int i = threadIdx.x; i < kPlanWaves * R; i += blockDim.x) wtag[i] = 0;
  __syncthreads();
  single_send_rounds<kPlanWaves>(idx, 0, (int64_t)T * k, k, E, R, T * k, s_rank, run, wcnt, wtag,
                                 lead, ss_row, ss_token);
}

__global__ __launch_bounds__(kPlanThreads) void layout_small_kernel(
    const int32_t* __restrict__ idx, int T, int E, int k, int R,
    const int32_t* __restrict__ assign, const int32_t* __restrict__ rep, int maxrep,
    int32_t* __restrict__ rank_of, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ pos, int32_t* __restrict__ src,
    int32_t* __restrict__ dedup, int32_t* __restrict__ ss_rank_offsets,
    int32_t* __restrict__ ss_row, int32_t* __restrict__ ss_token, int32_t* __restrict__ lead) {
  extern __shared__ __align__(16) int smem[];
  __shared__ int s_wave[kPlanWaves];
  __shared__ int s_wave2[kPlanWaves];
  layout_small_block(idx, T, E, k, R, assign, rep, maxrep, rank_of, expert_offsets, rank_offsets,
                     pos, src, dedup, ss_rank_offsets, ss_row, ss_token, lead, smem, s_wave,
                     s_wave2);
}

// The routing plan of a small batch after the top-k kernel, in one
// workgroup: the demand vector as the column sums of the route's per-block
// histogram rows, the greedy replica assignment (greedy.hpp) and the whole
// layout, with the counts and the assignment kept in LDS between the steps.
// Outputs equal those of the separate column-sum, assignment and layout
// kernels. Dynamic LDS: counts [E] and assign [E], then a region the
// assignment's scratch and the layout's tables use in turn.
__host__ __device__ constexpr int plan_greedy_ints(int E, int R) {
  // act (at least 64 entries), ncand (E bytes), cand (E * kMaxRep halves)
  return (R > kWave ? R : kWave) + (E + 3) / 4 + E * kMaxRep / 2;
}

__host__ __device__ constexpr int plan_small_ints(int E, int R) {
  const int g = plan_greedy_ints(E, R), l = small_layout_ints(E, R);
  return 2 * ((E + 3) & ~3) + (g > l ? g : l);
}

__global__ __launch_bounds__(kPlanThreads) void route_plan_small_kernel(
    const int32_t* __restrict__ hist, int nblk, const int32_t* __restrict__ idx, int T, int E,
    int k, int R, const int32_t* __restrict__ rep, int maxrep, int id_order,
    int32_t* __restrict__ counts, int32_t* __restrict__ assign, int32_t* __restrict__ active,
    int32_t* __restrict__ rank_of, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ pos, int32_t* __restrict__ src,
    int32_t* __restrict__ dedup) {
  extern __shared__ __align__(16) int smem[];
  __shared__ int s_wave[kPlanWaves];
  __shared__ int s_wave2[kPlanWaves];
  const int e4 = (E + 3) & ~3;
  int* s_counts = smem;            // [E]
  int* s_assign = smem + e4;       // [E]
  int* region = smem + 2 * e4;     // greedy scratch, then the layout's tables
  const int tid = threadIdx.x;
  // demand vector: column sums of the [nblk, E] histogram rows, the rows
  // split among max(1, 1024 / E) thread groups per column (integer adds)
  for (int e = tid; e < E; e += blockDim.x) s_counts[e] = 0;
  __syncthreads();
  {
    const int groups = E >= kPlanThreads ? 1 : kPlanThreads / E;
    const int g = tid / E;
    for (int e = tid % E; g < groups && e < E; e += kPlanThreads) {
      int acc = 0;
      for (int r = g; r < nblk; r += groups) acc += hist[(size_t)r * E + e];
      atomicAdd(&s_counts[e], acc);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) counts[e] = s_counts[e];
  // greedy replica assignment into LDS
  int* act = region;
  unsigned char* ncand = reinterpret_cast<unsigned char*>(region + (R > kWave ? R : kWave));
  unsigned short* cand = reinterpret_cast<unsigned short*>(region + (R > kWave ? R : kWave) + (E + 3) / 4);
  assign_block(s_counts, E, R, rep, maxrep, id_order, s_assign, act, ncand, cand);
  for (int e = tid; e < E; e += blockDim.x) assign[e] = s_assign[e];
  for (int g = tid; g < R; g += blockDim.x) active[g] = act[g];
  __syncthreads();  // the region is reused below
  layout_small_block(idx, T, E, k, R, s_assign, rep, maxrep, rank_of, expert_offsets, rank_offsets,
                     pos, src, dedup, nullptr, nullptr, nullptr, nullptr, region, s_wave, s_wave2);
}

}  // namespace

hipError_t launch_layout(const int32_t* idx, int T, int E, int k, int R, const int32_t* assign,
                         const int32_t* rep, int maxrep, int32_t* rank_of, int32_t* expert_offsets,
                         int32_t* rank_offsets, int32_t* pos, int32_t* src, int32_t* dedup,
                         int32_t* ss_rank_offsets, int32_t* ss_row, int32_t* ss_token,
                         int32_t* ws, hipStream_t s) {
  const Blocking bl = blocking_for(T, E, R);
  const int nblk = T > 0 ? bl.layout_nblk : 0;
  const bool ss = ss_rank_offsets != nullptr;
  int32_t* hist = ws;                                   // [nblk, E]
  int32_t* ded = ws + (size_t)bl.layout_nblk * E;       // [nblk, R]
  int32_t* lead = ded + (size_t)bl.layout_nblk * R;     // [T] leader masks (single-send)
  {
    const size_t small_ints = small_layout_ints(E, R);
    // dynamic LDS under 64 KiB with room for the kernel's static 128 bytes
    if (T > 0 && (int64_t)T * k <= kSmallPairs && small_ints <= kSmallLdsInts) {
      layout_small_kernel<<<1, kPlanThreads, small_ints * sizeof(int), s>>>(
          idx, T, E, k, R, assign, rep, maxrep, rank_of, expert_offsets, rank_offsets, pos, src,
          dedup, ss_rank_offsets, ss_row, ss_token, lead);
      return hipGetLastError();
    }
  }
  if (nblk > 0) {
    layout_count_kernel<<<nblk, kCountThreads, (2 * E + R) * sizeof(int), s>>>(
        idx, T, E, k, R, bl.layout_tpb, assign, rep, maxrep, hist, ded, ss ? lead : nullptr);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  layout_plan_kernel<<<1, kPlanThreads, 0, s>>>(T, E, k, R, nblk, hist, ded, assign, rep, maxrep,
                                               rank_of, expert_offsets, rank_offsets, dedup,
                                               ss_rank_offsets);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nblk == 0) return err;
  if (ss) {
    // permutation and single-send rows in one launch; 16 waves when blocks
    // hold many pairs and both phases' tables stay small
    const bool w16 = (int64_t)bl.layout_tpb * k >= 1024 && E <= 256 && E + 33 * R <= 12 * 1024;
    const int W = w16 ? 16 : 4;
    const size_t pe = (size_t)(1 + 2 * W) * E, pr = (size_t)E + (size_t)(1 + 2 * W) * R;
    const size_t lds = (pe > pr ? pe : pr) * sizeof(int);
    if (w16)
      layout_permute_ss_kernel<16><<<nblk, 16 * kWave, lds, s>>>(
          idx, T, E, k, R, bl.layout_tpb, hist, expert_offsets, rank_of, ded, ss_rank_offsets,
          lead, pos, src, ss_row, ss_token);
    else
      layout_permute_ss_kernel<4><<<nblk, 4 * kWave, lds, s>>>(
          idx, T, E, k, R, bl.layout_tpb, hist, expert_offsets, rank_of, ded, ss_rank_offsets,
          lead, pos, src, ss_row, ss_token);
    return hipGetLastError();
  }
  // 16 waves per permute block when blocks hold many pairs and the per-wave
  // LDS tables (33 E ints) fit comfortably; else 4 waves (9 E ints)
  if (E <= 256 && (int64_t)bl.layout_tpb * k >= 1024)
    layout_permute_kernel<16><<<nblk, 16 * kWave, 33 * E * sizeof(int), s>>>(
        idx, T, E, k, bl.layout_tpb, hist, expert_offsets, pos, src);
  else
    layout_permute_kernel<4><<<nblk, 4 * kWave, 9 * E * sizeof(int), s>>>(
        idx, T, E, k, bl.layout_tpb, hist, expert_offsets, pos, src);
  return hipGetLastError();
}

hipError_t launch_route_assign_layout(const float* logits, int T, int E, int k, int R,
                                      const int32_t* rep, int maxrep, bool id_order, int32_t* idx,
                                      float* w, int32_t* counts, int32_t* assign, int32_t* active,
                                      int32_t* rank_of, int32_t* expert_offsets,
                                      int32_t* rank_offsets, int32_t* pos, int32_t* src,
                                      int32_t* dedup, int32_t* ws, hipStream_t s) {
  const size_t plan_ints = plan_small_ints(E, R);
  if (T > 0 && (int64_t)T * k <= kSmallPairs && plan_ints <= kSmallLdsInts) {
    hipError_t err = launch_route_topk(logits, T, E, k, idx, w, ws, s);
    if (err != hipSuccess) return err;
    route_plan_small_kernel<<<1, kPlanThreads, plan_ints * sizeof(int), s>>>(
        ws, blocking_for(T, E, R).route_nblk, idx, T, E, k, R, rep, rep ? maxrep : 1,
        id_order ? 1 : 0, counts, assign, active, rank_of, expert_offsets, rank_offsets, pos, src,
        dedup);
    return hipGetLastError();
  }
  hipError_t err = launch_route(logits, T, E, k, idx, w, counts, ws, s);
  if (err != hipSuccess) return err;
  err = launch_assign(counts, E, R, rep, rep ? maxrep : 1, id_order, assign, active, s);
  if (err != hipSuccess) return err;
  return launch_layout(idx, T, E, k, R, assign, rep, rep ? maxrep : 1, rank_of, expert_offsets,
                       rank_offsets, pos, src, dedup, nullptr, nullptr, nullptr, ws, s);
}

}  // namespace moe
