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
//
// The one-call route + assignment + layout (launch_route_assign_layout)
// picks, after the top-k kernel:
//  - a decode-sized batch (T <= 1024, T k <= 8192): route_plan_mask_kernel,
//    one workgroup with one round trip to global memory, the demand vector
//    and the pairs' places from per-expert token bitmasks (the top-k kernel
//    then writes no histogram rows), the places counted while the greedy
//    walks;
//  - a batch of up to 8192 pairs whose tables fit: route_plan_small_kernel;
//  - a larger batch without a replica table: plan_scan_kernel and
//    layout_permute_scan_kernel, from the top-k kernel's per-block expert
//    and rank rows (three launches in all);
//  - else the kernels of the separate route, assignment and layout calls.
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
template <int NT>
__device__ __forceinline__ void count_tokens(const int32_t* __restrict__ idx, int t0, int t1, int E, int k,
                             const int* s_rank, int* s_hist, int* s_ded,
                             int32_t* __restrict__ lead_mask) {
  const size_t i0 = (size_t)t0 * k, i1 = (size_t)t1 * k;
  const size_t nt = NT;
  // four loads in flight at a time: clamped indices, and an add of 0 for a
  // slot past the end (a value used only under a condition has its load
  // moved under that condition, and waited for on its own)
  for (size_t i = i0 + threadIdx.x; i < i1; i += 4 * nt) {
    int v[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) v[b] = idx[i + b * nt < i1 ? i + b * nt : i1 - 1];
#pragma unroll
    for (int b = 0; b < 4; ++b) atomicAdd(&s_hist[clamp_expert(v[b], E)], i + b * nt < i1 ? 1 : 0);
  }
  for (int t = t0 + threadIdx.x; t < t1; t += NT) {
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
  for (int e = threadIdx.x; e < E; e += kCountThreads) {
    s_rank[e] = expert_rank(e, E, R, assign, rep, maxrep);
    s_hist[e] = 0;
  }
  for (int r = threadIdx.x; r < R; r += kCountThreads) s_ded[r] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * tpb;
  count_tokens<kCountThreads>(idx, t0, min(T, t0 + tpb), E, k, s_rank, s_hist, s_ded, lead_mask);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kCountThreads) hist[(size_t)blockIdx.x * E + e] = s_hist[e];
  for (int r = threadIdx.x; r < R; r += kCountThreads) ded[(size_t)blockIdx.x * R + r] = s_ded[r];
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
  for (int e = threadIdx.x; e < E; e += WAVES * kWave) {
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
    for (int e = threadIdx.x; e < E; e += WAVES * kWave) {
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
  for (int e = threadIdx.x; e < E; e += WAVES * kWave) s_rank[e] = rank_of[e];
  for (int r = threadIdx.x; r < R; r += WAVES * kWave) {
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
  for (int e = threadIdx.x; e < E; e += kPlanThreads) {
    s_rank[e] = expert_rank(e, E, R, assign, rep, maxrep);
    s_cnt[e] = 0;
  }
  for (int r = threadIdx.x; r < R; r += kPlanThreads) {
    s_ded[r] = 0;
    s_rtok[r] = 0;
  }
  __syncthreads();
  count_tokens<kPlanThreads>(idx, 0, T, E, k, s_rank, s_cnt, s_ded, ss ? lead : nullptr);
  __syncthreads();
  plan_finish(E, R, s_rank, s_cnt, s_ded, s_rtok, s_roff, s_wave, s_wave2, rank_of,
              expert_offsets, rank_offsets, dedup, ss_rank_offsets, run, s_ssoff);
  for (int i = threadIdx.x; i < kPlanWaves * E; i += kPlanThreads) wtag[i] = 0;
  __syncthreads();
  permute_rounds<kPlanWaves>(idx, 0, (int64_t)T * k, E, T * k, run, wcnt, wtag, pos, src);
  if (!ss) return;  // uniform: a kernel argument
  for (int r = threadIdx.x; r < R; r += kPlanThreads) run[r] = s_ssoff[r];
  for (int i = threadIdx.x; i < kPlanWaves * R; i += kPlanThreads) wtag[i] = 0;
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
  for (int e = tid; e < E; e += kPlanThreads) s_counts[e] = 0;
  __syncthreads();
  {
    const int groups = E >= kPlanThreads ? 1 : kPlanThreads / E;
    const int g = tid / E;
    for (int e = tid % E; g < groups && e < E; e += kPlanThreads) {
      // sixteen rows' loads in flight at a time (clamped rows, masked after)
      int acc = 0;
      for (int r0 = g; r0 < nblk; r0 += 16 * groups) {
        int v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = hist[(size_t)min(r0 + i * groups, nblk - 1) * E + e];
#pragma unroll
        for (int i = 0; i < 16; ++i) acc += r0 + i * groups < nblk ? v[i] : 0;
      }
      atomicAdd(&s_counts[e], acc);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPlanThreads) counts[e] = s_counts[e];
  // greedy replica assignment into LDS
  int* act = region;
  unsigned char* ncand = reinterpret_cast<unsigned char*>(region + (R > kWave ? R : kWave));
  unsigned short* cand = reinterpret_cast<unsigned short*>(region + (R > kWave ? R : kWave) + (E + 3) / 4);
  assign_block(s_counts, E, R, rep, maxrep, id_order, s_assign, act, ncand, cand);
  for (int e = tid; e < E; e += kPlanThreads) assign[e] = s_assign[e];
  for (int g = tid; g < R; g += kPlanThreads) active[g] = act[g];
  __syncthreads();  // the region is reused below
  layout_small_block(idx, T, E, k, R, s_assign, rep, maxrep, rank_of, expert_offsets, rank_offsets,
                     pos, src, dedup, nullptr, nullptr, nullptr, nullptr, region, s_wave, s_wave2);
}

// The one-call plan of a batch without a replica table (contiguous
// partition: expert e on rank e / per), after a top-k kernel that wrote one
// expert-histogram row and one per-rank count row per route block. There is
// no choice to make, and the send order (rank, expert) is expert order, so
// the plan is two launches: this column scan, then the permutation with the
// expert-offset scan in its prologue.
//
// One workgroup per task of 64 columns: the expert tasks replace their
// columns of the histogram rows with exclusive prefixes over blocks (the
// block's first row per expert) and write the totals as counts, with
// rank_of and assign; the rank tasks sum their columns into dedup (and with
// ded_prefix replace them with their exclusive prefixes as well: the
// block's first single-send row per rank). The 16
// waves split the rows (at most kSumRows each, so 512 route blocks) and load
// their segment at once.
constexpr int kSumRows = 32;

__global__ __launch_bounds__(kPlanThreads) void plan_scan_kernel(
    int32_t* __restrict__ hist, int32_t* __restrict__ ded, int nblk, int E, int R, int per,
    int32_t* __restrict__ counts, int32_t* __restrict__ assign, int32_t* __restrict__ rank_of,
    int32_t* __restrict__ dedup, int ded_prefix) {
  __shared__ int part[kPlanWaves][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int ch_h = (E + kWave - 1) / kWave;
  const bool is_h = static_cast<int>(blockIdx.x) < ch_h;
  const int cols = is_h ? E : R;
  const int c = (is_h ? blockIdx.x : blockIdx.x - ch_h) * kWave + lane;
  const int32_t* M = is_h ? hist : ded;
  const int seg = (nblk + kPlanWaves - 1) / kPlanWaves;
  const int r_lo = min(nblk, wave * seg), r_hi = min(nblk, r_lo + seg);
  int v[kSumRows];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kSumRows; ++i) {
    const int r = r_lo + i;
    v[i] = (c < cols && r < r_hi) ? M[(size_t)r * cols + c] : 0;
    sum += v[i];
  }
  part[wave][lane] = sum;
  __syncthreads();
  int pre = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kPlanWaves; ++i) {
    const int x = part[i][lane];
    pre += (i < wave) ? x : 0;
    all += x;
  }
  if (c >= cols) return;
  if (is_h) {
    int run = pre;
#pragma unroll
    for (int i = 0; i < kSumRows; ++i) {
      const int r = r_lo + i;
      if (r < r_hi) hist[(size_t)r * E + c] = run;
      run += v[i];
    }
    if (wave == 0) {
      counts[c] = all;
      rank_of[c] = c / per;
      assign[c] = all > 0 ? c / per : -1;
    }
  } else {
    if (ded_prefix) {  // uniform: a kernel argument
      int run = pre;
#pragma unroll
      for (int i = 0; i < kSumRows; ++i) {
        const int r = r_lo + i;
        if (r < r_hi) ded[(size_t)r * R + c] = run;
        run += v[i];
      }
    }
    if (wave == 0) dedup[c] = all;
  }
}

// Permutation of one route block's pairs for a batch without a replica
// table, after plan_scan_kernel. Prologue: the exclusive scan of counts over
// experts (each thread a run of up to 4 consecutive experts, then a block
// scan) gives expert_offsets; a block's cursors are those plus its
// histogram prefix (base). Block 0 also writes expert_offsets, rank_offsets
// (the offset of each rank's first expert; [R] = T k) and active (experts
// with rows, per rank). Then the permutation rounds of layout_permute_kernel.
// LDS: (1 + 2 WAVES) E + R ints.
template <int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void layout_permute_scan_kernel(
    const int32_t* __restrict__ idx, int T, int E, int k, int R, int per, int tpb,
    const int32_t* __restrict__ base, const int32_t* __restrict__ counts,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ rank_offsets,
    int32_t* __restrict__ active, int32_t* __restrict__ pos, int32_t* __restrict__ src) {
  constexpr int kThreads = WAVES * kWave;
  constexpr int kRun = (kMaxE + kThreads - 1) / kThreads;
  extern __shared__ int smem[];
  int* run = smem;                   // [E] next free row of each expert
  int* wcnt = smem + E;              // [WAVES][E]
  int* wtag = smem + E + WAVES * E;  // [WAVES][E]
  int* s_act = wtag + WAVES * E;     // [R] (block 0)
  __shared__ int s_wsum[WAVES];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int n_run = (E + kThreads - 1) / kThreads;
  const int e0 = threadIdx.x * n_run;
  int c[kRun], bs[kRun];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kRun; ++i) {
    const int e = e0 + i;
    const bool ok = i < n_run && e < E;
    c[i] = ok ? counts[e] : 0;
    bs[i] = ok ? base[(size_t)b * E + e] : 0;
    sum += c[i];
  }
  for (int i = threadIdx.x; i < WAVES * E; i += kThreads) wtag[i] = 0;
  if (b == 0)
    for (int r = threadIdx.x; r < R; r += kThreads) s_act[r] = 0;
  const int incl = wave_incl_scan(sum, lane);
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  int off = incl - sum;
#pragma unroll
  for (int i = 0; i < WAVES; ++i) off += (i < wave) ? s_wsum[i] : 0;
#pragma unroll
  for (int i = 0; i < kRun; ++i) {
    const int e = e0 + i;
    if (i < n_run && e < E) {
      run[e] = off + bs[i];
      if (b == 0) {
        expert_offsets[e] = off;
        if (e % per == 0) rank_offsets[e / per] = off;
        if (c[i] > 0) atomicAdd(&s_act[e / per], 1);
      }
      off += c[i];
    }
  }
  __syncthreads();
  if (b == 0) {
    for (int r = threadIdx.x; r < R; r += kThreads) active[r] = s_act[r];
    if (threadIdx.x == 0) rank_offsets[R] = T * k;
  }
  const int64_t i0 = (int64_t)b * tpb * k;
  const int64_t i1 = min((int64_t)T * k, i0 + (int64_t)tpb * k);
  permute_rounds<WAVES>(idx, i0, i1, E, T * k, run, wcnt, wtag, pos, src);
}

// The permutation and the single-send rows of one route block for a batch
// without a replica table, after plan_scan_kernel with ded_prefix (ss_base:
// the block's first single-send row per rank, relative to the rank's
// start). Prologue: the expert scan of layout_permute_scan_kernel (block 0
// writing expert_offsets, rank_offsets and active) and, beside it, the
// exclusive scan of dedup over ranks (block 0 writing ss_rank_offsets); the
// block's single-send cursors stay in registers through the permutation
// rounds. Then the single-send rounds of layout_permute_ss_kernel, reusing
// the permutation's LDS tables, with rank e / per for expert e.
// LDS: max((1 + 2 WAVES) E + R, E + (1 + 2 WAVES) R) ints.
template <int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void layout_permute_ss_scan_kernel(
    const int32_t* __restrict__ idx, int T, int E, int k, int R, int per, int tpb,
    const int32_t* __restrict__ base, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ ss_base, const int32_t* __restrict__ dedup,
    const int32_t* __restrict__ lead_mask, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ active, int32_t* __restrict__ pos,
    int32_t* __restrict__ src, int32_t* __restrict__ ss_rank_offsets, int32_t* __restrict__ ss_row,
    int32_t* __restrict__ ss_token) {
  constexpr int kThreads = WAVES * kWave;
  constexpr int kRun = (kMaxE + kThreads - 1) / kThreads;
  constexpr int kRunR = (kMaxR + kThreads - 1) / kThreads;
  extern __shared__ int smem[];
  __shared__ int s_wsum[WAVES];
  __shared__ int s_wsum_r[WAVES];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  // every load first: counts and this block's expert prefixes, dedup and
  // this block's single-send prefixes, each thread a run of consecutive ids
  const int n_run = (E + kThreads - 1) / kThreads;
  const int e0 = threadIdx.x * n_run;
  const int n_run_r = (R + kThreads - 1) / kThreads;
  const int q0 = threadIdx.x * n_run_r;
  int c[kRun], bs[kRun], cr[kRunR], sb[kRunR];
  int sum = 0, sum_r = 0;
#pragma unroll
  for (int i = 0; i < kRun; ++i) {
    const int e = e0 + i;
    const bool ok = i < n_run && e < E;
    c[i] = ok ? counts[e] : 0;
    bs[i] = ok ? base[(size_t)b * E + e] : 0;
  }
#pragma unroll
  for (int i = 0; i < kRunR; ++i) {
    const int r = q0 + i;
    const bool ok = i < n_run_r && r < R;
    cr[i] = ok ? dedup[r] : 0;
    sb[i] = ok ? ss_base[(size_t)b * R + r] : 0;
  }
#pragma unroll
  for (int i = 0; i < kRun; ++i) sum += c[i];
#pragma unroll
  for (int i = 0; i < kRunR; ++i) sum_r += cr[i];
  int* run = smem;                   // [E] next free row of each expert
  int* wcnt = smem + E;              // [WAVES][E]
  int* wtag = smem + E + WAVES * E;  // [WAVES][E]
  int* s_act = wtag + WAVES * E;     // [R] (block 0)
  for (int i = threadIdx.x; i < WAVES * E; i += kThreads) wtag[i] = 0;
  if (b == 0)
    for (int r = threadIdx.x; r < R; r += kThreads) s_act[r] = 0;
  const int incl = wave_incl_scan(sum, lane);
  const int incl_r = wave_incl_scan(sum_r, lane);
  if (lane == kWave - 1) {
    s_wsum[wave] = incl;
    s_wsum_r[wave] = incl_r;
  }
  __syncthreads();
  int off = incl - sum, off_r = incl_r - sum_r, n_ss = 0;
#pragma unroll
  for (int i = 0; i < WAVES; ++i) {
    off += (i < wave) ? s_wsum[i] : 0;
    off_r += (i < wave) ? s_wsum_r[i] : 0;
    n_ss += s_wsum_r[i];
  }
#pragma unroll
  for (int i = 0; i < kRun; ++i) {
    const int e = e0 + i;
    if (i < n_run && e < E) {
      run[e] = off + bs[i];
      if (b == 0) {
        expert_offsets[e] = off;
        if (e % per == 0) rank_offsets[e / per] = off;
        if (c[i] > 0) atomicAdd(&s_act[e / per], 1);
      }
      off += c[i];
    }
  }
#pragma unroll
  for (int i = 0; i < kRunR; ++i) {  // the block's single-send cursors, kept in sb
    const int r = q0 + i;
    if (i < n_run_r && r < R) {
      if (b == 0) ss_rank_offsets[r] = off_r;
      sb[i] += off_r;
      off_r += cr[i];
    }
  }
  __syncthreads();
  if (b == 0) {
    for (int r = threadIdx.x; r < R; r += kThreads) active[r] = s_act[r];
    if (threadIdx.x == 0) {
      rank_offsets[R] = T * k;
      ss_rank_offsets[R] = n_ss;
    }
  }
  const int64_t i0 = (int64_t)b * tpb * k;
  const int64_t i1 = min((int64_t)T * k, i0 + (int64_t)tpb * k);
  permute_rounds<WAVES>(idx, i0, i1, E, T * k, run, wcnt, wtag, pos, src);  // ends with a barrier
  int* s_rank = smem;                    // [E]
  int* run_r = smem + E;                 // [R] next free single-send row of each rank
  int* wcnt_r = smem + E + R;            // [WAVES][R]
  int* wtag_r = smem + E + R + WAVES * R;  // [WAVES][R]
  for (int e = threadIdx.x; e < E; e += kThreads) s_rank[e] = e / per;
  for (int i = threadIdx.x; i < WAVES * R; i += kThreads) wtag_r[i] = 0;
#pragma unroll
  for (int i = 0; i < kRunR; ++i) {
    const int r = q0 + i;
    if (i < n_run_r && r < R) run_r[r] = sb[i];
  }
  __syncthreads();
  single_send_rounds<WAVES>(idx, i0, i1, k, E, R, T * k, s_rank, run_r, wcnt_r, wtag_r, lead_mask,
                            ss_row, ss_token);
}

// The routing plan of a decode-sized batch (T <= 1024 tokens, T k <= 8192
// pairs) after the top-k kernel, in one workgroup with one round trip to
// global memory: the expert ids and the replica rows are loaded at the
// start. Each expert gets a bitmask of the tokens that chose it; its count
// is the number of bits set (a token chooses an expert at most once), and
// the place of pair (t, e) inside e's segment is the number of bits of e's
// mask below t, the stable rank. The places do not depend on the
// assignment, so they are counted while the greedy walks. The walkers
// (waves 0..3, one per component group of the GPU graph, with at most 64
// GPUs; else wave 0) visit the multi-copy experts in order (greedy_walk, or
// greedy_walk_packed for tables of at most 4 columns) while the other waves
// count those bits. Then the ranks of the experts, the per-token dedup
// counts and the offsets (finish_few_ranks for up to 64 ranks, else
// plan_finish), and pos = expert offset + place.
// Outputs equal those of route_plan_small_kernel.
constexpr int kMaskMaxT = 1024;
constexpr int kMaskPairsPerThread = kSmallPairs / kPlanThreads;

__host__ __device__ constexpr int round4(int n) { return (n + 3) & ~3; }

// Bits set in the first W <= N words of an LDS row, the N reads issued
// before any is used (words past W reread the last and count nothing).
template <int N>
__device__ __forceinline__ int popc_words(const unsigned long long* row, int W) {
  unsigned long long w[N];
#pragma unroll
  for (int q = 0; q < N; ++q) w[q] = row[q < W ? q : W - 1];
  int c = 0;
#pragma unroll
  for (int q = 0; q < N; ++q) c += q < W ? __popcll(w[q]) : 0;
  return c;
}

// LDS ints of route_plan_mask_kernel; with ss, room for the single-send rows
// (at most 64 ranks).
__host__ __device__ constexpr int mask_plan_ints(int T, int E, int k, int R, bool ss = false) {
  const int W = (T + 63) / 64, e8 = (E + 8) & ~7;
  return round4(2 * W * E) + 2 * round4(e8) + 2 * round4(E) + 3 * round4(R) +
         round4(R > kWave ? R : kWave) + round4((E + 3) / 4) + round4(E * kMaxRep / 2) +
         2 * round4((T * k + 1) / 2) +
         (R <= kWave ? round4(kPlanWaves * R) + round4(R + 1) + 2 * round4(E) + 2 * kWave : 0) +
         (ss && R <= kWave ? 2 * round4(kPlanWaves * R) + round4(R) + 2 * kPlanWaves * R : 0);
}

// The destination ranks of one token's k slots as a 64-bit set (ranks < 64):
// the N slot reads issued together (slots past k reread slot k - 1), then
// their ranks.
template <int N>
__device__ __forceinline__ unsigned long long token_rank_set(const unsigned short* row, int k,
                                                             const int* s_rank) {
  int ids[N];
#pragma unroll
  for (int j = 0; j < N; ++j) ids[j] = row[j < k ? j : k - 1];
  unsigned long long rm = 0ull;
#pragma unroll
  for (int j = 0; j < N; ++j) rm |= 1ull << s_rank[ids[j]];
  return rm;
}

// Exclusive prefix sums of in[0, n) into out[0, n) by one wave, lane l
// taking the run l P .. l P + P - 1 (P <= N): the run's reads issued
// together, its sum, a wave scan of the sums, then the run written out.
// Returns the total (wave-uniform).
template <int N>
__device__ __forceinline__ int wave_excl_scan_runs(const int* in, int* out, int n, int P, int lane) {
  const int base = lane * P;
  int v[N];
#pragma unroll
  for (int q = 0; q < N; ++q) {
    const int i = base + q;
    v[q] = in[i < n ? i : n - 1];
    v[q] = (q < P && i < n) ? v[q] : 0;
  }
  int sum = 0;
#pragma unroll
  for (int q = 0; q < N; ++q) sum += v[q];
  const int incl = wave_incl_scan(sum, lane);
  int run = incl - sum;
#pragma unroll
  for (int q = 0; q < N; ++q) {
    const int i = base + q;
    if (q < P && i < n) out[i] = run;
    run += v[q];
  }
  return __builtin_amdgcn_readlane(incl, kWave - 1);
}

// The end of the bitmask plan for at most 64 ranks, after s_rank holds every
// expert's rank (all threads take part; ends with a barrier):
//  - dedup: each token's ranks as a 64-bit set, counted per rank with one
//    ballot per rank and wave;
//  - the experts in (rank, id) order: each expert's place among the experts
//    of its rank from ballot matching on the rank bits (lower lanes) and
//    per-wave counts (earlier waves), plus the experts of lower ranks;
//  - one scan of the counts in that order, by a single wave
//    (wave_excl_scan_runs), gives every expert's offset, and a rank's offset
//    is the scan at its first place.
// s_wr [16][R], s_rbase [R + 1], s_ord [E], s_scan [E] are LDS scratch
// (s_wr zeroed by the caller); s_wave[0] carries the total.
__device__ __forceinline__ void finish_few_ranks(
    int T, int E, int k, int R, const int* s_rank, const int* s_counts,
    const unsigned short* s_idx, int* s_ded, int* s_wr, int* s_rbase, int* s_ord, int* s_scan,
    int* s_eoff, int* s_wave, int32_t* __restrict__ rank_of, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ dedup, int* s_ssw = nullptr,
    int* s_ssoff = nullptr, int* s_ssbase = nullptr, uint64_t* s_ssb = nullptr,
    int32_t* __restrict__ ss_rank_offsets = nullptr, int32_t* __restrict__ ss_row = nullptr,
    int32_t* __restrict__ ss_token = nullptr) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const bool ss = ss_rank_offsets != nullptr;  // uniform: an argument
  const int n_tw = (T + kWave - 1) / kWave;     // waves holding tokens
  unsigned long long rm = 0ull;                 // this thread's token's ranks
  if (wave < n_tw) {  // uniform per wave
    // the token's ids are read with loads issued together (in a bucket of
    // 4, 8 or 16 slots; slots past k reread slot k - 1), then their ranks
    if (tid < T) {
      const unsigned short* row = s_idx + tid * k;
      rm = k <= 4 ? token_rank_set<4>(row, k, s_rank)
         : k <= 8 ? token_rank_set<8>(row, k, s_rank) : token_rank_set<kMaxK>(row, k, s_rank);
    }
    // the wave's count for rank r lands in lane r (independent ballots,
    // then one LDS add per rank)
    int cnt = 0;
    for (int r = 0; r < R; ++r) {
      const uint64_t br = ballot((rm >> r) & 1ull);
      cnt = lane == r ? __popcll(br) : cnt;
      if (ss && lane == 0) s_ssb[wave * R + r] = br;  // the wave's tokens on rank r
    }
    if (lane < R && cnt > 0) atomicAdd(&s_ded[lane], cnt);
    if (ss && lane < R) s_ssw[wave * R + lane] = cnt;  // the wave's tokens per rank
  }
  const int r = tid < E ? s_rank[tid] : R;  // R: past every rank
  const int nbits = 32 - __builtin_clz(static_cast<unsigned>(R));
  uint64_t peers = ballot(true);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool x = (r >> bit) & 1;
    const uint64_t m = ballot(x);
    peers &= x ? m : ~m;
  }
  const int within = __popcll(peers & lanemask_lt(lane));
  if (tid < E && __builtin_ctzll(peers) == lane) s_wr[wave * R + r] = __popcll(peers);
  __syncthreads();
  if (wave == 0) {
    int ne = 0;
    if (lane < R)
      for (int w = 0; w < kPlanWaves; ++w) ne += s_wr[w * R + lane];
    const int incl = wave_incl_scan(ne, lane);
    const int nd = lane < R ? s_ded[lane] : 0;
    if (lane < R) {
      s_rbase[lane] = incl - ne;
      dedup[lane] = nd;
    }
    if (ss) {  // single-send offsets: the dedup totals scanned over ranks
      const int incl_d = wave_incl_scan(nd, lane);
      if (lane < R) {
        s_ssoff[lane] = incl_d - nd;
        ss_rank_offsets[lane] = incl_d - nd;
      }
      if (lane == kWave - 1) ss_rank_offsets[R] = incl_d;
    }
  }
  __syncthreads();
  int place = 0;
  if (tid < E) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += s_wr[w * R + r];
    place = s_rbase[r] + before + within;
    s_ord[place] = s_counts[tid];
    rank_of[tid] = r;
  }
  if (ss && tid < n_tw * R) {  // wave w's first single-send row on rank q
    const int w = tid / R, q = tid - w * R;
    int base = s_ssoff[q];
    for (int v = 0; v < w; ++v) base += s_ssw[v * R + q];
    s_ssbase[tid] = base;
  }
  __syncthreads();
  // one wave scans the counts in (rank, id) order, P = ceil(E / 64) per
  // lane; lane 63's inclusive sum is the total
  if (wave == 0) {
    const int P = (E + kWave - 1) / kWave;
    const int all = P <= 4 ? wave_excl_scan_runs<4>(s_ord, s_scan, E, P, lane)
                  : P <= 8 ? wave_excl_scan_runs<8>(s_ord, s_scan, E, P, lane)
                           : wave_excl_scan_runs<kMaxE / kWave>(s_ord, s_scan, E, P, lane);
    if (lane == 0) s_wave[0] = all;
  }
  __syncthreads();
  const int total = s_wave[0];
  if (tid < E) {
    const int o = s_scan[place];
    expert_offsets[tid] = o;
    s_eoff[tid] = o;
  }
  if (tid < R) rank_offsets[tid] = s_rbase[tid] < E ? s_scan[s_rbase[tid]] : total;
  if (tid == 0) rank_offsets[R] = total;
  if (ss && tid < T) {
    // single-send rows: for rank q the tokens holding it, in token order; a
    // slot's row is its wave's first row on q plus the lower lanes holding q
    // (from the wave's ballot); the token's first slot on q writes the row's
    // token
    const uint64_t lt = lanemask_lt(lane);
    const unsigned short* row_ids = s_idx + tid * k;
    for (int j = 0; j < k; ++j) {
      const int q = s_rank[row_ids[j]];
      const int row = s_ssbase[wave * R + q] + __popcll(s_ssb[wave * R + q] & lt);
      ss_row[(size_t)tid * k + j] = row;
      bool first = true;
      for (int jj = 0; jj < j; ++jj) first &= s_rank[row_ids[jj]] != q;
      if (first) ss_token[row] = tid;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kPlanThreads) void route_plan_mask_kernel(
    const int32_t* __restrict__ idx, int T, int E,
    int k, int R, const int32_t* __restrict__ rep, int maxrep, int id_order,
    int32_t* __restrict__ counts, int32_t* __restrict__ assign, int32_t* __restrict__ active,
    int32_t* __restrict__ rank_of, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ pos, int32_t* __restrict__ src,
    int32_t* __restrict__ dedup, int32_t* __restrict__ ss_rank_offsets,
    int32_t* __restrict__ ss_row, int32_t* __restrict__ ss_token) {
  extern __shared__ __align__(16) int smem[];
  __shared__ int s_wave[kPlanWaves];
  __shared__ int s_wave2[kPlanWaves];
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int W = (T + 63) / 64;  // mask words per expert
  const int n = T * k;
  const int e8 = (E + 8) & ~7;
  unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem);  // [E][W]
  int* p = smem + round4(2 * W * E);
  int* s_counts = p; p += round4(e8);  // the demand vector (plan_finish pads it)
  int* s_rank = p;   p += round4(e8);
  int* s_eoff = p;   p += round4(E);
  int* s_assign = p; p += round4(E);
  int* s_ded = p;    p += round4(R);
  int* s_rtok = p;   p += round4(R);
  int* s_roff = p;   p += round4(R);
  int* act = p;      p += round4(R > kWave ? R : kWave);
  unsigned char* ncand = reinterpret_cast<unsigned char*>(p); p += round4((E + 3) / 4);
  unsigned short* cand = reinterpret_cast<unsigned short*>(p);
  uint32_t* word = reinterpret_cast<uint32_t*>(p); p += round4(E * kMaxRep / 2);  // cand or word [E]
  unsigned short* s_idx = reinterpret_cast<unsigned short*>(p); p += round4((n + 1) / 2);
  unsigned short* s_rk = reinterpret_cast<unsigned short*>(p); p += round4((n + 1) / 2);
  const bool few = R <= kWave;  // the ballot-based end (finish_few_ranks)
  // the packed walk: at most 64 GPUs and kPackedRep table columns
  const bool packed = few && rep != nullptr && maxrep <= kPackedRep;
  int* s_wr = p;    p += few ? round4(kPlanWaves * R) : 0;
  int* s_rbase = p; p += few ? round4(R + 1) : 0;
  int* s_ord = p;   p += few ? round4(E) : 0;
  int* s_scan = p;  p += few ? round4(E) : 0;
  unsigned long long* adj = reinterpret_cast<unsigned long long*>(p);  // [64] when few
  p += few ? 2 * kWave : 0;
  // single-send rows (used only with the single-send outputs): per-wave
  // token counts and first rows per rank, the rank offsets, and each wave's
  // ballot of its tokens on each rank
  int* s_ssw = p;    p += few ? round4(kPlanWaves * R) : 0;
  int* s_ssbase = p; p += few ? round4(kPlanWaves * R) : 0;
  int* s_ssoff = p;  p += few ? round4(R) : 0;
  uint64_t* s_ssb = reinterpret_cast<uint64_t*>(p);  // [kPlanWaves][R]

  // every global load first, all in flight together: expert ids and replica
  // rows. Each load reads an index clamped into its array (T, k, maxrep >= 1
  // here) and is masked afterwards: a load under its own condition is
  // waited for before the next one is issued.
  int pe[kMaskPairsPerThread];
#pragma unroll
  for (int j = 0; j < kMaskPairsPerThread; ++j) pe[j] = idx[min(tid + j * kPlanThreads, n - 1)];
  int rr[kMaxRep];
  {
    const int32_t* row = rep + (size_t)min(tid, E - 1) * maxrep;  // read only with a table
#pragma unroll
    for (int s = 0; s < kMaxRep; ++s) rr[s] = (rep != nullptr && s < maxrep) ? row[s] : -1;  // uniform
  }
#pragma unroll
  for (int j = 0; j < kMaskPairsPerThread; ++j)
    pe[j] = tid + j * kPlanThreads < n ? clamp_expert(pe[j], E) : 0;
#pragma unroll
  for (int s = 0; s < kMaxRep; ++s)
    rr[s] = (rep != nullptr && tid < E && s < maxrep) ? rr[s] : -1;

  for (int i = tid; i < W * E; i += kPlanThreads) mask[i] = 0ull;
  for (int i = E + tid; i < e8; i += kPlanThreads) s_counts[i] = 0;  // the padding
  for (int i = tid; i < R; i += kPlanThreads) {
    s_ded[i] = 0;
    s_rtok[i] = 0;
  }
  for (int i = tid; i < (R > kWave ? R : kWave); i += kPlanThreads) act[i] = 0;
  if (few) {
    for (int i = tid; i < kPlanWaves * R; i += kPlanThreads) s_wr[i] = 0;
    if (tid < kWave) adj[tid] = 0ull;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kMaskPairsPerThread; ++j) {
    const int i = tid + j * kPlanThreads;
    if (i < n) {
      const int t = i / k;
      atomicOr(&mask[pe[j] * W + (t >> 6)], 1ull << (t & 63));
      s_idx[i] = static_cast<unsigned short>(pe[j]);
    }
  }
  __syncthreads();
  // The place of pair i inside its expert's segment: the tokens before it in
  // the expert's mask. Pairs first..n-1 in steps of `step`.
  auto places = [&](int first, int step) {
    for (int i = first; i < n; i += step) {
      const int e = s_idx[i], t = i / k, wt = t >> 6;
      const unsigned long long* m = mask + e * W;
      int c = __popcll(m[wt] & ((1ull << (t & 63)) - 1ull));
      for (int q = 0; q < wt; ++q) c += __popcll(m[q]);
      s_rk[i] = static_cast<unsigned short>(c);
    }
  };
  // the demand vector: an expert's count is the number of bits of its mask
  // (a token selects an expert at most once); active experts' valid
  // candidates to LDS; single-copy experts (and every expert without a
  // table) are placed at once
  if (tid < E) {
    // the expert's W mask words, loaded together in the narrowest of 4, 8
    // or 16 reads (W is uniform)
    const unsigned long long* mrow = mask + tid * W;
    const int c = W <= 4 ? popc_words<4>(mrow, W)
                : W <= 8 ? popc_words<8>(mrow, W) : popc_words<kMaskMaxT / 64>(mrow, W);
    s_counts[tid] = c;
    counts[tid] = c;
    if (rep == nullptr) {
      const int per = E / R;
      s_assign[tid] = c > 0 ? tid / per : -1;
      if (c > 0) atomicAdd(&act[tid / per], 1);
    } else {
      // the valid candidates, from the replica row in registers: packed in
      // one word (packed walk) or listed in cand
      int nc = 0, g0 = 0;
      uint32_t wd = 0u;
      unsigned long long cm = 0ull;
      if (c > 0) {
#pragma unroll
        for (int s = 0; s < kMaxRep; ++s) {
          if (s >= maxrep) break;  // uniform
          const int g = rr[s];
          if (g >= 0 && g < R) {
            g0 = nc == 0 ? g : g0;
            if (packed) wd |= static_cast<uint32_t>(g) << (6 * nc);
            else cand[tid * kMaxRep + nc] = static_cast<unsigned short>(g);
            cm |= 1ull << (g & 63);
            ++nc;
          }
        }
      }
      if (packed) word[tid] = wd | (static_cast<uint32_t>(nc) << 24);
      else ncand[tid] = static_cast<unsigned char>(nc);
      if (nc == 0) s_assign[tid] = -1;
      if (!id_order && nc == 1) {
        s_assign[tid] = g0;
        atomicAdd(&act[g0], 1);
      }
      // the GPU graph of the walked experts: each candidate learns the others
      if (few && nc >= (id_order ? 1 : 2)) {
#pragma unroll
        for (int s = 0; s < kMaxRep; ++s) {
          if (s >= maxrep) break;  // uniform
          if (rr[s] >= 0 && rr[s] < R) atomicOr(&adj[rr[s]], cm);
        }
      }
    }
  }
  __syncthreads();
  // With at most 64 GPUs the walk is split over waves 0..3 (one per SIMD),
  // each taking whole components of the GPU graph; else wave 0 walks. The
  // other waves find the pairs' places meanwhile.
  const int walkers = (few && rep != nullptr) ? 4 : 1;
  if (wave < walkers) {
    if (rep != nullptr) {
      if (packed) {
        if (maxrep <= 2) greedy_walk_packed<2>(E, maxrep, id_order, word, act, s_assign, adj, R, wave, walkers);
        else greedy_walk_packed<kPackedRep>(E, maxrep, id_order, word, act, s_assign, adj, R, wave, walkers);
      } else if (few) {
        const uint64_t gpus = walker_gpus(adj, R, wave, walkers);
        if (gpus != 0ull) greedy_walk<true>(E, maxrep, id_order, ncand, cand, act, s_assign, gpus);
      } else {
        greedy_walk<false>(E, maxrep, id_order, ncand, cand, act, s_assign);
      }
    }
  } else {
    places(tid - walkers * kWave, kPlanThreads - walkers * kWave);
  }
  __syncthreads();
  if (tid < E) {  // an expert's rank: its assignment, else its first-listed copy (in rr[0])
    const int a = s_assign[tid];
    assign[tid] = a;
    const int r = a >= 0 ? a : (rep != nullptr ? rr[0] : tid / (E / R));
    s_rank[tid] = r < 0 ? 0 : (r >= R ? R - 1 : r);
  }
  for (int g = tid; g < R; g += kPlanThreads) active[g] = act[g];
  __syncthreads();
  if (few) {
    finish_few_ranks(T, E, k, R, s_rank, s_counts, s_idx, s_ded, s_wr, s_rbase, s_ord, s_scan,
                     s_eoff, s_wave, rank_of, expert_offsets, rank_offsets, dedup, s_ssw, s_ssoff,
                     s_ssbase, s_ssb, ss_rank_offsets, ss_row, ss_token);
  } else {
    if (tid < T) {  // distinct destination ranks of the token
      int rk[kMaxK];
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) rk[j] = j < k ? s_rank[s_idx[tid * k + j]] : -1 - j;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        bool seen = false;
#pragma unroll
        for (int jj = 0; jj < j; ++jj) seen |= (rk[jj] == rk[j]);
        if (j < k && !seen) atomicAdd(&s_ded[rk[j]], 1);
      }
    }
    plan_finish(E, R, s_rank, s_counts, s_ded, s_rtok, s_roff, s_wave, s_wave2, rank_of,
                expert_offsets, rank_offsets, dedup, nullptr, s_eoff, nullptr);
    __syncthreads();
  }
  for (int i = tid; i < n; i += kPlanThreads) {
    const int q = s_eoff[s_idx[i]] + s_rk[i];
    pos[i] = q;
    if (static_cast<unsigned>(q) < static_cast<unsigned>(n)) src[q] = i;
  }
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
  if (T > 0 && T <= kMaskMaxT && (int64_t)T * k <= kSmallPairs &&
      mask_plan_ints(T, E, k, R) <= kSmallLdsInts) {
    // the plan counts the experts from idx itself: no histogram rows
    hipError_t err = launch_route_topk(logits, T, E, k, idx, w, nullptr, s);
    if (err != hipSuccess) return err;
    route_plan_mask_kernel<<<1, kPlanThreads, mask_plan_ints(T, E, k, R) * sizeof(int), s>>>(
        idx, T, E, k, R, rep, rep ? maxrep : 1,
        id_order ? 1 : 0, counts, assign, active, rank_of, expert_offsets, rank_offsets, pos, src,
        dedup, nullptr, nullptr, nullptr);
    return hipGetLastError();
  }
  if (T > 0 && (int64_t)T * k <= kSmallPairs && plan_ints <= kSmallLdsInts) {
    hipError_t err = launch_route_topk(logits, T, E, k, idx, w, ws, s);
    if (err != hipSuccess) return err;
    route_plan_small_kernel<<<1, kPlanThreads, plan_ints * sizeof(int), s>>>(
        ws, blocking_for(T, E, R).route_nblk, idx, T, E, k, R, rep, rep ? maxrep : 1,
        id_order ? 1 : 0, counts, assign, active, rank_of, expert_offsets, rank_offsets, pos, src,
        dedup);
    return hipGetLastError();
  }
  if (rep == nullptr && T > 0) {
    // no replica table: top-k with per-block counts, column scan, permutation
    const Blocking bl = blocking_for(T, E, R);
    const int nblk = bl.route_nblk, per = E / R;
    int32_t* hist = ws;                          // [nblk, E]
    int32_t* ded = ws + (size_t)nblk * E;        // [nblk, R]
    hipError_t err = launch_route_topk(logits, T, E, k, idx, w, hist, s, ded, R);
    if (err != hipSuccess) return err;
    const int tasks = (E + kWave - 1) / kWave + (R + kWave - 1) / kWave;
    plan_scan_kernel<<<tasks, kPlanThreads, 0, s>>>(hist, ded, nblk, E, R, per, counts, assign,
                                                    rank_of, dedup, 0);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (E <= 256 && (int64_t)bl.route_tpb * k >= 1024)
      layout_permute_scan_kernel<16><<<nblk, 16 * kWave, (33 * E + R) * sizeof(int), s>>>(
          idx, T, E, k, R, per, bl.route_tpb, hist, counts, expert_offsets, rank_offsets, active,
          pos, src);
    else
      layout_permute_scan_kernel<4><<<nblk, 4 * kWave, (9 * E + R) * sizeof(int), s>>>(
          idx, T, E, k, R, per, bl.route_tpb, hist, counts, expert_offsets, rank_offsets, active,
          pos, src);
    return hipGetLastError();
  }
  hipError_t err = launch_route(logits, T, E, k, idx, w, counts, ws, s);
  if (err != hipSuccess) return err;
  err = launch_assign(counts, E, R, rep, rep ? maxrep : 1, id_order, assign, active, s);
  if (err != hipSuccess) return err;
  return launch_layout(idx, T, E, k, R, assign, rep, rep ? maxrep : 1, rank_of, expert_offsets,
                       rank_offsets, pos, src, dedup, nullptr, nullptr, nullptr, ws, s);
}

hipError_t launch_route_assign_layout_single_send(
    const float* logits, int T, int E, int k, int R, const int32_t* rep, int maxrep, bool id_order,
    int32_t* idx, float* w, int32_t* counts, int32_t* assign, int32_t* active, int32_t* rank_of,
    int32_t* expert_offsets, int32_t* rank_offsets, int32_t* pos, int32_t* src, int32_t* dedup,
    int32_t* ss_rank_offsets, int32_t* ss_row, int32_t* ss_token, int32_t* ws, hipStream_t s) {
  if (T > 0 && T <= kMaskMaxT && (int64_t)T * k <= kSmallPairs && R <= kWave &&
      mask_plan_ints(T, E, k, R, true) <= kSmallLdsInts) {
    // a decode-sized batch: the top-k kernel, then one workgroup that also
    // lays out the single-send rows (by ballots over each rank's tokens)
    hipError_t err = launch_route_topk(logits, T, E, k, idx, w, nullptr, s);
    if (err != hipSuccess) return err;
    route_plan_mask_kernel<<<1, kPlanThreads, mask_plan_ints(T, E, k, R, true) * sizeof(int), s>>>(
        idx, T, E, k, R, rep, rep ? maxrep : 1, id_order ? 1 : 0, counts, assign, active, rank_of,
        expert_offsets, rank_offsets, pos, src, dedup, ss_rank_offsets, ss_row, ss_token);
    return hipGetLastError();
  }
  if (rep == nullptr && T > 0) {
    // no replica table: top-k with per-block counts and leader masks, the
    // column scan (expert and rank columns to prefixes), then the
    // permutation and the single-send rows
    const Blocking bl = blocking_for(T, E, R);
    const int nblk = bl.route_nblk, per = E / R;
    int32_t* hist = ws;                          // [nblk, E]
    int32_t* ded = ws + (size_t)nblk * E;        // [nblk, R]
    int32_t* lead = ded + (size_t)nblk * R;      // [T]
    hipError_t err = launch_route_topk(logits, T, E, k, idx, w, hist, s, ded, R, lead);
    if (err != hipSuccess) return err;
    const int tasks = (E + kWave - 1) / kWave + (R + kWave - 1) / kWave;
    plan_scan_kernel<<<tasks, kPlanThreads, 0, s>>>(hist, ded, nblk, E, R, per, counts, assign,
                                                    rank_of, dedup, 1);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const bool w16 = (int64_t)bl.route_tpb * k >= 1024 && E <= 256 && E + 33 * R <= 12 * 1024;
    const int W = w16 ? 16 : 4;
    const size_t pe = (size_t)(1 + 2 * W) * E + R, pr = (size_t)E + (size_t)(1 + 2 * W) * R;
    const size_t lds = (pe > pr ? pe : pr) * sizeof(int);
    if (w16)
      layout_permute_ss_scan_kernel<16><<<nblk, 16 * kWave, lds, s>>>(
          idx, T, E, k, R, per, bl.route_tpb, hist, counts, ded, dedup, lead, expert_offsets,
          rank_offsets, active, pos, src, ss_rank_offsets, ss_row, ss_token);
    else
      layout_permute_ss_scan_kernel<4><<<nblk, 4 * kWave, lds, s>>>(
          idx, T, E, k, R, per, bl.route_tpb, hist, counts, ded, dedup, lead, expert_offsets,
          rank_offsets, active, pos, src, ss_rank_offsets, ss_row, ss_token);
    return hipGetLastError();
  }
  hipError_t err = launch_route(logits, T, E, k, idx, w, counts, ws, s);
  if (err != hipSuccess) return err;
  err = launch_assign(counts, E, R, rep, rep ? maxrep : 1, id_order, assign, active, s);
  if (err != hipSuccess) return err;
  return launch_layout(idx, T, E, k, R, assign, rep, rep ? maxrep : 1, rank_of, expert_offsets,
                       rank_offsets, pos, src, dedup, ss_rank_offsets, ss_row, ss_token, ws, s);
}

}  // namespace moe
