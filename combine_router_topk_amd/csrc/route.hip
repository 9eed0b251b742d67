// Router top-k, gate weights and the global expert demand vector.
//
// "METRO AllGather vs AllToAll for MoE decode", section "METRO AllGather vs
// AllToAll changes the routing information": every token's top-k is taken and
// one demand count per expert is formed from all of them.
//
// Kernel 1 (route_topk, E <= 128): a group of L = 16 or 32 lanes owns one
// token's row of E logits (V = E/L values per lane, coalesced loads; the next
// token's logits are in flight while the current one is processed). Each of
// the k rounds takes the group maximum of order-preserving 32-bit keys with
// DPP butterflies (and readlane across 16-lane rows) and then the lowest
// expert id holding that key with ballots, so ties resolve to the lower id
// without 64-bit exchanges. Lane j of the group keeps slot j; the softmax over
// the selected logits is evaluated in fp64 by lanes 0..k-1 in parallel and
// summed with a fixed-order DPP tree. Selections are counted in an LDS
// histogram per block, written as one row of a [blocks, E] matrix: no global
// atomics.
// Kernel 1' (route_topk_wave, E > 128): one token per wave, each lane holding
// contiguous experts, so every step that decides a selection is wave-uniform
// (see the kernel's comment); measured 51 us against 60 us for the grouped
// kernel at T = 65536, E = 256, k = 8.
// Kernel 2 (column_sum): counts[e] = sum of column e of that matrix.
#include "device.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kRouteThreads = 1024;
constexpr int kRouteThreadsSmall = 256;  // small batches (see blocking_for)
constexpr int kRouteTargetBlocks = 512;

// With ded_rows set (contiguous partition, per = E / R experts per rank),
// each block also counts, per rank, its tokens with at least one selected
// expert on that rank (the single-send counts), written as one row of a
// [blocks, R] matrix beside the expert histogram; with lead set as well,
// lead[t] is token t's leader mask (bit j: slot j is the token's first slot
// on its rank).
template <int L, int V, int NT>
__global__ __launch_bounds__(NT) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int tpb, int32_t* __restrict__ idx,
    float* __restrict__ w, int32_t* __restrict__ block_hist, int32_t* __restrict__ ded_rows, int R,
    int per, int32_t* __restrict__ lead) {
  extern __shared__ int s_hist[];
  int* s_ded = s_hist + E;  // [R], used with ded_rows
  constexpr int TPW = kWave / L;  // tokens per wave step
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = NT / kWave;
  const int grp = lane / L;
  const int sl = lane % L;
  const uint64_t gmask = (L == 64) ? ~0ull : ((1ull << L) - 1ull) << (grp * L);

  const int t_begin = blockIdx.x * tpb;
  const int t_end = min(T, t_begin + tpb);

  // the next step's logits are loaded before the current token is processed
  const int tstep = nwaves * TPW;
  float nxt[V];
  {
    const int t = t_begin + wave * TPW + grp;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = sl + v * L;
      nxt[v] = (t < t_end && e < E) ? logits[(size_t)t * E + e] : 0.0f;
    }
  }
  if (block_hist != nullptr)  // uniform: a kernel argument
    for (int e = threadIdx.x; e < E; e += NT) s_hist[e] = 0;  // loads in flight meanwhile
  if (ded_rows != nullptr)
    for (int r = threadIdx.x; r < R; r += NT) s_ded[r] = 0;
  __syncthreads();
  for (int t0 = t_begin + wave * TPW; t0 < t_end; t0 += tstep) {
    const int t = t0 + grp;
    const bool valid = t < t_end;
    uint32_t key[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = sl + v * L;
      key[v] = (valid && e < E) ? logit_key(nxt[v]) : 0u;
    }
    {
      const int tn = t + tstep;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int e = sl + v * L;
        nxt[v] = (tn < t_end && e < E) ? logits[(size_t)tn * E + e] : 0.0f;
      }
    }
    int my_e = 0;
    uint32_t my_key = 0u, top_key = 0u;
    for (int j = 0; j < k; ++j) {
      uint32_t best = key[0];
#pragma unroll
      for (int v = 1; v < V; ++v) best = key[v] > best ? key[v] : best;
      best = group_max<L>(best);
      // lowest expert id e = v*L + lane-in-group whose key equals the maximum
      int e_sel = 0;
      bool found = false;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const uint64_t m = ballot(key[v] == best) & gmask;
        if (!found && m != 0ull) {
          e_sel = v * L + (__builtin_ctzll(m) - grp * L);
          found = true;
        }
      }
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (v * L + sl == e_sel) key[v] = 0u;  // taken: never chosen again
      if (sl == j) {
        my_e = e_sel;
        my_key = best;
      }
      if (j == 0) top_key = best;
    }

    // softmax over the k selected logits in fp64, lanes 0..k-1 of the group
    double ex = 0.0;
    if (sl < k) ex = exp(static_cast<double>(key_logit(my_key)) -
                         static_cast<double>(key_logit(top_key)));
    const double sum = group_sum16_f64<L>(ex);  // lanes >= k hold 0
    if (valid && sl < k) {
      const size_t o = (size_t)t * k + sl;
      idx[o] = my_e;
      w[o] = static_cast<float>(ex / sum);
      if (block_hist != nullptr) atomicAdd(&s_hist[my_e], 1);
    }
    if (ded_rows != nullptr) {  // uniform: a kernel argument
      // a slot counts for its rank unless a lower slot of the token has it
      const int rk = my_e / per;
      bool dup = false;
      for (int jj = 0; jj < k; ++jj) {
        const int o = __shfl(rk, grp * L + jj, kWave);
        dup |= (jj < sl) && (o == rk);
      }
      if (valid && sl < k && !dup) atomicAdd(&s_ded[rk], 1);
      if (lead != nullptr) {  // uniform: a kernel argument
        // bit j: slot j is the token's first slot on its rank
        const uint64_t lm = (ballot(valid && sl < k && !dup) & gmask) >> (grp * L);
        if (valid && sl == 0) lead[t] = static_cast<int32_t>(lm);
      }
    }
  }
  __syncthreads();
  if (block_hist != nullptr) {
    int32_t* row = block_hist + (size_t)blockIdx.x * E;
    for (int e = threadIdx.x; e < E; e += NT) row[e] = s_hist[e];
  }
  if (ded_rows != nullptr) {
    int32_t* drow = ded_rows + (size_t)blockIdx.x * R;
    for (int r = threadIdx.x; r < R; r += NT) drow[r] = s_ded[r];
  }
}

// One token per wave for wide rows (E > 128): lane l holds the V contiguous
// experts l*V .. l*V+V-1, so among equal keys the lowest expert id sits in
// the lowest lane holding that key, at the lowest slot of that lane. Each of
// the k rounds is then: the lane maximum, the wave maximum (uniform), one
// ballot for the lowest lane holding it, a readlane of that lane's first
// matching slot, a masked clear, and a select that records the choice in
// lane j. Everything that decides the selection is wave-uniform, so the
// scalar unit does little and the vector unit only O(V) work per round.
// The fp64 softmax waits until 64 / KP tokens have been selected (KP = k
// rounded up to a power of two): token s of a batch keeps its slot j in lane
// s KP + j, and one fp64 pass evaluates the whole batch. Evaluated per token,
// the softmax used k of the 64 lanes for the cost of all.
// ded_rows, R, per and lead as in route_topk_kernel.
template <int V, int KP, int NT>
__global__ __launch_bounds__(NT) void route_topk_wave_kernel(
    const float* __restrict__ logits, int T, int E, int k, int tpb, int32_t* __restrict__ idx,
    float* __restrict__ w, int32_t* __restrict__ block_hist, int32_t* __restrict__ ded_rows, int R,
    int per, int32_t* __restrict__ lead) {
  extern __shared__ int s_hist[];
  int* s_ded = s_hist + E;  // [R], used with ded_rows
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = NT / kWave;
  const int e0 = lane * V;
  const bool vec = (E & 3) == 0;  // rows are whole 16-byte chunks
  const int t_begin = blockIdx.x * tpb;
  const int t_end = min(T, t_begin + tpb);

  auto load_row = [&](int t, float (&f)[V]) {
    const float* row = logits + (size_t)t * E;
    if (vec) {
#pragma unroll
      for (int c = 0; c < V; c += 4) {
        if (t < t_end && e0 + c < E) {
          const float4 q = *reinterpret_cast<const float4*>(row + e0 + c);
          f[c] = q.x; f[c + 1] = q.y; f[c + 2] = q.z; f[c + 3] = q.w;
        } else {
          f[c] = f[c + 1] = f[c + 2] = f[c + 3] = 0.0f;
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v) f[v] = (t < t_end && e0 + v < E) ? row[e0 + v] : 0.0f;
    }
  };

  constexpr int kBatch = kWave / KP;  // tokens per softmax batch
  int slot = 0;                        // the current token's place in the batch
  uint32_t b_e = 0u, b_key = 0u, b_top = 0u;
  int b_t = 0;
  auto flush = [&](int filled) {
    const int j = lane % KP;
    const bool on = lane / KP < filled && j < k;
    double ex = 0.0;
    if (on) ex = exp(static_cast<double>(key_logit(b_key)) - static_cast<double>(key_logit(b_top)));
    const double sum = group_sum_f64<KP>(ex);  // lanes j >= k hold 0
    if (on) {
      const size_t o = (size_t)b_t * k + j;
      idx[o] = static_cast<int32_t>(b_e);
      w[o] = static_cast<float>(ex / sum);
      if (block_hist != nullptr) atomicAdd(&s_hist[b_e], 1);
    }
    if (ded_rows != nullptr) {  // uniform: a kernel argument
      // a slot counts for its rank unless a lower slot of the token has it
      const int rk = static_cast<int>(b_e) / per;
      bool dup = false;
#pragma unroll
      for (int jj = 0; jj < KP; ++jj) {
        const int o = __shfl(rk, (lane & ~(KP - 1)) + jj, kWave);
        dup |= (jj < j) && (o == rk);
      }
      if (on && !dup) atomicAdd(&s_ded[rk], 1);
      if (lead != nullptr) {  // uniform: a kernel argument
        // bit j: slot j is the token's first slot on its rank
        const uint64_t lm = ballot(on && !dup) >> (lane & ~(KP - 1));
        if (on && j == 0) lead[b_t] = static_cast<int32_t>(lm & ((KP < 64 ? (1ull << KP) : 0ull) - 1ull));
      }
    }
  };

  float nxt[V];
  load_row(t_begin + wave, nxt);
  if (block_hist != nullptr)  // uniform: a kernel argument
    for (int e = threadIdx.x; e < E; e += NT) s_hist[e] = 0;  // the load in flight meanwhile
  if (ded_rows != nullptr)
    for (int r = threadIdx.x; r < R; r += NT) s_ded[r] = 0;
  __syncthreads();
  for (int t = t_begin + wave; t < t_end; t += nwaves) {
    uint32_t key[V];
#pragma unroll
    for (int v = 0; v < V; ++v) key[v] = (e0 + v < E) ? logit_key(nxt[v]) : 0u;
    load_row(t + nwaves, nxt);  // the wave's next token, in flight meanwhile

    uint32_t top_key = 0u;
    for (int j = 0; j < k; ++j) {
      uint32_t lm = key[0];
#pragma unroll
      for (int v = 1; v < V; ++v) lm = umax(lm, key[v]);
      const uint32_t best = wave_max_u32(lm);
      const int l = __builtin_ctzll(ballot(lm == best));  // lowest lane holding it
      int fv = V - 1;
#pragma unroll
      for (int v = V - 2; v >= 0; --v) fv = key[v] == best ? v : fv;
      const int fvs = __builtin_amdgcn_readlane(fv, l);
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (v == fvs) key[v] = lane == l ? 0u : key[v];  // taken: never chosen again
      const int e_sel = l * V + fvs;
      if (lane == slot * KP + j) {
        b_e = static_cast<uint32_t>(e_sel);
        b_key = best;
      }
      if (j == 0) top_key = best;
    }
    if (lane / KP == slot) {
      b_top = top_key;
      b_t = t;
    }
    if (++slot == kBatch) {  // softmax over the k selected logits of each token, in fp64
      flush(kBatch);
      slot = 0;
    }
  }
  if (slot > 0) flush(slot);
  __syncthreads();
  if (block_hist != nullptr) {
    int32_t* row = block_hist + (size_t)blockIdx.x * E;
    for (int e = threadIdx.x; e < E; e += NT) row[e] = s_hist[e];
  }
  if (ded_rows != nullptr) {
    int32_t* drow = ded_rows + (size_t)blockIdx.x * R;
    for (int r = threadIdx.x; r < R; r += NT) drow[r] = s_ded[r];
  }
}

// out[c] = sum over rows of M[rows, cols]; one block per 64 columns, the 16
// waves split the rows (at most kSumSeg each) and meet in LDS. Each lane
// issues its whole segment of loads at once. Deterministic, no atomics.
constexpr int kSumSeg = 32;  // route blocks <= 16 * 32 = 512 (see blocking_for)

__global__ __launch_bounds__(1024) void column_sum_kernel(const int32_t* __restrict__ M, int rows,
                                                          int cols, int32_t* __restrict__ out) {
  __shared__ int part[16][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int c = blockIdx.x * kWave + lane;
  const int seg = (rows + 15) / 16;
  const int r_lo = min(rows, wave * seg), r_hi = min(rows, r_lo + seg);
  int acc = 0;
  if (c < cols) {
#pragma unroll
    for (int i = 0; i < kSumSeg; ++i) {
      const int r = r_lo + i;
      acc += (r < r_hi) ? M[(size_t)r * cols + c] : 0;
    }
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && c < cols) {
    int s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += part[i][lane];
    out[c] = s;
  }
}

struct TopkArgs {
  const float* logits;
  int T, E, k, tpb, nblk, threads;
  int32_t* idx;
  float* w;
  int32_t* hist;
  int32_t* ded;  // null: no per-rank counts
  int R, per;
  int32_t* lead;  // null: no leader masks (needs ded)
  size_t lds() const { return (size_t)(E + (ded != nullptr ? R : 0)) * sizeof(int); }
};

template <int L, int V>
hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.threads == kRouteThreadsSmall)
    route_topk_kernel<L, V, kRouteThreadsSmall><<<a.nblk, kRouteThreadsSmall, a.lds(), s>>>(
        a.logits, a.T, a.E, a.k, a.tpb, a.idx, a.w, a.hist, a.ded, a.R, a.per, a.lead);
  else
    route_topk_kernel<L, V, kRouteThreads><<<a.nblk, kRouteThreads, a.lds(), s>>>(
        a.logits, a.T, a.E, a.k, a.tpb, a.idx, a.w, a.hist, a.ded, a.R, a.per, a.lead);
  return hipGetLastError();
}

template <int V, int NT>
hipError_t launch_wave_nt(const TopkArgs& a, hipStream_t s) {
#define MOE_WAVE(KP)                                                                    \
  route_topk_wave_kernel<V, KP, NT><<<a.nblk, NT, a.lds(), s>>>(                        \
      a.logits, a.T, a.E, a.k, a.tpb, a.idx, a.w, a.hist, a.ded, a.R, a.per, a.lead)
  if (a.k <= 1) MOE_WAVE(1);
  else if (a.k <= 2) MOE_WAVE(2);
  else if (a.k <= 4) MOE_WAVE(4);
  else if (a.k <= 8) MOE_WAVE(8);
  else MOE_WAVE(16);
#undef MOE_WAVE
  return hipGetLastError();
}

template <int V>
hipError_t launch_wave(const TopkArgs& a, hipStream_t s) {
  return a.threads == kRouteThreadsSmall ? launch_wave_nt<V, kRouteThreadsSmall>(a, s)
                                         : launch_wave_nt<V, kRouteThreads>(a, s);
}

// Lanes per token: about four logits per lane measured fastest (T = 65536,
// E = 256, k = 8: 56 us at 64 lanes x 4 against 74 us at 16 x 16 and 85 us at
// 32 x 8; T = 16384, E = 64, k = 2: 6.6 us at 16 x 4 against 8.2 us at 64 x 1).
// At least 16 lanes, so lanes 0..k-1 can hold the k <= 16 slots.
int lanes_per_token(int E) {
  int L = 16;
  while (L < 64 && L * 4 < E) L *= 2;
  return L;
}

}  // namespace

Blocking blocking_for(int T, int E, int R) {
  Blocking b{};
  const int tpw = kWave / lanes_per_token(E);
  // A small batch takes 256-thread blocks of one token step per wave: the
  // blocks spread over four times the CUs with one wave per SIMD (in a
  // 1024-thread block four waves share each SIMD and the block waits for
  // the last). Only while the one-workgroup plans, which sum the blocks'
  // histogram rows per column with 1024 / E thread groups, keep at most 16
  // rows per group (and at most 64 blocks).
  const int step_small = tpw * (kRouteThreadsSmall / kWave);
  const int groups = E >= 1024 ? 1 : 1024 / E;
  const int nblk_small = (T + step_small - 1) / step_small;
  if (nblk_small <= 64 && nblk_small <= 16 * groups) {
    b.route_threads = kRouteThreadsSmall;
    b.route_tpb = step_small;
    b.route_nblk = nblk_small;
  } else {
    const int step = tpw * (kRouteThreads / kWave);
    int tpb = (T + kRouteTargetBlocks - 1) / kRouteTargetBlocks;
    tpb = ((tpb + step - 1) / step) * step;
    if (tpb < step) tpb = step;
    b.route_threads = kRouteThreads;
    b.route_tpb = tpb;
    b.route_nblk = (T + tpb - 1) / tpb;
  }
  // The layout plan scans [blocks, E] and [blocks, R] in tasks of 64 columns
  // with 16 waves; each wave may own at most 48 rows of one task, so the
  // block count is capped at 48 * (waves per task), and at 256.
  const int tasks = (E + kWave - 1) / kWave + (R + kWave - 1) / kWave;
  const int waves_per_task = tasks >= 16 ? 1 : 16 / tasks;
  const int max_nblk = 48 * waves_per_task < 256 ? 48 * waves_per_task : 256;
  int ltpb = 64;
  while ((T + ltpb - 1) / ltpb > max_nblk) ltpb *= 2;
  b.layout_tpb = ltpb;
  b.layout_nblk = (T + ltpb - 1) / ltpb;
  return b;
}

size_t workspace_bytes(int T, int E, int R) {
  const Blocking b = blocking_for(T, E, R);
  // route rows [blocks, E], plus [blocks, R] of per-rank counts when the
  // one-call plan takes them from the top-k kernel, plus T leader masks when
  // the one-call single-send plan does
  const size_t route = ((size_t)b.route_nblk * (E + R) + (size_t)T) * sizeof(int32_t);
  const size_t layout = ((size_t)b.layout_nblk * (E + R) + (size_t)T) * sizeof(int32_t);
  size_t n = route > layout ? route : layout;
  n = (n + 255) & ~(size_t)255;
  return n < 256 ? 256 : n;
}

size_t route_assign_layout_ws_bytes(int T, int E, int R) {
  const Blocking b = blocking_for(T, E, R);
  const size_t route = (size_t)b.route_nblk * (E + R) * sizeof(int32_t);
  const size_t layout = (size_t)b.layout_nblk * (E + R) * sizeof(int32_t);
  size_t n = route > layout ? route : layout;
  n = (n + 255) & ~(size_t)255;
  return n < 256 ? 256 : n;
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                             int32_t* ws, hipStream_t s, int32_t* ded_rows, int R,
                             int32_t* lead) {
  if (T == 0) return hipSuccess;
  const Blocking b = blocking_for(T, E, 1);
  const int L = lanes_per_token(E);
  const int V = (E + L - 1) / L;  // L = 16: 1..4; 32: 3..4; 64: 3..16
  const TopkArgs a{logits, T, E, k, b.route_tpb, b.route_nblk, b.route_threads, idx, w, ws, ded_rows, R,
                   ded_rows != nullptr ? E / R : 1, ded_rows != nullptr ? lead : nullptr};
  if (L == 16 && V == 1) return launch_topk<16, 1>(a, s);
  if (L == 16 && V == 2) return launch_topk<16, 2>(a, s);
  if (L == 16) return launch_topk<16, 4>(a, s);
  if (L == 32) return launch_topk<32, 4>(a, s);
  if (V <= 4) return launch_wave<4>(a, s);
  if (V <= 8) return launch_wave<8>(a, s);
  return launch_wave<16>(a, s);
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                        int32_t* counts, int32_t* ws, hipStream_t s) {
  const Blocking b = blocking_for(T, E, 1);
  const hipError_t err = launch_route_topk(logits, T, E, k, idx, w, ws, s);
  if (err != hipSuccess) return err;
  const int rows = T > 0 ? b.route_nblk : 0;
  column_sum_kernel<<<(E + kWave - 1) / kWave, 1024, 0, s>>>(ws, rows, E, counts);
  return hipGetLastError();
}

}  // namespace moe
