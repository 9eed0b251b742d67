// Greedy replica assignment as a device function of one 1024-thread
// workgroup, shared by the assignment kernel and the fused small-batch
// routing plan.
//
// "METRO AllGather vs AllToAll for MoE decode", section "METRO AllGather vs
// AllToAll changes the routing information" (each active expert is served by
// one replica, on the GPU with the fewest experts activated so far) and
// section "Add the expert-weight traffic term" (a greedy pass, not the
// optimum). Ties go to the lower GPU index.
//
// The activated-expert counters and every active expert's valid candidates
// live in LDS. Experts with a single candidate have no choice; in the default
// (most-constrained-first) order they are all counted first, in parallel with
// LDS atomics (integer adds commute, so the result is order-free). Experts
// with c >= 2 candidates are then visited in ascending (c, id): wave 0
// compacts each 64-expert chunk with a ballot and walks the set bits in
// order, so every choice sees the counters left by all earlier choices. The
// ascending-id order visits every active expert in the sequential walk. A
// choice takes the candidate with the fewest activated experts, the lower GPU
// index on ties.
#pragma once

#include "device.hpp"

namespace moe {

constexpr int kMaxRep = 16;  // replica-table columns (the C ABI caps maxrep)
constexpr int kGreedyThreads = 1024;  // the workgroup of assign_block


// The sequential part of the greedy, run by one wave. Multi-candidate experts
// are visited in ascending (candidates, id) (or ascending id): each 64-expert
// chunk is compacted with a ballot and its candidate lists are loaded into
// registers once; each choice is then the scalar minimum of
// (activated << 16 | gpu) over the expert's candidates, which is the fewest
// activated experts with ties to the lower GPU index. With IN_REG the keys
// themselves live in a register (lane g holds act[g] << 16 | g, at most 64
// GPUs), so a candidate's key is one readlane; else the counters are in LDS.
// Every value that decides a choice is wave-uniform.
// `gpus` (IN_REG only) restricts the walk to the experts whose candidates lie
// in that set of GPUs (tested on the first candidate), and only those GPUs'
// counters are written back: walkers given disjoint unions of whole
// components of the GPU graph (GPUs joined by a shared expert) make the
// same choices as one walker, since an expert's choice reads and changes
// only counters of its own component.
template <bool IN_REG>
__device__ __forceinline__ void greedy_walk(int E, int maxrep, int id_order, const unsigned char* ncand,
                                            const unsigned short* cand, int* act,
                                            int32_t* __restrict__ assign, uint64_t gpus = ~0ull) {
  const int lane = threadIdx.x & (kWave - 1);
  // lanes >= R hold keys never read
  uint32_t key_reg = IN_REG ? (static_cast<uint32_t>(act[lane]) << 16) | static_cast<uint32_t>(lane) : 0u;
  const int c_lo = id_order ? 0 : 2;     // class 0: any active expert
  const int c_hi = id_order ? 0 : maxrep;
  for (int c = c_lo; c <= c_hi; ++c) {
    for (int base = 0; base < E; base += kWave) {
      const int e = base + lane;
      const int ce = e < E ? ncand[e] : 0;
      const int g_first = ce > 0 ? cand[e * kMaxRep] : 0;
      uint64_t m = ballot((c == 0 ? ce > 0 : ce == c) && ((gpus >> (g_first & 63)) & 1ull));
      if (m == 0ull) continue;
      uint32_t cpk[kMaxRep / 2];  // this lane's expert: candidates as 16-bit pairs
#pragma unroll
      for (int i = 0; i < kMaxRep / 2; ++i)
        cpk[i] = (e < E && 2 * i < maxrep) ? reinterpret_cast<const uint32_t*>(cand + e * kMaxRep)[i] : 0u;
      while (m != 0ull) {
        const int b = __builtin_ctzll(m);
        m &= m - 1ull;
        const int n = __builtin_amdgcn_readlane(ce, b);
        uint32_t best = 0xFFFFFFFFu;
        auto consider = [&](uint32_t g) {
          const uint32_t key = IN_REG ? static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(key_reg), g))
                                      : (static_cast<uint32_t>(act[g]) << 16) | g;
          best = key < best ? key : best;
        };
#pragma unroll
        for (int q = 0; q < kMaxRep / 2; ++q) {
          if (2 * q >= n) break;
          const uint32_t pr = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(cpk[q]), b));
          consider(pr & 0xFFFFu);
          if (2 * q + 1 < n) consider(pr >> 16);
        }
        const int g = static_cast<int>(best & 0xFFFFu);
        if (IN_REG) key_reg += (lane == g) ? 0x10000u : 0u;
        else act[g] = static_cast<int>(best >> 16) + 1;  // every lane writes the same value
        if (lane == 0) assign[base + b] = g;
      }
    }
  }
  // act holds at least 64 entries (see assign_block)
  if (IN_REG && ((gpus >> lane) & 1ull)) act[lane] = static_cast<int>(key_reg >> 16);
}

// The walk of greedy_walk<true> (at most 64 GPUs) for tables of at most
// kPackedRep columns, with each expert's valid candidates packed in one
// 32-bit word: candidate q in bits 6q..6q+5, their number in bits 24..31
// (0 for an inactive expert). Every 64-expert chunk of words is loaded into
// registers before the walk, so a choice is one readlane of its expert's
// word and one readlane of a key per candidate, with no LDS access; the
// choices of a chunk are gathered in a register and stored once. Same
// visiting order and same choices as greedy_walk; the walker's GPUs are
// found with walker_gpus (adj, R, walker, walkers as there) while the
// words and counters are in flight.
constexpr int kPackedRep = 4;

__device__ __forceinline__ uint64_t walker_gpus(const unsigned long long* adj, int R, int walker,
                                                int walkers);

// NC: the most candidates an expert can have (maxrep <= NC <= kPackedRep).
template <int NC>
__device__ __forceinline__ void greedy_walk_packed(int E, int maxrep, int id_order,
                                                   const uint32_t* word, int* act,
                                                   int32_t* __restrict__ assign,
                                                   const unsigned long long* adj, int R,
                                                   int walker, int walkers) {
  constexpr int kChunks = kMaxE / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int nch = (E + kWave - 1) / kWave;
  uint32_t key_reg = (static_cast<uint32_t>(act[lane]) << 16) | static_cast<uint32_t>(lane);
  uint32_t wv[kChunks];
#pragma unroll
  for (int ch = 0; ch < kChunks; ++ch) {
    const int e = ch * kWave + lane;
    wv[ch] = ch < nch ? word[e < E ? e : E - 1] : 0u;  // uniform test; clamped index
    wv[ch] = e < E ? wv[ch] : 0u;
  }
  const uint64_t gpus = walker_gpus(adj, R, walker, walkers);
  if (gpus == 0ull) return;  // uniform
  const int c_lo = id_order ? 0 : 2;  // class 0: any active expert
  const int c_hi = id_order ? 0 : maxrep;
  for (int c = c_lo; c <= c_hi; ++c) {
#pragma unroll
    for (int ch = 0; ch < kChunks; ++ch) {
      if (ch >= nch) break;
      const uint32_t wd = wv[ch];
      const int ce = static_cast<int>(wd >> 24);
      const uint64_t walked = ballot((c == 0 ? ce > 0 : ce == c) && ((gpus >> (wd & 63u)) & 1ull));
      uint64_t m = walked;
      int gsel = -1;
      while (m != 0ull) {
        const int b = __builtin_ctzll(m);
        m &= m - 1ull;
        const uint32_t x = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wd), b));
        const int n = static_cast<int>(x >> 24);
        auto key = [&](int q) {
          return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(key_reg), (x >> (6 * q)) & 63u));
        };
        uint32_t best = key(0);
#pragma unroll
        for (int q = 1; q < NC; ++q) {
          const uint32_t kq = key(q);
          best = (q < n && kq < best) ? kq : best;
        }
        const int g = static_cast<int>(best & 0xFFFFu);
        // lane g's key becomes best with one more activated expert (a
        // uniform value: one select); lane b records g
        const uint32_t bumped = best + 0x10000u;
        key_reg = (lane == g) ? bumped : key_reg;
        gsel = (lane == b) ? g : gsel;
      }
      if ((walked >> lane) & 1ull) assign[ch * kWave + lane] = gsel;
    }
  }
  if ((gpus >> lane) & 1ull) act[lane] = static_cast<int>(key_reg >> 16);
}

// The components of the GPU graph in which two GPUs are joined when some
// walked expert has both as candidates, found by one wave (R <= 64, lane g
// for GPU g): adj is each GPU's union of the candidate sets of the walked
// experts that list it (symmetric, so a GPU joins a component exactly when
// its adj meets it, one ballot per step). Component i, in the order of their
// lowest GPU, goes to walker i % walkers; returns the GPUs of `walker`'s
// components. Wave-uniform.
__device__ __forceinline__ uint64_t walker_gpus(const unsigned long long* adj, int R, int walker,
                                                int walkers) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t a = lane < R ? adj[lane] : 0ull;
  uint64_t todo = ballot(a != 0ull);
  uint64_t mine = 0ull;
  for (int i = 0; todo != 0ull; ++i) {
    // start from the lowest remaining GPU's whole row (it lists the GPU
    // itself), which already holds its neighbours
    const int g0 = __builtin_ctzll(todo);
    uint64_t comp = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(a >> 32), g0))) << 32) |
                    static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(a), g0));
    for (;;) {
      const uint64_t grown = comp | ballot((a & comp) != 0ull);
      if (grown == comp) break;
      comp = grown;
    }
    if (i % walkers == walker) mine |= comp;
    todo &= ~comp;
  }
  return mine;
}

// The whole assignment by one 1024-thread workgroup. counts [E] (read) and
// assign [E] (write) may be global or LDS; act (max(R, 64) ints), ncand
// (E bytes) and cand (E * kMaxRep 16-bit entries, 4-byte aligned) are LDS
// scratch. On return (after a barrier) act[g] holds the activated experts of
// GPU g. All threads take part.
__device__ __forceinline__ void assign_block(const int32_t* counts, int E, int R,
                                    const int32_t* __restrict__ rep, int maxrep, int id_order,
                                    int32_t* assign, int* act, unsigned char* ncand,
                                    unsigned short* cand) {
  const int tid = threadIdx.x;
  for (int g = tid; g < (R > kWave ? R : kWave); g += kGreedyThreads) act[g] = 0;
  __syncthreads();
  if (rep == nullptr) {
    const int per = E / R;
    for (int e = tid; e < E; e += kGreedyThreads) {
      const bool on = counts[e] > 0;
      assign[e] = on ? e / per : -1;
      if (on) atomicAdd(&act[e / per], 1);
    }
  } else {
    // in parallel: each active expert's valid candidates go to LDS, so the
    // sequential walk below never waits on global memory (the count and the
    // replica row are loaded together)
    for (int e = tid; e < E; e += kGreedyThreads) {
      const int cnt = counts[e];
      const int32_t* row = rep + (size_t)e * maxrep;
      int x[kMaxRep];
#pragma unroll
      for (int s = 0; s < kMaxRep; ++s) x[s] = s < maxrep ? row[s] : -1;  // uniform test
      int c = 0;
      if (cnt > 0) {
#pragma unroll
        for (int s = 0; s < kMaxRep; ++s)
          if (s < maxrep && x[s] >= 0 && x[s] < R) cand[e * kMaxRep + c++] = static_cast<unsigned short>(x[s]);
      }
      ncand[e] = static_cast<unsigned char>(c);
      if (c == 0) assign[e] = -1;  // inactive (or no valid candidate)
      if (!id_order && c == 1) {
        const int g = cand[e * kMaxRep];
        assign[e] = g;
        atomicAdd(&act[g], 1);
      }
    }
    __syncthreads();
    if (tid < kWave) {
      if (R <= kWave) greedy_walk<true>(E, maxrep, id_order, ncand, cand, act, assign);
      else greedy_walk<false>(E, maxrep, id_order, ncand, cand, act, assign);
    }
  }
  __syncthreads();
}

}  // namespace moe
