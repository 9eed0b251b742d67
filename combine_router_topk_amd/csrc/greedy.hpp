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

// The sequential part of the greedy, run by one wave. Multi-candidate experts
// are visited in ascending (candidates, id) (or ascending id): each 64-expert
// chunk is compacted with a ballot and its candidate lists are loaded into
// registers once; each choice is then the scalar minimum of
// (activated << 16 | gpu) over the expert's candidates, which is the fewest
// activated experts with ties to the lower GPU index. With IN_REG the keys
// themselves live in a register (lane g holds act[g] << 16 | g, at most 64
// GPUs), so a candidate's key is one readlane; else the counters are in LDS.
// Every value that decides a choice is wave-uniform.
template <bool IN_REG>
__device__ void greedy_walk(int E, int maxrep, int id_order, const unsigned char* ncand,
                            const unsigned short* cand, int* act, int32_t* __restrict__ assign) {
  const int lane = threadIdx.x & (kWave - 1);
  // lanes >= R hold keys never read
  uint32_t key_reg = IN_REG ? (static_cast<uint32_t>(act[lane]) << 16) | static_cast<uint32_t>(lane) : 0u;
  const int c_lo = id_order ? 0 : 2;     // class 0: any active expert
  const int c_hi = id_order ? 0 : maxrep;
  for (int c = c_lo; c <= c_hi; ++c) {
    for (int base = 0; base < E; base += kWave) {
      const int e = base + lane;
      const int ce = e < E ? ncand[e] : 0;
      uint64_t m = ballot(c == 0 ? ce > 0 : ce == c);
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
  if (IN_REG) act[lane] = static_cast<int>(key_reg >> 16);  // act holds at least 64 entries (see assign_block)
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
  for (int g = tid; g < (R > kWave ? R : kWave); g += blockDim.x) act[g] = 0;
  __syncthreads();
  if (rep == nullptr) {
    const int per = E / R;
    for (int e = tid; e < E; e += blockDim.x) {
      const bool on = counts[e] > 0;
      assign[e] = on ? e / per : -1;
      if (on) atomicAdd(&act[e / per], 1);
    }
  } else {
    // in parallel: each active expert's valid candidates go to LDS, so the
    // sequential walk below never waits on global memory
    for (int e = tid; e < E; e += blockDim.x) {
      int c = 0;
      if (counts[e] > 0) {
        for (int s = 0; s < maxrep; ++s) {
          const int x = rep[e * maxrep + s];
          if (x >= 0 && x < R) cand[e * kMaxRep + c++] = static_cast<unsigned short>(x);
        }
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
