// Greedy replica assignment: the kernel that keeps the activated experts per GPU small.
//
// "METRO AllGather vs AllToAll for MoE decode", section "METRO AllGather vs
// AllToAll changes the routing information" (each active expert is served by
// one replica, on the GPU with the fewest experts activated so far) and
// section "Add the expert-weight traffic term" (a greedy pass, not the
// optimum). Ties go to the lower GPU index.
//
// One workgroup. The activated-expert counters live in LDS. Experts with a
// single candidate have no choice; in the default (most-constrained-first)
// order they are all counted first, in parallel with LDS atomics (integer
// adds commute, so the result is order-free). Experts with c >= 2 candidates
// are then visited in ascending (c, id): wave 0 compacts each 64-expert chunk
// with a ballot and walks the set bits in order, so every choice sees the
// counters left by all earlier choices. The ascending-id order visits every
// active expert in the sequential walk.
#include "device.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kAssignThreads = 1024;

__device__ __forceinline__ int n_candidates(const int32_t* __restrict__ rep, int e, int maxrep,
                                            int R) {
  int n = 0;
  for (int s = 0; s < maxrep; ++s) {
    const int g = rep[e * maxrep + s];
    n += (g >= 0 && g < R) ? 1 : 0;
  }
  return n;
}

// Candidate of expert e with the fewest activated experts; lower GPU index on
// ties. Uniform across the wave (e is uniform). Returns -1 if none is valid.
__device__ __forceinline__ int pick_replica(const int32_t* __restrict__ rep, int e, int maxrep,
                                            int R, const int* act) {
  int best_g = -1, best_a = 0;
  for (int s = 0; s < maxrep; ++s) {
    const int g = rep[e * maxrep + s];
    if (g < 0 || g >= R) continue;
    const int a = act[g];
    if (best_g < 0 || a < best_a || (a == best_a && g < best_g)) {
      best_g = g;
      best_a = a;
    }
  }
  return best_g;
}

__global__ __launch_bounds__(kAssignThreads) void assign_kernel(
    const int32_t* __restrict__ counts, int E, int R, const int32_t* __restrict__ rep, int maxrep,
    int id_order, int32_t* __restrict__ assign, int32_t* __restrict__ active) {
  __shared__ int act[kMaxR];
  __shared__ unsigned char ncand[kMaxE];
  const int tid = threadIdx.x;
  for (int g = tid; g < R; g += blockDim.x) act[g] = 0;
  __syncthreads();

  if (rep == nullptr) {
    const int per = E / R;
    for (int e = tid; e < E; e += blockDim.x) {
      const bool on = counts[e] > 0;
      assign[e] = on ? e / per : -1;
      if (on) atomicAdd(&act[e / per], 1);
    }
  } else {
    for (int e = tid; e < E; e += blockDim.x) {
      const int c = counts[e] > 0 ? n_candidates(rep, e, maxrep, R) : 0;
      ncand[e] = static_cast<unsigned char>(c);
      if (c == 0) assign[e] = -1;  // inactive (or no valid candidate)
      if (!id_order && c == 1) {
        int g = -1;
        for (int s = 0; s < maxrep && g < 0; ++s) {
          const int x = rep[e * maxrep + s];
          if (x >= 0 && x < R) g = x;
        }
        assign[e] = g;
        atomicAdd(&act[g], 1);
      }
    }
    __syncthreads();
    if (tid < kWave) {
      const int lane = tid;
      // visiting classes: id order walks every active expert once (class 0
      // means "any"); constrained order walks classes 2..maxrep
      const int c_lo = id_order ? 0 : 2;
      const int c_hi = id_order ? 0 : maxrep;
      for (int c = c_lo; c <= c_hi; ++c) {
        for (int base = 0; base < E; base += kWave) {
          const int e = base + lane;
          const int ce = e < E ? ncand[e] : 0;
          uint64_t m = ballot(c == 0 ? ce > 0 : ce == c);
          while (m != 0ull) {
            const int b = __builtin_ctzll(m);
            m &= m - 1ull;
            const int ee = base + b;
            // every lane reads the same counters and applies the same
            // update, so each lane's view stays consistent in program order
            const int g = pick_replica(rep, ee, maxrep, R, act);
            if (g >= 0) {
              act[g] = act[g] + 1;
              if (lane == 0) assign[ee] = g;
            }
          }
        }
      }
    }
  }
  __syncthreads();
  for (int g = tid; g < R; g += blockDim.x) active[g] = act[g];
}

}  // namespace

hipError_t launch_assign(const int32_t* counts, int E, int R, const int32_t* rep, int maxrep,
                         bool id_order, int32_t* assign, int32_t* active, hipStream_t s) {
  assign_kernel<<<1, kAssignThreads, 0, s>>>(counts, E, R, rep, maxrep, id_order ? 1 : 0, assign,
                                            active);
  return hipGetLastError();
}

}  // namespace moe
