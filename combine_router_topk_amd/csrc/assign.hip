// Greedy replica assignment: the kernel that keeps the activated experts per
// GPU small, one workgroup running assign_block (greedy.hpp, which holds the
// algorithm and its source).
#include "device.hpp"
#include "greedy.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kAssignThreads = kGreedyThreads;

__global__ __launch_bounds__(kAssignThreads) void assign_kernel(
    const int32_t* __restrict__ counts, int E, int R, const int32_t* __restrict__ rep, int maxrep,
    int id_order, int32_t* __restrict__ assign, int32_t* __restrict__ active) {
  __shared__ int act[kMaxR];
  __shared__ unsigned char ncand[kMaxE];
  __shared__ __align__(16) unsigned short cand[kMaxE * kMaxRep];  // valid candidates, table order
  assign_block(counts, E, R, rep, maxrep, id_order, assign, act, ncand, cand);
  for (int g = threadIdx.x; g < R; g += kAssignThreads) active[g] = act[g];
}

}  // namespace

hipError_t launch_assign(const int32_t* counts, int E, int R, const int32_t* rep, int maxrep,
                         bool id_order, int32_t* assign, int32_t* active, hipStream_t s) {
  assign_kernel<<<1, kAssignThreads, 0, s>>>(counts, E, R, rep, maxrep, id_order ? 1 : 0, assign,
                                            active);
  return hipGetLastError();
}

}  // namespace moe
