// Internal launch interface between the C ABI (abi.hip) and the kernels.
// Shapes are validated by the caller; these functions only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Token blocking used by the route and layout kernels. One function decides
// it so the workspace size and the launches always agree.
struct Blocking {
  int route_tpb;          // tokens per route block
  int route_nblk;         // route blocks (<= 512)
  int route_threads;      // threads per route block (1024, or 256 for a small batch)
  int layout_tpb;         // tokens per layout block
  int layout_nblk;        // layout blocks (<= 32 * waves per column task, <= 256)
};
Blocking blocking_for(int T, int E, int R);

// LDS reservations of the one-row kernels (a kernel declares its dynamic LDS
// with declare_lds_reserve and never touches it): a launch passes one to cap
// how many blocks share a CU. Launches of fewer than 16 blocks per CU take
// none, since there a cap on resident blocks only adds rounds of blocks
// (decode fan-out, 2048 blocks: 9.8 us without, 11.0 us with 32 KiB).
constexpr size_t kKiB = 1024;
constexpr long long kMinBlocksToCap = 16 * 256;
inline size_t if_many_blocks(size_t res, long long blocks) {
  return blocks >= kMinBlocksToCap ? res : 0;
}

// Sliced launches (see slice_of_block) take at most kMaxSliceBlocks blocks
// each, whole rows, which keeps every grid far below the 2^32 work-items a
// launch can address; every workload here fits one launch (T = 65536 at
// H = 7168: 458,752 blocks for the dispatch, 3,670,016 for the stand-in's
// T k rows). slice_launches calls launch(first_row, blocks) for each launch
// of `rows` rows of S slices.
constexpr long long kMaxSliceBlocks = 1 << 22;
// A kernel slices its rows only in launches of at least `min_slices`
// slices (kMinBlocksToCap unless its launcher names more): smaller launches
// are latency-bound, and there one-row blocks, which issue their index loads
// alongside the row loads, finish sooner (decode, T = 256, k = 8,
// H = 4096: combine 9.9 us in 1024 slices against 6.9 us in 256 one-row
// blocks; dispatch backward 10.4 against 9.4 us).
inline bool enough_slices(long long rows, int slices, long long min_slices = kMinBlocksToCap) {
  return rows * slices >= min_slices;
}
template <typename F>
inline void slice_launches(int rows, int S, F&& launch) {
  const long long per_ll = kMaxSliceBlocks / S;
  const int per = per_ll > 0 ? static_cast<int>(per_ll) : 1;
  for (int r0 = 0; r0 < rows; r0 += per) {
    const int n = rows - r0 < per ? rows - r0 : per;
    launch(r0, static_cast<unsigned>(n) * static_cast<unsigned>(S));
  }
}

// Workspace bytes for route and layout (the larger of the two).
size_t workspace_bytes(int T, int E, int R);

// The part of that workspace launch_route_assign_layout uses: the route's
// block rows or the layout's block matrices, without the single-send leader
// masks.
size_t route_assign_layout_ws_bytes(int T, int E, int R);

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                        int32_t* counts, int32_t* ws, hipStream_t s);

// The top-k kernel of launch_route alone: idx, w, and one histogram row per
// route block in ws ([blocking_for(T, E, R).route_nblk, E]; none when ws is
// null), no counts.
// With ded_rows (and ws; R | E, contiguous partition), also one row per route block
// of per-rank token counts ([route_nblk, R]: tokens of the block with at
// least one selected expert on the rank), and with lead as well each token's
// leader mask ([T]: bit j set when slot j is the token's first slot on its
// rank).
hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                             int32_t* ws, hipStream_t s, int32_t* ded_rows = nullptr, int R = 1,
                             int32_t* lead = nullptr);

// route, assign and layout of one batch: for a small batch the top-k kernel
// and one workgroup that does everything else, else the three launches.
hipError_t launch_route_assign_layout(const float* logits, int T, int E, int k, int R,
                                      const int32_t* rep, int maxrep, bool id_order, int32_t* idx,
                                      float* w, int32_t* counts, int32_t* assign, int32_t* active,
                                      int32_t* rank_of, int32_t* expert_offsets,
                                      int32_t* rank_offsets, int32_t* pos, int32_t* src,
                                      int32_t* dedup, int32_t* ws, hipStream_t s);

// route, assign and layout with the single-send rows: for a batch without a
// replica table the top-k kernel (with leader masks), the column scan and
// one permutation + single-send launch; else the separate calls' kernels.
// ws as for launch_route_assign_layout plus T ints.
hipError_t launch_route_assign_layout_single_send(
    const float* logits, int T, int E, int k, int R, const int32_t* rep, int maxrep, bool id_order,
    int32_t* idx, float* w, int32_t* counts, int32_t* assign, int32_t* active, int32_t* rank_of,
    int32_t* expert_offsets, int32_t* rank_offsets, int32_t* pos, int32_t* src, int32_t* dedup,
    int32_t* ss_rank_offsets, int32_t* ss_row, int32_t* ss_token, int32_t* ws, hipStream_t s);

hipError_t launch_assign(const int32_t* counts, int E, int R, const int32_t* rep, int maxrep,
                         bool id_order, int32_t* assign, int32_t* active, hipStream_t s);

// ss_rank_offsets, ss_row and ss_token are all null (plain layout) or all set
// (also the single-send rows).
hipError_t launch_layout(const int32_t* idx, int T, int E, int k, int R, const int32_t* assign,
                         const int32_t* rep, int maxrep, int32_t* rank_of, int32_t* expert_offsets,
                         int32_t* rank_offsets, int32_t* pos, int32_t* src, int32_t* dedup,
                         int32_t* ss_rank_offsets, int32_t* ss_row, int32_t* ss_token,
                         int32_t* ws, hipStream_t s);

hipError_t launch_single_send_dispatch(const void* x, const int32_t* ss_row, void* send_ss,
                                       int ss_capacity, int T, int k, int H, hipStream_t s);

hipError_t launch_single_send_expand(const void* send_ss, const int32_t* ss_rank_offsets,
                                     const int32_t* ss_token, const int32_t* ss_row,
                                     const int32_t* pos, int ss_capacity, void* send, int T, int k,
                                     int R, int H, hipStream_t s);

hipError_t launch_dispatch(const void* x, const int32_t* pos, void* send, int T, int k, int H,
                           hipStream_t s);

hipError_t launch_standin(const void* send, const int32_t* src, const int32_t* idx, void* y, int T,
                          int E, int k, int H, int act, hipStream_t s);

hipError_t launch_combine(const void* y, const int32_t* pos, const float* w, void* out, int T, int k,
                          int H, int act, bool out_f32, hipStream_t s);

hipError_t launch_combine_backward(const void* dout, const void* y, const int32_t* pos,
                                   const float* w, void* dy, float* dw, int T, int k, int H,
                                   int act, hipStream_t s);
hipError_t launch_dispatch_backward(const void* dsend, const int32_t* pos, void* dx, int T, int k,
                                    int H, int act, bool out_f32, hipStream_t s);

hipError_t launch_routing_stats(const int32_t* idx, const int32_t* rank_of, const int32_t* counts,
                                int T, int E, int k, int R, int32_t* S, int32_t* C, double* stats,
                                hipStream_t s);

hipError_t launch_token_balanced_split(const int32_t* idx, const int32_t* counts,
                                       const int32_t* pos, const int32_t* expert_offsets,
                                       const int32_t* rep, int maxrep, int T, int E, int k, int R,
                                       int32_t* gpu_of_pair, int32_t* active, int32_t* tokens,
                                       hipStream_t s);

}  // namespace moe
