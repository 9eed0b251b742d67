// Row movement: dispatch of token rows into the rank-grouped send buffer, the
// expert stand-in, and the weighted combine back to token order; also the
// single-send dispatch (one row per token and destination rank) and its
// receiver fan-out back to the expert-grouped rows.
//
// "METRO AllGather vs AllToAll for MoE decode", section "Work the 8-GPU
// payload example" (the dispatch payload is token activation rows) and
// section "METRO AllGather vs AllToAll changes the routing information"
// (expert outputs come back through a combine); news summary of correlated
// expert placement and token shuffling, section "Why communication is the
// target" (each layer dispatches tokens and combines results).
//
// All are HBM-bound streams of 16-byte chunks. A row is split over a
// team of lanes (a power of two, up to the block: 256 threads, or 128 for
// the dispatch's 129-256-chunk and longest rows); small rows pack several
// tokens into one block. Each lane issues all of its loads
// before its stores or arithmetic so many 16-byte requests are in flight.
// Dispatch reads each token row once and writes its k copies (the minimum
// traffic); combine reads the k rows of a token and writes one.
#include "device.hpp"
#include "launch.hpp"

namespace moe {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowThreads = 256;

__device__ __forceinline__ uint4 to_uint4(u32x4 v) { return make_uint4(v.x, v.y, v.z, v.w); }
__device__ __forceinline__ u32x4 to_vec(uint4 v) { return u32x4{v.x, v.y, v.z, v.w}; }

// Row teams. With ONE = true a block is one row: the row index is uniform,
// so the row's pos / w / src entries come through scalar loads and the lane
// stride is the compile-time block size. With ONE = false (short rows: under
// 64 chunks, or up to 128 chunks for the dispatch) a block holds NT / tpt
// rows of tpt lanes each.
template <int NT, bool ONE>
__device__ __forceinline__ void row_team(int tpt, int& row, int& lane, int& stride) {
  if constexpr (ONE) {
    row = blockIdx.x;
    lane = threadIdx.x;
    stride = NT;
  } else {
    row = blockIdx.x * (NT / tpt) + threadIdx.x / tpt;
    lane = threadIdx.x % tpt;
    stride = tpt;
  }
}

// Each lane loads its U chunks of the token row, then stores them to the
// row's k send rows.
//
// With SS (single-send dispatch), pos is the token's single-send row per slot
// and n_rows the buffer's row capacity; a row shared by several slots (the
// same destination rank) is written once, by its first slot.
//
// With PREF (one-row blocks), lanes 0..k-1 of each wave load the token's k
// send rows before the row loads and each slot's row is a readlane, so that
// load's latency overlaps the row loads; without it the rows are scalar
// loads issued once the row data has arrived. Measured on MI355X (cold
// cache): PREF is 3% faster for rows of 129-256 chunks (H = 2048, k = 6:
// 83.4 against 85.9 us) but 9% slower for 257-512 chunks (H = 4096, k = 2:
// 75.5 against 69.2 us, and no LDS reservation from 0 to 64 KiB recovers
// it): the stores then start sooner and more scattered write streams are
// open at once. At H = 7168 it made no difference.
template <int NT, int U, bool ONE, bool SS = false, bool PREF = false>
__global__ __launch_bounds__(NT) void dispatch_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ pos, u32x4* __restrict__ send, int T,
    int k, int cpr, int tpt, int capacity = 0) {
  declare_lds_reserve(cpr);
  int t, lt, stride;
  row_team<NT, ONE>(tpt, t, lt, stride);
  if (t >= T) return;
  const int n_rows = SS ? capacity : T * k;
  const u32x4* xr = x + (size_t)t * cpr;
  const int32_t* pr = pos + (size_t)t * k;
  static_assert(!PREF || ONE, "the row prefetch needs one row per block");
  int my_r = 0;
  if constexpr (PREF) {
    if (__lane_id() < k) my_r = pr[__lane_id()];
  }
  auto slot_row = [&](int j) -> int {
    if constexpr (PREF) return __builtin_amdgcn_readlane(my_r, j);
    else return pr[j];
  };
  // SS: bit j set when slot j is the first of the token to carry its row;
  // formed once, while the first row loads are in flight
  uint32_t first = 0;
  for (int c0 = lt; c0 < cpr; c0 += stride * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * stride;
      if (c < cpr) v[u] = __builtin_nontemporal_load(xr + c);
    }
    if constexpr (SS) {
      if (c0 == lt) {
        for (int j = 0; j < k; ++j) {
          const int r = slot_row(j);
          bool dup = false;
          for (int jj = 0; jj < j; ++jj) dup |= (slot_row(jj) == r);
          first |= dup ? 0u : (1u << j);
        }
      }
    }
    for (int j = 0; j < k; ++j) {
      const int r = slot_row(j);
      if (static_cast<unsigned>(r) >= static_cast<unsigned>(n_rows)) continue;  // bad pos: skipped
      if constexpr (SS) {
        if (!((first >> j) & 1u)) continue;
      }
      u32x4* dst = send + (size_t)r * cpr;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * stride;
        if (c < cpr) __builtin_nontemporal_store(v[u], dst + c);
      }
    }
  }
}

// Wide rows, one block per row slice (slice_of_block): each block reads
// 2 KiB of a token's row and writes it to the token's k send rows; SS and
// the bad-row skip as in dispatch_kernel.
template <bool SS>
__global__ __launch_bounds__(kSliceChunks) void dispatch_slice_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ pos, u32x4* __restrict__ send, int k,
    int cpr, int S, int first, int n_rows) {
  declare_lds_reserve(cpr);
  int t, c;
  slice_of_block(S, first, t, c);
  const int32_t* pr = pos + (size_t)t * k;
  u32x4 v;
  if (c < cpr) v = __builtin_nontemporal_load(x + (size_t)t * cpr + c);
  for (int j = 0; j < k; ++j) {
    const int r = pr[j];
    if (static_cast<unsigned>(r) >= static_cast<unsigned>(n_rows)) continue;  // bad pos: skipped
    if constexpr (SS) {
      bool dup = false;  // an earlier slot carries this row
      for (int jj = 0; jj < j; ++jj) dup |= (pr[jj] == r);
      if (dup) continue;
    }
    if (c < cpr) __builtin_nontemporal_store(v, send + (size_t)r * cpr + c);
  }
}

// Up to U chunks per lane are loaded before the row's expert id (two
// dependent loads: src, then idx) is looked up, so the id's latency overlaps
// the row loads (H = 2048, k = 6: 125 against 139 us; H = 4096: 2% less).
template <int ACT, bool ONE, int U>
__global__ __launch_bounds__(kRowThreads) void standin_kernel(
    const u32x4* send, const int32_t* __restrict__ src, const int32_t* __restrict__ idx, u32x4* y,
    int n, int E, int cpr, int tpt) {  // y may alias send: each chunk is read, then written, by one lane
  int r, lt, stride;
  declare_lds_reserve(cpr);
  row_team<kRowThreads, ONE>(tpt, r, lt, stride);
  if (r >= n) return;
  const u32x4* in = send + (size_t)r * cpr;
  u32x4* out = y + (size_t)r * cpr;
  auto expert_scale = [&]() {
    const int sr = src[r];
    const int e = static_cast<unsigned>(sr) < static_cast<unsigned>(n) ? idx[sr] : 0;
    return 1.0f + static_cast<float>(e) / static_cast<float>(E);
  };
  auto convert = [&](u32x4 v, float scale, int c) {
    float f[8];
    unpack8<ACT>(to_uint4(v), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = keep_f32(f[i] * scale);  // product rounded to fp32
    __builtin_nontemporal_store(to_vec(pack8<ACT>(f)), out + c);
  };
  float scale = 0.0f;
  for (int c0 = lt; c0 < cpr; c0 += stride * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * stride;
      if (c < cpr) v[u] = __builtin_nontemporal_load(in + c);
    }
    if (c0 == lt) scale = expert_scale();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * stride;
      if (c >= cpr) break;
      convert(v[u], scale, c);
    }
  }
}

// The stand-in over row slices (rows over 512 chunks), one chunk per lane:
// the chunk's load, then the row's expert id, then the scaled store. y may
// alias send (each chunk is read, then written, by one lane).
template <int ACT>
__global__ __launch_bounds__(kSliceChunks) void standin_slice_kernel(
    const u32x4* send, const int32_t* __restrict__ src, const int32_t* __restrict__ idx, u32x4* y,
    int n, int E, int cpr, int S, int first) {
  declare_lds_reserve(cpr);
  int r, c;
  slice_of_block(S, first, r, c);
  u32x4 v;
  if (c < cpr) v = __builtin_nontemporal_load(send + (size_t)r * cpr + c);
  const int sr = src[r];
  const int e = static_cast<unsigned>(sr) < static_cast<unsigned>(n) ? idx[sr] : 0;
  const float scale = 1.0f + static_cast<float>(e) / static_cast<float>(E);
  if (c < cpr) {
    float f[8];
    unpack8<ACT>(to_uint4(v), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = keep_f32(f[i] * scale);  // product rounded to fp32
    __builtin_nontemporal_store(to_vec(pack8<ACT>(f)), y + (size_t)r * cpr + c);
  }
}

template <int ACT, bool OUT_F32>
__device__ __forceinline__ void combine_store(void* __restrict__ out, size_t chunk, const float (&acc)[8]) {
  if constexpr (OUT_F32) {
    f32x4* o = reinterpret_cast<f32x4*>(out) + chunk * 2;
    __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, o);
    __builtin_nontemporal_store(f32x4{acc[4], acc[5], acc[6], acc[7]}, o + 1);
  } else {
    __builtin_nontemporal_store(to_vec(pack8<ACT>(acc)), reinterpret_cast<u32x4*>(out) + chunk);
  }
}

// out[t] = sum_j (ascending) w[t,j] * y[pos[t,j]] in fp32. Two code shapes,
// each the faster one where it is used (measured on MI355X, cold cache):
//  - U == 1: per chunk position, the k row loads, then the math and store;
//    the token's pos / w entries are read per slot (scalar loads when the
//    row index is uniform). Used for short rows and rows of <= 256 chunks
//    (H = 2048, k = 6: 83 us against 96 us for the batched shape).
//  - U == 2 (one-row blocks, rows of more than 256 chunks, except the large
//    launches with k >= 5 that go out in slices, see combine_sliced): lanes 0..k-1 of
//    each wave fetch the k pos / w entries in one vector load and broadcast
//    them with readlane; each lane then issues the loads of two chunk
//    positions before any math; with EXACT, k == KMAX is a compile-time
//    constant so no slot is guarded (H = 4096, k = 2: 69 us against 73 us;
//    H = 7168, k = 8: 1.58 ms against 1.62 ms).
template <int ACT, int KMAX, bool OUT_F32, bool ONE, int U, bool EXACT>
__global__ __launch_bounds__(kRowThreads) void combine_kernel(
    const u32x4* __restrict__ y, const int32_t* __restrict__ pos, const float* __restrict__ w,
    void* __restrict__ out, int T, int k_rt, int cpr, int tpt) {
  const int k = EXACT ? KMAX : k_rt;
  int t, lt, stride;
  declare_lds_reserve(cpr);
  row_team<kRowThreads, ONE>(tpt, t, lt, stride);
  if (t >= T) return;
  size_t row[KMAX];
  float wt[KMAX];
  if constexpr (U == 1) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        const int r = pos[(size_t)t * k + j];
        const bool ok = static_cast<unsigned>(r) < static_cast<unsigned>(T * k);
        row[j] = ok ? (size_t)r * cpr : 0;  // a bad pos reads row 0 with weight 0
        wt[j] = ok ? w[(size_t)t * k + j] : 0.0f;
      }
    }
    for (int c = lt; c < cpr; c += stride) {
      u32x4 v[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < k) v[j] = __builtin_nontemporal_load(y + row[j] + c);
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
          float f[8];
          unpack8<ACT>(to_uint4(v[j]), f);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(wt[j], f[i], acc[i]);
        }
      }
      combine_store<ACT, OUT_F32>(out, (size_t)t * cpr + c, acc);
    }
  } else {
    static_assert(ONE, "the batched shape needs one row per block");
    const int ln = __lane_id();
    const int my_r = ln < k ? pos[(size_t)t * k + ln] : 0;
    const float my_w = ln < k ? w[(size_t)t * k + ln] : 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        const int r = __builtin_amdgcn_readlane(my_r, j);
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
        const bool ok = static_cast<unsigned>(r) < static_cast<unsigned>(T * k);
        row[j] = ok ? (size_t)r * cpr : 0;  // a bad pos reads row 0 with weight 0
        wt[j] = ok ? wj : 0.0f;
      }
    }
    for (int c0 = lt; c0 < cpr; c0 += stride * U) {
      u32x4 v[U][KMAX];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * stride;
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (j < k && c < cpr) v[u][j] = __builtin_nontemporal_load(y + row[j] + c);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * stride;
        if (c >= cpr) break;
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          if (j < k) {
            float f[8];
            unpack8<ACT>(to_uint4(v[u][j]), f);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = fmaf(wt[j], f[i], acc[i]);
          }
        }
        combine_store<ACT, OUT_F32>(out, (size_t)t * cpr + c, acc);
      }
    }
  }
}

// The combine over row slices (rows over 256 chunks with k >= 5): a block
// reads one 128-chunk slice of each of the token's k rows and writes that
// slice of out, with the arithmetic of combine_kernel (fp32 FMAs in
// ascending slot order, a bad pos read as row 0 with weight 0).
template <int ACT, int KMAX, bool OUT_F32>
__global__ __launch_bounds__(kSliceChunks) void combine_slice_kernel(
    const u32x4* __restrict__ y, const int32_t* __restrict__ pos, const float* __restrict__ w,
    void* __restrict__ out, int T, int k, int cpr, int S, int first) {
  declare_lds_reserve(cpr);
  int t, c;
  slice_of_block(S, first, t, c);
  size_t row[KMAX];
  float wt[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      const int r = pos[(size_t)t * k + j];
      const bool ok = static_cast<unsigned>(r) < static_cast<unsigned>(T * k);
      row[j] = ok ? (size_t)r * cpr : 0;
      wt[j] = ok ? w[(size_t)t * k + j] : 0.0f;
    }
  }
  if (c >= cpr) return;
  u32x4 v[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (j < k) v[j] = __builtin_nontemporal_load(y + row[j] + c);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      float f[8];
      unpack8<ACT>(to_uint4(v[j]), f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(wt[j], f[i], acc[i]);
    }
  }
  combine_store<ACT, OUT_F32>(out, (size_t)t * cpr + c, acc);
}

// Receiver fan-out of single-send rows: each single-send row q (token t =
// ss_token[q]) is read once and written to the expert rows pos[t*k + j] of
// every slot j that it carries (ss_row[t*k + j] == q). One row per block, so
// the token, its slots' rows and their destinations are uniform. Rows at or
// beyond n_ss = ss_rank_offsets[R] exit at once.
//
// With PREF the row's first loads go out before its token and the token's
// (ss_row, pos) entries are looked up (lanes 0..k-1 of each wave load one
// slot's entries, which are then readlanes), so those dependent lookups
// overlap the row loads; without it they are scalar loads, the token's
// before the row loads and each slot's after the row data arrived. PREF
// measured faster for rows of at most 256 chunks (H = 2048, k = 6: 1.3%) and
// for launches too small for the occupancy cap (decode, 1344 rows: 4.4%),
// slower for long rows in large launches (H = 4096, k = 2: 3.6%; H = 7168,
// k = 8: 8.9%), where more scattered write streams are then open at once.
template <int NT, int U, bool PREF>
__global__ __launch_bounds__(NT) void fanout_kernel(
    const u32x4* __restrict__ send_ss, const int32_t* __restrict__ n_ss_ptr,
    const int32_t* __restrict__ ss_token, const int32_t* __restrict__ ss_row,
    const int32_t* __restrict__ pos, u32x4* __restrict__ send, int T, int k, int cpr) {
  declare_lds_reserve(cpr);
  const int q = blockIdx.x;
  if (q >= *n_ss_ptr) return;
  const int n_rows = T * k;
  const u32x4* in = send_ss + (size_t)q * cpr;
  if constexpr (PREF) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = threadIdx.x + u * NT;
      if (c < cpr) v[u] = __builtin_nontemporal_load(in + c);
    }
    const int t = ss_token[q];
    if (static_cast<unsigned>(t) >= static_cast<unsigned>(T)) return;  // uniform over the block
    int my_s = -1, my_p = 0;
    if (__lane_id() < k) {
      my_s = ss_row[(size_t)t * k + __lane_id()];
      my_p = pos[(size_t)t * k + __lane_id()];
    }
    for (int c0 = threadIdx.x; c0 < cpr; c0 += NT * U) {
      if (c0 != threadIdx.x) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * NT;
          if (c < cpr) v[u] = __builtin_nontemporal_load(in + c);
        }
      }
      for (int j = 0; j < k; ++j) {
        const int r = __builtin_amdgcn_readlane(my_p, j);
        if (__builtin_amdgcn_readlane(my_s, j) != q ||
            static_cast<unsigned>(r) >= static_cast<unsigned>(n_rows)) continue;
        u32x4* dst = send + (size_t)r * cpr;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * NT;
          if (c < cpr) __builtin_nontemporal_store(v[u], dst + c);
        }
      }
    }
  } else {
    const int t = ss_token[q];
    if (static_cast<unsigned>(t) >= static_cast<unsigned>(T)) return;
    const int32_t* sr = ss_row + (size_t)t * k;
    const int32_t* pr = pos + (size_t)t * k;
    for (int c0 = threadIdx.x; c0 < cpr; c0 += NT * U) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * NT;
        if (c < cpr) v[u] = __builtin_nontemporal_load(in + c);
      }
      for (int j = 0; j < k; ++j) {
        const int r = pr[j];
        if (sr[j] != q || static_cast<unsigned>(r) >= static_cast<unsigned>(n_rows)) continue;
        u32x4* dst = send + (size_t)r * cpr;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * NT;
          if (c < cpr) __builtin_nontemporal_store(v[u], dst + c);
        }
      }
    }
  }
}

// Rows of at least this many 16-byte chunks get a block each (the dispatch
// decides by dispatch_multi_row instead).
constexpr int kOneRowChunks = 64;

// Threads per row for short rows: enough for one 16-byte chunk each.
int threads_per_row(int cpr) {
  int tpt = 16;
  while (tpt < cpr && tpt < kRowThreads) tpt *= 2;
  return tpt;
}

// LDS reservations (see declare_lds_reserve): fewer resident blocks per CU
// mean fewer concurrent scattered row streams, which the memory system
// serves faster once each block keeps enough bytes in flight. A CU then
// holds at most 160 KiB / reservation blocks, fewer where registers bind
// first (32 and 40 KiB measured alike). The values below come from
// cold-cache sweeps on MI355X of
// every one-row kernel over H = 2048, 4096, 7168 and k = 2..8 (reservations
// 0 to 64 KiB); each rule names the measured gain over no reservation.

// Dispatch (plain and single-send), per launch shape (see launch_dispatch):
//  - row slices (dispatch_sliced), 128-thread blocks: 14 KiB for rows over
//    512 chunks, 12 KiB for 257-512 chunks. The rate peaks sharply: at
//    T = 65536, E = 256, k = 8, H = 7168, 1.53 ms at 14-15 KiB against
//    1.59-1.73 ms at 8-13 KiB and 1.56-1.60 ms at 16-24 KiB; at T = 16384,
//    E = 64, 12 KiB was 1-4% faster than 14 KiB, which serves both;
//  - 257-512 chunks with k <= 4, 256-thread blocks: 64 KiB at k = 4
//    (H = 4096: 9%), else 48 KiB (H = 4096, k = 2: 71 vs 81 us);
//  - 129-256 chunks, 128-thread blocks: 24 KiB (measured with the shape);
//  - at most 128 chunks, several rows per 256-thread block: 48 KiB.
size_t dispatch_reserve(int k, int cpr, bool sliced) {
  if (sliced) return (cpr > 512 ? 14 : 12) * kKiB;
  if (cpr > 512) return 0;  // unsliced only in launches too small for a cap
  if (cpr > 256) return (k >= 4 ? 64 : 48) * kKiB;
  if (cpr > 128) return 24 * kKiB;
  return 48 * kKiB;
}

// Rows the dispatch cuts into slices (dispatch_slice_kernel): rows over 512
// chunks, and rows of 257-512 chunks with k >= 5. Against one block per
// token row (cold cache, T = 16384, E = 64 unless named): H = 7168, k = 2:
// 113-118 against 123 us; k = 8: 368-380 against 392 us; T = 65536,
// E = 256, k = 8: 1.53 against 1.61 ms; H = 8192, k = 2: 128-135 against
// 143 us; H = 5120, k = 8: 265-272 against 278 us; H = 4096, k = 6: 160
// against 181 us; k = 8: 211 against 235 us; H = 3072, k = 8: 160 against
// 175 us. At H = 4096 with k = 2 and 4 slices were 1-2% slower (69.8
// against 68.9 us, 112.6 against 110.7 us), at H = 2048, k = 8 equal.
// The single-send dispatch writes fewer rows per token (one per distinct
// rank) and is sliced only for rows over 512 chunks (T = 65536, E = 256,
// k = 8, H = 7168: 1.42 against 1.48 ms); at 257-512 chunks slices were
// mixed (H = 4096, k = 6: 125.5 against 123.7 us; k = 8: 160.8 against
// 165.3 us; decode: 6.5 against 6.2 us).
// Rows of 257-512 chunks need launches of 16384 slices: at H = 4096, k = 8
// slices were slower at T = 1100 and 2048 (16.9 against 16.0 us, 29.9
// against 29.0 us) and faster from T = 4096 (55.6 against 59.8 us); rows
// over 512 chunks were faster from the smallest launch sliced (H = 7168,
// k = 8, T = 600: 15.1 against 17.8 us).
bool dispatch_sliced(int T, int k, int cpr) {
  if (cpr > 512) return enough_slices(T, slices_per_row(cpr));
  return cpr > 256 && k >= 5 && enough_slices(T, slices_per_row(cpr), 16384);
}
bool ss_dispatch_sliced(int T, int cpr) { return cpr > 512 && enough_slices(T, slices_per_row(cpr)); }

// The dispatch gives a block several rows whenever a row needs fewer than
// kRowThreads lanes (rows of at most 128 chunks), so no lane idles while the
// LDS reservation caps the blocks per CU: at H = 512, k = 8 one row per
// block took 116 us and four rows 62 us; at H = 1024, k = 2, 77 against
// 45 us. Rows of 129 to 256 chunks keep one row per block (the several-row
// kernel with one row was 7% slower there).
bool dispatch_multi_row(int cpr) { return threads_per_row(cpr) < kRowThreads; }

// Blocks of a dispatch launch (all launches of a sliced one).
long long dispatch_blocks(int T, int cpr, bool sliced) {
  if (sliced) return (long long)T * slices_per_row(cpr);
  if (!dispatch_multi_row(cpr)) return T;
  const int per_blk = kRowThreads / threads_per_row(cpr);
  return (T + per_blk - 1) / per_blk;
}

// Stand-in: one-row blocks (rows of 64-512 chunks) were fastest with no
// reservation. Rows over 512 chunks go out in slices, also with none (any
// reservation from 4 to 32 KiB was slower); against one-row blocks with
// 24 KiB (cold cache, T = 16384, E = 64 unless named): T = 65536, E = 256,
// k = 8, H = 7168: 2.29 against 2.35 ms; H = 7168, k = 2: 149 against
// 158 us; k = 8: 577 against 597 us; H = 8192, k = 2: 171 against 174 us.
// Slices of 257-512-chunk rows were mixed (H = 4096, k = 8: 333 against
// 339 us; k = 2: 86.5 against 84.6 us; H = 3072, k = 2: 69.5 against
// 63.5 us).
bool standin_sliced(int n, int cpr) { return cpr > 512 && enough_slices(n, slices_per_row(cpr)); }

// Fan-out, two chunks per lane (rows over 256 chunks): 32 KiB at every k
// measured (6-15%); rows of 256 chunks or fewer were fastest with none.
size_t fanout_reserve(int cpr) { return cpr > 256 ? 32 * kKiB : 0; }

// Combine, batched shape (rows over 256 chunks, k <= 8): the row loads in
// flight per block grow with k, so the best block count falls with k:
// k >= 6: 64 KiB (6-9%); k = 3..5: 48 KiB (6%); k <= 2: 32 KiB for rows over
// 512 chunks (7%), none for shorter rows. The one-chunk shape (rows of
// 64-256 chunks) was fastest with none.
size_t combine_reserve(int k, int cpr) {
  if (cpr <= kRowThreads || k > 8) return 0;
  if (k >= 6) return 64 * kKiB;
  if (k >= 3) return 48 * kKiB;
  return cpr > 512 ? 32 * kKiB : 0;
}

// Rows over 256 chunks with k >= 5 are combined in slices
// (combine_slice_kernel), 24 KiB at k >= 7 and 16 KiB below. Against the
// batched one-row shape (cold cache, T = 16384, E = 64 unless named):
// T = 65536, E = 256, k = 8, H = 7168: 1.34 against 1.43-1.45 ms; H = 7168,
// k = 8: 331 against 354 us; H = 4096, k = 8: 193 against 202 us; k = 6:
// 151 against 160 us; H = 3072, k = 8: 149 against 160 us. With k <= 4
// slices were slower or equal (H = 4096, k = 2: 70.3 against 66.7 us; k = 4:
// 108.9 against 107.1 us; H = 7168, k = 4: 192.5 against 191.6 us).
// Only in launches of at least 12288 slices: below, the one-row shape was
// faster (k = 8, H = 7168, T = 1024: 25.7 against 27.6 us in slices;
// H = 4096, T = 2048: 28.3 against 30.5 us); above, slices (H = 7168,
// T = 2048: 48.4 against 49.5 us; H = 4096, T = 4096: 54.0 against 55.6 us).
bool combine_sliced(int T, int k, int cpr) {
  return cpr > kRowThreads && k >= 5 && enough_slices(T, slices_per_row(cpr), 12288);
}
size_t combine_slice_reserve(int k) { return (k >= 7 ? 24 : 16) * kKiB; }

template <int ACT, bool OUT_F32, bool ONE>
hipError_t launch_combine_k(const u32x4* y, const int32_t* pos, const float* w, void* out, int T,
                            int k, int cpr, int tpt, int grid, hipStream_t s) {
  const size_t res = ONE ? if_many_blocks(combine_reserve(k, cpr), grid) : 0;
#define MOE_COMBINE(KM, ONE_, U, EX) \
  combine_kernel<ACT, KM, OUT_F32, ONE_, U, EX><<<grid, kRowThreads, res, s>>>(y, pos, w, out, T, k, cpr, tpt)
  if (ONE && cpr > kRowThreads && k <= 8) {  // the batched shape, exact k
    switch (k) {
      case 1: MOE_COMBINE(1, true, 2, true); break;
      case 2: MOE_COMBINE(2, true, 2, true); break;
      case 3: MOE_COMBINE(3, true, 2, true); break;
      case 4: MOE_COMBINE(4, true, 2, true); break;
      case 5: MOE_COMBINE(5, true, 2, true); break;
      case 6: MOE_COMBINE(6, true, 2, true); break;
      case 7: MOE_COMBINE(7, true, 2, true); break;
      default: MOE_COMBINE(8, true, 2, true); break;
    }
  } else if (k <= 2) {
    MOE_COMBINE(2, ONE, 1, false);
  } else if (k <= 4) {
    MOE_COMBINE(4, ONE, 1, false);
  } else if (k <= 8) {
    MOE_COMBINE(8, ONE, 1, false);
  } else {
    MOE_COMBINE(16, ONE, 1, false);
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

template <int ACT, bool OUT_F32>
hipError_t launch_combine_a(const u32x4* y, const int32_t* pos, const float* w, void* out, int T,
                            int k, int cpr, hipStream_t s) {
  if (combine_sliced(T, k, cpr)) {
    const int S = slices_per_row(cpr);
    const size_t res = if_many_blocks(combine_slice_reserve(k), (long long)T * S);
    slice_launches(T, S, [&](int first, unsigned blocks) {
#define MOE_COMBINE_SLICE(KM) \
  combine_slice_kernel<ACT, KM, OUT_F32><<<blocks, kSliceChunks, res, s>>>(y, pos, w, out, T, k, cpr, S, first)
      if (k <= 8) MOE_COMBINE_SLICE(8);
      else MOE_COMBINE_SLICE(16);
#undef MOE_COMBINE_SLICE
    });
    return hipGetLastError();
  }
  if (cpr >= kOneRowChunks) return launch_combine_k<ACT, OUT_F32, true>(y, pos, w, out, T, k, cpr, kRowThreads, T, s);
  const int tpt = threads_per_row(cpr);
  const int per_blk = kRowThreads / tpt;
  return launch_combine_k<ACT, OUT_F32, false>(y, pos, w, out, T, k, cpr, tpt, (T + per_blk - 1) / per_blk, s);
}

}  // namespace

// Launch shape of the dispatch, from measurements on MI355X (cold cache),
// each with the LDS reservation of dispatch_reserve:
//  - rows of at most 128 chunks: several rows per 256-thread block (see
//    dispatch_multi_row);
//  - 129-256 chunks: 128-thread blocks, two chunks per lane, one row per
//    block. Against 256-thread blocks with one chunk per lane (48 KiB):
//    H = 2048, k = 2: 70 vs 90 us; H = 1536, k = 2: 56 vs 85 us; H = 1280,
//    k = 4: 77 vs 98 us; H = 2048, k = 6: 86 us either way;
//  - longer rows, and 257-512 chunks with k >= 5, in launches of at least
//    kMinBlocksToCap slices: 128-chunk row slices, one block each (see
//    dispatch_sliced). One 128-thread block per token row, ceil(cpr / 128)
//    chunks per lane with serialized row loads, took 1.61-1.63 ms at
//    H = 7168, k = 8 (256-thread blocks: 1.69-1.77 ms);
//  - other rows over 256 chunks (k <= 4, the single-send dispatch at
//    257-512 chunks, and small launches): 256-thread blocks, two chunks per
//    lane, looping over rows beyond 512 chunks.

hipError_t launch_dispatch(const void* x, const int32_t* pos, void* send, int T, int k, int H,
                           hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int cpr = H / 8;
  const u32x4* xv = static_cast<const u32x4*>(x);
  u32x4* sv = static_cast<u32x4*>(send);
  const bool sliced = dispatch_sliced(T, k, cpr);
  const size_t res = if_many_blocks(dispatch_reserve(k, cpr, sliced), dispatch_blocks(T, cpr, sliced));
  if (sliced) {
    const int S = slices_per_row(cpr);
    slice_launches(T, S, [&](int first, unsigned blocks) {
      dispatch_slice_kernel<false><<<blocks, kSliceChunks, res, s>>>(xv, pos, sv, k, cpr, S, first, T * k);
    });
  } else if (dispatch_multi_row(cpr)) {
    const int tpt = threads_per_row(cpr);
    const int per_blk = kRowThreads / tpt;
    dispatch_kernel<kRowThreads, 1, false><<<(T + per_blk - 1) / per_blk, kRowThreads, res, s>>>(
        xv, pos, sv, T, k, cpr, tpt);
  } else if (cpr <= 256) {
    dispatch_kernel<128, 2, true, false, true><<<T, 128, res, s>>>(xv, pos, sv, T, k, cpr, 0);
  } else {
    dispatch_kernel<kRowThreads, 2, true><<<T, kRowThreads, res, s>>>(xv, pos, sv, T, k, cpr, 0);
  }
  return hipGetLastError();
}

hipError_t launch_single_send_dispatch(const void* x, const int32_t* ss_row, void* send_ss,
                                       int ss_capacity, int T, int k, int H, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int cpr = H / 8;
  const u32x4* xv = static_cast<const u32x4*>(x);
  u32x4* sv = static_cast<u32x4*>(send_ss);
  const bool sliced = ss_dispatch_sliced(T, cpr);
  const size_t res = if_many_blocks(dispatch_reserve(k, cpr, sliced), dispatch_blocks(T, cpr, sliced));
  const int cap = ss_capacity;
  if (sliced) {
    const int S = slices_per_row(cpr);
    slice_launches(T, S, [&](int first, unsigned blocks) {
      dispatch_slice_kernel<true><<<blocks, kSliceChunks, res, s>>>(xv, ss_row, sv, k, cpr, S, first, cap);
    });
  } else if (dispatch_multi_row(cpr)) {
    const int tpt = threads_per_row(cpr);
    const int per_blk = kRowThreads / tpt;
    dispatch_kernel<kRowThreads, 1, false, true><<<(T + per_blk - 1) / per_blk, kRowThreads, res, s>>>(
        xv, ss_row, sv, T, k, cpr, tpt, cap);
  } else if (cpr <= 256) {
    dispatch_kernel<128, 2, true, true, true><<<T, 128, res, s>>>(xv, ss_row, sv, T, k, cpr, 0, cap);
  } else {
    dispatch_kernel<kRowThreads, 2, true, true><<<T, kRowThreads, res, s>>>(xv, ss_row, sv, T, k, cpr, 0, cap);
  }
  return hipGetLastError();
}

hipError_t launch_single_send_expand(const void* send_ss, const int32_t* ss_rank_offsets,
                                     const int32_t* ss_token, const int32_t* ss_row,
                                     const int32_t* pos, int ss_capacity, void* send, int T, int k,
                                     int R, int H, hipStream_t s) {
  if (T == 0 || ss_capacity == 0) return hipSuccess;
  const int cpr = H / 8;
  const u32x4* in = static_cast<const u32x4*>(send_ss);
  u32x4* out = static_cast<u32x4*>(send);
  const int32_t* n_ss = ss_rank_offsets + R;
  // there are at most T*k single-send rows, so blocks past that would only exit
  const int grid = ss_capacity < T * k ? ss_capacity : T * k;
  const size_t res = if_many_blocks(fanout_reserve(cpr), grid);
  if (cpr <= 256)
    fanout_kernel<kRowThreads, 1, true><<<grid, kRowThreads, res, s>>>(in, n_ss, ss_token, ss_row,
                                                                      pos, out, T, k, cpr);
  else if (grid < kMinBlocksToCap)
    fanout_kernel<kRowThreads, 2, true><<<grid, kRowThreads, res, s>>>(in, n_ss, ss_token, ss_row,
                                                                      pos, out, T, k, cpr);
  else
    fanout_kernel<kRowThreads, 2, false><<<grid, kRowThreads, res, s>>>(in, n_ss, ss_token, ss_row,
                                                                       pos, out, T, k, cpr);
  return hipGetLastError();
}

hipError_t launch_standin(const void* send, const int32_t* src, const int32_t* idx, void* y, int T,
                          int E, int k, int H, int act, hipStream_t s) {
  const int n = T * k;
  if (n == 0) return hipSuccess;
  const int cpr = H / 8;
  const u32x4* in = static_cast<const u32x4*>(send);
  u32x4* out = static_cast<u32x4*>(y);
  if (standin_sliced(n, cpr)) {
    const int S = slices_per_row(cpr);
    slice_launches(n, S, [&](int first, unsigned blocks) {
      if (act == 1) standin_slice_kernel<1><<<blocks, kSliceChunks, 0, s>>>(in, src, idx, out, n, E, cpr, S, first);
      else standin_slice_kernel<2><<<blocks, kSliceChunks, 0, s>>>(in, src, idx, out, n, E, cpr, S, first);
    });
  } else if (cpr >= kOneRowChunks) {
    if (act == 1) standin_kernel<1, true, 4><<<n, kRowThreads, 0, s>>>(in, src, idx, out, n, E, cpr, 0);
    else standin_kernel<2, true, 4><<<n, kRowThreads, 0, s>>>(in, src, idx, out, n, E, cpr, 0);
  } else {
    const int tpt = threads_per_row(cpr);
    const int per_blk = kRowThreads / tpt;
    const int grid = (n + per_blk - 1) / per_blk;
    if (act == 1) standin_kernel<1, false, 4><<<grid, kRowThreads, 0, s>>>(in, src, idx, out, n, E, cpr, tpt);
    else standin_kernel<2, false, 4><<<grid, kRowThreads, 0, s>>>(in, src, idx, out, n, E, cpr, tpt);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const void* y, const int32_t* pos, const float* w, void* out, int T, int k,
                          int H, int act, bool out_f32, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int cpr = H / 8;
  const u32x4* yv = static_cast<const u32x4*>(y);
  if (act == 1)
    return out_f32 ? launch_combine_a<1, true>(yv, pos, w, out, T, k, cpr, s)
                   : launch_combine_a<1, false>(yv, pos, w, out, T, k, cpr, s);
  return out_f32 ? launch_combine_a<2, true>(yv, pos, w, out, T, k, cpr, s)
                 : launch_combine_a<2, false>(yv, pos, w, out, T, k, cpr, s);
}

}  // namespace moe
