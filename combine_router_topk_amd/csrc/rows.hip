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
// row's k send rows. With SERIAL, each load completes before the next is
// issued: for long rows with many copies (H = 7168, k = 8: 56 stores per
// lane) this staggers the waves' store bursts and measured 7% faster
// (1.63 vs 1.76 ms); for shorter rows it does not help.
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
template <int NT, int U, bool ONE, bool SERIAL = false, bool SS = false, bool PREF = false>
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
      if constexpr (SERIAL) __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
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

// U > 1: up to U chunks per lane are loaded before the row's expert id (two
// dependent loads: src, then idx) is looked up, so the id's latency overlaps
// the row loads (H = 2048, k = 6: 125 against 139 us; H = 4096: 2% less).
// U == 1 (rows of more than 512 chunks): the id first, then one chunk at a
// time; batching the loads there measured 11% slower (H = 7168, k = 8:
// 2.61 against 2.35 ms).
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
  if constexpr (U == 1) {
    const float scale = expert_scale();
    for (int c = lt; c < cpr; c += stride) convert(__builtin_nontemporal_load(in + c), scale, c);
  } else {
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
//  - U == 2 (one-row blocks, rows of more than 256 chunks): lanes 0..k-1 of
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
//  - rows over 512 chunks, 128-thread blocks: 24 KiB at k <= 2, 32 KiB above
//    (H = 7168: 5-8%);
//  - 257-512 chunks, 256-thread blocks: 64 KiB at k >= 4 (H = 4096, k = 4:
//    9%), else 48 KiB (H = 4096, k = 2: 71 vs 81 us);
//  - 129-256 chunks, 128-thread blocks: 24 KiB (measured with the shape);
//  - at most 128 chunks, several rows per 256-thread block: 48 KiB.
size_t dispatch_reserve(int k, int cpr) {
  if (cpr > 512) return (k <= 2 ? 24 : 32) * kKiB;
  if (cpr > 256) return (k >= 4 ? 64 : 48) * kKiB;
  if (cpr > 128) return 24 * kKiB;
  return 48 * kKiB;
}

// The dispatch gives a block several rows whenever a row needs fewer than
// kRowThreads lanes (rows of at most 128 chunks), so no lane idles while the
// LDS reservation caps the blocks per CU: at H = 512, k = 8 one row per
// block took 116 us and four rows 62 us; at H = 1024, k = 2, 77 against
// 45 us. Rows of 129 to 256 chunks keep one row per block (the several-row
// kernel with one row was 7% slower there).
bool dispatch_multi_row(int cpr) { return threads_per_row(cpr) < kRowThreads; }

// Blocks of a dispatch launch.
long long dispatch_blocks(int T, int cpr) {
  if (!dispatch_multi_row(cpr)) return T;
  const int per_blk = kRowThreads / threads_per_row(cpr);
  return (T + per_blk - 1) / per_blk;
}

// Stand-in: rows over 512 chunks, 24 KiB (H = 7168: 5-12%); shorter rows
// were fastest with none.
size_t standin_reserve(int cpr) { return cpr > 512 ? 24 * kKiB : 0; }

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
//  - 257-512 chunks: 256-thread blocks, two chunks per lane;
//  - longer rows (H = 7168): 128-thread blocks with ceil(cpr / 128) chunks
//    per lane and serialized row loads (1.63 ms against 1.69-1.77 ms for
//    256-thread shapes at full occupancy).

hipError_t launch_dispatch(const void* x, const int32_t* pos, void* send, int T, int k, int H,
                           hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int cpr = H / 8;
  const u32x4* xv = static_cast<const u32x4*>(x);
  u32x4* sv = static_cast<u32x4*>(send);
  const size_t res = if_many_blocks(dispatch_reserve(k, cpr), dispatch_blocks(T, cpr));
  if (dispatch_multi_row(cpr)) {
    const int tpt = threads_per_row(cpr);
    const int per_blk = kRowThreads / tpt;
    dispatch_kernel<kRowThreads, 1, false><<<(T + per_blk - 1) / per_blk, kRowThreads, res, s>>>(
        xv, pos, sv, T, k, cpr, tpt);
  } else if (cpr <= 256) {
    dispatch_kernel<128, 2, true, false, false, true><<<T, 128, res, s>>>(xv, pos, sv, T, k, cpr, 0);
  } else if (cpr <= 512) {
    dispatch_kernel<kRowThreads, 2, true><<<T, kRowThreads, res, s>>>(xv, pos, sv, T, k, cpr, 0);
  } else {
    // ceil(cpr / 128) chunks per lane (a loop covers rows beyond 8 * 128)
    const int u = (cpr + 127) / 128;
    if (u <= 5) dispatch_kernel<128, 5, true, true><<<T, 128, res, s>>>(xv, pos, sv, T, k, cpr, 0);
    else if (u == 6) dispatch_kernel<128, 6, true, true><<<T, 128, res, s>>>(xv, pos, sv, T, k, cpr, 0);
    else if (u == 7) dispatch_kernel<128, 7, true, true><<<T, 128, res, s>>>(xv, pos, sv, T, k, cpr, 0);
    else dispatch_kernel<128, 8, true, true><<<T, 128, res, s>>>(xv, pos, sv, T, k, cpr, 0);
  }
  return hipGetLastError();
}

hipError_t launch_single_send_dispatch(const void* x, const int32_t* ss_row, void* send_ss,
                                       int ss_capacity, int T, int k, int H, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int cpr = H / 8;
  const u32x4* xv = static_cast<const u32x4*>(x);
  u32x4* sv = static_cast<u32x4*>(send_ss);
  const size_t res = if_many_blocks(dispatch_reserve(k, cpr), dispatch_blocks(T, cpr));
  const int cap = ss_capacity;
  if (dispatch_multi_row(cpr)) {
    const int tpt = threads_per_row(cpr);
    const int per_blk = kRowThreads / tpt;
    dispatch_kernel<kRowThreads, 1, false, false, true><<<(T + per_blk - 1) / per_blk, kRowThreads, res, s>>>(
        xv, ss_row, sv, T, k, cpr, tpt, cap);
  } else if (cpr <= 256) {
    dispatch_kernel<128, 2, true, false, true, true><<<T, 128, res, s>>>(xv, ss_row, sv, T, k, cpr, 0, cap);
  } else if (cpr <= 512) {
    dispatch_kernel<kRowThreads, 2, true, false, true><<<T, kRowThreads, res, s>>>(xv, ss_row, sv, T, k, cpr, 0, cap);
  } else {
    dispatch_kernel<128, 8, true, true, true><<<T, 128, res, s>>>(xv, ss_row, sv, T, k, cpr, 0, cap);
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
  if (cpr >= kOneRowChunks) {
    const size_t res = if_many_blocks(standin_reserve(cpr), n);
    if (cpr > 512) {
      if (act == 1) standin_kernel<1, true, 1><<<n, kRowThreads, res, s>>>(in, src, idx, out, n, E, cpr, 0);
      else standin_kernel<2, true, 1><<<n, kRowThreads, res, s>>>(in, src, idx, out, n, E, cpr, 0);
    } else {
      if (act == 1) standin_kernel<1, true, 4><<<n, kRowThreads, res, s>>>(in, src, idx, out, n, E, cpr, 0);
      else standin_kernel<2, true, 4><<<n, kRowThreads, res, s>>>(in, src, idx, out, n, E, cpr, 0);
    }
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
