// Backward of the combine and of the dispatch.
//
// News summary of correlated expert placement and token shuffling, section
// "Why communication is the target": each MoE layer dispatches tokens and
// combines results in the backward pass as in the forward. Differentiating
// the forward maps out[t] = sum_j w[t,j] y[pos[t*k+j]] and
// send[pos[i]] = x[i/k] gives
//   dy[pos[t*k+j]] = w[t,j] * dout[t]          (a dispatch-shaped weighted scatter)
//   dw[t,j]        = <y[pos[t*k+j]], dout[t]>  (row dot products)
//   dx[t]          = sum_j dsend[pos[t*k+j]]   (a combine-shaped gather-sum)
//
// Both kernels give each token a team of lanes (a whole 256-thread block for
// rows of 64 chunks or more, else 16-64 lanes inside one wave) that walks the
// token's row in 16-byte chunks, so every gradient row is read once and
// every output row written once: (1 + 2k) T H b bytes for the combine
// backward with both outputs, (1 + k) T H b for the dispatch backward.
#include "device.hpp"
#include "launch.hpp"

namespace moe {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGradThreads = 256;
constexpr int kGradWaves = kGradThreads / kWave;
constexpr int kGradOneRowChunks = 64;  // rows of at least this many chunks get a block each

__device__ __forceinline__ uint4 as_uint4(u32x4 v) { return make_uint4(v.x, v.y, v.z, v.w); }
__device__ __forceinline__ u32x4 as_vec(uint4 v) { return u32x4{v.x, v.y, v.z, v.w}; }

// The token a lane works on, its index inside the token's team, and the
// team's width (the chunk stride).
template <bool ONE>
__device__ __forceinline__ void grad_team(int tpt, int& t, int& lt, int& stride) {
  if constexpr (ONE) {
    t = blockIdx.x;
    lt = threadIdx.x;
    stride = kGradThreads;
  } else {
    t = blockIdx.x * (kGradThreads / tpt) + threadIdx.x / tpt;
    lt = threadIdx.x % tpt;
    stride = tpt;
  }
}

// dy and dw for one token per team. dy (nullable) = rne16(fp32(w * dout));
// dw (nullable) = fp32 dot products, summed per lane over its chunks in
// order, then over the team (a butterfly inside the wave, then the block's
// waves in order). Slots whose pos is out of range write no dy row and a dw
// of 0. dy may alias y: every chunk of y is read before the same lane
// writes that chunk of dy.
template <int ACT, int KMAX, bool ONE, int U>
__global__ __launch_bounds__(kGradThreads) void combine_backward_kernel(
    const u32x4* __restrict__ dout, const u32x4* y, const int32_t* __restrict__ pos,
    const float* __restrict__ w, u32x4* dy, float* __restrict__ dw, int T, int k, int cpr,
    int tpt) {
  __shared__ float s_part[kGradWaves][KMAX];
  declare_lds_reserve(cpr);
  int t, lt, stride;
  grad_team<ONE>(tpt, t, lt, stride);
  const bool live = t < T;
  if (ONE && !live) return;  // uniform over the block
  const bool do_dy = dy != nullptr;
  const bool do_dw = dw != nullptr;
  const int n_rows = T * k;
  size_t row[KMAX];
  bool ok[KMAX];
  float wt[KMAX];
  float part[KMAX];
  // One-row blocks: lanes 0..k-1 of each wave load the token's pos and w
  // entries (one vector load per array), then the first step's dout chunks
  // are requested before those entries are waited for; each slot's entry
  // is a readlane.
  int my_r = 0;
  float my_w = 0.0f;
  u32x4 gv[U];
  const u32x4* g_row = dout + (size_t)t * cpr;
  if constexpr (ONE) {
    const int ln = __lane_id();
    if (ln < k) {
      my_r = pos[(size_t)t * k + ln];
      if (w != nullptr) my_w = w[(size_t)t * k + ln];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = lt + u * stride;
      if (c < cpr) gv[u] = __builtin_nontemporal_load(g_row + c);
    }
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    part[j] = 0.0f;
    ok[j] = false;
    row[j] = 0;
    wt[j] = 0.0f;
    if (live && j < k) {
      int r;
      if constexpr (ONE) {
        r = __builtin_amdgcn_readlane(my_r, j);
        wt[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
      } else {
        r = pos[(size_t)t * k + j];
        wt[j] = w != nullptr ? w[(size_t)t * k + j] : 0.0f;
      }
      ok[j] = static_cast<unsigned>(r) < static_cast<unsigned>(n_rows);
      row[j] = ok[j] ? (size_t)r * cpr : 0;
    }
  }
  if (live) {
    // U chunk positions per step: every load of the step (U dout chunks and,
    // for dw, U * k y chunks) is issued before any math or store
    for (int c0 = lt; c0 < cpr; c0 += stride * U) {
      u32x4 v[U][KMAX];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * stride;
        if (c < cpr && (!ONE || c0 != lt)) gv[u] = __builtin_nontemporal_load(g_row + c);
        if (do_dw) {
#pragma unroll
          for (int j = 0; j < KMAX; ++j)
            if (j < k && ok[j] && c < cpr) v[u][j] = __builtin_nontemporal_load(y + row[j] + c);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * stride;
        if (c >= cpr) break;
        float g[8];
        unpack8<ACT>(as_uint4(gv[u]), g);
        if (do_dw) {
#pragma unroll
          for (int j = 0; j < KMAX; ++j) {
            if (j < k && ok[j]) {
              float f[8];
              unpack8<ACT>(as_uint4(v[u][j]), f);
              float s = part[j];
#pragma unroll
              for (int i = 0; i < 8; ++i) s = fmaf(f[i], g[i], s);
              part[j] = s;
            }
          }
        }
        if (do_dy) {
#pragma unroll
          for (int j = 0; j < KMAX; ++j) {
            if (j < k && ok[j]) {
              float p[8];
#pragma unroll
              for (int i = 0; i < 8; ++i) p[i] = keep_f32(wt[j] * g[i]);  // fp32 product, then one rounding
              __builtin_nontemporal_store(as_vec(pack8<ACT>(p)), dy + row[j] + c);
            }
          }
        }
      }
    }
  }
  if (!do_dw) return;  // uniform: a kernel argument
  // team sum of each slot's partial dot product
  const int width = ONE ? kWave : tpt;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      float s = part[j];
      for (int off = width / 2; off > 0; off /= 2) s += __shfl_xor(s, off, width);
      part[j] = s;
    }
  }
  if constexpr (ONE) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < k) s_part[wave][j] = part[j];
    }
    __syncthreads();
    if (threadIdx.x < k) {
      const int j = threadIdx.x;
      float s = 0.0f;
#pragma unroll
      for (int v = 0; v < kGradWaves; ++v) s += s_part[v][j];
      const int r = pos[(size_t)t * k + j];
      dw[(size_t)t * k + j] = static_cast<unsigned>(r) < static_cast<unsigned>(n_rows) ? s : 0.0f;
    }
  } else {
    if (live && lt == 0) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < k) dw[(size_t)t * k + j] = ok[j] ? part[j] : 0.0f;
    }
  }
}

// dy alone over row slices (see combine_backward_split): a block loads one
// 128-chunk slice of dout and writes w[t,j] * dout, rounded as in
// combine_backward_kernel, to the same slice of each valid slot's dy row.
template <int ACT>
__global__ __launch_bounds__(kSliceChunks) void combine_backward_dy_slice_kernel(
    const u32x4* __restrict__ dout, const int32_t* __restrict__ pos, const float* __restrict__ w,
    u32x4* dy, int T, int k, int cpr, int S, int first) {
  declare_lds_reserve(cpr);
  int t, c;
  slice_of_block(S, first, t, c);
  const int n_rows = T * k;
  u32x4 gv;
  if (c < cpr) gv = __builtin_nontemporal_load(dout + (size_t)t * cpr + c);
  for (int j = 0; j < k; ++j) {
    const int r = pos[(size_t)t * k + j];
    if (static_cast<unsigned>(r) >= static_cast<unsigned>(n_rows)) continue;
    const float wj = w[(size_t)t * k + j];
    if (c < cpr) {
      float gf[8], p[8];
      unpack8<ACT>(as_uint4(gv), gf);
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = keep_f32(wj * gf[i]);  // fp32 product, then one rounding
      __builtin_nontemporal_store(as_vec(pack8<ACT>(p)), dy + (size_t)r * cpr + c);
    }
  }
}

template <int ACT, bool OUT_F32>
__device__ __forceinline__ void grad_store(void* __restrict__ out, size_t chunk, const float (&acc)[8]) {
  if constexpr (OUT_F32) {
    f32x4* o = reinterpret_cast<f32x4*>(out) + chunk * 2;
    __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, o);
    __builtin_nontemporal_store(f32x4{acc[4], acc[5], acc[6], acc[7]}, o + 1);
  } else {
    __builtin_nontemporal_store(as_vec(pack8<ACT>(acc)), reinterpret_cast<u32x4*>(out) + chunk);
  }
}

// dx[t] = sum_j (ascending) dsend[pos[t*k+j]] in fp32, stored in the
// activation format (one rounding) or as fp32. The k row loads of a chunk
// position are issued before the sums. Slots whose pos is out of range add
// nothing. With PREF (one-row blocks) the k pos entries come in one vector
// load by lanes 0..k-1 and are broadcast with readlane, in place of one
// scalar load per slot: measured 2.6% faster for rows of 64-256 chunks
// (H = 2048, k = 6) and 4% slower for 512 chunks (H = 4096, k = 2), where
// the rows' loads then start sooner and more of them are open at once.
template <int ACT, int KMAX, bool OUT_F32, bool ONE, bool PREF>
__global__ __launch_bounds__(kGradThreads) void dispatch_backward_kernel(
    const u32x4* __restrict__ dsend, const int32_t* __restrict__ pos, void* __restrict__ dx, int T,
    int k, int cpr, int tpt) {
  declare_lds_reserve(cpr);
  int t, lt, stride;
  grad_team<ONE>(tpt, t, lt, stride);
  if (t >= T) return;
  const int n_rows = T * k;
  size_t row[KMAX];
  bool ok[KMAX];
  static_assert(!PREF || ONE, "the vector pos load needs one row per block");
  int my_r = 0;
  if constexpr (PREF) {
    if (__lane_id() < k) my_r = pos[(size_t)t * k + __lane_id()];
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    ok[j] = false;
    row[j] = 0;
    if (j < k) {
      const int r = PREF ? __builtin_amdgcn_readlane(my_r, j) : pos[(size_t)t * k + j];
      ok[j] = static_cast<unsigned>(r) < static_cast<unsigned>(n_rows);
      row[j] = ok[j] ? (size_t)r * cpr : 0;
    }
  }
  for (int c = lt; c < cpr; c += stride) {
    u32x4 v[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k && ok[j]) v[j] = __builtin_nontemporal_load(dsend + row[j] + c);
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k && ok[j]) {
        float f[8];
        unpack8<ACT>(as_uint4(v[j]), f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += f[i];
      }
    }
    grad_store<ACT, OUT_F32>(dx, (size_t)t * cpr + c, acc);
  }
}

// dx over row slices (rows over 256 chunks): a block sums one 128-chunk
// slice of each of the token's k rows, with the arithmetic of
// dispatch_backward_kernel.
template <int ACT, int KMAX, bool OUT_F32>
__global__ __launch_bounds__(kSliceChunks) void dispatch_backward_slice_kernel(
    const u32x4* __restrict__ dsend, const int32_t* __restrict__ pos, void* __restrict__ dx, int T,
    int k, int cpr, int S, int first) {
  declare_lds_reserve(cpr);
  int t, c;
  slice_of_block(S, first, t, c);
  const int n_rows = T * k;
  size_t row[KMAX];
  bool ok[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    ok[j] = false;
    row[j] = 0;
    if (j < k) {
      const int r = pos[(size_t)t * k + j];
      ok[j] = static_cast<unsigned>(r) < static_cast<unsigned>(n_rows);
      row[j] = ok[j] ? (size_t)r * cpr : 0;
    }
  }
  if (c >= cpr) return;
  u32x4 v[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (j < k && ok[j]) v[j] = __builtin_nontemporal_load(dsend + row[j] + c);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k && ok[j]) {
      float f[8];
      unpack8<ACT>(as_uint4(v[j]), f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += f[i];
    }
  }
  grad_store<ACT, OUT_F32>(dx, (size_t)t * cpr + c, acc);
}

int grad_threads_per_row(int cpr) {
  int tpt = 16;
  while (tpt < cpr && tpt < kWave) tpt *= 2;
  return tpt;
}

template <int ACT, int KMAX>
hipError_t launch_cb(const u32x4* dout, const u32x4* y, const int32_t* pos, const float* w,
                     u32x4* dy, float* dw, int T, int k, int cpr, hipStream_t s) {
  if constexpr (KMAX <= 8) {
    if (cpr > kGradThreads) {  // long rows: two chunk positions per step
      combine_backward_kernel<ACT, KMAX, true, 2><<<T, kGradThreads, 0, s>>>(
          dout, y, pos, w, dy, dw, T, k, cpr, kGradThreads);
      return hipGetLastError();
    }
  }
  if (cpr >= kGradOneRowChunks) {
    // rows of 64-256 chunks: a 32 KiB LDS reservation (see if_many_blocks)
    // measured 3% faster (H = 2048, k = 6: 155.6 against 161.4 us); longer
    // rows, above, were within 1% under every reservation from 0 to 48 KiB
    const size_t res = if_many_blocks(32 * kKiB, T);
    combine_backward_kernel<ACT, KMAX, true, 1><<<T, kGradThreads, res, s>>>(dout, y, pos, w, dy, dw,
                                                                            T, k, cpr, kGradThreads);
  } else {
    const int tpt = grad_threads_per_row(cpr);
    const int per_blk = kGradThreads / tpt;
    combine_backward_kernel<ACT, KMAX, false, 1><<<(T + per_blk - 1) / per_blk, kGradThreads, 0, s>>>(
        dout, y, pos, w, dy, dw, T, k, cpr, tpt);
  }
  return hipGetLastError();
}

// With wide rows and many slots the combine backward runs as two launches:
// dw alone (combine_backward_kernel without dy: dout and the k y rows read,
// nothing but dw written), then dy alone in row slices, dispatch-shaped
// (reservations as the dispatch's slices: 14 KiB over 512 chunks, else
// 12 KiB). That reads dout twice, (2k + 2) H b per token instead of
// (2k + 1) H b, but each half runs at its own kernel's rate: at T = 65536,
// E = 256, k = 8, H = 7168 the fused kernel took 3.11 ms, dw alone 1.26 ms
// and dy alone 1.75 ms in one-row blocks; split, with dy in slices, it
// takes 2.80 ms. Split only in launches of at least 8192 slices with
// k >= 5 and rows over 256 chunks whose k dy rows hold at least 64 KiB
// (k * cpr >= 4096), where it measured faster (cold cache,
// T = 16384, E = 64): H = 7168, k = 5: 454 against 485 us; k = 6: 534
// against 576 us; H = 4096, k = 8: 415 against 433 us. Below that it was
// slower: H = 4096, k = 5: 270 against 265 us; k = 6: 321 against 316 us;
// H = 3072, k = 8: 329 against 319 us; and at train top-2 the one-row
// halves took 75.7 + 64.8 us against 127.2 us fused.
// Smaller launches stay fused (H = 4096, k = 8, T = 1100: 37.3 against
// 35.6 us fused; T = 2048: 59.1 against 60.1 us).
bool combine_backward_split(int T, int k, int cpr) {
  return cpr > 256 && k >= 5 && k * cpr >= 4096 && enough_slices(T, slices_per_row(cpr), 8192);
}

template <int ACT>
hipError_t launch_cb_k(const u32x4* dout, const u32x4* y, const int32_t* pos, const float* w,
                       u32x4* dy, float* dw, int T, int k, int cpr, hipStream_t s) {
  if (k <= 2) return launch_cb<ACT, 2>(dout, y, pos, w, dy, dw, T, k, cpr, s);
  if (k <= 4) return launch_cb<ACT, 4>(dout, y, pos, w, dy, dw, T, k, cpr, s);
  if (k <= 8) return launch_cb<ACT, 8>(dout, y, pos, w, dy, dw, T, k, cpr, s);
  return launch_cb<ACT, 16>(dout, y, pos, w, dy, dw, T, k, cpr, s);
}

// The dispatch backward cuts rows over 256 chunks into slices
// (dispatch_backward_slice_kernel) in launches of at least 12288 slices
// (below); shorter rows, and smaller launches, keep one-row blocks, fastest
// with no LDS reservation. The slices' reservation grows
// with k, which sets the row loads in flight per block: none at k <= 2,
// 4 KiB at k = 3, 16 KiB at k = 4..6, 24 KiB above. Against one-row blocks
// with their best reservations (cold cache, T = 16384, E = 64 unless
// named): T = 65536, E = 256, k = 8, H = 7168: 1.37 against 1.52 ms;
// H = 7168, k = 8: 331 against 379 us; k = 2: 110 against 118 us;
// H = 4096, k = 2: 67.4 against 69.2 us; k = 3: 84.1 against 92.5 us;
// k = 4: 108 against 111 us; k = 6: 152 against 165 us; H = 3072, k = 2:
// 50.8 against 57.1 us; k = 8: 152 against 166 us.
// Launches of at least 12288 slices: at k = 8 slices were slower in smaller
// ones (H = 7168, T = 1024: 27.6 against 26.7 us; H = 4096, T = 2048: 30.7
// against 29.9 us) and faster from there (H = 7168, T = 2048: 48.6 against
// 52.7 us; H = 4096, T = 4096: 54.5 against 56.1 us).
bool dispatch_backward_sliced(int T, int cpr) {
  return cpr > 256 && enough_slices(T, slices_per_row(cpr), 12288);
}
size_t dispatch_backward_slice_reserve(int k) {
  if (k <= 2) return 0;
  if (k == 3) return 4 * kKiB;
  return (k <= 6 ? 16 : 24) * kKiB;
}

template <int ACT, int KMAX, bool OUT_F32>
hipError_t launch_db(const u32x4* dsend, const int32_t* pos, void* dx, int T, int k, int cpr,
                     hipStream_t s) {
  if (dispatch_backward_sliced(T, cpr)) {
    const int S = slices_per_row(cpr);
    const size_t res = if_many_blocks(dispatch_backward_slice_reserve(k), (long long)T * S);
    slice_launches(T, S, [&](int first, unsigned blocks) {
      dispatch_backward_slice_kernel<ACT, KMAX, OUT_F32><<<blocks, kSliceChunks, res, s>>>(
          dsend, pos, dx, T, k, cpr, S, first);
    });
  } else if (cpr >= kGradOneRowChunks && cpr <= 256) {
    dispatch_backward_kernel<ACT, KMAX, OUT_F32, true, true><<<T, kGradThreads, 0, s>>>(
        dsend, pos, dx, T, k, cpr, kGradThreads);
  } else if (cpr > 256) {
    dispatch_backward_kernel<ACT, KMAX, OUT_F32, true, false><<<T, kGradThreads, 0, s>>>(
        dsend, pos, dx, T, k, cpr, kGradThreads);
  } else {
    const int tpt = grad_threads_per_row(cpr);
    const int per_blk = kGradThreads / tpt;
    dispatch_backward_kernel<ACT, KMAX, OUT_F32, false, false>
        <<<(T + per_blk - 1) / per_blk, kGradThreads, 0, s>>>(dsend, pos, dx, T, k, cpr, tpt);
  }
  return hipGetLastError();
}

template <int ACT, bool OUT_F32>
hipError_t launch_db_k(const u32x4* dsend, const int32_t* pos, void* dx, int T, int k, int cpr,
                       hipStream_t s) {
  if (k <= 2) return launch_db<ACT, 2, OUT_F32>(dsend, pos, dx, T, k, cpr, s);
  if (k <= 4) return launch_db<ACT, 4, OUT_F32>(dsend, pos, dx, T, k, cpr, s);
  if (k <= 8) return launch_db<ACT, 8, OUT_F32>(dsend, pos, dx, T, k, cpr, s);
  return launch_db<ACT, 16, OUT_F32>(dsend, pos, dx, T, k, cpr, s);
}

}  // namespace

hipError_t launch_combine_backward(const void* dout, const void* y, const int32_t* pos,
                                   const float* w, void* dy, float* dw, int T, int k, int H,
                                   int act, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int cpr = H / 8;
  const u32x4* g = static_cast<const u32x4*>(dout);
  const u32x4* yv = static_cast<const u32x4*>(y);
  u32x4* dyv = static_cast<u32x4*>(dy);
  if (dy != nullptr && combine_backward_split(T, k, cpr)) {
    // dw first: it reads y, which dy may alias
    if (dw != nullptr) {
      const hipError_t e = act == 1 ? launch_cb_k<1>(g, yv, pos, w, nullptr, dw, T, k, cpr, s)
                                    : launch_cb_k<2>(g, yv, pos, w, nullptr, dw, T, k, cpr, s);
      if (e != hipSuccess) return e;
    }
    const int S = slices_per_row(cpr);
    const size_t res = if_many_blocks((cpr > 512 ? 14 : 12) * kKiB, (long long)T * S);
    slice_launches(T, S, [&](int first, unsigned blocks) {
      if (act == 1)
        combine_backward_dy_slice_kernel<1><<<blocks, kSliceChunks, res, s>>>(g, pos, w, dyv, T, k, cpr, S, first);
      else
        combine_backward_dy_slice_kernel<2><<<blocks, kSliceChunks, res, s>>>(g, pos, w, dyv, T, k, cpr, S, first);
    });
    return hipGetLastError();
  }
  return act == 1 ? launch_cb_k<1>(g, yv, pos, w, dyv, dw, T, k, cpr, s)
                  : launch_cb_k<2>(g, yv, pos, w, dyv, dw, T, k, cpr, s);
}

hipError_t launch_dispatch_backward(const void* dsend, const int32_t* pos, void* dx, int T, int k,
                                    int H, int act, bool out_f32, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int cpr = H / 8;
  const u32x4* d = static_cast<const u32x4*>(dsend);
  if (act == 1)
    return out_f32 ? launch_db_k<1, true>(d, pos, dx, T, k, cpr, s)
                   : launch_db_k<1, false>(d, pos, dx, T, k, cpr, s);
  return out_f32 ? launch_db_k<2, true>(d, pos, dx, T, k, cpr, s)
                 : launch_db_k<2, false>(d, pos, dx, T, k, cpr, s);
}

}  // namespace moe
