// Row movement: dispatch of token rows into the rank-grouped send buffer, the
// expert stand-in, and the weighted combine back to token order.
//
// "METRO AllGather vs AllToAll for MoE decode", section "Work the 8-GPU
// payload example" (the dispatch payload is token activation rows) and
// section "METRO AllGather vs AllToAll changes the routing information"
// (expert outputs come back through a combine); news summary of correlated
// expert placement and token shuffling, section "Why communication is the
// target" (each layer dispatches tokens and combines results).
//
// All three are HBM-bound streams of 16-byte chunks. A row is split over a
// team of TPT lanes (TPT a power of two, up to the 256-thread block); small
// rows pack several tokens into one block. Each lane issues all of its loads
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

template <int U>
__global__ __launch_bounds__(kRowThreads) void dispatch_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ pos, u32x4* __restrict__ send, int T,
    int k, int cpr, int tpt) {
  const int n_rows = T * k;
  const int per_blk = kRowThreads / tpt;
  const int t = blockIdx.x * per_blk + threadIdx.x / tpt;
  if (t >= T) return;
  const int lt = threadIdx.x % tpt;
  const u32x4* xr = x + (size_t)t * cpr;
  const int32_t* pr = pos + (size_t)t * k;
  for (int c0 = lt; c0 < cpr; c0 += tpt * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * tpt;
      if (c < cpr) v[u] = __builtin_nontemporal_load(xr + c);
    }
    for (int j = 0; j < k; ++j) {
      const int r = pr[j];
      if (static_cast<unsigned>(r) >= static_cast<unsigned>(n_rows)) continue;  // bad pos: skipped
      u32x4* dst = send + (size_t)r * cpr;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * tpt;
        if (c < cpr) __builtin_nontemporal_store(v[u], dst + c);
      }
    }
  }
}

template <int ACT>
__global__ __launch_bounds__(kRowThreads) void standin_kernel(
    const u32x4* send, const int32_t* __restrict__ src, const int32_t* __restrict__ idx, u32x4* y,
    int n, int E, int cpr, int tpt) {  // y may alias send: each chunk is read, then written, by one lane
  const int per_blk = kRowThreads / tpt;
  const int r = blockIdx.x * per_blk + threadIdx.x / tpt;
  if (r >= n) return;
  const int lt = threadIdx.x % tpt;
  const int sr = src[r];
  const int e = static_cast<unsigned>(sr) < static_cast<unsigned>(n) ? idx[sr] : 0;
  const float scale = 1.0f + static_cast<float>(e) / static_cast<float>(E);
  const u32x4* in = send + (size_t)r * cpr;
  u32x4* out = y + (size_t)r * cpr;
  for (int c = lt; c < cpr; c += tpt) {
    float f[8];
    unpack8<ACT>(to_uint4(__builtin_nontemporal_load(in + c)), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = keep_f32(f[i] * scale);  // product rounded to fp32
    __builtin_nontemporal_store(to_vec(pack8<ACT>(f)), out + c);
  }
}

template <int ACT, int KMAX, bool OUT_F32>
__global__ __launch_bounds__(kRowThreads) void combine_kernel(
    const u32x4* __restrict__ y, const int32_t* __restrict__ pos, const float* __restrict__ w,
    void* __restrict__ out, int T, int k, int cpr, int tpt) {
  const int per_blk = kRowThreads / tpt;
  const int t = blockIdx.x * per_blk + threadIdx.x / tpt;
  if (t >= T) return;
  const int lt = threadIdx.x % tpt;
  size_t row[KMAX];
  float wt[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      const int r = pos[(size_t)t * k + j];
      const bool ok = static_cast<unsigned>(r) < static_cast<unsigned>(T * k);
      row[j] = ok ? (size_t)r * cpr : 0;  // a bad pos reads row 0 with weight 0
      wt[j] = ok ? w[(size_t)t * k + j] : 0.0f;
    }
  }
  for (int c = lt; c < cpr; c += tpt) {
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
    if constexpr (OUT_F32) {
      f32x4* o = reinterpret_cast<f32x4*>(out) + ((size_t)t * cpr + c) * 2;
      __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, o);
      __builtin_nontemporal_store(f32x4{acc[4], acc[5], acc[6], acc[7]}, o + 1);
    } else {
      u32x4* o = reinterpret_cast<u32x4*>(out) + (size_t)t * cpr + c;
      __builtin_nontemporal_store(to_vec(pack8<ACT>(acc)), o);
    }
  }
}

// Threads per row: enough for one 16-byte chunk each, at most the block.
int threads_per_row(int cpr) {
  int tpt = 16;
  while (tpt < cpr && tpt < kRowThreads) tpt *= 2;
  return tpt;
}

template <int ACT, bool OUT_F32>
hipError_t launch_combine_k(const u32x4* y, const int32_t* pos, const float* w, void* out, int T,
                            int k, int cpr, int tpt, int grid, hipStream_t s) {
  if (k <= 1) combine_kernel<ACT, 1, OUT_F32><<<grid, kRowThreads, 0, s>>>(y, pos, w, out, T, k, cpr, tpt);
  else if (k <= 2) combine_kernel<ACT, 2, OUT_F32><<<grid, kRowThreads, 0, s>>>(y, pos, w, out, T, k, cpr, tpt);
  else if (k <= 4) combine_kernel<ACT, 4, OUT_F32><<<grid, kRowThreads, 0, s>>>(y, pos, w, out, T, k, cpr, tpt);
  else if (k <= 8) combine_kernel<ACT, 8, OUT_F32><<<grid, kRowThreads, 0, s>>>(y, pos, w, out, T, k, cpr, tpt);
  else combine_kernel<ACT, 16, OUT_F32><<<grid, kRowThreads, 0, s>>>(y, pos, w, out, T, k, cpr, tpt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch(const void* x, const int32_t* pos, void* send, int T, int k, int H,
                           hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int cpr = H / 8;
  const int tpt = threads_per_row(cpr);
  const int per_blk = kRowThreads / tpt;
  const int grid = (T + per_blk - 1) / per_blk;
  const int per_lane = (cpr + tpt - 1) / tpt;
  const u32x4* xv = static_cast<const u32x4*>(x);
  u32x4* sv = static_cast<u32x4*>(send);
  if (per_lane <= 1) dispatch_kernel<1><<<grid, kRowThreads, 0, s>>>(xv, pos, sv, T, k, cpr, tpt);
  else if (per_lane <= 2) dispatch_kernel<2><<<grid, kRowThreads, 0, s>>>(xv, pos, sv, T, k, cpr, tpt);
  else dispatch_kernel<4><<<grid, kRowThreads, 0, s>>>(xv, pos, sv, T, k, cpr, tpt);
  return hipGetLastError();
}

hipError_t launch_standin(const void* send, const int32_t* src, const int32_t* idx, void* y, int T,
                          int E, int k, int H, int act, hipStream_t s) {
  const int n = T * k;
  if (n == 0) return hipSuccess;
  const int cpr = H / 8;
  const int tpt = threads_per_row(cpr);
  const int per_blk = kRowThreads / tpt;
  const int grid = (n + per_blk - 1) / per_blk;
  const u32x4* in = static_cast<const u32x4*>(send);
  u32x4* out = static_cast<u32x4*>(y);
  if (act == 1) standin_kernel<1><<<grid, kRowThreads, 0, s>>>(in, src, idx, out, n, E, cpr, tpt);
  else standin_kernel<2><<<grid, kRowThreads, 0, s>>>(in, src, idx, out, n, E, cpr, tpt);
  return hipGetLastError();
}

hipError_t launch_combine(const void* y, const int32_t* pos, const float* w, void* out, int T, int k,
                          int H, int act, bool out_f32, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int cpr = H / 8;
  const int tpt = threads_per_row(cpr);
  const int per_blk = kRowThreads / tpt;
  const int grid = (T + per_blk - 1) / per_blk;
  const u32x4* yv = static_cast<const u32x4*>(y);
  if (act == 1)
    return out_f32 ? launch_combine_k<1, true>(yv, pos, w, out, T, k, cpr, tpt, grid, s)
                   : launch_combine_k<1, false>(yv, pos, w, out, T, k, cpr, tpt, grid, s);
  return out_f32 ? launch_combine_k<2, true>(yv, pos, w, out, T, k, cpr, tpt, grid, s)
                 : launch_combine_k<2, false>(yv, pos, w, out, T, k, cpr, tpt, grid, s);
}

}  // namespace moe
