// Device helpers shared by the routing kernels: 16-bit float conversions,
// order-preserving integer keys for fp32 logits, and wave64 utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxE = 1024;  // largest expert count the kernels size LDS for
constexpr int kMaxR = 1024;  // largest virtual-rank count
constexpr int kMaxK = 16;    // largest number of experts per token

// ---- 16-bit activation formats --------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

// Hardware conversion in the default round-to-nearest-even mode.
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

template <int ACT>
__device__ __forceinline__ float act_to_f32(uint32_t bits16) {
  if constexpr (ACT == 1) return f16_to_f32(bits16);
  else return bf16_to_f32(bits16);
}

template <int ACT>
__device__ __forceinline__ uint32_t f32_to_act(float f) {
  if constexpr (ACT == 1) return f32_to_f16(f);
  else return f32_to_bf16(f);
}

// 8 packed 16-bit values <-> 8 floats.
template <int ACT>
__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = act_to_f32<ACT>(w[i] & 0xffffu);
    f[2 * i + 1] = act_to_f32<ACT>(w[i] >> 16);
  }
}

template <int ACT>
__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = f32_to_act<ACT>(f[2 * i]) | (f32_to_act<ACT>(f[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Pins a value as an fp32 register so the compiler cannot fold the
// conversions around it into a mixed-precision FMA (which would round the
// product directly to 16 bits and add +0.0, losing the sign of -0.0).
__device__ __forceinline__ float keep_f32(float v) {
  __asm__ volatile("" : "+v"(v));
  return v;
}

// Declares the launch's dynamic LDS so that a launch can reserve some: the
// runtime allocates dynamic LDS only for a kernel that references it. The
// reservation is never read or written (never_negative is a row length); it
// only caps how many blocks share a CU's 160 KiB of LDS.
__device__ __forceinline__ void declare_lds_reserve(int never_negative) {
  extern __shared__ int lds_reserve[];
  if (never_negative < 0) lds_reserve[threadIdx.x] = 0;
}

// Row slices: wide rows are cut into slices of kSliceChunks 16-byte chunks,
// one 128-thread block per slice and one chunk per lane. Block b of a launch
// whose first row is `first` takes slice b mod S of row first + b / S (S
// slices per row), so the slices of a row are dispatched together; c is the
// lane's chunk in the row (at most S * kSliceChunks - 1: lanes past the row
// end hold no chunk).
constexpr int kSliceChunks = 128;
__host__ __device__ constexpr int slices_per_row(int cpr) { return (cpr + kSliceChunks - 1) / kSliceChunks; }

__device__ __forceinline__ void slice_of_block(int S, int first, int& row, int& c) {
  const int rr = static_cast<int>(blockIdx.x) / S;
  row = first + rr;
  c = (static_cast<int>(blockIdx.x) - rr * S) * kSliceChunks + static_cast<int>(threadIdx.x);
}

// ---- order-preserving keys for top-k ---------------------------------------
// Larger key = better logit. Finite values and +-inf map monotonically into
// [0x007fffff, 0xff800000]; -0.0 is folded onto +0.0 so the two tie; any NaN
// maps to 1 (below every number); 0 is reserved for "no candidate".

__device__ __forceinline__ uint32_t logit_key(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 1u;     // NaN
  if ((u << 1) == 0u) u = 0u;                          // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_logit(uint32_t key) {
  if (key == 1u) return __uint_as_float(0x7fc00000u);
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
  return __uint_as_float(u);
}

// ---- wave64 helpers --------------------------------------------------------

__device__ __forceinline__ uint64_t ballot(bool pred) { return __ballot(pred); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// ---- DPP lane exchanges (gfx9 encodings) ----------------------------------
// Each is a VALU modifier, not an LDS round trip.
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;      // lane i <- lane 15-i within 16

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint32_t readlane(uint32_t v, int lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
}

// Max over aligned groups of L lanes (L in {8, 16, 32, 64}); every lane of the
// group receives the result. Butterfly within rows of 16 lanes, then the row
// maxima are read into scalar registers for groups wider than a row.
template <int L>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
  v = umax(v, dpp<kDppXor1>(v));
  v = umax(v, dpp<kDppXor2>(v));
  v = umax(v, dpp<kDppHalfMirror>(v));
  if constexpr (L >= 16) v = umax(v, dpp<kDppMirror>(v));
  if constexpr (L == 32) {
    const uint32_t g0 = umax(readlane(v, 0), readlane(v, 16));
    const uint32_t g1 = umax(readlane(v, 32), readlane(v, 48));
    v = (__lane_id() < 32) ? g0 : g1;
  } else if constexpr (L == 64) {
    v = umax(umax(readlane(v, 0), readlane(v, 16)), umax(readlane(v, 32), readlane(v, 48)));
  }
  return v;
}

constexpr int kDppRowShr1 = 0x111;     // lane i <- lane i-1 within a row of 16
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row -> every lane of the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 -> every lane of rows 2 and 3

// Row-masked DPP move: rows outside ROW_MASK receive 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_rows(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROW_MASK, 0xF, false));
}

// Max over the 64 lanes of a wave, returned as a wave-uniform value: a
// butterfly inside each row of 16 lanes, then the row maxima are carried
// forward with row broadcasts (rows 1 and 3 take rows 0 and 2, rows 2 and 3
// take row 1), so lane 63 ends with the maximum.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = umax(v, dpp<kDppXor1>(v));
  v = umax(v, dpp<kDppXor2>(v));
  v = umax(v, dpp<kDppHalfMirror>(v));
  v = umax(v, dpp<kDppMirror>(v));
  v = umax(v, dpp_rows<kDppRowBcast15, 0xA>(v));
  v = umax(v, dpp_rows<kDppRowBcast31, 0xC>(v));
  return readlane(v, 63);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = __double_as_longlong(x);
  const uint64_t lo = dpp<CTRL>(static_cast<uint32_t>(u));
  const uint64_t hi = dpp<CTRL>(static_cast<uint32_t>(u >> 32));
  return __longlong_as_double(static_cast<long long>(lo | (hi << 32)));
}

__device__ __forceinline__ double readlane_f64(double x, int lane) {
  const uint64_t u = __double_as_longlong(x);
  const uint64_t lo = readlane(static_cast<uint32_t>(u), lane);
  const uint64_t hi = readlane(static_cast<uint32_t>(u >> 32), lane);
  return __longlong_as_double(static_cast<long long>(lo | (hi << 32)));
}

// Sum over the first min(L, 16) lanes of each aligned group of L lanes (the
// other lanes of a group must hold 0, or be ignored by the caller when
// L <= 16); every lane of the group receives it. Fixed tree order, so the
// result is deterministic.
template <int L>
__device__ __forceinline__ double group_sum16_f64(double x) {
  x += dpp_f64<kDppXor1>(x);
  x += dpp_f64<kDppXor2>(x);
  x += dpp_f64<kDppHalfMirror>(x);
  if constexpr (L >= 16) x += dpp_f64<kDppMirror>(x);
  if constexpr (L == 32) {
    const double g0 = readlane_f64(x, 0), g1 = readlane_f64(x, 32);
    x = (__lane_id() < 32) ? g0 : g1;
  } else if constexpr (L == 64) {
    x = readlane_f64(x, 0);
  }
  return x;
}

// Sum over each aligned group of KP lanes (KP in {1, 2, 4, 8, 16}); every
// lane of the group receives it. Fixed tree order, so the result is
// deterministic.
template <int KP>
__device__ __forceinline__ double group_sum_f64(double x) {
  if constexpr (KP >= 2) x += dpp_f64<kDppXor1>(x);
  if constexpr (KP >= 4) x += dpp_f64<kDppXor2>(x);
  if constexpr (KP >= 8) x += dpp_f64<kDppHalfMirror>(x);
  if constexpr (KP >= 16) x += dpp_f64<kDppMirror>(x);
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave (every lane active), in
// DPP moves rather than LDS permutes: shifts by 1, 2, 4 and 8 lanes inside
// each row of 16 (a lane shifted in from outside its row reads 0) give the
// row prefixes; then lane 15's sum is added to row 1 and lane 47's to row 3
// (row_bcast:15), and lane 31's to rows 2 and 3 (row_bcast:31). `lane` is
// kept for the callers' convenience.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
  (void)lane;
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr1, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr2, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr4, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr8, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xC, 0xF, false);
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// One token's k (<= kMaxK) entries of a [T, k] int table, read so that every
// load is issued before any is used: the bucket of k is a uniform branch,
// and inside it the loads are unconditional (slots from k on reread slot
// k - 1, and callers ignore them), so one wait covers them all. Loads behind
// a per-slot condition were each waited for in turn (statistics count kernel
// at T = 65536, k = 8: 28.8 us that way, 24.8 us with this).
template <int N>
__device__ __forceinline__ void load_slots_n(const int32_t* __restrict__ row, int k,
                                             int (&v)[kMaxK]) {
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) v[j] = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = row[j < k ? j : k - 1];
}

__device__ __forceinline__ void load_slots(const int32_t* __restrict__ row, int k, int (&v)[kMaxK]) {
  if (k <= 2) load_slots_n<2>(row, k, v);
  else if (k <= 4) load_slots_n<4>(row, k, v);
  else if (k <= 8) load_slots_n<8>(row, k, v);
  else load_slots_n<kMaxK>(row, k, v);
}

// Destination rank of expert e: its assigned replica if active, else its
// primary copy, else the contiguous partition. Clamped so a bad table can
// never index out of bounds.
__device__ __forceinline__ int expert_rank(int e, int E, int R, const int* __restrict__ assign,
                                           const int* __restrict__ rep, int maxrep) {
  // both loads issued before either is used (the null tests are uniform);
  // the empty asm takes both values, so the compiler cannot move the second
  // load under a test of the first and wait for them in turn
  int a = assign != nullptr ? assign[e] : -1;
  int p = rep != nullptr ? rep[(size_t)e * maxrep] : e / (E / R);
  asm volatile("" : "+v"(a), "+v"(p));
  const int r = a >= 0 ? a : p;
  return r < 0 ? 0 : (r >= R ? R - 1 : r);
}

}  // namespace moe
