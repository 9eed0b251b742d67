// C ABI of the routing library: argument checks on the host, then kernel
// launches on the caller's stream. Declarations and the meaning of every
// argument are in include/moe_route.h.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "launch.hpp"
#include "moe_route.h"

// Scratch of moe_route_assign_layout_noalloc: a static device array, so the
// call needs no allocation. Each GPU the library runs on holds its own copy
// for the life of the process. In host code `scratch` names a host-side
// stand-in, never the device memory: kernels are given the device address
// that hipGetSymbolAddress returns for the current device (static_scratch
// below).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

// Set by the build to a digest of the sources and flags; a library compiled
// any other way reports "unknown", which no loader accepts.
#ifndef MOE_BUILD_ID
#define MOE_BUILD_ID "unknown"
#endif

namespace {

thread_local char g_last_error[256] = "";

moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

// Drop a stale error left by earlier unrelated HIP calls on this thread so a
// launch failure reported by a call is that call's own.
void clear_stale_error() { (void)hipGetLastError(); }

moe_status hip_status(hipError_t err, const char* where) {
  if (err == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(err));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr uint32_t kKnownFlags = MOE_FLAG_GREEDY_ID_ORDER | MOE_FLAG_OUT_F32;

moe_status check_problem(const moe_problem* p, const char* fn) {
  if (p == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: problem is NULL", fn);
  if (p->T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T=%d < 0", fn, p->T);
  if (p->E < 1 || p->E > MOE_MAX_E) return fail(MOE_ERR_INVALID_ARG, "%s: E=%d outside [1, %d]", fn, p->E, MOE_MAX_E);
  if (p->k < 1 || p->k > MOE_MAX_K || p->k > p->E)
    return fail(MOE_ERR_INVALID_ARG, "%s: k=%d outside [1, min(E, %d)]", fn, p->k, MOE_MAX_K);
  if (p->R < 1 || p->R > MOE_MAX_R) return fail(MOE_ERR_INVALID_ARG, "%s: R=%d outside [1, %d]", fn, p->R, MOE_MAX_R);
  if (p->H <= 0 || p->H % 8 != 0) return fail(MOE_ERR_INVALID_ARG, "%s: H=%d is not a positive multiple of 8", fn, p->H);
  if (p->act_dtype != MOE_F16 && p->act_dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "%s: act_dtype=%d is neither MOE_F16 nor MOE_BF16", fn, p->act_dtype);
  if (p->flags & ~kKnownFlags) return fail(MOE_ERR_INVALID_ARG, "%s: unknown flag bits 0x%x", fn, p->flags & ~kKnownFlags);
  if ((int64_t)p->T * p->k > MOE_MAX_ROWS)
    return fail(MOE_ERR_INVALID_ARG, "%s: T*k=%lld exceeds %d", fn, (long long)p->T * p->k, MOE_MAX_ROWS);
  return MOE_OK;
}

moe_status need(const void* ptr, size_t align, const char* fn, const char* name) {
  if (ptr == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);
  if (!aligned(ptr, align)) return fail(MOE_ERR_INVALID_ARG, "%s: %s is not %zu-byte aligned", fn, name, align);
  return MOE_OK;
}

moe_status check_rep(const moe_problem* p, const int32_t* rep, int32_t maxrep, const char* fn) {
  if (rep == nullptr) {
    if (p->E % p->R != 0)
      return fail(MOE_ERR_INVALID_ARG, "%s: no replica table and R=%d does not divide E=%d", fn, p->R, p->E);
    return MOE_OK;
  }
  if (maxrep < 1 || maxrep > MOE_MAX_REP)
    return fail(MOE_ERR_INVALID_ARG, "%s: maxrep=%d outside [1, %d]", fn, maxrep, MOE_MAX_REP);
  return need(rep, 4, fn, "rep");
}

#define CHECK(x)                        \
  do {                                  \
    const moe_status _st = (x);         \
    if (_st != MOE_OK) return _st;      \
  } while (0)

// Device address of the current device's copy of `scratch`, looked up once
// per device (with that device current) and kept.
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status static_scratch(void** out, const char* fn) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_status(err, fn);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "%s: device %d beyond the %d the library tracks", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return hip_status(err, fn);
    if (ptr == nullptr) return fail(MOE_ERR_HIP, "%s: no device address for the static scratch", fn);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// Argument checks shared by the two route + assignment + layout calls.
moe_status check_route_assign_layout(const moe_problem* p, const float* logits, const int32_t* rep,
                                     int32_t maxrep, const int32_t* idx, const float* w,
                                     const int32_t* counts, const int32_t* assign,
                                     const int32_t* active, const int32_t* rank_of,
                                     const int32_t* expert_offsets, const int32_t* rank_offsets,
                                     const int32_t* pos, const int32_t* src, const int32_t* dedup,
                                     const char* fn) {
  CHECK(check_problem(p, fn));
  CHECK(check_rep(p, rep, maxrep, fn));
  CHECK(need(counts, 4, fn, "counts"));
  CHECK(need(assign, 4, fn, "assign"));
  CHECK(need(active, 4, fn, "active"));
  CHECK(need(rank_of, 4, fn, "rank_of"));
  CHECK(need(expert_offsets, 4, fn, "expert_offsets"));
  CHECK(need(rank_offsets, 4, fn, "rank_offsets"));
  CHECK(need(dedup, 4, fn, "dedup"));
  if (p->T > 0) {
    CHECK(need(logits, 4, fn, "logits"));
    CHECK(need(idx, 4, fn, "idx"));
    CHECK(need(w, 4, fn, "w"));
    CHECK(need(pos, 4, fn, "pos"));
    CHECK(need(src, 4, fn, "src"));
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_version(void) { return 1 * 10000 + 2 * 100 + 0; }

const char* moe_build_id(void) { return MOE_BUILD_ID; }

const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_last_error; }

moe_status moe_workspace_bytes(const moe_problem* p, size_t* bytes) {
  CHECK(check_problem(p, "moe_workspace_bytes"));
  if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_workspace_bytes: bytes is NULL");
  *bytes = moe::workspace_bytes(p->T, p->E, p->R);
  return MOE_OK;
}

moe_status moe_route(const moe_problem* p, const float* logits, int32_t* idx, float* w,
                     int32_t* counts, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_route";
  CHECK(check_problem(p, fn));
  CHECK(need(counts, 4, fn, "counts"));
  CHECK(need(ws, 256, fn, "ws"));
  if (p->T > 0) {
    CHECK(need(logits, 4, fn, "logits"));
    CHECK(need(idx, 4, fn, "idx"));
    CHECK(need(w, 4, fn, "w"));
  }
  const size_t req = moe::workspace_bytes(p->T, p->E, p->R);
  if (ws_bytes < req) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, req);
  clear_stale_error();
  return hip_status(moe::launch_route(logits, p->T, p->E, p->k, idx, w, counts,
                                      static_cast<int32_t*>(ws), static_cast<hipStream_t>(stream)),
                    fn);
}

moe_status moe_assign_replicas(const moe_problem* p, const int32_t* counts, const int32_t* rep,
                               int32_t maxrep, int32_t* assign, int32_t* active, void* stream) {
  const char* fn = "moe_assign_replicas";
  CHECK(check_problem(p, fn));
  CHECK(check_rep(p, rep, maxrep, fn));
  CHECK(need(counts, 4, fn, "counts"));
  CHECK(need(assign, 4, fn, "assign"));
  CHECK(need(active, 4, fn, "active"));
  clear_stale_error();
  return hip_status(moe::launch_assign(counts, p->E, p->R, rep, rep ? maxrep : 1,
                                       (p->flags & MOE_FLAG_GREEDY_ID_ORDER) != 0, assign, active,
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

moe_status moe_route_assign_layout(const moe_problem* p, const float* logits, const int32_t* rep,
                                   int32_t maxrep, int32_t* idx, float* w, int32_t* counts,
                                   int32_t* assign, int32_t* active, int32_t* rank_of,
                                   int32_t* expert_offsets, int32_t* rank_offsets, int32_t* pos,
                                   int32_t* src, int32_t* dedup, void* ws, size_t ws_bytes,
                                   void* stream) {
  const char* fn = "moe_route_assign_layout";
  CHECK(check_route_assign_layout(p, logits, rep, maxrep, idx, w, counts, assign, active, rank_of,
                                  expert_offsets, rank_offsets, pos, src, dedup, fn));
  CHECK(need(ws, 256, fn, "ws"));
  const size_t req = moe::workspace_bytes(p->T, p->E, p->R);
  if (ws_bytes < req) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, req);
  clear_stale_error();
  return hip_status(moe::launch_route_assign_layout(
                        logits, p->T, p->E, p->k, p->R, rep, maxrep,
                        (p->flags & MOE_FLAG_GREEDY_ID_ORDER) != 0, idx, w, counts, assign, active,
                        rank_of, expert_offsets, rank_offsets, pos, src, dedup,
                        static_cast<int32_t*>(ws), static_cast<hipStream_t>(stream)),
                    fn);
}

moe_status moe_route_assign_layout_single_send(
    const moe_problem* p, const float* logits, const int32_t* rep, int32_t maxrep, int32_t* idx,
    float* w, int32_t* counts, int32_t* assign, int32_t* active, int32_t* rank_of,
    int32_t* expert_offsets, int32_t* rank_offsets, int32_t* pos, int32_t* src, int32_t* dedup,
    int32_t* ss_rank_offsets, int32_t* ss_row, int32_t* ss_token, void* ws, size_t ws_bytes,
    void* stream) {
  const char* fn = "moe_route_assign_layout_single_send";
  CHECK(check_route_assign_layout(p, logits, rep, maxrep, idx, w, counts, assign, active, rank_of,
                                  expert_offsets, rank_offsets, pos, src, dedup, fn));
  CHECK(need(ss_rank_offsets, 4, fn, "ss_rank_offsets"));
  if (p->T > 0) {
    CHECK(need(ss_row, 4, fn, "ss_row"));
    CHECK(need(ss_token, 4, fn, "ss_token"));
  }
  CHECK(need(ws, 256, fn, "ws"));
  const size_t req = moe::workspace_bytes(p->T, p->E, p->R);
  if (ws_bytes < req) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, req);
  clear_stale_error();
  return hip_status(moe::launch_route_assign_layout_single_send(
                        logits, p->T, p->E, p->k, p->R, rep, maxrep,
                        (p->flags & MOE_FLAG_GREEDY_ID_ORDER) != 0, idx, w, counts, assign, active,
                        rank_of, expert_offsets, rank_offsets, pos, src, dedup, ss_rank_offsets,
                        ss_row, ss_token, static_cast<int32_t*>(ws),
                        static_cast<hipStream_t>(stream)),
                    fn);
}

moe_status moe_route_assign_layout_noalloc(const moe_problem* p, const float* logits,
                                           const int32_t* rep, int32_t maxrep, int32_t* idx,
                                           float* w, int32_t* counts, int32_t* assign,
                                           int32_t* active, int32_t* rank_of,
                                           int32_t* expert_offsets, int32_t* rank_offsets,
                                           int32_t* pos, int32_t* src, int32_t* dedup,
                                           void* stream) {
  const char* fn = "moe_route_assign_layout_noalloc";
  CHECK(check_route_assign_layout(p, logits, rep, maxrep, idx, w, counts, assign, active, rank_of,
                                  expert_offsets, rank_offsets, pos, src, dedup, fn));
  const size_t req = moe::route_assign_layout_ws_bytes(p->T, p->E, p->R);
  if (req > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE, "%s: this problem needs %zu bytes of scratch, the static scratch holds %zu "
                "(use moe_route_assign_layout with a workspace)", fn, req, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  CHECK(static_scratch(&ws, fn));
  clear_stale_error();
  return hip_status(moe::launch_route_assign_layout(
                        logits, p->T, p->E, p->k, p->R, rep, maxrep,
                        (p->flags & MOE_FLAG_GREEDY_ID_ORDER) != 0, idx, w, counts, assign, active,
                        rank_of, expert_offsets, rank_offsets, pos, src, dedup,
                        static_cast<int32_t*>(ws), static_cast<hipStream_t>(stream)),
                    fn);
}

moe_status moe_layout(const moe_problem* p, const int32_t* idx, const int32_t* assign,
                      const int32_t* rep, int32_t maxrep, int32_t* rank_of,
                      int32_t* expert_offsets, int32_t* rank_offsets, int32_t* pos, int32_t* src,
                      int32_t* dedup, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_layout";
  CHECK(check_problem(p, fn));
  CHECK(check_rep(p, rep, maxrep, fn));
  if (assign != nullptr) CHECK(need(assign, 4, fn, "assign"));
  CHECK(need(rank_of, 4, fn, "rank_of"));
  CHECK(need(expert_offsets, 4, fn, "expert_offsets"));
  CHECK(need(rank_offsets, 4, fn, "rank_offsets"));
  CHECK(need(dedup, 4, fn, "dedup"));
  CHECK(need(ws, 256, fn, "ws"));
  if (p->T > 0) {
    CHECK(need(idx, 4, fn, "idx"));
    CHECK(need(pos, 4, fn, "pos"));
    CHECK(need(src, 4, fn, "src"));
  }
  const size_t req = moe::workspace_bytes(p->T, p->E, p->R);
  if (ws_bytes < req) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, req);
  clear_stale_error();
  return hip_status(moe::launch_layout(idx, p->T, p->E, p->k, p->R, assign, rep, rep ? maxrep : 1,
                                       rank_of, expert_offsets, rank_offsets, pos, src, dedup,
                                       nullptr, nullptr, nullptr, static_cast<int32_t*>(ws),
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

moe_status moe_layout_single_send(const moe_problem* p, const int32_t* idx, const int32_t* assign,
                                  const int32_t* rep, int32_t maxrep, int32_t* rank_of,
                                  int32_t* expert_offsets, int32_t* rank_offsets, int32_t* pos,
                                  int32_t* src, int32_t* dedup, int32_t* ss_rank_offsets,
                                  int32_t* ss_row, int32_t* ss_token, void* ws, size_t ws_bytes,
                                  void* stream) {
  const char* fn = "moe_layout_single_send";
  CHECK(check_problem(p, fn));
  CHECK(check_rep(p, rep, maxrep, fn));
  if (assign != nullptr) CHECK(need(assign, 4, fn, "assign"));
  CHECK(need(rank_of, 4, fn, "rank_of"));
  CHECK(need(expert_offsets, 4, fn, "expert_offsets"));
  CHECK(need(rank_offsets, 4, fn, "rank_offsets"));
  CHECK(need(dedup, 4, fn, "dedup"));
  CHECK(need(ss_rank_offsets, 4, fn, "ss_rank_offsets"));
  CHECK(need(ws, 256, fn, "ws"));
  if (p->T > 0) {
    CHECK(need(idx, 4, fn, "idx"));
    CHECK(need(pos, 4, fn, "pos"));
    CHECK(need(src, 4, fn, "src"));
    CHECK(need(ss_row, 4, fn, "ss_row"));
    CHECK(need(ss_token, 4, fn, "ss_token"));
  }
  const size_t req = moe::workspace_bytes(p->T, p->E, p->R);
  if (ws_bytes < req) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, req);
  clear_stale_error();
  return hip_status(moe::launch_layout(idx, p->T, p->E, p->k, p->R, assign, rep, rep ? maxrep : 1,
                                       rank_of, expert_offsets, rank_offsets, pos, src, dedup,
                                       ss_rank_offsets, ss_row, ss_token,
                                       static_cast<int32_t*>(ws), static_cast<hipStream_t>(stream)),
                    fn);
}

moe_status moe_single_send_dispatch(const moe_problem* p, const void* x, const int32_t* ss_row,
                                    void* send_ss, int32_t ss_capacity, void* stream) {
  const char* fn = "moe_single_send_dispatch";
  CHECK(check_problem(p, fn));
  if (ss_capacity < 0) return fail(MOE_ERR_INVALID_ARG, "%s: ss_capacity=%d < 0", fn, ss_capacity);
  if (p->T == 0 || ss_capacity == 0) return MOE_OK;
  CHECK(need(x, 16, fn, "x"));
  CHECK(need(ss_row, 4, fn, "ss_row"));
  CHECK(need(send_ss, 16, fn, "send_ss"));
  clear_stale_error();
  return hip_status(moe::launch_single_send_dispatch(x, ss_row, send_ss, ss_capacity, p->T, p->k,
                                                     p->H, static_cast<hipStream_t>(stream)),
                    fn);
}

moe_status moe_single_send_expand(const moe_problem* p, const void* send_ss,
                                  const int32_t* ss_rank_offsets, const int32_t* ss_token,
                                  const int32_t* ss_row, const int32_t* pos, int32_t ss_capacity,
                                  void* send, void* stream) {
  const char* fn = "moe_single_send_expand";
  CHECK(check_problem(p, fn));
  if (ss_capacity < 0) return fail(MOE_ERR_INVALID_ARG, "%s: ss_capacity=%d < 0", fn, ss_capacity);
  if (p->T == 0 || ss_capacity == 0) return MOE_OK;
  CHECK(need(send_ss, 16, fn, "send_ss"));
  CHECK(need(ss_rank_offsets, 4, fn, "ss_rank_offsets"));
  CHECK(need(ss_token, 4, fn, "ss_token"));
  CHECK(need(ss_row, 4, fn, "ss_row"));
  CHECK(need(pos, 4, fn, "pos"));
  CHECK(need(send, 16, fn, "send"));
  clear_stale_error();
  return hip_status(moe::launch_single_send_expand(send_ss, ss_rank_offsets, ss_token, ss_row, pos,
                                                   ss_capacity, send, p->T, p->k, p->R, p->H,
                                                   static_cast<hipStream_t>(stream)),
                    fn);
}

moe_status moe_dispatch(const moe_problem* p, const void* x, const int32_t* pos, void* send,
                        void* stream) {
  const char* fn = "moe_dispatch";
  CHECK(check_problem(p, fn));
  if (p->T == 0) return MOE_OK;
  CHECK(need(x, 16, fn, "x"));
  CHECK(need(pos, 4, fn, "pos"));
  CHECK(need(send, 16, fn, "send"));
  clear_stale_error();
  return hip_status(moe::launch_dispatch(x, pos, send, p->T, p->k, p->H,
                                         static_cast<hipStream_t>(stream)),
                    fn);
}

moe_status moe_expert_standin(const moe_problem* p, const void* send, const int32_t* src,
                              const int32_t* idx, void* y, void* stream) {
  const char* fn = "moe_expert_standin";
  CHECK(check_problem(p, fn));
  if (p->T == 0) return MOE_OK;
  CHECK(need(send, 16, fn, "send"));
  CHECK(need(src, 4, fn, "src"));
  CHECK(need(idx, 4, fn, "idx"));
  CHECK(need(y, 16, fn, "y"));
  clear_stale_error();
  return hip_status(moe::launch_standin(send, src, idx, y, p->T, p->E, p->k, p->H, p->act_dtype,
                                        static_cast<hipStream_t>(stream)),
                    fn);
}

moe_status moe_combine(const moe_problem* p, const void* y, const int32_t* pos, const float* w,
                       void* out, void* stream) {
  const char* fn = "moe_combine";
  CHECK(check_problem(p, fn));
  if (p->T == 0) return MOE_OK;
  CHECK(need(y, 16, fn, "y"));
  CHECK(need(pos, 4, fn, "pos"));
  CHECK(need(w, 4, fn, "w"));
  CHECK(need(out, 16, fn, "out"));
  clear_stale_error();
  return hip_status(moe::launch_combine(y, pos, w, out, p->T, p->k, p->H, p->act_dtype,
                                        (p->flags & MOE_FLAG_OUT_F32) != 0,
                                        static_cast<hipStream_t>(stream)),
                    fn);
}

moe_status moe_combine_backward(const moe_problem* p, const void* dout, const void* y,
                                const int32_t* pos, const float* w, void* dy, float* dw,
                                void* stream) {
  const char* fn = "moe_combine_backward";
  CHECK(check_problem(p, fn));
  if (p->T == 0) return MOE_OK;
  if (dy == nullptr && dw == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: dy and dw are both NULL", fn);
  CHECK(need(dout, 16, fn, "dout"));
  CHECK(need(pos, 4, fn, "pos"));
  if (dy != nullptr) {
    CHECK(need(w, 4, fn, "w"));
    CHECK(need(dy, 16, fn, "dy"));
  }
  if (dw != nullptr) {
    CHECK(need(y, 16, fn, "y"));
    CHECK(need(dw, 4, fn, "dw"));
  }
  clear_stale_error();
  return hip_status(moe::launch_combine_backward(dout, y, pos, w, dy, dw, p->T, p->k, p->H,
                                                 p->act_dtype, static_cast<hipStream_t>(stream)),
                    fn);
}

moe_status moe_dispatch_backward(const moe_problem* p, const void* dsend, const int32_t* pos,
                                 void* dx, void* stream) {
  const char* fn = "moe_dispatch_backward";
  CHECK(check_problem(p, fn));
  if (p->T == 0) return MOE_OK;
  CHECK(need(dsend, 16, fn, "dsend"));
  CHECK(need(pos, 4, fn, "pos"));
  CHECK(need(dx, 16, fn, "dx"));
  clear_stale_error();
  return hip_status(moe::launch_dispatch_backward(dsend, pos, dx, p->T, p->k, p->H, p->act_dtype,
                                                  (p->flags & MOE_FLAG_OUT_F32) != 0,
                                                  static_cast<hipStream_t>(stream)),
                    fn);
}

moe_status moe_routing_stats(const moe_problem* p, const int32_t* idx, const int32_t* counts,
                             const int32_t* rank_of, int32_t* send_counts, int32_t* coselect,
                             double* stats, void* stream) {
  const char* fn = "moe_routing_stats";
  CHECK(check_problem(p, fn));
  CHECK(need(counts, 4, fn, "counts"));
  CHECK(need(rank_of, 4, fn, "rank_of"));
  CHECK(need(send_counts, 4, fn, "send_counts"));
  CHECK(need(stats, 8, fn, "stats"));
  if (coselect != nullptr) CHECK(need(coselect, 4, fn, "coselect"));
  if (p->T > 0) CHECK(need(idx, 4, fn, "idx"));
  clear_stale_error();
  return hip_status(moe::launch_routing_stats(idx, rank_of, counts, p->T, p->E, p->k, p->R,
                                              send_counts, coselect, stats,
                                              static_cast<hipStream_t>(stream)),
                    fn);
}

moe_status moe_token_balanced_split(const moe_problem* p, const int32_t* idx,
                                    const int32_t* counts, const int32_t* pos,
                                    const int32_t* expert_offsets, const int32_t* rep,
                                    int32_t maxrep, int32_t* gpu_of_pair, int32_t* active,
                                    int32_t* tokens, void* stream) {
  const char* fn = "moe_token_balanced_split";
  CHECK(check_problem(p, fn));
  CHECK(check_rep(p, rep, maxrep, fn));
  CHECK(need(counts, 4, fn, "counts"));
  CHECK(need(active, 4, fn, "active"));
  CHECK(need(tokens, 4, fn, "tokens"));
  if (p->T > 0 && gpu_of_pair != nullptr) {
    CHECK(need(idx, 4, fn, "idx"));
    CHECK(need(pos, 4, fn, "pos"));
    CHECK(need(expert_offsets, 4, fn, "expert_offsets"));
    CHECK(need(gpu_of_pair, 4, fn, "gpu_of_pair"));
  }
  clear_stale_error();
  return hip_status(moe::launch_token_balanced_split(idx, counts, pos, expert_offsets, rep,
                                                     rep ? maxrep : 1, p->T, p->E, p->k, p->R,
                                                     gpu_of_pair, active, tokens,
                                                     static_cast<hipStream_t>(stream)),
                    fn);
}

}  // extern "C"
