/*
 * moe_route.h -- C ABI of the single-GPU MoE token-routing path for AMD
 * Instinct MI355X (gfx950): router top-k with gate weights, the expert demand
 * vector, METRO-style greedy replica assignment, the rank-grouped dispatch
 * layout with single-send dedup counts, the row dispatch, an expert stand-in,
 * and the weighted combine; around them, single-send dispatch (one row per
 * token and destination rank) with its receiver fan-out, the backward of the
 * combine and the dispatch, routing statistics, and token-balanced replica
 * routing as the greedy's baseline.
 *
 * Sources (web pages on MoE dispatch and combine):
 *   [METRO]  "METRO AllGather vs AllToAll for MoE decode".
 *   [CORR]   News summary of "correlated expert placement and token
 *            shuffling" for MoE pretraining.
 *   [DODOCO] "Diagnosing Overhead in Dispatch Operations: Cross-architecture
 *            Observatory".
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every array argument is a DEVICE pointer allocated and owned by the
 *    caller. The library never allocates or frees device memory, never
 *    synchronises, and only enqueues kernels on `stream` (a hipStream_t;
 *    NULL means the null stream). Results are valid once the stream has
 *    reached that point. Calls are stateless and may run concurrently on
 *    different streams with different buffers.
 *  - Every call returns a moe_status and never aborts. Host-side argument
 *    checks happen before anything is enqueued: MOE_ERR_INVALID_ARG for a bad
 *    shape, dtype, flag, a NULL pointer where data is needed, or a
 *    misaligned pointer; MOE_ERR_WORKSPACE for a workspace smaller than
 *    moe_workspace_bytes(). A failed kernel launch returns MOE_ERR_HIP.
 *    moe_last_error() gives a one-line description of the last failure on
 *    the calling thread.
 *  - Data-dependent faults are not detected: expert ids in `idx` outside
 *    [0, E), replica entries outside [-1, R), or `pos` / `src` values that
 *    are not the permutation moe_layout wrote give an unspecified result,
 *    but every kernel keeps its memory accesses inside the buffers the shape
 *    describes (out-of-range entries are clamped or skipped).
 *  - T = 0 is valid: per-token outputs are empty, per-expert and per-rank
 *    outputs are written (zero counts, no active experts, zero offsets).
 *  - Token activations are 16-bit floats (fp16 or bf16) in row-major [rows, H]
 *    with H a multiple of 8, so each row is a whole number of 16-byte chunks;
 *    activation pointers must be 16-byte aligned.
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4
} moe_status;

/* Activation formats. */
enum { MOE_F16 = 1, MOE_BF16 = 2 };

/* Flags (bit set). */
enum {
  /* Greedy replica assignment visits active experts in ascending id instead
   * of the default most-constrained-first order (fewest replicas, then id). */
  MOE_FLAG_GREEDY_ID_ORDER = 1u << 0,
  /* moe_combine writes fp32 rows instead of the activation format. */
  MOE_FLAG_OUT_F32 = 1u << 1
};

/* Limits checked on the host. */
/* MOE_MAX_ROWS bounds T*k: kernels that give each send row a 256-thread
 * block launch up to T*k blocks, and one launch holds fewer than 2^32
 * work-items. */
enum { MOE_MAX_E = 1024, MOE_MAX_K = 16, MOE_MAX_R = 1024, MOE_MAX_REP = 16,
       MOE_MAX_ROWS = (1 << 24) - 1 };

/* One routing problem.
 *   T  tokens, T >= 0, T*k <= MOE_MAX_ROWS (2^24 - 1)
 *   E  experts, 1 <= E <= 1024
 *   k  experts selected per token, 1 <= k <= min(E, 16)
 *   H  hidden width (elements per activation row), H > 0, H % 8 == 0
 *   R  virtual expert-parallel ranks (= virtual GPUs), 1 <= R <= 1024; a
 *      layout inside this GPU's memory, nothing is communicated
 *   act_dtype  MOE_F16 or MOE_BF16
 *   flags      MOE_FLAG_* bits                                               */
typedef struct {
  int32_t T, E, k, H, R;
  int32_t act_dtype;
  uint32_t flags;
} moe_problem;

/* Version of this ABI (major * 10000 + minor * 100 + patch). */
int32_t moe_version(void);

/* Identity of the build: 16 hex digits of a SHA-256 over the compile flags
 * and the bytes of every source and header the library was compiled from
 * ("unknown" when built without the package's build script). A loader
 * compares it with the digest of the sources beside it to refuse a stale
 * library. Static string; host only. */
const char* moe_build_id(void);

/* Static text for a status code ("unknown status" for other values). */
const char* moe_status_string(int32_t status);

/* Description of the last non-OK status returned on this thread ("" if none). */
const char* moe_last_error(void);

/* Bytes of device workspace moe_route, moe_layout, moe_layout_single_send and
 * the one-call plans need for this problem (one buffer of this size serves
 * all of them; its contents need no initialisation and are not meaningful
 * between calls).
 * Host only; enqueues nothing. */
moe_status moe_workspace_bytes(const moe_problem* p, size_t* bytes);

/* Router top-k, gate weights and the global expert demand vector.
 * [METRO] section "METRO AllGather vs AllToAll changes the routing
 * information": top-k over every token, then one count per expert.
 *   logits  f32 [T, E] row-major (read)
 *   idx     i32 [T, k] (write): the k selected experts of each token, slot 0
 *           the largest logit; ties go to the lower expert id, -0.0 ties
 *           +0.0, a NaN logit ranks below every number
 *   w       f32 [T, k] (write): softmax over the k selected logits, evaluated
 *           in fp64 and rounded once to fp32 (the pages give no gate rule;
 *           this is the reading taken)
 *   counts  i32 [E] (write): number of (token, slot) pairs that chose e;
 *           sums to T*k
 *   ws      workspace of at least moe_workspace_bytes() bytes             */
moe_status moe_route(const moe_problem* p, const float* logits, int32_t* idx, float* w,
                     int32_t* counts, void* ws, size_t ws_bytes, void* stream);

/* Greedy replica assignment: every active expert (counts[e] > 0) goes to one
 * of its replicas, on the virtual GPU with the fewest experts activated so
 * far; ties go to the lower GPU index. [METRO] sections "METRO AllGather vs
 * AllToAll changes the routing information" and "Add the expert-weight
 * traffic term" (greedy, not the optimal min-max assignment).
 * Visiting order: most-constrained first (ascending number of replicas, then
 * id) unless MOE_FLAG_GREEDY_ID_ORDER is set.
 *   counts  i32 [E] (read)
 *   rep     i32 [E, maxrep] (read) virtual GPU ids in [0, R) holding a copy of
 *           each expert, -1 padded; rep[e][0] is the primary copy and must be
 *           valid. NULL means no replicas: expert e lives on GPU e / (E / R)
 *           (needs R | E).
 *   maxrep  columns of rep, 1..16 (ignored when rep is NULL)
 *   assign  i32 [E] (write): chosen GPU, or -1 for an inactive expert
 *   active  i32 [R] (write): activated experts per virtual GPU              */
moe_status moe_assign_replicas(const moe_problem* p, const int32_t* counts, const int32_t* rep,
                               int32_t maxrep, int32_t* assign, int32_t* active, void* stream);

/* Dispatch layout and single-send dedup counts.
 * [METRO] section "Work the 8-GPU payload example" (an all-to-all sends one
 * chunk per destination rank) and section "Distinguish METRO from backend
 * names" (variable-size all-to-all driven by destination counts); [CORR]
 * section "Two locality techniques" (a token is sent to a GPU at most once).
 * The send buffer has exactly T*k rows, grouped by destination rank, inside a
 * rank by expert id, inside an expert by token (stable).
 *   idx      i32 [T, k] (read), as written by moe_route; an id outside
 *            [0, E) is clamped into it
 *   assign   i32 [E] or NULL (read): destination of active experts; inactive
 *            experts (-1) and the NULL case use the primary copy
 *   rep, maxrep  as in moe_assign_replicas (NULL: contiguous partition)
 *   rank_of         i32 [E]   (write) destination rank of each expert
 *   expert_offsets  i32 [E]   (write) first send row of expert e's segment
 *   rank_offsets    i32 [R+1] (write) first send row of each rank; [R] = T*k
 *   pos   i32 [T*k] (write) send row of pair (t, j) at index t*k + j
 *   src   i32 [T*k] (write) inverse of pos: flat (t, j) index of each row
 *   dedup i32 [R]   (write) tokens with at least one expert on rank r: the
 *                   rows a single-send dispatcher sends to r               */
moe_status moe_layout(const moe_problem* p, const int32_t* idx, const int32_t* assign,
                      const int32_t* rep, int32_t maxrep, int32_t* rank_of,
                      int32_t* expert_offsets, int32_t* rank_offsets, int32_t* pos,
                      int32_t* src, int32_t* dedup, void* ws, size_t ws_bytes, void* stream);

/* Everything moe_layout computes, plus the single-send rows: one send row
 * per (token, destination rank) instead of one per (token, slot), so a token
 * goes to each virtual GPU once. [CORR] section "Two locality techniques"
 * (a dispatcher that sends each token to a GPU once; with correlated expert
 * placement it removes dispatched rows).
 * Single-send rows are grouped by destination rank, inside a rank by token.
 *   ss_rank_offsets i32 [R+1] (write) first single-send row of each rank;
 *                   [R] = n_ss = sum(dedup), the number of rows
 *   ss_row          i32 [T*k] (write) the single-send row carrying pair
 *                   (t, j) at index t*k + j; the pairs of one token whose
 *                   experts sit on the same rank share one row
 *   ss_token        i32 [T*k] (write) token of each single-send row; entries
 *                   from n_ss on are left untouched
 * The other arguments are those of moe_layout. The workspace is the same
 * size (moe_workspace_bytes).                                              */
moe_status moe_layout_single_send(const moe_problem* p, const int32_t* idx, const int32_t* assign,
                                  const int32_t* rep, int32_t maxrep, int32_t* rank_of,
                                  int32_t* expert_offsets, int32_t* rank_offsets, int32_t* pos,
                                  int32_t* src, int32_t* dedup, int32_t* ss_rank_offsets,
                                  int32_t* ss_row, int32_t* ss_token, void* ws, size_t ws_bytes,
                                  void* stream);

/* moe_route, moe_assign_replicas and moe_layout in one call, with the same
 * arguments and outputs as those three calls made in that order (assign is
 * both an output and the layout's input). For a decode batch fixed latency
 * rather than bytes sets the time ([METRO] section "Find the crossover
 * instead of copying 2 MB": below the crossover payload a fixed overhead
 * dominates), so the steps share launches:
 *   - a batch with T*k <= 8192 whose tables fit in 64 KiB of LDS: two
 *     launches, the top-k kernel, then one workgroup that sums the demand
 *     vector, runs the greedy and lays out the batch;
 *   - a larger batch without a replica table (rep NULL): three launches,
 *     the top-k kernel (which also counts each block's tokens per rank), a
 *     column scan, and the permutation;
 *   - a larger batch with a replica table: the kernels of the three calls.
 * ws is one workspace of moe_workspace_bytes().                             */
moe_status moe_route_assign_layout(const moe_problem* p, const float* logits, const int32_t* rep,
                                   int32_t maxrep, int32_t* idx, float* w, int32_t* counts,
                                   int32_t* assign, int32_t* active, int32_t* rank_of,
                                   int32_t* expert_offsets, int32_t* rank_offsets, int32_t* pos,
                                   int32_t* src, int32_t* dedup, void* ws, size_t ws_bytes,
                                   void* stream);

/* moe_route, moe_assign_replicas and moe_layout_single_send in one call, with
 * the same arguments and outputs as those three calls made in that order:
 * the routing and the plain layout, plus the single-send rows of a
 * dispatcher that sends each token to a GPU once (news summary of correlated
 * expert placement and token shuffling, section "Two locality techniques").
 *   - a batch with T <= 1024, T*k <= 8192 and R <= 64 whose tables fit in
 *     64 KiB of LDS: two launches, the top-k kernel, then one workgroup that
 *     sums the demand vector, runs the greedy and lays out the batch and its
 *     single-send rows;
 *   - a larger batch without a replica table (rep NULL): three launches, the
 *     top-k kernel (which also counts each block's tokens per rank and
 *     records each token's first slot on each of its ranks), a column scan,
 *     and one launch for the permutation and the single-send rows;
 *   - otherwise (a larger batch with a replica table, or T = 0): the kernels
 *     of the three calls.
 *   ss_rank_offsets, ss_row, ss_token as for moe_layout_single_send (ss_row
 *   and ss_token i32 [T*k], unused when T = 0).
 * ws is one workspace of moe_workspace_bytes().                             */
moe_status moe_route_assign_layout_single_send(
    const moe_problem* p, const float* logits, const int32_t* rep, int32_t maxrep, int32_t* idx,
    float* w, int32_t* counts, int32_t* assign, int32_t* active, int32_t* rank_of,
    int32_t* expert_offsets, int32_t* rank_offsets, int32_t* pos, int32_t* src, int32_t* dedup,
    int32_t* ss_rank_offsets, int32_t* ss_row, int32_t* ss_token, void* ws, size_t ws_bytes,
    void* stream);

/* Bytes of the static device scratch behind moe_route_assign_layout_noalloc
 * (2 MiB per GPU). */
#define MOE_NOALLOC_SCRATCH_BYTES (2u << 20)

/* moe_route_assign_layout without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). The scratch is a static device
 * array of MOE_NOALLOC_SCRATCH_BYTES that each GPU holds from the first call
 * on it until the process ends; the call itself allocates nothing.
 * Arguments and outputs are those of moe_route_assign_layout (the caller
 * still allocates every input and output), and so are the results.
 *   - A problem whose route and layout tables need more scratch than the
 *     array holds (E + R above 1024, with enough tokens; every
 *     problem with E + R <= 1024 fits) returns MOE_ERR_WORKSPACE before
 *     anything is enqueued.
 *   - The first call on a device looks up that device's copy of the array
 *     (a failure returns MOE_ERR_HIP).
 *   - The scratch needs no initialisation, and its contents are not
 *     meaningful between calls.
 *   - Every call on one GPU uses that GPU's one array: calls that overlap on
 *     one GPU (different streams, or host threads enqueueing concurrently)
 *     race on it and give unspecified results. Order them on one stream.   */
moe_status moe_route_assign_layout_noalloc(const moe_problem* p, const float* logits,
                                           const int32_t* rep, int32_t maxrep, int32_t* idx,
                                           float* w, int32_t* counts, int32_t* assign,
                                           int32_t* active, int32_t* rank_of,
                                           int32_t* expert_offsets, int32_t* rank_offsets,
                                           int32_t* pos, int32_t* src, int32_t* dedup,
                                           void* stream);

/* Single-send dispatch: each token row x[t] is copied once to each distinct
 * single-send row among ss_row[t*k .. t*k+k). [CORR] section "Two locality
 * techniques".
 *   x        16-bit [T, H] (read)   ss_row i32 [T*k] (read), from
 *            moe_layout_single_send
 *   send_ss  16-bit [ss_capacity, H] (write); ss_capacity >= n_ss rows
 *            (rows at or beyond ss_capacity are skipped)                   */
moe_status moe_single_send_dispatch(const moe_problem* p, const void* x, const int32_t* ss_row,
                                    void* send_ss, int32_t ss_capacity, void* stream);

/* Receiver-side fan-out of single-send rows to the expert-grouped layout:
 * send[pos[i]] = send_ss[ss_row[i]] for every pair i < T*k, which equals what
 * moe_dispatch writes. [CORR] section "Two locality techniques" (each GPU
 * receives a token once and serves every selected expert it holds). Each
 * single-send row is read once and written to the expert rows of all the
 * slots it carries.
 *   send_ss          16-bit [ss_capacity, H] (read)
 *   ss_rank_offsets  i32 [R+1] (read; [R] = n_ss)   ss_token i32 [n_ss] (read)
 *   ss_row, pos      i32 [T*k] (read), from moe_layout_single_send
 *   send             16-bit [T*k, H] (write)
 * Single-send rows at or beyond min(n_ss, ss_capacity), and out-of-range
 * tokens or positions, are skipped: their destination rows are left
 * untouched.                                                               */
moe_status moe_single_send_expand(const moe_problem* p, const void* send_ss,
                                  const int32_t* ss_rank_offsets, const int32_t* ss_token,
                                  const int32_t* ss_row, const int32_t* pos, int32_t ss_capacity,
                                  void* send, void* stream);

/* Row dispatch: send[pos[i]] = x[i / k] for every i < T*k, a bit copy.
 * [METRO] section "Work the 8-GPU payload example" (the dispatch payload is
 * token activation rows).
 *   x     16-bit [T, H] (read)    pos  i32 [T*k] (read)
 *   send  16-bit [T*k, H] (write); must not overlap x
 * A slot whose pos is outside [0, T*k) is skipped: no row is written for
 * it.                                                                      */
moe_status moe_dispatch(const moe_problem* p, const void* x, const int32_t* pos, void* send,
                        void* stream);

/* Expert stand-in (the pages' expert GEMMs need trained weights): for send
 * row r routed to expert e = idx[src[r]], y[r] = round16(fp32(send[r]) * s)
 * with s = 1 + e/E, s and the product each rounded to fp32, round16 to
 * nearest-even in the activation format.
 *   send 16-bit [T*k, H] (read)  src i32 [T*k]  idx i32 [T, k]
 *   y    16-bit [T*k, H] (write); may alias send
 * A row whose src is outside [0, T*k) is scaled as expert 0 (s = 1).      */
moe_status moe_expert_standin(const moe_problem* p, const void* send, const int32_t* src,
                              const int32_t* idx, void* y, void* stream);

/* Weighted combine back to token order:
 * out[t] = sum over j = 0..k-1 (ascending) of w[t, j] * y[pos[t*k + j]],
 * accumulated in fp32, written in the activation format (round to
 * nearest-even) or as fp32 with MOE_FLAG_OUT_F32.
 * [METRO] section "METRO AllGather vs AllToAll changes the routing
 * information" (expert outputs return through a combine); [CORR] section
 * "Why communication is the target".
 *   y    16-bit [T*k, H] (read)  pos i32 [T*k]  w f32 [T, k]
 *   out  [T, H] in the activation format or fp32 (write); must not overlap y
 * A slot whose pos is outside [0, T*k) takes weight 0 on row 0: it adds
 * nothing while row 0 is finite.                                           */
moe_status moe_combine(const moe_problem* p, const void* y, const int32_t* pos, const float* w,
                       void* out, void* stream);

/* Backward of the combine. With dout [T, H] the gradient of out:
 *   dy[pos[t*k + j]] = round16(fp32(w[t, j] * dout[t]))   (one rounding
 *                      of the fp32 product to the activation format)
 *   dw[t, j]         = <y[pos[t*k + j]], dout[t]>, summed in fp32
 * Derived from the forward definition of moe_combine; [CORR] section "Why
 * communication is the target" (the combine also runs in the backward
 * pass). One kernel reads each dout row once and, per slot, writes the dy
 * row and reads the y row for the dot product.
 *   dout 16-bit [T, H] (read)   pos i32 [T*k] (read)
 *   w    f32 [T, k] (read; may be NULL when dy is NULL)
 *   y    16-bit [T*k, H] (read; may be NULL when dw is NULL)
 *   dy   16-bit [T*k, H] (write, or NULL to skip); may alias y, must not
 *        overlap dout
 *   dw   f32 [T, k] (write, or NULL to skip)
 * With T > 0 at least one of dy, dw must be non-NULL (else
 * MOE_ERR_INVALID_ARG). A slot whose pos is out of range
 * writes no dy row and a dw of 0.                                          */
moe_status moe_combine_backward(const moe_problem* p, const void* dout, const void* y,
                                const int32_t* pos, const float* w, void* dy, float* dw,
                                void* stream);

/* Backward of the dispatch: dx[t] = sum over j = 0..k-1 (ascending) of
 * dsend[pos[t*k + j]], accumulated in fp32, written in the activation format
 * (round to nearest-even) or as fp32 with MOE_FLAG_OUT_F32. Derived from the
 * forward definition of moe_dispatch; [CORR] section "Why communication is
 * the target".
 *   dsend 16-bit [T*k, H] (read)   pos i32 [T*k] (read)
 *   dx    [T, H] in the activation format or fp32 (write); must not overlap
 *         dsend. A slot whose pos is out of range adds nothing.           */
moe_status moe_dispatch_backward(const moe_problem* p, const void* dsend, const int32_t* pos,
                                 void* dx, void* stream);

/* Routing statistics of one batch. [DODOCO] section "Methodology" (three
 * scalar summaries of the send-counts matrix: per-expert max/mean, Gini of
 * the per-rank load, a fitted symmetric Dirichlet alpha); [CORR] sections
 * "Correlations in router choices" (experts chosen together) and "Two
 * locality techniques" (share of assignments served on the token's own GPU).
 * Token t comes from virtual rank floor(t R / T).
 *   idx         i32 [T, k] (read)   counts i32 [E] (read, from moe_route)
 *   rank_of     i32 [E] (read, from moe_layout)
 *   send_counts i32 [R, R] (write): [s][d] = (token, slot) pairs from
 *               source rank s whose expert sits on rank d
 *   coselect    i32 [E, E] (write, or NULL to skip): [a][b] for a < b = the
 *               tokens that chose both a and b; 0 elsewhere
 *   stats       f64 [4] (write): with N = T k and L[d] = sum_s S[s][d],
 *               [0] max_e counts[e] / (N / E)
 *               [1] Gini of L: sum_i sum_j |L_i - L_j| / (2 R N)
 *               [2] symmetric Dirichlet alpha fitted by moments to the
 *                   shares L / N: ((R - 1) / (R D) - 1) / R with
 *                   D = sum_i (L_i / N - 1/R)^2; +inf when D = 0
 *               [3] locality: sum_r S[r][r] / N
 *               all four NaN when T = 0.
 * Every count is exact (integer adds); the ratios are a few fp64 operations
 * on exact integers.                                                        */
moe_status moe_routing_stats(const moe_problem* p, const int32_t* idx, const int32_t* counts,
                             const int32_t* rank_of, int32_t* send_counts, int32_t* coselect,
                             double* stats, void* stream);

/* Token-balanced (EPLB-style) replica routing, the baseline the greedy of
 * moe_assign_replicas is compared against. [METRO] section "Add the
 * expert-weight traffic term" (balancing tokens over an expert's replicas
 * activates more replicas per GPU than grouping them; the greedy is
 * reported against EPLB's token routing).
 * The n pairs routed to expert e, in the order of e's send segment (token
 * order), are cut into contiguous shares over e's valid replicas (entries
 * of rep[e] in [0, R), in table order): with m of them, replica j takes
 * n / m pairs, plus one when j < n mod m. rep = NULL: one copy per expert,
 * on rank e / (E / R).
 *   idx            i32 [T, k] (read)   counts i32 [E] (read, from moe_route)
 *   pos            i32 [T*k] (read)    expert_offsets i32 [E] (read), both
 *                  from moe_layout (any rank order: only the place of a
 *                  pair inside its expert's segment is used)
 *   rep, maxrep    as for moe_assign_replicas
 *   gpu_of_pair    i32 [T*k] (write, or NULL to skip): the GPU serving each
 *                  pair; -1 for an expert without a valid replica
 *   active         i32 [R] (write): replicas with a non-empty share per GPU
 *   tokens         i32 [R] (write): pairs served per GPU                    */
moe_status moe_token_balanced_split(const moe_problem* p, const int32_t* idx,
                                    const int32_t* counts, const int32_t* pos,
                                    const int32_t* expert_offsets, const int32_t* rep,
                                    int32_t maxrep, int32_t* gpu_of_pair, int32_t* active,
                                    int32_t* tokens, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H */
