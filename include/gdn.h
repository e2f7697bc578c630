/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated delta rule chunked prefill.
 *
 * The operator is the GDN ("Gated Delta Rule") chunked prefill that the
 * FlashQLA pages describe: the FlashQLA article's "高级 API 示例" section
 * (chunk_gated_delta_rule(q, k, v, g, beta, scale, initial_state,
 * output_final_state, cu_seqlens) -> (o, final_state)) and its "底层 API"
 * section (chunk_gated_delta_rule_fwd -> (g, A, o, h, final_state) and
 * chunk_gated_delta_rule_bwd(q, k, v, g, beta, A, do, dht, scale,
 * initial_state, cu_seqlens) -> (dq, dk, dv, db, dg, dh0)).  The pages print
 * the signatures and the input shapes only.  The recurrence computed, per
 * sequence n and v-head h, with the state S stored K x V (fp32):
 *
 *   S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *   o_t = scale * S_t^T q_t
 *
 * with S_{-1} = initial_state[n, h] (or 0) and final_state[n, h] = the last
 * S.  v-head h reads q/k head h / (Hv / Hq).
 *
 * Layouts (all row-major, contiguous, device memory unless stated):
 *   q, k        [B, T, Hq, K]      dtype of the problem (GDN_F32 or GDN_BF16)
 *   v, o, do    [B, T, Hv, V]      problem dtype
 *   beta        [B, T, Hv]         problem dtype
 *   g           [B, T, Hv]         fp32, the raw log-gate (decay = exp(g))
 *   initial_state, final_state, dht, dh0
 *               [N, Hv, K, V]      fp32
 *   g_cum       [B, T, Hv]         fp32, gate cumsum inside each 64-token chunk
 *   A           [B, T, Hv, 64]     fp32, per chunk the unit-lower-triangular
 *                                  T = (I + strict_lower(diag(beta) K K^T *
 *                                  exp(gamma_r - gamma_j)))^-1; row r of a
 *                                  chunk is stored at that row's token
 *   h           [NC, Hv, K, V]     fp32, state entering each chunk; NC is the
 *                                  total chunk count (sum over sequences of
 *                                  ceil(len / 64)), chunks numbered in token
 *                                  order
 *   dq, dk      [B, T, Hq, K]      problem dtype (summed over each q/k group)
 *   dv          [B, T, Hv, V], dbeta [B, T, Hv]: problem dtype; dg [B,T,Hv] fp32
 * With cu_seqlens, B must be 1, T is the total packed length and sequence n
 * covers tokens [cu[n], cu[n+1]); chunks never cross sequences.
 * Alignment: q, k, v, o, A, state_cache (forward) and q, k, v, do, dq, dk,
 * dv, A, state_cache (backward) 16 bytes (they are read or written 16 bytes
 * a lane); every other buffer 4 bytes; the workspace 256 bytes.
 *
 * Ownership: every buffer belongs to the caller.  The operator calls
 * (gdn_chunk_fwd, gdn_chunk_bwd) allocate no device memory; their scratch
 * comes from the caller's workspace (size from the *_workspace_size calls,
 * 256-byte aligned).  The one exception in the library is the diagnostic
 * gdn_selftest, which allocates, synchronises on and frees three small
 * device buffers of its own.  The library keeps no state between calls
 * apart from the thread-local error message.
 *
 * Asynchrony: work is enqueued on `stream` (a hipStream_t, NULL = default
 * stream) and the call returns without waiting for it.  No host
 * synchronisation happens inside.
 *
 * Errors: a non-zero return means nothing was enqueued (validation errors)
 * or a launch failed (GDN_ERR_HIP); gdn_last_error() then describes it.
 * Nothing is thrown across this boundary.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype_t;

enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = 1, /* null required pointer, bad dims, bad cu_seqlens */
  GDN_ERR_UNSUPPORTED = 2, /* Hv % Hq != 0, K or V not in {32, 64, 128}, dtype */
  GDN_ERR_LAYOUT = 3,      /* pointer not aligned as documented below */
  GDN_ERR_WORKSPACE = 4,   /* workspace missing, too small or misaligned */
  GDN_ERR_HIP = 5          /* a HIP launch or runtime call failed */
};

typedef struct {
  int32_t B, T, Hq, Hv, K, V; /* T = total packed tokens when cu_seqlens set */
  int32_t N;                  /* sequences: B, or len(cu_seqlens) - 1 */
  int32_t dtype;              /* gdn_dtype_t */
  float scale;                /* output scale; callers usually pass K^-0.5 */
  const int32_t *cu_seqlens;      /* device [N+1] or NULL */
  const int32_t *cu_seqlens_host; /* host copy of the same; required iff
                                     cu_seqlens != NULL (sizes the launch
                                     without a device->host read) */
  int32_t cp_mode; /* intra-GPU context parallelism: -1 automatic, 0 off,
                      n > 0 = split sequences into segments of n chunks */
  int32_t qk_l2norm; /* 1: every q and k row (one token, one q/k head) is
                        L2-normalised inside the library before use,
                        x * (sum x^2 + 1e-6)^-1/2 (the pages state no such
                        step; it is the plain reading of the upstream q/k
                        normalisation), and dq, dk are gradients with respect
                        to the raw q, k.  0: q, k are used as given. */
} gdn_problem_t;

/* Workspace bytes gdn_chunk_fwd / gdn_chunk_bwd need for this problem
 * (0 if the problem is invalid; gdn_last_error() says why). */
size_t gdn_chunk_fwd_workspace_size(const gdn_problem_t *p);
size_t gdn_chunk_bwd_workspace_size(const gdn_problem_t *p);

/* Bytes of the state cache of this problem (0 if invalid).  The cache is an
 * opaque hand-over from gdn_chunk_fwd to gdn_chunk_bwd, the memory-for-
 * compute trade of training: it holds the state entering every chunk (in the
 * element type, K * V elements per chunk and v-head, [chunks][Hv] in token
 * order, each state in the library's internal element order) and every
 * chunk's T = (I + A)^-1 (element type, [chunks][Hv][64][64], at the next
 * 256-byte boundary).  With qk_l2norm it also holds the normalised q and k
 * rows (element type, [tokens][Hq][K] each) and their factors
 * (sum x^2 + 1e-6)^-1/2 (fp32, [tokens][Hq] for q, then for k), each piece
 * at the next 256-byte boundary: the forward normalises every row once and
 * the backward reads the rows back.  With the cache the backward neither
 * recomputes those states nor rebuilds T, and ignores its A argument. */
size_t gdn_state_cache_size(const gdn_problem_t *p);

/* Forward (chunk_gated_delta_rule_fwd of the FlashQLA article, "底层 API").
 * Required: q k v g beta o.  Optional (NULL = not wanted / absent):
 * h0 (initial state, else zero), ht (final state = output_final_state),
 * g_cum, A, h (per-chunk entering states, the training-mode extras),
 * state_cache (gdn_state_cache_size bytes, 16-byte aligned, filled for the
 * backward). */
int gdn_chunk_fwd(const gdn_problem_t *p, const void *q, const void *k,
                  const void *v, const float *g, const void *beta,
                  const float *h0, void *o, float *ht, float *g_cum, float *A,
                  float *h, void *state_cache, void *workspace, size_t ws_bytes,
                  void *stream);

/* Backward (chunk_gated_delta_rule_bwd of the same section).  g is the raw
 * log-gate; dg is with respect to it.  A (as written by gdn_chunk_fwd) is
 * optional: NULL recomputes it.  h0 and dht are optional (zero), dh0 is
 * optional output.  state_cache is optional: the cache a gdn_chunk_fwd of
 * the same problem, inputs and h0 filled (then the per-chunk states are not
 * recomputed; NULL recomputes them).  Required: q k v g beta do dq dk dv
 * dbeta dg. */
int gdn_chunk_bwd(const gdn_problem_t *p, const void *q, const void *k,
                  const void *v, const float *g, const void *beta,
                  const float *A, const float *h0, const void *do_,
                  const float *dht, void *dq, void *dk, void *dv, void *dbeta,
                  float *dg, float *dh0, const void *state_cache,
                  void *workspace, size_t ws_bytes, void *stream);

/* gdn_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Its scratch is a fixed device array of
 * gdn_chunk_fwd_noalloc_max_bytes() bytes (128 MiB) inside the library, one
 * per device, allocated with the library's code object and held until the
 * process ends; the call itself allocates nothing.  Arguments, layouts and
 * results are those of gdn_chunk_fwd.  A problem whose workspace
 * (gdn_chunk_fwd_workspace_size) exceeds the fixed size is rejected with
 * GDN_ERR_WORKSPACE before anything is enqueued.  Every call on one device
 * shares that device's array: calls that may overlap on one device (other
 * streams, other threads) race and must be serialised by the caller. */
int gdn_chunk_fwd_noalloc(const gdn_problem_t *p, const void *q,
                          const void *k, const void *v, const float *g,
                          const void *beta, const float *h0, void *o,
                          float *ht, float *g_cum, float *A, float *h,
                          void *state_cache, void *stream);
size_t gdn_chunk_fwd_noalloc_max_bytes(void);

/* Number of context-parallel segments the forward would launch for this
 * problem (host-only planning query; 0 if invalid). */
int64_t gdn_plan_segments(const gdn_problem_t *p);

/* Kernel timing for benchmarks.  While enabled on the calling thread, every
 * kernel the library enqueues is bracketed by a pair of HIP events recorded
 * on the same stream (no host synchronisation).  gdn_timing_collect() waits
 * for the recorded events, writes for each distinct kernel name (in first
 * launch order, at most max_kernels): the name (NUL-terminated, 32 bytes per
 * entry in `names`), the number of launches and their summed duration in
 * milliseconds; it then forgets the record.  Returns the number of entries,
 * or a negative error code.  Any output pointer may be NULL. */
int gdn_timing_enable(int on); /* returns the previous setting */
int gdn_timing_collect(int max_kernels, char *names, int32_t *counts,
                       double *ms_total);

/* Thread-local description of the last non-zero return ("" if none). */
const char *gdn_last_error(void);

/* Runs the library's MFMA lane-layout self-check on the current device:
 * 0 when the bf16 and fp32 matrix instructions give the products the
 * kernels assume, GDN_ERR_HIP otherwise.  Diagnostics only: unlike the
 * operator calls it allocates (and frees) its own small device buffers and
 * waits for the device before it returns. */
int gdn_selftest(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
