// Internal interface between the C ABI layer (gdn_api.cpp: validation,
// planning, workspace carving) and the HIP kernel launchers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace gdn {

// Host-side plan of one problem.  Sequences are cut into 64-token chunks
// (never crossing a sequence end) and the chunks of a sequence into
// segments of `seg_chunks` chunks, the unit of intra-GPU context parallelism.
struct Plan {
  int N = 0;
  int seg_chunks = 1;
  int64_t total_chunks = 0;  // sum over sequences of ceil(len / 64)
  int64_t total_segs = 0;    // sum over sequences of ceil(chunks / seg_chunks)
  int max_segs_per_seq = 0;
  bool has_empty = false;   // some sequence has no tokens
  int64_t total_tokens = 0;
  int cus = 256;            // compute units of the device
};

// Byte offsets of the pieces of a workspace (all 256-byte aligned).
struct FwdWorkspace {
  size_t chunk_prefix = 0;  // int32 [N+1]
  size_t seg_prefix = 0;    // int32 [N+1]
  size_t tmat = 0;          // element type [NC][Hv][64][64]: per-chunk T
  size_t hseg = 0;          // fp32 [NS][Hv][K][V]: segment end states (pass 1)
  size_t eseg = 0;          // fp32 [NS][Hv][K][V]: propagated starts (pass 2)
  size_t flags = 0;         // int32 [NS][Hv]: eseg non-zero
  size_t total = 0;
};

struct BwdWorkspace {
  FwdWorkspace fwd;  // forward state recompute (its own pieces)
  size_t hstates = 0;   // element type [NC][Hv][K*V]: state entering each chunk, lane layout (gdn_seg.hpp)
  size_t dstates = 0;   // element type [NC][Hv][K*V]: gradient of the state leaving each chunk, lane layout
  size_t dseg = 0;      // fp32 [NS][Hv][K][V]: reverse segment partials
  size_t deseg = 0;     // fp32 [NS][Hv][K][V]
  size_t dflags = 0;    // int32 [NS][Hv]
  size_t total = 0;
};

struct Problem {
  int B, T, Hq, Hv, K, V, N;
  int dtype;  // 0 fp32, 1 bf16
  float scale;
  const int32_t *cu;  // device, or null (uniform rows of T tokens)
  // in-library q/k L2 normalisation: every kernel normalises the q and k
  // rows it loads (l2n_piece) before they reach LDS
  int l2;
};

struct FwdArgs {
  Problem p;
  Plan plan;
  const void *q, *k, *v, *beta;
  const float *g, *h0;
  void *o;
  float *ht, *g_cum, *A, *h;
  void *h_e;  // per-chunk states in the element type (backward's internal copy)
  void *tm_ext = nullptr;  // per-chunk T there instead of the workspace (state cache)
  // with l2 and a state cache: prep writes the normalised q, k rows and their
  // factors here, and the passes after it read those rows
  void *qn_out = nullptr, *kn_out = nullptr;
  float *rq_out = nullptr, *rk_out = nullptr;
  char *ws;
  FwdWorkspace wl;
};

struct BwdArgs {
  Problem p;
  Plan plan;
  const void *q, *k, *v, *beta, *dout;
  const float *g, *A, *h0, *dht;
  void *dq, *dk, *dv, *dbeta;
  float *dg, *dh0;
  // set when q, k point at rows the forward normalised (state cache, l2):
  // their factors, for the chain rule of dq, dk
  const float *rq = nullptr, *rk = nullptr;
  // the forward's state cache ([chunks][Hv][K*V], element type, lane layout), or null:
  // then the states are recomputed into the workspace
  const void *hcache = nullptr;
  const void *tm_ext = nullptr;  // per-chunk T of the same cache
  char *ws;
  BwdWorkspace wl;
};

hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream);
// pass 1 of the forward with the recurrence in registers (gdn_fwd_slice.hip):
// bf16, K = V = 128
bool fwd_slice_supported(const FwdArgs &a);
hipError_t launch_fwd_slice_main(const FwdArgs &a, hipStream_t stream);
// states only (a.h), no output; T from Ain ([B,T,Hv,64] fp32) when given
hipError_t launch_bwd_prep(const FwdArgs &a, const float *Ain, hipStream_t stream);
hipError_t launch_fwd_states(const FwdArgs &a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream);
// reverse pass 1 of the backward with the gradient in registers
// (gdn_rev_slice.hip): bf16, K = V = 128
bool rev_slice_supported(const BwdArgs &a);
hipError_t launch_rev_slice_main(const BwdArgs &a, hipStream_t stream);
// local gradients on 32x32 tiles (gdn_grad_slice.hip): bf16, K = V = 128,
// q and k given normalised
bool grad_slice_supported(const BwdArgs &a);
hipError_t launch_grad_slice(const BwdArgs &a, hipStream_t stream);
// q_hat, k_hat (element type) and their per-row factors from raw q, k

// Benchmark timing: while enabled on the calling thread, each KernelTimer
// scope records a HIP event before and after the kernel launched inside it,
// on the launch stream (see gdn_timing_enable / gdn_timing_collect).
class KernelTimer {
 public:
  KernelTimer(const char *name, hipStream_t stream);
  ~KernelTimer();
  KernelTimer(const KernelTimer &) = delete;
  KernelTimer &operator=(const KernelTimer &) = delete;

 private:
  int slot_;
  hipStream_t stream_;
};
int run_selftest();

}  // namespace gdn
