// C ABI of the GDN chunked prefill: argument validation, planning (chunks,
// context-parallel segments), workspace carving and kernel dispatch.
// Validation and planning are plain host code that runs before any HIP call,
// so every error path is reachable without a GPU.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Compute units of the device the process first plans on (256 on MI355X;
// also the value used when no device can be queried).  Cached, so that the
// workspace-size query and the launch always plan alike.
int64_t device_compute_units() {
  static std::atomic<int> cached{0};
  int c = cached.load(std::memory_order_relaxed);
  if (c > 0) return c;
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      n > 0) {
    c = n;
  } else {
    (void)hipGetLastError();  // leave no error behind for the caller's next HIP call
    c = 256;
  }
  cached.store(c, std::memory_order_relaxed);
  return c;
}

bool aligned(const void *ptr, size_t a) {
  return ((uintptr_t)ptr % a) == 0;
}

// (K, V) pairs the kernels are compiled for.  fp32 tiles take twice the LDS,
// so fp32 stops at 64.
bool supported_kv(int dtype, int k, int v) {
  if (dtype == GDN_BF16)
    return (k == v && (k == 32 || k == 64 || k == 128)) || (k == 64 && v == 128) ||
           (k == 128 && v == 64);
  return (k == 32 || k == 64) && (v == 32 || v == 64);
}

// Validates the problem description; fills plan on success.
int validate(const gdn_problem_t *p, gdn::Plan *plan) {
  if (!p) return fail(GDN_ERR_INVALID_ARG, "problem descriptor is NULL");
  if (p->B <= 0 || p->T < 0 || p->Hq <= 0 || p->Hv <= 0 || p->K <= 0 || p->V <= 0)
    return fail(GDN_ERR_INVALID_ARG,
                "dimensions must be positive (B=%d T=%d Hq=%d Hv=%d K=%d V=%d)",
                p->B, p->T, p->Hq, p->Hv, p->K, p->V);
  if (p->dtype != GDN_F32 && p->dtype != GDN_BF16)
    return fail(GDN_ERR_UNSUPPORTED, "dtype %d is not GDN_F32 or GDN_BF16", p->dtype);
  if (p->Hv % p->Hq != 0)
    return fail(GDN_ERR_UNSUPPORTED, "Hv=%d is not a multiple of Hq=%d", p->Hv, p->Hq);
  if (!supported_kv(p->dtype, p->K, p->V))
    return fail(GDN_ERR_UNSUPPORTED,
                "K=%d V=%d not supported for this dtype (bf16: K == V in {32, 64, "
                "128}, (64, 128), (128, 64); fp32: K, V in {32, 64})",
                p->K, p->V);
  if (!(p->scale == p->scale)) return fail(GDN_ERR_INVALID_ARG, "scale is NaN");
  if (p->qk_l2norm != 0 && p->qk_l2norm != 1)
    return fail(GDN_ERR_INVALID_ARG, "qk_l2norm must be 0 or 1 (got %d)", p->qk_l2norm);
  gdn::Plan pl;
  int64_t maxlen = 0;
  if (p->cu_seqlens) {
    if (!p->cu_seqlens_host)
      return fail(GDN_ERR_INVALID_ARG,
                  "cu_seqlens given without its host copy cu_seqlens_host");
    if (p->B != 1)
      return fail(GDN_ERR_INVALID_ARG, "B must be 1 with cu_seqlens (got %d)", p->B);
    if (p->N <= 0) return fail(GDN_ERR_INVALID_ARG, "N must be positive (got %d)", p->N);
    const int32_t *cu = p->cu_seqlens_host;
    if (cu[0] != 0) return fail(GDN_ERR_INVALID_ARG, "cu_seqlens[0] = %d, must be 0", cu[0]);
    for (int n = 0; n < p->N; ++n) {
      if (cu[n + 1] < cu[n])
        return fail(GDN_ERR_INVALID_ARG, "cu_seqlens decreases at %d (%d -> %d)", n,
                    cu[n], cu[n + 1]);
      const int64_t len = cu[n + 1] - cu[n];
      maxlen = std::max(maxlen, len);
      if (len == 0) pl.has_empty = true;
      pl.total_chunks += (len + 63) / 64;
    }
    if (cu[p->N] != p->T)
      return fail(GDN_ERR_INVALID_ARG, "cu_seqlens[N] = %d but T = %d", cu[p->N], p->T);
    pl.N = p->N;
  } else {
    if (p->cu_seqlens_host)
      return fail(GDN_ERR_INVALID_ARG, "cu_seqlens_host given without cu_seqlens");
    if (p->N != p->B)
      return fail(GDN_ERR_INVALID_ARG, "N must equal B without cu_seqlens (N=%d B=%d)",
                  p->N, p->B);
    pl.N = p->B;
    maxlen = p->T;
    pl.has_empty = p->T == 0;
    pl.total_chunks = (int64_t)p->B * ((p->T + 63) / 64);
  }
  pl.total_tokens = (int64_t)p->B * p->T;
  if ((int64_t)p->B * p->T * std::max(p->Hq, p->Hv) * std::max(p->K, p->V) >
      ((int64_t)1 << 40))
    return fail(GDN_ERR_UNSUPPORTED, "problem too large");
  // context-parallel segment length (in chunks)
  int cp = p->cp_mode;
  if (cp == -1) {
    const char *env = getenv("GDN_CP");
    if (env && *env) cp = atoi(env);
  }
  if (cp < -1) return fail(GDN_ERR_INVALID_ARG, "cp_mode %d invalid (-1, 0 or n > 0)", cp);
  const int64_t maxchunks = (maxlen + 63) / 64;
  int64_t seg;
  if (cp == 0) {
    seg = std::max<int64_t>(maxchunks, 1);
  } else if (cp > 0) {
    seg = cp;
  } else {
    // automatic: every (segment, v-head) work item of the segment passes
    // holds one compute unit (its LDS use leaves room for one workgroup), so
    // a pass takes ceil(items / CUs) rounds of up to `seg` chunk steps each.
    // Choose the segment length with the least estimated critical path,
    // rounds x (seg + kItemCost): kItemCost is the fixed cost of one work
    // item (state load, first-chunk latency, its fix-up item) in chunk steps,
    // measured along the head-count sweep.  On ties the longer segment wins.
    // Segments shorter than 4 chunks are not considered.
    std::vector<int64_t> nc;
    if (p->cu_seqlens) {
      for (int n = 0; n < p->N; ++n)
        nc.push_back((p->cu_seqlens_host[n + 1] - p->cu_seqlens_host[n] + 63) / 64);
    } else {
      nc.assign(p->B, (p->T + 63) / 64);
    }
    const int64_t cus = device_compute_units();
    seg = std::max<int64_t>(maxchunks, 1);
    int64_t best_cost = INT64_MAX;
    for (int64_t sl = std::max<int64_t>(maxchunks, 1); sl >= std::min<int64_t>(4, maxchunks);
         --sl) {
      if (sl <= 0) break;
      int64_t items = 0;
      for (int64_t c : nc) items += (int64_t)p->Hv * ((c + sl - 1) / sl);
      constexpr int64_t kItemCost = 6;
      const int64_t cost = ((items + cus - 1) / cus) * (sl + kItemCost);
      if (cost < best_cost) {
        best_cost = cost;
        seg = sl;
      }
    }
  }
  pl.seg_chunks = (int)std::min<int64_t>(seg, 1 << 30);
  pl.cus = (int)device_compute_units();
  pl.total_segs = 0;
  pl.max_segs_per_seq = 0;
  auto add_seq = [&](int64_t len) {
    const int64_t nc = (len + 63) / 64;
    const int64_t ns = (nc + pl.seg_chunks - 1) / pl.seg_chunks;
    pl.total_segs += ns;
    pl.max_segs_per_seq = std::max<int>(pl.max_segs_per_seq, (int)ns);
  };
  if (p->cu_seqlens) {
    for (int n = 0; n < p->N; ++n) add_seq(p->cu_seqlens_host[n + 1] - p->cu_seqlens_host[n]);
  } else {
    for (int n = 0; n < p->B; ++n) add_seq(p->T);
  }
  if (pl.total_segs * p->Hv >= ((int64_t)1 << 31) ||
      pl.total_chunks * p->Hv >= ((int64_t)1 << 31))
    return fail(GDN_ERR_UNSUPPORTED, "problem too large for the launch grid");
  *plan = pl;
  return GDN_OK;
}

gdn::FwdWorkspace fwd_layout(const gdn_problem_t *p, const gdn::Plan &pl, size_t base) {
  gdn::FwdWorkspace w;
  size_t off = base;
  const size_t es = p->dtype == GDN_BF16 ? 2 : 4;
  const size_t kv = (size_t)p->K * p->V * 4;
  w.chunk_prefix = off;
  off = align256(off + (size_t)(pl.N + 1) * 4);
  w.seg_prefix = off;
  off = align256(off + (size_t)(pl.N + 1) * 4);
  w.tmat = off;
  off = align256(off + (size_t)pl.total_chunks * p->Hv * 64 * 64 * es);
  w.hseg = off;
  off = align256(off + (size_t)pl.total_segs * p->Hv * kv);
  w.eseg = off;
  off = align256(off + (size_t)pl.total_segs * p->Hv * kv);
  w.flags = off;
  off = align256(off + (size_t)pl.total_segs * p->Hv * 4);
  w.total = off;
  return w;
}

gdn::BwdWorkspace bwd_layout(const gdn_problem_t *p, const gdn::Plan &pl) {
  gdn::BwdWorkspace w;
  w.fwd = fwd_layout(p, pl, 0);
  size_t off = w.fwd.total;
  const size_t kv = (size_t)p->K * p->V * 4;
  const size_t kve = (size_t)p->K * p->V * (p->dtype == GDN_BF16 ? 2 : 4);
  w.hstates = off;
  off = align256(off + (size_t)pl.total_chunks * p->Hv * kve);
  w.dstates = off;
  off = align256(off + (size_t)pl.total_chunks * p->Hv * kve);
  w.dseg = off;
  off = align256(off + (size_t)pl.total_segs * p->Hv * kv);
  w.deseg = off;
  off = align256(off + (size_t)pl.total_segs * p->Hv * kv);
  w.dflags = off;
  off = align256(off + (size_t)pl.total_segs * p->Hv * 4);
  w.total = off;
  return w;
}

gdn::Problem to_problem(const gdn_problem_t *p) {
  gdn::Problem q;
  q.B = p->B;
  q.T = p->T;
  q.Hq = p->Hq;
  q.Hv = p->Hv;
  q.K = p->K;
  q.V = p->V;
  q.N = p->cu_seqlens ? p->N : p->B;
  q.dtype = p->dtype;
  q.scale = p->scale;
  q.cu = p->cu_seqlens;
  q.l2 = p->qk_l2norm;
  return q;
}

struct TimedLaunch {
  const char *name;
  hipEvent_t start, stop;
};
thread_local bool g_timing = false;
thread_local std::vector<TimedLaunch> g_launches;

}  // namespace

namespace gdn {

KernelTimer::KernelTimer(const char *name, hipStream_t stream) : slot_(-1), stream_(stream) {
  if (!g_timing) return;
  TimedLaunch t{name, nullptr, nullptr};
  if (hipEventCreate(&t.start) != hipSuccess) return;
  if (hipEventCreate(&t.stop) != hipSuccess) {
    (void)hipEventDestroy(t.start);
    return;
  }
  (void)hipEventRecord(t.start, stream);
  slot_ = (int)g_launches.size();
  g_launches.push_back(t);
}

KernelTimer::~KernelTimer() {
  if (slot_ >= 0) (void)hipEventRecord(g_launches[slot_].stop, stream_);
}

}  // namespace gdn

// ---- fixed device scratch of gdn_chunk_fwd_noalloc
// The workspace of the forward for callers that cannot allocate: one array
// per device, allocated with the code object and held until the process
// ends.  Every call on a device uses the same array; nothing in it has to
// start at zero (each piece a kernel reads is written earlier in the same
// call), and calls that overlap on one device race on it.
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device (the host-side name of the array is not a device address).
int scratch_of_current_device(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GDN_ERR_UNSUPPORTED, "device %d beyond the %d devices the scratch table holds",
                dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(GDN_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_timing_enable(int on) {
  const int prev = g_timing ? 1 : 0;
  g_timing = on != 0;
  return prev;
}

int gdn_timing_collect(int max_kernels, char *names, int32_t *counts, double *ms_total) {
  g_err.clear();
  std::map<std::string, std::pair<int32_t, double>> acc;
  std::vector<std::string> order;
  int rc = 0;
  for (TimedLaunch &t : g_launches) {
    float ms = 0.f;
    if (hipEventSynchronize(t.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, t.start, t.stop) != hipSuccess)
      rc = GDN_ERR_HIP;
    if (!acc.count(t.name)) order.push_back(t.name);
    auto &e = acc[t.name];
    e.first += 1;
    e.second += ms;
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  g_launches.clear();
  if (rc) return -fail(rc, "timing events could not be read");
  int n = 0;
  for (const std::string &k : order) {
    if (n >= max_kernels) break;
    if (names) {
      snprintf(names + 32 * n, 32, "%s", k.c_str());
    }
    if (counts) counts[n] = acc[k].first;
    if (ms_total) ms_total[n] = acc[k].second;
    ++n;
  }
  return n;
}


const char *gdn_last_error(void) { return g_err.c_str(); }

size_t gdn_chunk_fwd_workspace_size(const gdn_problem_t *p) {
  gdn::Plan pl;
  if (validate(p, &pl) != GDN_OK) return 0;
  return fwd_layout(p, pl, 0).total;
}

size_t gdn_chunk_bwd_workspace_size(const gdn_problem_t *p) {
  gdn::Plan pl;
  if (validate(p, &pl) != GDN_OK) return 0;
  return bwd_layout(p, pl).total;
}

// State cache layout: the per-chunk states ([chunks][Hv][K*V] in the lane layout, element
// type), then at a 256-byte boundary the per-chunk T ([chunks][Hv][64][64]).
// Byte offsets of the state cache's pieces: the states, T, and with qk_l2norm
// the normalised q, k rows and their factors.
struct CacheLayout {
  size_t t = 0, qn = 0, kn = 0, rq = 0, rk = 0, total = 0;
};
static CacheLayout cache_layout(const gdn_problem_t *p, const gdn::Plan &pl) {
  const size_t es = p->dtype == GDN_BF16 ? 2 : 4;
  CacheLayout c;
  c.t = align256((size_t)pl.total_chunks * p->Hv * p->K * p->V * es);
  size_t off = c.t + (size_t)pl.total_chunks * p->Hv * 64 * 64 * es;
  if (p->qk_l2norm) {
    const size_t rows = (size_t)pl.total_tokens * p->Hq;
    c.qn = off = align256(off);
    off += rows * p->K * es;
    c.kn = off = align256(off);
    off += rows * p->K * es;
    c.rq = off = align256(off);
    off += rows * 4;
    c.rk = off = align256(off);
    off += rows * 4;
  }
  c.total = off;
  return c;
}

size_t gdn_state_cache_size(const gdn_problem_t *p) {
  gdn::Plan pl;
  if (validate(p, &pl) != GDN_OK) return 0;
  const size_t n = cache_layout(p, pl).total;
  return n > 0 ? n : 256;  // a valid size even for an empty problem
}

int64_t gdn_plan_segments(const gdn_problem_t *p) {
  gdn::Plan pl;
  if (validate(p, &pl) != GDN_OK) return 0;
  return pl.total_segs;
}

}  // extern "C"

namespace {

// Checks of the forward's arguments other than the workspace (no HIP call).
int fwd_check(const gdn_problem_t *p, gdn::Plan *pl, const void *q, const void *k,
              const void *v, const float *g, const void *beta, const float *h0, const void *o,
              const float *ht, const float *g_cum, const float *A, const float *h,
              const void *state_cache) {
  int rc = validate(p, pl);
  if (rc != GDN_OK) return rc;
  if (pl->total_tokens > 0 && (!q || !k || !v || !g || !beta || !o))
    return fail(GDN_ERR_INVALID_ARG, "q, k, v, g, beta and o are required");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(g, 4) || !aligned(h0, 4) || !aligned(ht, 4) || !aligned(A, 16) ||
      !aligned(h, 4) || !aligned(g_cum, 4) || !aligned(state_cache, 16))
    return fail(GDN_ERR_LAYOUT,
                "q, k, v, o, A, state_cache must be 16-byte aligned; fp32 buffers 4-byte");
  return GDN_OK;
}

// The forward's launches on a checked problem and a large enough workspace.
int fwd_run(const gdn_problem_t *p, const gdn::Plan &pl, const gdn::FwdWorkspace &wl,
            const void *q, const void *k, const void *v, const float *g, const void *beta,
            const float *h0, void *o, float *ht, float *g_cum, float *A, float *h,
            void *state_cache, void *workspace, void *stream) {
  gdn::FwdArgs a;
  a.p = to_problem(p);
  a.plan = pl;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.g = g;
  a.h0 = h0;
  a.o = o;
  a.ht = ht;
  a.g_cum = g_cum;
  a.A = A;
  a.h = h;
  a.h_e = state_cache;  // the segment passes store the states they run through
  if (state_cache) {
    char *sc = static_cast<char *>(state_cache);
    const CacheLayout cl = cache_layout(p, pl);
    a.tm_ext = sc + cl.t;
    if (p->qk_l2norm && pl.total_tokens > 0) {
      a.qn_out = sc + cl.qn;
      a.kn_out = sc + cl.kn;
      a.rq_out = reinterpret_cast<float *>(sc + cl.rq);
      a.rk_out = reinterpret_cast<float *>(sc + cl.rk);
    }
  }
  a.ws = static_cast<char *>(workspace);
  a.wl = wl;
  const hipError_t e = gdn::launch_fwd(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(GDN_ERR_HIP, "forward launch failed: %s", hipGetErrorString(e));
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_chunk_fwd(const gdn_problem_t *p, const void *q, const void *k, const void *v,
                  const float *g, const void *beta, const float *h0, void *o, float *ht,
                  float *g_cum, float *A, float *h, void *state_cache, void *workspace,
                  size_t ws_bytes, void *stream) {
  g_err.clear();
  gdn::Plan pl;
  int rc = fwd_check(p, &pl, q, k, v, g, beta, h0, o, ht, g_cum, A, h, state_cache);
  if (rc != GDN_OK) return rc;
  const gdn::FwdWorkspace wl = fwd_layout(p, pl, 0);
  if (!workspace || ws_bytes < wl.total)
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", wl.total,
                workspace ? ws_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(GDN_ERR_WORKSPACE, "workspace not 256-byte aligned");
  return fwd_run(p, pl, wl, q, k, v, g, beta, h0, o, ht, g_cum, A, h, state_cache, workspace,
                 stream);
}

int gdn_chunk_bwd(const gdn_problem_t *p, const void *q, const void *k, const void *v,
                  const float *g, const void *beta, const float *A, const float *h0,
                  const void *do_, const float *dht, void *dq, void *dk, void *dv,
                  void *dbeta, float *dg, float *dh0, const void *state_cache,
                  void *workspace, size_t ws_bytes, void *stream) {
  g_err.clear();
  gdn::Plan pl;
  int rc = validate(p, &pl);
  if (rc != GDN_OK) return rc;
  if (pl.total_tokens > 0 &&
      (!q || !k || !v || !g || !beta || !do_ || !dq || !dk || !dv || !dbeta || !dg))
    return fail(GDN_ERR_INVALID_ARG,
                "q, k, v, g, beta, do, dq, dk, dv, dbeta and dg are required");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(do_, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(g, 4) ||
      !aligned(dbeta, 4) || !aligned(A, 16) || !aligned(h0, 4) || !aligned(dht, 4) ||
      !aligned(dh0, 4) || !aligned(dg, 4) || !aligned(state_cache, 16))
    return fail(GDN_ERR_LAYOUT,
                "q, k, v, do, dq, dk, dv, A, state_cache must be 16-byte aligned; "
                "dbeta and fp32 buffers 4-byte");
  const gdn::BwdWorkspace wl = bwd_layout(p, pl);
  if (!workspace || ws_bytes < wl.total)
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", wl.total,
                workspace ? ws_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(GDN_ERR_WORKSPACE, "workspace not 256-byte aligned");
  gdn::BwdArgs a;
  a.p = to_problem(p);
  a.plan = pl;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.dout = do_;
  a.g = g;
  a.A = A;
  a.h0 = h0;
  a.dht = dht;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dbeta = dbeta;
  a.dg = dg;
  a.dh0 = dh0;
  a.hcache = state_cache;
  if (state_cache) {
    const char *sc = static_cast<const char *>(state_cache);
    const CacheLayout cl = cache_layout(p, pl);
    a.tm_ext = sc + cl.t;
    if (p->qk_l2norm && pl.total_tokens > 0) {
      // the rows the forward normalised, and their factors for dq, dk
      a.q = sc + cl.qn;
      a.k = sc + cl.kn;
      a.rq = reinterpret_cast<const float *>(sc + cl.rq);
      a.rk = reinterpret_cast<const float *>(sc + cl.rk);
      a.p.l2 = 0;
    }
  }
  a.ws = static_cast<char *>(workspace);
  a.wl = wl;
  const hipError_t e = gdn::launch_bwd(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(GDN_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return GDN_OK;
}

size_t gdn_chunk_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

int gdn_chunk_fwd_noalloc(const gdn_problem_t *p, const void *q, const void *k, const void *v,
                          const float *g, const void *beta, const float *h0, void *o,
                          float *ht, float *g_cum, float *A, float *h, void *state_cache,
                          void *stream) {
  g_err.clear();
  gdn::Plan pl;
  int rc = fwd_check(p, &pl, q, k, v, g, beta, h0, o, ht, g_cum, A, h, state_cache);
  if (rc != GDN_OK) return rc;
  const gdn::FwdWorkspace wl = fwd_layout(p, pl, 0);
  if (wl.total > kScratchBytes)
    return fail(GDN_ERR_WORKSPACE,
                "problem needs %zu bytes of scratch; the fixed scratch of "
                "gdn_chunk_fwd_noalloc holds %zu (use gdn_chunk_fwd with a workspace)",
                wl.total, kScratchBytes);
  void *ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc != GDN_OK) return rc;
  return fwd_run(p, pl, wl, q, k, v, g, beta, h0, o, ht, g_cum, A, h, state_cache, ws, stream);
}

int gdn_selftest(void) {
  g_err.clear();
  int rc = gdn::run_selftest();
  if (rc != 0) return fail(GDN_ERR_HIP, "MFMA self-test failed (code %d)", rc);
  return GDN_OK;
}

}  // extern "C"
