// Forward kernels of the GDN chunked prefill for gfx950.
//
// The FlashQLA pages describe the method only in words: a chunked prefill of
// the gated delta rule whose forward returns a processed gate g, a matrix A,
// o, per-chunk states h and the final state (FlashQLA article, "底层 API"),
// built from a few medium-grained fused kernels rather than one kernel per
// step or one monolithic kernel (same article, "FlashQLA 架构图"; aiwebcool
// "flashqla-resource", section 三, third feature), with an exact algebraic
// reformulation (section 三, second feature) and a gate-driven automatic
// split of long sequences across the compute units (section 三, first
// feature).  The kernels here are this library's own design for CDNA4.
//
// Per 64-token chunk of one (sequence, v-head), with entering state S
// (K x V, fp32) and gamma = inclusive cumsum of g inside the chunk:
//   A  = strict_lower(diag(beta) K K^T * exp(gamma_r - gamma_j))
//   T  = (I + A)^-1                         (prep kernel, chunk-parallel)
//   R  = diag(beta) (V - diag(exp(gamma)) K S)
//   Vn = T R                                (= u - w S of the WY form)
//   O  = scale (diag(exp(gamma)) Q S + lower_incl(Q K^T * E) Vn)
//   S' = exp(gamma_L) S + K^T diag(exp(gamma_L - gamma)) Vn
// Folding w S and u into one product T R is exact: w = T diag(beta e^gamma) K
// and u = T diag(beta) V, so u - w S = T (diag(beta)(V - diag(e^gamma) K S)).
//
// Context parallelism: the chunks of a sequence are cut into segments.
//   pass 1 (segment_kernel<kMain>): every segment runs from a zero state
//          (segment 0 from the initial state), writing O and its end state H.
//   pass 2 (segment_kernel<kFix>): segment j >= 1 propagates D = H_{j-1}
//          through its chunks with the homogeneous recurrence (v = 0) and adds
//          the resulting output corrections; it stops as soon as D is exactly
//          zero (the gates decay it geometrically), recording the leftover
//          E_j otherwise.
//   pass 3 (serial_kernel): per (sequence, head), carries the remaining
//          residual rho_{j+1} = E_j + Phi_j(rho_j) through the segments and
//          writes the final state H_last + rho.  Every step is exact by
//          linearity of the recurrence in the state.
#include "gdn_common.hpp"
#include "gdn_internal.h"

namespace gdn {

struct SeqInfo {
  int64_t tok0;
  int len;
  int nchunks;
};

__device__ __forceinline__ SeqInfo seq_info(const Problem &p, int n) {
  SeqInfo s;
  if (p.cu) {
    s.tok0 = p.cu[n];
    s.len = p.cu[n + 1] - p.cu[n];
  } else {
    s.tok0 = (int64_t)n * p.T;
    s.len = p.T;
  }
  s.nchunks = (s.len + kChunk - 1) / kChunk;
  return s;
}

// ------------------------------------------------------------------- plan
// Chunk and segment prefix sums over sequences (one thread; N is small).
__global__ void plan_kernel(Problem p, int seg_chunks, int32_t *chunk_prefix,
                            int32_t *seg_prefix) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  int32_t c = 0, s = 0;
  chunk_prefix[0] = 0;
  seg_prefix[0] = 0;
  for (int n = 0; n < p.N; ++n) {
    const int len = p.cu ? p.cu[n + 1] - p.cu[n] : p.T;
    const int nc = (len + kChunk - 1) / kChunk;
    c += nc;
    s += (nc + seg_chunks - 1) / seg_chunks;
    chunk_prefix[n + 1] = c;
    seg_prefix[n + 1] = s;
  }
}

// ------------------------------------------------------------------- prep
// One wavefront per (chunk, v-head): gate cumsum, the strictly lower
// beta * K K^T * decay matrix (MFMA), and its unit-lower-triangular inverse
// by forward substitution with one lane per column (fp32).
template <typename E, int K>
struct PrepCfg {
  static constexpr int PAD = 16 / (int)sizeof(E);
  static constexpr int LDK = K + PAD;
  static constexpr int LDA = 68;
  static constexpr int bytesK = 64 * LDK * (int)sizeof(E);
  static constexpr int bytesA = 64 * LDA * 4;
  static constexpr int bytes = bytesK > bytesA ? bytesK : bytesA;
};

template <typename E, int K>
__global__ __launch_bounds__(64) void prep_kernel(FwdArgs a) {
  using C = PrepCfg<E, K>;
  using M = Mma<E>;
  __shared__ __attribute__((aligned(16))) char smem[C::bytes];
  __shared__ float sGam[64], sBet[64];
  E *sK = reinterpret_cast<E *>(smem);
  float *sA = reinterpret_cast<float *>(smem);
  const Problem &p = a.p;
  const int lane = threadIdx.x;
  const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
  const int h = (int)(wid % p.Hv);
  const int64_t gid = wid / p.Hv;
  const int32_t *chunk_prefix =
      reinterpret_cast<const int32_t *>(a.ws + a.wl.chunk_prefix);
  const int n = find_seq(chunk_prefix, p.N, gid);
  const SeqInfo si = seq_info(p, n);
  const int c = (int)(gid - chunk_prefix[n]);
  const int64_t tok0 = si.tok0 + (int64_t)c * kChunk;
  const int rows = min(kChunk, si.len - c * kChunk);
  const int hq = h / (p.Hv / p.Hq);

  const E *kp = reinterpret_cast<const E *>(a.k);
  constexpr int VEC = 16 / (int)sizeof(E);
  constexpr int PR = K / VEC;
#pragma unroll
  for (int m = 0; m < PR; ++m) {
    const int idx = lane + 64 * m;
    const int r = idx / PR, cv = idx % PR;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (r < rows)
      val = *reinterpret_cast<const uint4 *>(kp + ((tok0 + r) * p.Hq + hq) * K +
                                             cv * VEC);
    *reinterpret_cast<uint4 *>(sK + r * C::LDK + cv * VEC) = val;
  }
  const int64_t gi = (tok0 + lane) * p.Hv + h;
  const float gv = lane < rows ? a.g[gi] : 0.f;
  const float bv =
      lane < rows ? to_f32(reinterpret_cast<const E *>(a.beta)[gi]) : 0.f;
  const float gam = wave_incl_scan(gv);
  sGam[lane] = gam;
  sBet[lane] = bv;
  __syncthreads();

  const int lr = lane & 15, lg = lane >> 4;
  f32x4 acc[10];
  {
    int t = 0;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct <= rt; ++ct) {
        f32x4 s = zero4();
#pragma unroll
        for (int ks = 0; ks < K / M::KS; ++ks) {
          auto x = M::ld(sK + (16 * rt + lr) * C::LDK + ks * M::KS + M::EPL * lg);
          auto y = M::ld(sK + (16 * ct + lr) * C::LDK + ks * M::KS + M::EPL * lg);
          s = M::mma(x, y, s);
        }
        acc[t++] = s;
      }
  }
  __syncthreads();  // sA aliases sK
  {
    int t = 0;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int j = 16 * ct + lr;
        const float gj = sGam[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * lg + i;
          float val = 0.f;
          if (ct <= rt && j < r) val = sBet[r] * expf(sGam[r] - gj) * acc[t][i];
          sA[r * C::LDA + j] = val;
        }
        if (ct <= rt) ++t;
      }
  }
  __syncthreads();

  // x = column `lane` of T = (I + A)^-1:  x_r = delta_{r,lane} - sum_{j<r} A_rj x_j
  float x[64];
#pragma unroll
  for (int r = 0; r < 64; ++r) x[r] = (r == lane) ? 1.f : 0.f;
#pragma unroll
  for (int r = 1; r < 64; ++r) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < r; j += 4) {
      const float4 a4 = *reinterpret_cast<const float4 *>(sA + r * C::LDA + j);
      s += a4.x * x[j];
      s += a4.y * x[j + 1];
      s += a4.z * x[j + 2];
      s += a4.w * x[j + 3];
    }
    x[r] -= s;
  }

  E *tm = reinterpret_cast<E *>(a.ws + a.wl.tmat) + (gid * p.Hv + h) * 64 * 64;
#pragma unroll
  for (int r = 0; r < 64; ++r) tm[r * 64 + lane] = from_f32<E>(x[r]);
  if (a.A) {
#pragma unroll
    for (int r = 0; r < 64; ++r)
      if (r < rows) a.A[((tok0 + r) * p.Hv + h) * 64 + lane] = x[r];
  }
  if (a.g_cum && lane < rows) a.g_cum[gi] = gam;
}

// ------------------------------------------------------ segment machinery
enum { kMain = 0, kFix = 1 };

template <typename E, int K, int V>
struct SegCfg {
  static constexpr int PAD = 16 / (int)sizeof(E);
  static constexpr int LDK = K + PAD;  // rows of length K (Q, K, S^T)
  static constexpr int LDV = V + PAD;  // rows of length V (V)
  static constexpr int LDC = 64 + PAD; // rows of length 64 (T, P, R^T, Vn^T)
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + 64 * LDK;
  static constexpr int oV = oK + 64 * LDK;
  static constexpr int oSt = oV + 64 * LDV;
  static constexpr int oT = oSt + V * LDK;
  static constexpr int oP = oT + 64 * LDC;
  static constexpr int oRt = oP + 64 * LDC;
  static constexpr int oVnt = oRt + V * LDC;
  static constexpr int nE = oVnt + V * LDC;
  static constexpr int bytes = nE * (int)sizeof(E);
  // state tile ownership: wave w holds RTW x CTW 16x16 tiles of S
  static constexpr int NCT = V / 16;
  static constexpr int RTW = K >= 64 ? K / 64 : 1;
  static constexpr int CTW = K >= 64 ? NCT : NCT / 2;
  static constexpr int NTS = RTW * CTW;
  __device__ static int rt0(int w) { return K >= 64 ? w * RTW : (w & 1); }
  __device__ static int ct0(int w) { return K >= 64 ? 0 : (w >> 1) * CTW; }
  // register prefetch of one chunk (16-byte pieces per thread)
  static constexpr int VEC = 16 / (int)sizeof(E);
  static constexpr int NQ = 64 * K / VEC / 256;
  static constexpr int NV = 64 * V / VEC / 256;
  static constexpr int NTM = 64 * 64 / VEC / 256;
};

template <typename E, int K, int V>
struct Pref {
  using C = SegCfg<E, K, V>;
  uint4 q[C::NQ], k[C::NQ], v[C::NV], t[C::NTM];
  float g, b;
  int rows;
};

struct Lds {
  char *base;
  float *sGam, *sEg, *sDec, *sBet;
  int *sFlag;
};

template <typename E, int K, int V, int MODE>
__device__ __forceinline__ void pref_load(Pref<E, K, V> &pf, const FwdArgs &a,
                                 int64_t tok0, int rows, int h, int64_t cgid) {
  using C = SegCfg<E, K, V>;
  const Problem &p = a.p;
  const int tid = threadIdx.x;
  const int hq = h / (p.Hv / p.Hq);
  const E *qp = reinterpret_cast<const E *>(a.q);
  const E *kp = reinterpret_cast<const E *>(a.k);
  const E *vp = reinterpret_cast<const E *>(a.v);
  constexpr int PK = K / C::VEC, PV = V / C::VEC;
  pf.rows = rows;
#pragma unroll
  for (int m = 0; m < C::NQ; ++m) {
    const int idx = tid + 256 * m;
    const int r = idx / PK, cv = idx % PK;
    uint4 z = make_uint4(0u, 0u, 0u, 0u), zq = z;
    if (r < rows) {
      const int64_t off = ((tok0 + r) * p.Hq + hq) * K + cv * C::VEC;
      zq = *reinterpret_cast<const uint4 *>(qp + off);
      z = *reinterpret_cast<const uint4 *>(kp + off);
    }
    pf.q[m] = zq;
    pf.k[m] = z;
  }
  if (MODE == kMain) {
#pragma unroll
    for (int m = 0; m < C::NV; ++m) {
      const int idx = tid + 256 * m;
      const int r = idx / PV, cv = idx % PV;
      uint4 z = make_uint4(0u, 0u, 0u, 0u);
      if (r < rows)
        z = *reinterpret_cast<const uint4 *>(vp + ((tok0 + r) * p.Hv + h) * V +
                                             cv * C::VEC);
      pf.v[m] = z;
    }
  }
  const E *tm = reinterpret_cast<const E *>(a.ws + a.wl.tmat) + (cgid * p.Hv + h) * 64 * 64;
#pragma unroll
  for (int m = 0; m < C::NTM; ++m)
    pf.t[m] = *reinterpret_cast<const uint4 *>(tm + (tid + 256 * m) * C::VEC);
  pf.g = 0.f;
  pf.b = 0.f;
  if (tid < 64 && tid < rows) {
    const int64_t gi = (tok0 + tid) * p.Hv + h;
    pf.g = a.g[gi];
    pf.b = to_f32(reinterpret_cast<const E *>(a.beta)[gi]);
  }
}

template <typename E, int K, int V, int MODE>
__device__ __forceinline__ void pref_commit(const Pref<E, K, V> &pf, const Lds &L) {
  using C = SegCfg<E, K, V>;
  E *sm = reinterpret_cast<E *>(L.base);
  const int tid = threadIdx.x;
  constexpr int PK = K / C::VEC, PV = V / C::VEC;
#pragma unroll
  for (int m = 0; m < C::NQ; ++m) {
    const int idx = tid + 256 * m;
    const int r = idx / PK, cv = idx % PK;
    *reinterpret_cast<uint4 *>(sm + C::oQ + r * C::LDK + cv * C::VEC) = pf.q[m];
    *reinterpret_cast<uint4 *>(sm + C::oK + r * C::LDK + cv * C::VEC) = pf.k[m];
  }
  if (MODE == kMain) {
#pragma unroll
    for (int m = 0; m < C::NV; ++m) {
      const int idx = tid + 256 * m;
      const int r = idx / PV, cv = idx % PV;
      *reinterpret_cast<uint4 *>(sm + C::oV + r * C::LDV + cv * C::VEC) = pf.v[m];
    }
  }
  constexpr int PT = 64 / C::VEC;
#pragma unroll
  for (int m = 0; m < C::NTM; ++m) {
    const int idx = tid + 256 * m;
    const int r = idx / PT, cv = idx % PT;
    *reinterpret_cast<uint4 *>(sm + C::oT + r * C::LDC + cv * C::VEC) = pf.t[m];
  }
  if (tid < 64) {
    const float gam = wave_incl_scan(pf.g);
    const float gL = __shfl(gam, 63, 64);
    L.sGam[tid] = gam;
    L.sEg[tid] = expf(gam);
    L.sDec[tid] = expf(gL - gam);
    L.sBet[tid] = pf.b;
  }
}

// Write the bf16/fp32 copy of the state (as S^T) into LDS for the products.
template <typename E, int K, int V>
__device__ __forceinline__ void state_to_lds(const TileArr<SegCfg<E, K, V>::NTS> &sacc,
                                    const Lds &L) {
  using C = SegCfg<E, K, V>;
  E *sSt = reinterpret_cast<E *>(L.base) + C::oSt;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int a = 0; a < C::RTW; ++a)
#pragma unroll
    for (int b = 0; b < C::CTW; ++b) {
      const int rt = C::rt0(w) + a, ct = C::ct0(w) + b;
      const f32x4 s = sacc[a * C::CTW + b];
      st4(sSt + (16 * ct + lr) * C::LDK + 16 * rt + 4 * lg, s[0], s[1], s[2], s[3]);
    }
}

// Global fp32 [K][V] <-> tile registers.
template <typename E, int K, int V>
__device__ __forceinline__ void load_state(TileArr<SegCfg<E, K, V>::NTS> &sacc,
                                  const float *src) {
  using C = SegCfg<E, K, V>;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int a = 0; a < C::RTW; ++a)
#pragma unroll
    for (int b = 0; b < C::CTW; ++b) {
      const int rt = C::rt0(w) + a, ct = C::ct0(w) + b;
      f32x4 s = zero4();
      if (src) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = src[(16 * rt + 4 * lg + i) * V + 16 * ct + lr];
      }
      sacc[a * C::CTW + b] = s;
    }
}

template <typename E, int K, int V>
__device__ __forceinline__ void store_state(const TileArr<SegCfg<E, K, V>::NTS> &sacc,
                                   float *dst, const float *add, bool accumulate) {
  using C = SegCfg<E, K, V>;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int a = 0; a < C::RTW; ++a)
#pragma unroll
    for (int b = 0; b < C::CTW; ++b) {
      const int rt = C::rt0(w) + a, ct = C::ct0(w) + b;
      const f32x4 s = sacc[a * C::CTW + b];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t off = (16 * rt + 4 * lg + i) * V + 16 * ct + lr;
        float x = s[i];
        if (add) x += add[off];
        if (accumulate) x += dst[off];
        dst[off] = x;
      }
    }
}

template <typename E, int K, int V>
__device__ __forceinline__ bool state_any_nonzero(const TileArr<SegCfg<E, K, V>::NTS> &sacc) {
  using C = SegCfg<E, K, V>;
  bool nz = false;
#pragma unroll
  for (int m = 0; m < C::NTS; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) nz |= (sacc[m][i] != 0.f);
  return nz;
}

// Runs chunks [c_begin, c_end) of one (sequence, v-head) starting from the
// state in sacc.  kMain: normal recurrence, O written.  kFix: homogeneous
// recurrence (v = 0), O incremented, stops early once the state is exactly
// zero.  h (optional) receives (kMain) or accumulates (kFix) the state
// entering each chunk.  Returns true when a kFix run ended on a zero state.
template <typename E, int K, int V, int MODE, bool WRITE_O>
__device__ __forceinline__ bool run_chunks(const FwdArgs &a, const Lds &L,
                           TileArr<SegCfg<E, K, V>::NTS> &sacc, const SeqInfo &si,
                           int64_t chunk_gid0, int c_begin, int c_end, int h) {
  using C = SegCfg<E, K, V>;
  using M = Mma<E>;
  constexpr int KS = M::KS, EPL = M::EPL;
  constexpr int NKK = K / KS;   // k-steps over the key dimension
  constexpr int NKC = 64 / KS;  // k-steps over the chunk dimension
  constexpr int NCT = C::NCT;
  const Problem &p = a.p;
  E *sm = reinterpret_cast<E *>(L.base);
  const E *sQ = sm + C::oQ;
  const E *sK = sm + C::oK;
  const E *sV = sm + C::oV;
  const E *sSt = sm + C::oSt;
  const E *sT = sm + C::oT;
  E *sP = sm + C::oP;
  E *sRt = sm + C::oRt;
  E *sVnt = sm + C::oVnt;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const float scale = p.scale;
  E *op = reinterpret_cast<E *>(a.o);

  Pref<E, K, V> pf;
  if (c_begin >= c_end) return MODE == kFix ? !state_any_nonzero<E, K, V>(sacc) : false;
  {
    const int rows = min(kChunk, si.len - c_begin * kChunk);
    pref_load<E, K, V, MODE>(pf, a, si.tok0 + (int64_t)c_begin * kChunk, rows, h,
                             chunk_gid0 + c_begin);
    pref_commit<E, K, V, MODE>(pf, L);
    state_to_lds<E, K, V>(sacc, L);
  }
  __syncthreads();
  bool zero_exit = false;
  for (int c = c_begin; c < c_end && !zero_exit; ++c) {
    const int64_t tok0 = si.tok0 + (int64_t)c * kChunk;
    const int rows = pf.rows;
    if (a.h) {
      float *hs = a.h + ((chunk_gid0 + c) * p.Hv + h) * (int64_t)K * V;
      store_state<E, K, V>(sacc, hs, nullptr, MODE == kFix);
    }
    // ---- phase A: Q K^T, Q S, K S for the wave's 16 chunk rows
    typename M::frag qa[NKK], ka[NKK];
#pragma unroll
    for (int ks = 0; ks < NKK; ++ks) {
      qa[ks] = M::ld(sQ + (16 * w + lr) * C::LDK + ks * KS + EPL * lg);
      ka[ks] = M::ld(sK + (16 * w + lr) * C::LDK + ks * KS + EPL * lg);
    }
    f32x4 qs[NCT], kss[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 x = zero4(), y = zero4();
#pragma unroll
      for (int ks = 0; ks < NKK; ++ks) {
        const auto b = M::ld(sSt + (16 * ct + lr) * C::LDK + ks * KS + EPL * lg);
        if (WRITE_O) x = M::mma(qa[ks], b, x);
        y = M::mma(ka[ks], b, y);
      }
      qs[ct] = x;
      kss[ct] = y;
    }
    float eg_r[4], b_r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * lg + i;
      eg_r[i] = L.sEg[r];
      b_r[i] = L.sBet[r];
    }
    if (WRITE_O) {
      float gam_r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) gam_r[i] = L.sGam[16 * w + 4 * lg + i];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        f32x4 x = zero4();
        if (ct <= w) {
#pragma unroll
          for (int ks = 0; ks < NKK; ++ks)
            x = M::mma(qa[ks], M::ld(sK + (16 * ct + lr) * C::LDK + ks * KS + EPL * lg), x);
        }
        const int j = 16 * ct + lr;
        const float gj = L.sGam[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * w + 4 * lg + i;
          const float val = (ct <= w && j <= r) ? x[i] * expf(gam_r[i] - gj) : 0.f;
          sP[r * C::LDC + j] = from_f32<E>(val);
        }
      }
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int vc = 16 * ct + lr;
      float rr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * lg + i;
        const float vv = MODE == kMain ? to_f32(sV[r * C::LDV + vc]) : 0.f;
        rr[i] = b_r[i] * (vv - eg_r[i] * kss[ct][i]);
      }
      st4(sRt + vc * C::LDC + 16 * w + 4 * lg, rr[0], rr[1], rr[2], rr[3]);
    }
    __syncthreads();
    // next chunk's inputs travel while phases B and C run
    if (c + 1 < c_end) {
      const int rows1 = min(kChunk, si.len - (c + 1) * kChunk);
      pref_load<E, K, V, MODE>(pf, a, tok0 + kChunk, rows1, h, chunk_gid0 + c + 1);
    }
    // ---- phase B: Vn = T R
    {
      typename M::frag ta[NKC];
#pragma unroll
      for (int ks = 0; ks < NKC; ++ks)
        ta[ks] = M::ld(sT + (16 * w + lr) * C::LDC + ks * KS + EPL * lg);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 x = zero4();
#pragma unroll
        for (int ks = 0; ks < NKC; ++ks)
          x = M::mma(ta[ks], M::ld(sRt + (16 * ct + lr) * C::LDC + ks * KS + EPL * lg), x);
        st4(sVnt + (16 * ct + lr) * C::LDC + 16 * w + 4 * lg, x[0], x[1], x[2], x[3]);
      }
    }
    __syncthreads();
    // ---- phase C: output rows of this wave, state update of its tiles
    if (WRITE_O) {
      typename M::frag pa[NKC];
#pragma unroll
      for (int ks = 0; ks < NKC; ++ks)
        pa[ks] = M::ld(sP + (16 * w + lr) * C::LDC + ks * KS + EPL * lg);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 x = qs[ct];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] *= eg_r[i];
#pragma unroll
        for (int ks = 0; ks < NKC; ++ks)
          x = M::mma(pa[ks], M::ld(sVnt + (16 * ct + lr) * C::LDC + ks * KS + EPL * lg), x);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * w + 4 * lg + i;
          if (r < rows) {
            E *dst = op + ((tok0 + r) * p.Hv + h) * V + 16 * ct + lr;
            float val = scale * x[i];
            if (MODE == kFix) val += to_f32(*dst);
            *dst = from_f32<E>(val);
          }
        }
      }
    }
    {
      const float egL = L.sEg[63];
      typename M::frag ka2[C::RTW][NKC];
#pragma unroll
      for (int aa = 0; aa < C::RTW; ++aa)
#pragma unroll
        for (int ks = 0; ks < NKC; ++ks) {
          const int t0 = ks * KS + EPL * lg;
          ka2[aa][ks] = M::ld_strided_scaled(sK + t0 * C::LDK + 16 * (C::rt0(w) + aa) + lr,
                                             C::LDK, L.sDec + t0);
        }
#pragma unroll
      for (int aa = 0; aa < C::RTW; ++aa)
#pragma unroll
        for (int bb = 0; bb < C::CTW; ++bb) {
          const int ct = C::ct0(w) + bb;
          f32x4 x = sacc[aa * C::CTW + bb];
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] *= egL;
#pragma unroll
          for (int ks = 0; ks < NKC; ++ks)
            x = M::mma(ka2[aa][ks],
                       M::ld(sVnt + (16 * ct + lr) * C::LDC + ks * KS + EPL * lg), x);
          sacc[aa * C::CTW + bb] = x;
        }
    }
    state_to_lds<E, K, V>(sacc, L);
    if (MODE == kFix) {
      const bool nz = state_any_nonzero<E, K, V>(sacc);
      const bool wnz = __any(nz);
      if (lane == 0) L.sFlag[w] = wnz ? 1 : 0;
    }
    __syncthreads();
    if (MODE == kFix) zero_exit = (L.sFlag[0] | L.sFlag[1] | L.sFlag[2] | L.sFlag[3]) == 0;
    if (c + 1 < c_end && !zero_exit) {
      pref_commit<E, K, V, MODE>(pf, L);
      __syncthreads();
    }
  }
  return zero_exit;
}

template <typename E, int K, int V>
struct SegSmem {
  using C = SegCfg<E, K, V>;
  static constexpr int bytes = C::bytes;
};

#define GDN_SEG_LDS(E, K, V)                                                  \
  __shared__ __attribute__((aligned(16))) char smem_[SegCfg<E, K, V>::bytes]; \
  __shared__ float sg_[4][64];                                                \
  __shared__ int sflag_[4];                                                   \
  Lds L;                                                                      \
  L.base = smem_;                                                             \
  L.sGam = sg_[0];                                                            \
  L.sEg = sg_[1];                                                             \
  L.sDec = sg_[2];                                                            \
  L.sBet = sg_[3];                                                            \
  L.sFlag = sflag_;

// pass 1 (kMain) and pass 2 (kFix) over (segment, v-head) work items.
template <typename E, int K, int V, int MODE, bool WRITE_O>
__global__ __launch_bounds__(256) void segment_kernel(FwdArgs a) {
  using C = SegCfg<E, K, V>;
  GDN_SEG_LDS(E, K, V)
  const Problem &p = a.p;
  const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
  const int h = (int)(wid % p.Hv);
  const int64_t sg = wid / p.Hv;
  const int32_t *chunk_prefix = reinterpret_cast<const int32_t *>(a.ws + a.wl.chunk_prefix);
  const int32_t *seg_prefix = reinterpret_cast<const int32_t *>(a.ws + a.wl.seg_prefix);
  const int n = find_seq(seg_prefix, p.N, sg);
  const int j = (int)(sg - seg_prefix[n]);
  if (MODE == kFix && j == 0) return;
  const SeqInfo si = seq_info(p, n);
  const int nseg = seg_prefix[n + 1] - seg_prefix[n];
  const int c_begin = j * a.plan.seg_chunks;
  const int c_end = min(c_begin + a.plan.seg_chunks, si.nchunks);
  const int64_t KV = (int64_t)K * V;
  float *hseg = reinterpret_cast<float *>(a.ws + a.wl.hseg);
  float *eseg = reinterpret_cast<float *>(a.ws + a.wl.eseg);
  int32_t *flags = reinterpret_cast<int32_t *>(a.ws + a.wl.flags);

  f32x4 sacc[C::NTS];
  if (MODE == kMain) {
    const float *src = (j == 0 && a.h0) ? a.h0 + ((int64_t)n * p.Hv + h) * KV : nullptr;
    load_state<E, K, V>(sacc, src);
  } else {
    load_state<E, K, V>(sacc, hseg + ((sg - 1) * p.Hv + h) * KV);
  }
  const bool zero = run_chunks<E, K, V, MODE, WRITE_O>(a, L, sacc, si, chunk_prefix[n],
                                                       c_begin, c_end, h);
  if (MODE == kMain) {
    store_state<E, K, V>(sacc, hseg + (sg * p.Hv + h) * KV, nullptr, false);
    if (nseg == 1 && a.ht)
      store_state<E, K, V>(sacc, a.ht + ((int64_t)n * p.Hv + h) * KV, nullptr, false);
  } else {
    if (!zero) store_state<E, K, V>(sacc, eseg + (sg * p.Hv + h) * KV, nullptr, false);
    if (threadIdx.x == 0) flags[sg * p.Hv + h] = zero ? 0 : 1;
  }
}

// pass 3: per (sequence, v-head), serial residual carry across segments.
template <typename E, int K, int V, bool WRITE_O>
__global__ __launch_bounds__(256) void serial_kernel(FwdArgs a) {
  using C = SegCfg<E, K, V>;
  GDN_SEG_LDS(E, K, V)
  const Problem &p = a.p;
  const int64_t wid = blockIdx.x;
  const int h = (int)(wid % p.Hv);
  const int n = (int)(wid / p.Hv);
  const int32_t *chunk_prefix = reinterpret_cast<const int32_t *>(a.ws + a.wl.chunk_prefix);
  const int32_t *seg_prefix = reinterpret_cast<const int32_t *>(a.ws + a.wl.seg_prefix);
  const SeqInfo si = seq_info(p, n);
  const int nseg = seg_prefix[n + 1] - seg_prefix[n];
  const int64_t KV = (int64_t)K * V;
  if (nseg == 0) {  // empty sequence: the final state is the initial one
    if (a.ht) {
      float *dst = a.ht + ((int64_t)n * p.Hv + h) * KV;
      const float *src = a.h0 ? a.h0 + ((int64_t)n * p.Hv + h) * KV : nullptr;
      for (int64_t i = threadIdx.x; i < KV; i += blockDim.x) dst[i] = src ? src[i] : 0.f;
    }
    return;
  }
  if (nseg == 1) return;
  const float *hseg = reinterpret_cast<const float *>(a.ws + a.wl.hseg);
  const float *eseg = reinterpret_cast<const float *>(a.ws + a.wl.eseg);
  const int32_t *flags = reinterpret_cast<const int32_t *>(a.ws + a.wl.flags);
  f32x4 sacc[C::NTS];
  load_state<E, K, V>(sacc, nullptr);
  bool nonzero = false;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int j = 1; j < nseg; ++j) {
    const int64_t sg = seg_prefix[n] + j;
    if (nonzero) {
      const int c_begin = j * a.plan.seg_chunks;
      const int c_end = min(c_begin + a.plan.seg_chunks, si.nchunks);
      run_chunks<E, K, V, kFix, WRITE_O>(a, L, sacc, si, chunk_prefix[n], c_begin, c_end, h);
      __syncthreads();
    }
    if (flags[sg * p.Hv + h]) {
      f32x4 e[C::NTS];
      load_state<E, K, V>(e, eseg + (sg * p.Hv + h) * KV);
#pragma unroll
      for (int m = 0; m < C::NTS; ++m) sacc[m] += e[m];
    }
    const bool wnz = __any(state_any_nonzero<E, K, V>(sacc));
    if (lane == 0) L.sFlag[w] = wnz ? 1 : 0;
    __syncthreads();
    nonzero = (L.sFlag[0] | L.sFlag[1] | L.sFlag[2] | L.sFlag[3]) != 0;
    __syncthreads();
  }
  if (a.ht) {
    const int64_t last = seg_prefix[n] + nseg - 1;
    store_state<E, K, V>(sacc, a.ht + ((int64_t)n * p.Hv + h) * KV,
                         hseg + (last * p.Hv + h) * KV, false);
  }
}

// ---------------------------------------------------------------- launch
template <typename E, int K, int V, bool WRITE_O>
static hipError_t launch_fwd_t(const FwdArgs &a, hipStream_t st) {
  const Problem &p = a.p;
  const Plan &pl = a.plan;
  plan_kernel<<<1, 64, 0, st>>>(p, pl.seg_chunks,
                                reinterpret_cast<int32_t *>(a.ws + a.wl.chunk_prefix),
                                reinterpret_cast<int32_t *>(a.ws + a.wl.seg_prefix));
  if (pl.total_chunks > 0) {
    prep_kernel<E, K><<<dim3((unsigned)(pl.total_chunks * p.Hv)), 64, 0, st>>>(a);
    segment_kernel<E, K, V, kMain, WRITE_O>
        <<<dim3((unsigned)(pl.total_segs * p.Hv)), 256, 0, st>>>(a);
    if (pl.max_segs_per_seq > 1)
      segment_kernel<E, K, V, kFix, WRITE_O>
          <<<dim3((unsigned)(pl.total_segs * p.Hv)), 256, 0, st>>>(a);
  }
  if (pl.max_segs_per_seq > 1 || pl.has_empty)
    serial_kernel<E, K, V, WRITE_O><<<dim3((unsigned)(p.N * p.Hv)), 256, 0, st>>>(a);
  return hipGetLastError();
}

template <bool WRITE_O>
static hipError_t dispatch_kv(const FwdArgs &a, hipStream_t st) {
  const int K = a.p.K, V = a.p.V;
#define GDN_KV(E, KK, VV) \
  if (K == KK && V == VV) return launch_fwd_t<E, KK, VV, WRITE_O>(a, st);
  if (a.p.dtype == 1) {
    GDN_KV(bf16, 128, 128)
    GDN_KV(bf16, 64, 64)
    GDN_KV(bf16, 32, 32)
    GDN_KV(bf16, 64, 128)
    GDN_KV(bf16, 128, 64)
  } else {
    GDN_KV(float, 32, 32)
    GDN_KV(float, 64, 64)
    GDN_KV(float, 32, 64)
    GDN_KV(float, 64, 32)
  }
#undef GDN_KV
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdArgs &a, hipStream_t st) { return dispatch_kv<true>(a, st); }

// Forward state recompute for the backward: states only, no output.
hipError_t launch_fwd_states(const FwdArgs &a, hipStream_t st) {
  return dispatch_kv<false>(a, st);
}

}  // namespace gdn
