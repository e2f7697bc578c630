// Backward kernels of the GDN chunked prefill for gfx950.
//
// The backward of the FlashQLA article's low-level API ("底层 API":
// chunk_gated_delta_rule_bwd(q, k, v, g, beta, A, do, dht, scale,
// initial_state, cu_seqlens) -> dq, dk, dv, db, dg, dh0) is the reverse mode
// of the chunked forward (see gdn_fwd.hip).  Per chunk, with S the entering
// state, D = dL/dS' the gradient of the leaving state, and the forward
// quantities recomputed (P = lower_incl(Q K^T * E), R, Vn = T R):
//   dVn = scale P^T dO + diag(exp(gamma_L - gamma)) K D
//   dR  = T^T dVn,      dA = -strict_lower(dR Vn^T)   (= -T^T dT T^T, dT = dVn R^T)
//   dP  = scale lower_incl(dO Vn^T)
//   dS  = exp(gamma_L) D + Q^T diag(scale e^gamma) dO - K^T diag(beta e^gamma) dR
//   dq  = diag(scale e^gamma) dO S^T + (dP * E) K
//   dk  = (dP * E)^T Q + (dKK + dKK^T) K - diag(beta e^gamma) dR S^T
//         + diag(exp(gamma_L - gamma)) Vn D^T,          dKK = diag(beta) dA * E
//   dv  = diag(beta) dR
//   dbeta, dgamma from the rows and columns of these products; dg is the
//   reverse cumulative sum of dgamma inside the chunk.
// Kernels: (1) forward state recompute (the forward segment kernels, states
// only), (2) the reverse recurrence for D, context-parallel with the same
// exact fix-up scheme mirrored (segments run from a zero leaving gradient,
// then the true one is propagated backwards with the homogeneous recurrence
// until it is zero or denormal in every element), (3) a chunk-parallel kernel for the local
// gradients, one workgroup per (chunk, q/k head) summing its v-heads' dq and
// dk in a fixed order (no atomics).
#include <stdlib.h>

#include "gdn_seg.hpp"

namespace gdn {

enum { kRMain = 0, kRFix = 1 };

// ------------------------------------------------- reverse recurrence for D
template <typename E, int K, int V>
struct RevLds {
  using G = Geo<E, K, V>;
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + 64 * G::LDK;
  static constexpr int oDO = oK + 64 * G::LDK;    // dO   [64][V]
  static constexpr int oDt = oDO + 64 * G::LDV;   // D^T  [V][K]
  static constexpr int oT = oDt + V * G::LDK;     // T    [64][64]
  static constexpr int oPt = oT + 64 * G::LDC;    // P^T  [64][64]
  static constexpr int oDVnt = oPt + 64 * G::LDC; // dVn^T [V][64]
  static constexpr int oXt = oDVnt + V * G::LDC;  // (-beta e^gamma T^T dVn)^T [V][64]
  static constexpr int nE = oXt + V * G::LDC;
  static constexpr int bytes = nE * (int)sizeof(E);
};

struct RSmem {
  char *base;
  GateLds gate;
  float *wq;  // scale * exp(gamma)
  float *wk;  // -beta * exp(gamma)
  int *flag;
};

template <typename E, int K, int V, bool MAIN>
__device__ __forceinline__ void rev_commit(const Pref<E, K, V> &pf, const RSmem &S, float scale,
                                           bool l2, int tid = threadIdx.x) {
  using G = Geo<E, K, V>;
  using L = RevLds<E, K, V>;
  E *sm = reinterpret_cast<E *>(S.base);
  constexpr int PK = K / G::VEC, PVr = V / G::VEC, PTr = 64 / G::VEC;
#pragma unroll
  for (int m = 0; m < G::NQ; ++m) {
    const int idx = tid + kThreads * m;
    const uint4 xq = l2 ? l2n_piece<E, PK>(pf.q[m]) : pf.q[m];
    const uint4 xk = l2 ? l2n_piece<E, PK>(pf.k[m]) : pf.k[m];
    if (idx < G::PQ) {
      const int r = idx / PK, cv = idx % PK;
      *reinterpret_cast<uint4 *>(sm + L::oQ + r * G::LDK + cv * G::VEC) = xq;
      *reinterpret_cast<uint4 *>(sm + L::oK + r * G::LDK + cv * G::VEC) = xk;
    }
  }
  // dO and T stay row-major; their transposed operands come from LDS
  // transpose reads
  if (MAIN) {
#pragma unroll
    for (int m = 0; m < G::NV; ++m) {
      const int idx = tid + kThreads * m;
      if (idx < G::PV) {
        const int r = idx / PVr, cv = idx % PVr;
        *reinterpret_cast<uint4 *>(sm + L::oDO + r * G::LDV + cv * G::VEC) = pf.v[m];
      }
    }
  }
#pragma unroll
  for (int m = 0; m < G::NTM; ++m) {
    const int idx = tid + kThreads * m;
    if (idx < G::PT) {
      const int r = idx / PTr, cv = idx % PTr;
      *reinterpret_cast<uint4 *>(sm + L::oT + r * G::LDC + cv * G::VEC) = pf.t[m];
    }
  }
  if (tid < 64) {
    const float gam = wave_incl_scan(pf.g) * kLog2e;
    const float gL = lane63(gam);
    const float eg = __builtin_amdgcn_exp2f(gam);
    S.gate.gam[tid] = gam;
    S.gate.eg[tid] = eg;
    S.gate.dec[tid] = __builtin_amdgcn_exp2f(gL - gam);
    S.gate.bet[tid] = pf.beta();
    S.wq[tid] = scale * eg;
    S.wk[tid] = -pf.beta() * eg;
  }
}

// Runs chunks c_end-1 down to c_begin of one (sequence, v-head), starting
// from the leaving-state gradient in `st`.  kRMain: full reverse step.
// kRFix: homogeneous reverse step (no dO), stops once the gradient is zero
// or denormal in every element.  The gradient leaving every visited chunk is
// stored (kRMain) or accumulated (kRFix) into dstates.
template <typename E, int K, int V, int MODE>
__device__ __forceinline__ bool rev_run(const BwdArgs &a, const RSmem &S,
                                        Tiles<Geo<E, K, V>::NTS> &st, const SeqInfo &si,
                                        int64_t chunk_gid0, int c_begin, int c_end, int h) {
  using G = Geo<E, K, V>;
  using L = RevLds<E, K, V>;
  using M = Mma<E>;
  constexpr int KS = M::KS, EPL = M::EPL;
  constexpr int NKK = K / KS;
  constexpr int NKC = 64 / KS;
  constexpr int NCH = G::NCH;
  constexpr bool MAIN = MODE == kRMain;
  const Problem &p = a.p;
  E *sm = reinterpret_cast<E *>(S.base);
  const E *sQ = sm + L::oQ;
  const E *sK = sm + L::oK;
  const E *sDO = sm + L::oDO;
  E *sDt = sm + L::oDt;
  const E *sT = sm + L::oT;
  E *sPt = sm + L::oPt;
  E *sDVnt = sm + L::oDVnt;
  E *sXt = sm + L::oXt;
  const int w = wave_of(threadIdx.x);
  const int rt = w & 3;
  const int ct0 = (w >> 2) * NCH;
  const float scale = p.scale;
  const E *qp = reinterpret_cast<const E *>(a.q);
  const E *kp = reinterpret_cast<const E *>(a.k);
  const E *dop = reinterpret_cast<const E *>(a.dout);
  const E *bp = reinterpret_cast<const E *>(a.beta);
  const E *tmat = reinterpret_cast<const E *>(a.tm_ext ? a.tm_ext : a.ws + a.wl.fwd.tmat);
  E *dstates = reinterpret_cast<E *>(a.ws + a.wl.dstates);

  if (c_begin >= c_end)
    return MODE == kRFix ? !block_any(tiles_significant<E, K, V>(st), S.flag) : false;
  const float thr = MODE == kRFix ? fix_threshold<E, K, V>(st, S.flag) : 0.f;
  Pref<E, K, V> pf;
  {
    const int c = c_end - 1;
    pref_load<E, K, V, MAIN>(pf, p, qp, kp, dop, tmat, a.g, bp, si.tok0 + (int64_t)c * kChunk,
                             min(kChunk, si.len - c * kChunk), h, chunk_gid0 + c);
    rev_commit<E, K, V, MAIN>(pf, S, scale, p.l2);
    tiles_to_lds_t<E, K, V>(st, sDt);
  }
  __syncthreads();
  bool zero_exit = false;
  for (int c = c_end - 1; c >= c_begin && !zero_exit; --c) {
    const int tid = opaque_tid(), lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    // per-chunk gradients (lane layout): pass 1 stores the LDS mirror written
    // last step; the fix-up pass adds its correction, reading the stored
    // values here and writing the sums after phase A
    E *ds = dstates + ((chunk_gid0 + c) * p.Hv + h) * (int64_t)K * V;
    TilesOld<E, K, V> dold;
    if (MODE == kRFix)
      tiles_old_l<E, K, V>(dold, ds, tid);
    else
      mirror_store_l<E, K, V>(sDt, ds, tid);
    // the previous chunk's inputs travel while this whole chunk is computed
    if (c - 1 >= c_begin) {
      const int c1 = c - 1;
      pref_load<E, K, V, MAIN>(pf, p, qp, kp, dop, tmat, a.g, bp,
                               si.tok0 + (int64_t)c1 * kChunk,
                               min(kChunk, si.len - c1 * kChunk), h, chunk_gid0 + c1, tid);
    }
    // ---- phase A: K D (rows of tile rt, half of V); P^T.  Fragments are
    // double-buffered over the k-steps; the two Q K^T tiles are formed
    // whether or not they lie below the diagonal (the mask below zeroes them).
    const int pc0 = 2 * (w >> 2);
    f32x4 kd[NCH];
    f32x4 qk[2] = {zero4(), zero4()};
#pragma unroll
    for (int c2 = 0; c2 < NCH; ++c2) kd[c2] = zero4();
    {
      typename M::frag fk[2], fq[2], fd[2][NCH], fkb[2][2];
      auto load_step = [&](int ks, int sl) {
        fk[sl] = M::ld(sK + (16 * rt + lr) * G::LDK + ks * KS + EPL * lg);
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2)
          fd[sl][c2] = M::ld(sDt + (16 * (ct0 + c2) + lr) * G::LDK + ks * KS + EPL * lg);
        if (MAIN) {
          fq[sl] = M::ld(sQ + (16 * rt + lr) * G::LDK + ks * KS + EPL * lg);
#pragma unroll
          for (int cc = 0; cc < 2; ++cc)
            fkb[sl][cc] = M::ld(sK + (16 * (pc0 + cc) + lr) * G::LDK + ks * KS + EPL * lg);
        }
      };
      load_step(0, 0);
#pragma unroll
      for (int ks = 0; ks < NKK; ++ks) {
        const int sl = ks & 1;
        if (ks + 1 < NKK) load_step(ks + 1, sl ^ 1);
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2) kd[c2] = M::mma(fk[sl], fd[sl][c2], kd[c2]);
        if (MAIN) {
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) qk[cc] = M::mma(fq[sl], fkb[sl][cc], qk[cc]);
        }
      }
    }
    if (MODE == kRFix) tiles_accumulate_l<E, K, V>(st, dold, ds, tid);
    if (MAIN) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int t = 16 * (pc0 + cc) + lr;
        const float gt = S.gate.gam[t];
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = 16 * rt + 4 * lg + i;
          pv[i] = (t <= s) ? qk[cc][i] * __builtin_amdgcn_exp2f(S.gate.gam[s] - gt) : 0.f;
        }
        st4(sPt + t * G::LDC + 16 * rt + 4 * lg, pv[0], pv[1], pv[2], pv[3]);
      }
    }
    __syncthreads();
    // ---- phase B: dVn = dec * (K D) + scale P^T dO
    {
      float dec_r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) dec_r[i] = S.gate.dec[16 * rt + 4 * lg + i];
      f32x4 x[NCH];
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2) x[c2] = zero4();
      if (MAIN) {
        typename M::frag pa[NKC];
#pragma unroll
        for (int ks = 0; ks < NKC; ++ks)
          pa[ks] = M::ld(sPt + (16 * rt + lr) * G::LDC + ks * KS + EPL * lg);
#pragma unroll
        for (int ks = 0; ks < NKC; ++ks)
#pragma unroll
          for (int c2 = 0; c2 < NCH; ++c2)
            x[c2] = M::mma(
                pa[ks], M::ld_tr(sDO + ks * KS * G::LDV + 16 * (ct0 + c2), G::LDV, lane),
                x[c2]);
      }
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2) {
        float y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = dec_r[i] * kd[c2][i] + scale * x[c2][i];
        st4(sDVnt + (16 * (ct0 + c2) + lr) * G::LDC + 16 * rt + 4 * lg, y[0], y[1], y[2], y[3]);
      }
    }
    __syncthreads();
    // ---- phase C: X = T^T dVn, scaled by -beta e^gamma
    {
      typename M::frag ta[NKC];
#pragma unroll
      for (int ks = 0; ks < NKC; ++ks)
        ta[ks] = M::ld_tr(sT + ks * KS * G::LDC + 16 * rt, G::LDC, lane);
      f32x4 x[NCH];
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2) x[c2] = zero4();
#pragma unroll
      for (int ks = 0; ks < NKC; ++ks)
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2)
          x[c2] = M::mma(
              ta[ks], M::ld(sDVnt + (16 * (ct0 + c2) + lr) * G::LDC + ks * KS + EPL * lg),
              x[c2]);
      float wk_r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) wk_r[i] = S.wk[16 * rt + 4 * lg + i];
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2)
        st4(sXt + (16 * (ct0 + c2) + lr) * G::LDC + 16 * rt + 4 * lg, wk_r[0] * x[c2][0],
            wk_r[1] * x[c2][1], wk_r[2] * x[c2][2], wk_r[3] * x[c2][3]);
    }
    __syncthreads();
    // ---- phase D: D <- exp(gamma_L) D + Q^T diag(scale e^g) dO + K^T Xs
    if (G::owns(w)) {
      const float egL = S.gate.eg[63];
      const int srt = G::srt(w), sct = G::sct(w);
#pragma unroll
      for (int m = 0; m < G::NTS; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[m][i] *= egL;
#pragma unroll
      for (int ks = 0; ks < NKC; ++ks) {
        const auto kt = M::ld_tr(sK + ks * KS * G::LDK + 16 * srt, G::LDK, lane);
#pragma unroll
        for (int m = 0; m < G::NTS; ++m)
          st[m] = M::mma(kt, M::ld(sXt + (16 * (sct + m) + lr) * G::LDC + ks * KS + EPL * lg),
                         st[m]);
        if (MAIN) {
          const auto qt =
              M::ld_tr_scaled(sQ + ks * KS * G::LDK + 16 * srt, G::LDK, S.wq + ks * KS, lane);
#pragma unroll
          for (int m = 0; m < G::NTS; ++m)
            st[m] = M::mma(qt, M::ld_tr(sDO + ks * KS * G::LDV + 16 * (sct + m), G::LDV, lane),
                           st[m]);
        }
      }
    }
    tiles_to_lds_t<E, K, V>(st, sDt, tid);
    if (MODE == kRFix) {
      zero_exit = !block_any(tiles_significant<E, K, V>(st, thr), S.flag);
    } else {
      __syncthreads();
    }
    if (c - 1 >= c_begin && !zero_exit) {
      rev_commit<E, K, V, MAIN>(pf, S, scale, p.l2, tid);
      __syncthreads();
    }
  }
  return zero_exit;
}

#define GDN_REV_LDS(E, K, V)                                                   \
  __shared__ __attribute__((aligned(16))) char smem_[RevLds<E, K, V>::bytes]; \
  __shared__ float sg_[6][64];                                                 \
  __shared__ int sflag_[kNW];                                                  \
  RSmem S;                                                                     \
  S.base = smem_;                                                              \
  S.gate.gam = sg_[0];                                                         \
  S.gate.eg = sg_[1];                                                          \
  S.gate.dec = sg_[2];                                                         \
  S.gate.bet = sg_[3];                                                         \
  S.wq = sg_[4];                                                               \
  S.wk = sg_[5];                                                               \
  S.flag = sflag_;

template <typename E, int K, int V, int MODE>
__global__ __launch_bounds__(kThreads) void rev_segment_kernel(BwdArgs a) {
  using G = Geo<E, K, V>;
  GDN_REV_LDS(E, K, V)
  const Problem &p = a.p;
  const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
  const int h = (int)(wid % p.Hv);
  const int64_t sg = wid / p.Hv;
  const SegLoc sl =
      locate_segment(p, a.plan.seg_chunks,
                     reinterpret_cast<const int32_t *>(a.ws + a.wl.fwd.chunk_prefix),
                     reinterpret_cast<const int32_t *>(a.ws + a.wl.fwd.seg_prefix), sg);
  if (MODE == kRFix && sl.j == sl.nseg - 1) return;
  const int64_t KV = (int64_t)K * V;
  float *dseg = reinterpret_cast<float *>(a.ws + a.wl.dseg);
  float *deseg = reinterpret_cast<float *>(a.ws + a.wl.deseg);
  int32_t *dflags = reinterpret_cast<int32_t *>(a.ws + a.wl.dflags);
  Tiles<G::NTS> st;
  if (MODE == kRMain) {
    const float *src = (sl.j == sl.nseg - 1 && a.dht)
                           ? a.dht + ((int64_t)sl.n * p.Hv + h) * KV : nullptr;
    tiles_load<E, K, V>(st, src);
  } else {
    tiles_load<E, K, V>(st, dseg + ((sg + 1) * p.Hv + h) * KV);
  }
  const bool zero =
      rev_run<E, K, V, MODE>(a, S, st, sl.si, sl.chunk0, sl.c_begin, sl.c_end, h);
  if (MODE == kRMain) {
    if (sl.nseg > 1) tiles_store<E, K, V>(st, dseg + (sg * p.Hv + h) * KV, nullptr, false);
    if (sl.nseg == 1 && a.dh0)
      tiles_store<E, K, V>(st, a.dh0 + ((int64_t)sl.n * p.Hv + h) * KV, nullptr, false);
  } else {
    if (!zero) tiles_store<E, K, V>(st, deseg + (sg * p.Hv + h) * KV, nullptr, false);
    if (threadIdx.x == 0) dflags[sg * p.Hv + h] = zero ? 0 : 1;
  }
}

template <typename E, int K, int V>
__global__ __launch_bounds__(kThreads) void rev_serial_kernel(BwdArgs a) {
  using G = Geo<E, K, V>;
  GDN_REV_LDS(E, K, V)
  const Problem &p = a.p;
  const int h = (int)(blockIdx.x % p.Hv);
  const int n = (int)(blockIdx.x / p.Hv);
  const SegLoc sl =
      locate_sequence(p, a.plan.seg_chunks,
                      reinterpret_cast<const int32_t *>(a.ws + a.wl.fwd.chunk_prefix),
                      reinterpret_cast<const int32_t *>(a.ws + a.wl.fwd.seg_prefix), n);
  const int64_t KV = (int64_t)K * V;
  if (sl.nseg == 0) {  // empty sequence: dh0 = dht
    if (a.dh0) {
      float *dst = a.dh0 + ((int64_t)n * p.Hv + h) * KV;
      const float *src = a.dht ? a.dht + ((int64_t)n * p.Hv + h) * KV : nullptr;
      copy_state<K, V>(dst, src);
    }
    return;
  }
  if (sl.nseg == 1) return;
  const float *dseg = reinterpret_cast<const float *>(a.ws + a.wl.dseg);
  const float *deseg = reinterpret_cast<const float *>(a.ws + a.wl.deseg);
  const int32_t *dflags = reinterpret_cast<const int32_t *>(a.ws + a.wl.dflags);
  bool any_flag = false;
  for (int j = (int)threadIdx.x; j < sl.nseg - 1; j += blockDim.x)
    any_flag |= dflags[(sl.seg0 + j) * p.Hv + h] != 0;
  if (!block_any(any_flag, S.flag)) {
    if (a.dh0) {
      float *dst = a.dh0 + ((int64_t)n * p.Hv + h) * KV;
      const float *src = dseg + (sl.seg0 * p.Hv + h) * KV;
      copy_state<K, V>(dst, src);
    }
    return;
  }
  Tiles<G::NTS> st;
  tiles_zero<E, K, V>(st);
  bool nonzero = false;
  for (int j = sl.nseg - 2; j >= 0; --j) {
    const int64_t sg = sl.seg0 + j;
    if (nonzero) {
      const int c_begin = j * a.plan.seg_chunks;
      const int c_end = min(c_begin + a.plan.seg_chunks, sl.si.nchunks);
      rev_run<E, K, V, kRFix>(a, S, st, sl.si, sl.chunk0, c_begin, c_end, h);
      __syncthreads();
    }
    if (dflags[sg * p.Hv + h]) {
      Tiles<G::NTS> e;
      tiles_load<E, K, V>(e, deseg + (sg * p.Hv + h) * KV);
#pragma unroll
      for (int m = 0; m < G::NTS; ++m) st[m] += e[m];
    }
    nonzero = block_any(tiles_significant<E, K, V>(st), S.flag);
  }
  if (a.dh0)
    tiles_store<E, K, V>(st, a.dh0 + ((int64_t)n * p.Hv + h) * KV,
                         dseg + (sl.seg0 * p.Hv + h) * KV, false);
}

// --------------------------------------------------------- local gradients
template <typename E, int K, int V>
struct LocCfg {
  using G = Geo<E, K, V>;
  // row pitches: bf16 rows pad 32 bytes, which keeps their 16-byte fragment
  // reads free of bank conflicts; fp32 V-block rows and S/D rows pad 16
  // bytes (the fp32 footprint has no room for more)
  static constexpr int PAD = 16 / (int)sizeof(E);   // 16 bytes
  static constexpr int PAD2 = 32 / (int)sizeof(E);  // 32 bytes
  static constexpr int PADB = sizeof(E) == 2 ? PAD2 : PAD;
  static constexpr int LDK = K + PAD2;
  static constexpr int LDC = 64 + PAD2;
  static constexpr int VB = (sizeof(E) == 4) ? 32 : (V < 64 ? V : 64);
  static constexpr int NVB = V / VB;
  static constexpr int LDB = VB + PADB;
  static constexpr int NCHB = VB / 32;  // V-block column tiles per half
  static constexpr int NCHK = K / 32;   // key column tiles per half
  static constexpr int LDSK = K + PADB;  // rows of the transposed S and D blocks
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + 64 * LDK;
  static constexpr int oT = oK + 64 * LDK;
  static constexpr int oPt = oT + 64 * LDC;
  // V-block buffers (dead after the V-block loop)
  // (every buffer of its own: no phase waits for another's readers before
  // it writes; row-scaled operands are scaled in registers)
  static constexpr int oS = oPt + 64 * LDC;      // S^T block [VB][LDSK]
  static constexpr int oD = oS + VB * LDSK;      // D^T block [VB][LDSK]
  static constexpr int oDO = oD + VB * LDSK;     // dO block [64][LDB]
  static constexpr int oRt = oDO + 64 * LDB;     // R^T [VB][LDC]
  static constexpr int oDVnt = oRt + VB * LDC;   // dVn^T [VB][LDC]
  static constexpr int oVn = oDVnt + VB * LDC;   // Vn [64][LDB]
  static constexpr int oDR = oVn + 64 * LDB;     // dR [64][LDB]
  static constexpr int oV = oDR + 64 * LDB;      // V block [64][LDB]; later dv
  static constexpr int nE = oV + 64 * LDB;
  // after the V-block loop: dP * E and dKK [64][LDC] reuse the block buffers
  static constexpr int oPE = oS;
  static constexpr int oKK = oPE + 64 * LDC;
  static_assert(oKK + 64 * LDC <= nE, "LDS reuse");
  static constexpr int bytes = nE * (int)sizeof(E);
};

// Per-row values of local_grad, kept at the start of its LDS so that their
// addresses fit the LDS instructions' immediate offsets.
struct LocSmall {
  float gam[64];  // gamma * log2(e)
  float eg[64];   // exp(gamma)
  float dec[64];  // exp(gamma_L - gamma)
  float bet[64];
  float rowp[4][2][64];  // [de, db, rs, c][half][row]
  float colp[4][64];     // [row tile][col]
  float rq[64], rk[64];  // L2-normalisation factors of the item's q, k rows
  float glp[kNW];
};

// One work item of local_grad: chunk gid (global id) of q/k head hq.
struct LocItem {
  int hq;
  int64_t gid;
  int64_t tok0;
  int rows;
};

// Registers that carry the next V block (S, D, dO, V pieces) and, at a v-head
// boundary, the next v-head's T piece and raw g, beta while the current block
// is computed.
template <typename E, int K, int V>
struct LocPref {
  using C = LocCfg<E, K, V>;
  static constexpr int PB = C::VB * (int)sizeof(E) / 16;  // 16-byte pieces per block row
  static constexpr int PK = K * (int)sizeof(E) / 16;  // 16-byte pieces per row of S^T, D^T
  static constexpr int NSP = (C::VB * PK + kThreads - 1) / kThreads;
  static constexpr int NOP = (64 * PB + kThreads - 1) / kThreads;
  static constexpr int NTP = (64 * 64 * (int)sizeof(E) / 16 + kThreads - 1) / kThreads;
  uint4 s[NSP], d[NSP], o[NOP], v[NOP], t[NTP];
  float g;
  E b;
};

template <typename E, int K, int V>
__global__ __launch_bounds__(kThreads) void local_grad_kernel(BwdArgs a) {
  using G = Geo<E, K, V>;
  using C = LocCfg<E, K, V>;
  using M = Mma<E>;
  constexpr int KS = M::KS, EPL = M::EPL;
  constexpr int NKK = K / KS;
  constexpr int NKC = 64 / KS;
  constexpr int NKB = C::VB / KS;
  constexpr int VB = C::VB, LDB = C::LDB, NCHB = C::NCHB, NCHK = C::NCHK;
  static_assert(sizeof(LocSmall) % 16 == 0, "LDS alignment");
  __shared__ __attribute__((aligned(16))) char smem_[sizeof(LocSmall) + C::bytes];
  LocSmall &ls = *reinterpret_cast<LocSmall *>(smem_);
  float *sgam = ls.gam, *seg = ls.eg, *sdec = ls.dec, *sbet = ls.bet;
  auto &rowp = ls.rowp;
  auto &colp = ls.colp;
  float *glp = ls.glp;
  E *sm = reinterpret_cast<E *>(smem_ + sizeof(LocSmall));
  E *sQ = sm + C::oQ;
  E *sK = sm + C::oK;
  E *sT = sm + C::oT;
  E *sPt = sm + C::oPt;
  E *sS = sm + C::oS;
  E *sD = sm + C::oD;
  E *sDR = sm + C::oDR;
  E *sDO = sm + C::oDO;
  E *sRt = sm + C::oRt;
  E *sDVnt = sm + C::oDVnt;
  E *sVn = sm + C::oVn;
  E *sPE = sm + C::oPE;
  E *sKK = sm + C::oKK;
  E *sV = sm + C::oV;

  const Problem &p = a.p;
  const int w = wave_of(threadIdx.x);
  const int rt = w & 3, ch = w >> 2;
  const int pc0 = 2 * ch;
  // Lane quantities; re-derived (opaquely) at the top of each loop iteration
  // so that the addresses built on them are not hoisted and held across it.
  int tid, lane, lr, lg, ra;  // ra: matrix row an A-operand fragment of this lane covers
  auto relane = [&]() {
    tid = opaque_tid();
    lane = tid & 63;
    lr = lane & 15;
    lg = lane >> 4;
    ra = 16 * rt + lr;
  };
  relane();
  const int Gq = p.Hv / p.Hq;
  // Work items are (chunk, q/k head) pairs; a workgroup takes items
  // blockIdx.x, + gridDim.x, ...  and loads the next item's q, k, first T,
  // gates and V block while it finishes the current one.
  const int64_t n_items = a.plan.total_chunks * p.Hq;
  auto item_of = [&](int64_t it) {
    LocItem x;
    x.hq = (int)(it % p.Hq);
    x.gid = it / p.Hq;
    const ChunkLoc cl =
        locate_chunk(p, reinterpret_cast<const int32_t *>(a.ws + a.wl.fwd.chunk_prefix), x.gid);
    x.tok0 = cl.si.tok0 + (int64_t)cl.c * kChunk;
    x.rows = min(kChunk, cl.si.len - cl.c * kChunk);
    return x;
  };
  const float scale = p.scale;
  const E *qp = reinterpret_cast<const E *>(a.q);
  const E *kp = reinterpret_cast<const E *>(a.k);
  const E *vp = reinterpret_cast<const E *>(a.v);
  const E *dop = reinterpret_cast<const E *>(a.dout);
  const E *bp = reinterpret_cast<const E *>(a.beta);
  const E *tmat = reinterpret_cast<const E *>(a.tm_ext ? a.tm_ext : a.ws + a.wl.fwd.tmat);
  const E *hst = reinterpret_cast<const E *>(a.hcache ? a.hcache : a.ws + a.wl.hstates);
  const E *dst = reinterpret_cast<const E *>(a.ws + a.wl.dstates);
  E *dqp = reinterpret_cast<E *>(a.dq);
  E *dkp = reinterpret_cast<E *>(a.dk);
  E *dvp = reinterpret_cast<E *>(a.dv);
  E *dbp = reinterpret_cast<E *>(a.dbeta);
  constexpr int VEC = G::VEC;
  // Per-workgroup tile bases (uniform, held in scalar registers) and 32-bit
  // byte offsets per lane: row strides of q/k and of v/do/dv in bytes.
  const uint32_t qk_rs = (uint32_t)(p.Hq * K * sizeof(E));
  const uint32_t v_rs = (uint32_t)(p.Hv * V * sizeof(E));
  // 4 per-row values of this lane's accumulator rows 16 rt + 4 lg + i
  auto row4 = [&](const float *arr) {
    return *reinterpret_cast<const f32x4 *>(arr + 16 * rt + 4 * lg);
  };

#define QA(ks) M::ld(sQ + ra * C::LDK + (ks) * KS + EPL * lg)
#define KA(ks) M::ld(sK + ra * C::LDK + (ks) * KS + EPL * lg)
  // raw Q K^T and (if wanted) K K^T tiles of this wave (fp32); recomputed
  // where needed rather than held across the v-block loop
  auto qk_tiles = [&](f32x4 *qk, f32x4 *kk) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      qk[cc] = zero4();
      if (kk) kk[cc] = zero4();
    }
#pragma unroll
    for (int ks = 0; ks < NKK; ++ks) {
      const auto qa = QA(ks);
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
        if (pc0 + cc <= rt) {
          const auto kb = M::ld(sK + (16 * (pc0 + cc) + lr) * C::LDK + ks * KS + EPL * lg);
          qk[cc] = M::mma(qa, kb, qk[cc]);
          if (kk) kk[cc] = M::mma(KA(ks), kb, kk[cc]);
        }
    }
  };
  // dq, dk of the q/k head: every term is accumulated in place
  f32x4 dq[NCHK], dk[NCHK];

  using LP = LocPref<E, K, V>;
  constexpr int PB = LP::PB;
  LP pf;
  // global loads of V block vb of v-head hl, in two parts: the S and D
  // blocks, then the dO and V rows (rows past the chunk end read 0)
  auto load_sd = [&](const LocItem &x, int hl, int vb) {
    const int h = x.hq * Gq + hl;
    const int64_t cg = x.gid * p.Hv + h;
    const int v0 = vb * VB;
    // columns v0 .. v0 + VB - 1 of the states and of their gradients: one
    // contiguous block of the lane layout each
    const char *hsb = reinterpret_cast<const char *>(hst + cg * (int64_t)K * V + v0 * K);
    const char *dsb = reinterpret_cast<const char *>(dst + cg * (int64_t)K * V + v0 * K);
#pragma unroll
    for (int m = 0; m < LP::NSP; ++m) {
      const int idx = tid + kThreads * m;
      uint4 zs = make_uint4(0u, 0u, 0u, 0u), zd = zs;
      if (idx < VB * LP::PK) {
        const uint32_t off = (uint32_t)idx * 16u;
        zs = *reinterpret_cast<const uint4 *>(hsb + off);
        zd = *reinterpret_cast<const uint4 *>(dsb + off);
      }
      pf.s[m] = zs;
      pf.d[m] = zd;
    }
  };
  auto load_ov = [&](const LocItem &x, int hl, int vb) {
    const int h = x.hq * Gq + hl;
    const int v0 = vb * VB;
    const char *vb_ = reinterpret_cast<const char *>(vp + (x.tok0 * p.Hv + h) * V + v0);
    const char *ob_ = reinterpret_cast<const char *>(dop + (x.tok0 * p.Hv + h) * V + v0);
#pragma unroll
    for (int m = 0; m < LP::NOP; ++m) {
      const int idx = tid + kThreads * m;
      const int r = idx / PB, cv = idx % PB;
      uint4 zo = make_uint4(0u, 0u, 0u, 0u), zv = zo;
      if (idx < 64 * PB && r < x.rows) {
        const uint32_t off = r * v_rs + (uint32_t)(cv * 16);
        zo = *reinterpret_cast<const uint4 *>(ob_ + off);
        zv = *reinterpret_cast<const uint4 *>(vb_ + off);
      }
      pf.o[m] = zo;
      pf.v[m] = zv;
    }
  };
  // global loads of v-head hl's T and raw gates
  auto load_head = [&](const LocItem &x, int hl) {
    const int h = x.hq * Gq + hl;
    const int64_t cg = x.gid * p.Hv + h;
    const char *tm = reinterpret_cast<const char *>(tmat + cg * 64 * 64);
#pragma unroll
    for (int m = 0; m < LP::NTP; ++m) {
      const int idx = tid + kThreads * m;
      pf.t[m] = idx < 64 * 64 / VEC ? *reinterpret_cast<const uint4 *>(tm + idx * 16)
                                    : make_uint4(0u, 0u, 0u, 0u);
    }
    pf.g = 0.f;
    pf.b = from_f32<E>(0.f);
    if (tid < x.rows) {
      const int64_t gi = (x.tok0 + tid) * p.Hv + h;
      pf.g = a.g[gi];
      pf.b = bp[gi];
    }
  };
  // q and k tiles of an item (shared by its v-heads) into registers
  constexpr int PK = K / VEC;
  constexpr int NQP = (64 * PK + kThreads - 1) / kThreads;
  uint4 zq[NQP], zk[NQP];
  auto load_qk = [&](const LocItem &x) {
    const char *qtile = reinterpret_cast<const char *>(qp + (x.tok0 * p.Hq + x.hq) * K);
    const char *ktile = reinterpret_cast<const char *>(kp + (x.tok0 * p.Hq + x.hq) * K);
#pragma unroll
    for (int m = 0; m < NQP; ++m) {
      const int idx = tid + kThreads * m;
      const int r = idx / PK, cv = idx % PK;
      zq[m] = make_uint4(0u, 0u, 0u, 0u);
      zk[m] = zq[m];
      if (idx < 64 * PK && r < x.rows) {
        const uint32_t off = r * qk_rs + cv * 16u;
        zq[m] = *reinterpret_cast<const uint4 *>(qtile + off);
        zk[m] = *reinterpret_cast<const uint4 *>(ktile + off);
      }
    }
  };
  if (blockIdx.x >= n_items) return;
  LocItem cur = item_of(blockIdx.x);
  load_head(cur, 0);
  load_sd(cur, 0, 0);
  load_ov(cur, 0, 0);
  load_qk(cur);

  for (int64_t it = blockIdx.x; it < n_items; it += gridDim.x) {
  relane();
  const int64_t it_next = it + gridDim.x;
  const bool has_next = it_next < n_items;
  const int hq = cur.hq;
  const int64_t tok0 = cur.tok0;
  const int rows = cur.rows;
#pragma unroll
  for (int m = 0; m < NQP; ++m) {
    const int idx = tid + kThreads * m;
    float fq = 0.f, fk = 0.f;
    const uint4 xq = p.l2 ? l2n_piece<E, PK>(zq[m], fq) : zq[m];
    const uint4 xk = p.l2 ? l2n_piece<E, PK>(zk[m], fk) : zk[m];
    if (idx < 64 * PK) {
      const int r = idx / PK, cv = idx % PK;
      *reinterpret_cast<uint4 *>(sQ + r * C::LDK + cv * VEC) = xq;
      *reinterpret_cast<uint4 *>(sK + r * C::LDK + cv * VEC) = xk;
      if (cv == 0) {
        ls.rq[r] = fq;
        ls.rk[r] = fk;
      }
    }
  }
#pragma unroll
  for (int m = 0; m < NCHK; ++m) {
    dq[m] = zero4();
    dk[m] = zero4();
  }
  __syncthreads();

  for (int hl = 0; hl < Gq; ++hl) {
    relane();
    const int h = hq * Gq + hl;
    // ---- per v-head inputs: T, gates (from the prefetch registers)
    {
      constexpr int PT = 64 / VEC;
#pragma unroll
      for (int m = 0; m < LP::NTP; ++m) {
        const int idx = tid + kThreads * m;
        if (idx < 64 * PT) {
          const int r = idx / PT, cv = idx % PT;
          *reinterpret_cast<uint4 *>(sT + r * C::LDC + cv * VEC) = pf.t[m];
        }
      }
      if (tid < 64) {
        const float gam = wave_incl_scan(pf.g) * kLog2e;
        const float gL = lane63(gam);
        sgam[tid] = gam;
        seg[tid] = __builtin_amdgcn_exp2f(gam);
        sdec[tid] = __builtin_amdgcn_exp2f(gL - gam);
        sbet[tid] = to_f32(pf.b);
      }
    }
    __syncthreads();
    char *dvtile = reinterpret_cast<char *>(dvp + (tok0 * p.Hv + h) * V);
    // P^T (P = lower_incl(Q K^T * E)) of this v-head into LDS
    {
    f32x4 qk[2];
    qk_tiles(qk, nullptr);
    const f32x4 gam_s = row4(sgam);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int t = 16 * (pc0 + cc) + lr;
      const float gt = sgam[t];
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 16 * rt + 4 * lg + i;
        pv[i] = (t <= s) ? qk[cc][i] * __builtin_amdgcn_exp2f(gam_s[i] - gt) : 0.f;
      }
      st4(sPt + t * C::LDC + 16 * rt + 4 * lg, pv[0], pv[1], pv[2], pv[3]);
    }
    }
    f32x4 dp[2], da[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      dp[cc] = zero4();
      da[cc] = zero4();
    }
    float de_p[4] = {0.f, 0.f, 0.f, 0.f}, db_p[4] = {0.f, 0.f, 0.f, 0.f};
    float c_p[4] = {0.f, 0.f, 0.f, 0.f};
    float gl_p = 0.f;

    for (int vb = 0; vb < C::NVB; ++vb) {
      relane();
      const int v0 = vb * VB;
      __syncthreads();  // previous readers of the block buffers are done
      // commit the prefetched S, D, dO, V block; <D, S> partial; scaled dO
      {
#pragma unroll
        for (int m = 0; m < LP::NSP; ++m) {
          const int idx = tid + kThreads * m;
          if (idx < VB * LP::PK) {
            gl_p = dot_piece<E>(pf.s[m], pf.d[m], gl_p);
            int r, k_lo, k_hi;
            if (sizeof(E) == 2) {
              lane_unit<K>(idx, r, k_lo, k_hi);
              const uint4 x = pf.s[m], y = pf.d[m];
              *reinterpret_cast<uint2 *>(sS + r * C::LDSK + k_lo) = make_uint2(x.x, x.y);
              *reinterpret_cast<uint2 *>(sS + r * C::LDSK + k_hi) = make_uint2(x.z, x.w);
              *reinterpret_cast<uint2 *>(sD + r * C::LDSK + k_lo) = make_uint2(y.x, y.y);
              *reinterpret_cast<uint2 *>(sD + r * C::LDSK + k_hi) = make_uint2(y.z, y.w);
            } else {
              lane_unit<K>(idx >> 1, r, k_lo, k_hi);
              const int k0 = (idx & 1) ? k_hi : k_lo;
              *reinterpret_cast<uint4 *>(sS + r * C::LDSK + k0) = pf.s[m];
              *reinterpret_cast<uint4 *>(sD + r * C::LDSK + k0) = pf.d[m];
            }
          }
        }
#pragma unroll
        for (int m = 0; m < LP::NOP; ++m) {
          const int idx = tid + kThreads * m;
          if (idx < 64 * PB) {
            const int r = idx / PB, cv = idx % PB;
            *reinterpret_cast<uint4 *>(sDO + r * LDB + cv * VEC) = pf.o[m];
            *reinterpret_cast<uint4 *>(sV + r * LDB + cv * VEC) = pf.v[m];
          }
        }
      }
      // the next block is loaded while this one is computed: its S and D
      // blocks here, its dO and V rows (and at a v-head boundary the next T
      // and gates) after phase 3's MFMAs.  Issued all at once here, the
      // eight waves' loads queue behind one another in the address unit.
      if (vb + 1 < C::NVB) {
        load_sd(cur, hl, vb + 1);
      } else if (hl + 1 < Gq) {
        load_sd(cur, hl + 1, 0);
      } else if (has_next) {  // the next item's first v-head
        load_sd(item_of(it_next), 0, 0);
      }
      __syncthreads();
      // ---- phase 2: K S, Q S; R; dq += (scale e^g dO) S^T
      f32x4 ks_[NCHB], qs_[NCHB];
#pragma unroll
      for (int m = 0; m < NCHB; ++m) {
        ks_[m] = zero4();
        qs_[m] = zero4();
      }
#pragma unroll
      for (int ks = 0; ks < NKK; ++ks) {
        const auto qa = QA(ks), ka = KA(ks);
#pragma unroll
        for (int m = 0; m < NCHB; ++m) {
          const auto b =
              M::ld(sS + (16 * (ch * NCHB + m) + lr) * C::LDSK + ks * KS + EPL * lg);
          ks_[m] = M::mma(ka, b, ks_[m]);
          qs_[m] = M::mma(qa, b, qs_[m]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      {
      const f32x4 bet_s = row4(sbet), eg_s = row4(seg);
#pragma unroll
      for (int m = 0; m < NCHB; ++m) {
        const int vc = 16 * (ch * NCHB + m) + lr;
        const f32x4 v4 = M::ld_acc(sV + 16 * rt * LDB + 16 * (ch * NCHB + m), LDB, lane);
        const f32x4 o4 = M::ld_acc(sDO + 16 * rt * LDB + 16 * (ch * NCHB + m), LDB, lane);
        float rr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          rr[i] = bet_s[i] * (v4[i] - eg_s[i] * ks_[m][i]);
          de_p[i] += scale * o4[i] * qs_[m][i];
        }
        st4(sRt + vc * C::LDC + 16 * rt + 4 * lg, rr[0], rr[1], rr[2], rr[3]);
      }
      }
      // dq += (scale e^g dO) S^T: the dO rows scaled in registers
      const float dq_s = scale * seg[ra];
#pragma unroll
      for (int ks = 0; ks < NKB; ++ks) {
        const auto da_ = M::scaled(M::ld(sDO + ra * LDB + ks * KS + EPL * lg), dq_s);
#pragma unroll
        for (int m = 0; m < NCHK; ++m)
          dq[m] = M::mma(da_, M::ld_tr(sS + ks * KS * C::LDSK + 16 * (ch * NCHK + m), C::LDSK),
                         dq[m]);
      }
      __syncthreads();
      // ---- phase 3: Vn = T R; K D; c_r = e^{gL-g_r} <Vn_r, (K D)_r>
      {
        f32x4 vn[NCHB], kd[NCHB];
#pragma unroll
        for (int m = 0; m < NCHB; ++m) {
          vn[m] = zero4();
          kd[m] = zero4();
        }
        // Vn built transposed (Vn^T = R^T T^T): each lane then holds 4
        // consecutive columns of row 16 rt + (l & 15)
#pragma unroll
        for (int ks = 0; ks < NKC; ++ks) {
          const auto ta = M::ld(sT + ra * C::LDC + ks * KS + EPL * lg);
#pragma unroll
          for (int m = 0; m < NCHB; ++m)
            vn[m] = M::mma(
                M::ld(sRt + (16 * (ch * NCHB + m) + lr) * C::LDC + ks * KS + EPL * lg), ta,
                vn[m]);
        }
#pragma unroll
        for (int ks = 0; ks < NKK; ++ks) {
          const auto ka = KA(ks);
#pragma unroll
          for (int m = 0; m < NCHB; ++m)
            kd[m] = M::mma(
                ka, M::ld(sD + (16 * (ch * NCHB + m) + lr) * C::LDSK + ks * KS + EPL * lg),
                kd[m]);
          __builtin_amdgcn_sched_barrier(0);
        }
        // second part of the next block's loads
        if (vb + 1 < C::NVB) {
          load_ov(cur, hl, vb + 1);
        } else if (hl + 1 < Gq) {
          load_head(cur, hl + 1);
          load_ov(cur, hl + 1, 0);
        } else if (has_next) {  // the next item's first v-head
          const LocItem nxt = item_of(it_next);
          load_head(nxt, 0);
          load_ov(nxt, 0, 0);
        }
        const f32x4 dec_s = row4(sdec);
        {
#pragma unroll
          for (int m = 0; m < NCHB; ++m)
            st4(sVn + ra * LDB + 16 * (ch * NCHB + m) + 4 * lg, vn[m][0], vn[m][1], vn[m][2],
                vn[m][3]);
          // c_r = e^{gL-g_r} <Vn_r, (K D)_r>: Vn read back at the K D tiles'
          // accumulator positions (this wave's own tiles)
#pragma unroll
          for (int m = 0; m < NCHB; ++m) {
            const f32x4 v4 = M::ld_acc(sVn + 16 * rt * LDB + 16 * (ch * NCHB + m), LDB, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) c_p[i] += dec_s[i] * v4[i] * kd[m][i];
          }
        }
        // ---- phase 4a: dVn = dec * (K D) + scale P^T dO
        f32x4 x[NCHB];
#pragma unroll
        for (int m = 0; m < NCHB; ++m) x[m] = zero4();
#pragma unroll
        for (int ks = 0; ks < NKC; ++ks) {
          const auto pa = M::ld(sPt + ra * C::LDC + ks * KS + EPL * lg);
#pragma unroll
          for (int m = 0; m < NCHB; ++m)
            x[m] = M::mma(
                pa, M::ld_tr(sDO + ks * KS * LDB + 16 * (ch * NCHB + m), LDB),
                x[m]);
        }
#pragma unroll
        for (int m = 0; m < NCHB; ++m) {
          const int vc = 16 * (ch * NCHB + m) + lr;
          float y[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) y[i] = dec_s[i] * kd[m][i] + scale * x[m][i];
          st4(sDVnt + vc * C::LDC + 16 * rt + 4 * lg, y[0], y[1], y[2], y[3]);
        }
      }
      __syncthreads();
      // ---- phase 4b: dk += (dec Vn) D^T;  phase 5: dR = T^T dVn, dv, dbeta/de rows
      // dk += (e^{gL-g} Vn) D^T: the Vn rows scaled in registers
      const float dk_s = sdec[ra];
#pragma unroll
      for (int ks = 0; ks < NKB; ++ks) {
        const auto vna = M::scaled(M::ld(sVn + ra * LDB + ks * KS + EPL * lg), dk_s);
#pragma unroll
        for (int m = 0; m < NCHK; ++m)
          dk[m] = M::mma(vna, M::ld_tr(sD + ks * KS * C::LDSK + 16 * (ch * NCHK + m), C::LDSK),
                         dk[m]);
      }
      f32x4 dr[NCHB];
#pragma unroll
      for (int m = 0; m < NCHB; ++m) dr[m] = zero4();
#pragma unroll
      for (int ks = 0; ks < NKC; ++ks) {
        const auto tta = M::ld_tr(sT + ks * KS * C::LDC + 16 * rt, C::LDC);
#pragma unroll
        for (int m = 0; m < NCHB; ++m)
          dr[m] = M::mma(
              tta, M::ld(sDVnt + (16 * (ch * NCHB + m) + lr) * C::LDC + ks * KS + EPL * lg),
              dr[m]);
      }
      {
      const f32x4 bet_s = row4(sbet), eg_s = row4(seg);
#pragma unroll
      for (int m = 0; m < NCHB; ++m) {
        const int vc = 16 * (ch * NCHB + m) + lr;
        const f32x4 v4 = M::ld_acc(sV + 16 * rt * LDB + 16 * (ch * NCHB + m), LDB, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = 16 * rt + 4 * lg + i;
          const float x = dr[m][i];
          sDR[s * LDB + vc] = from_f32<E>(x);
          // dv = beta dR replaces this lane's own V elements (read above)
          sV[s * LDB + vc] = from_f32<E>(bet_s[i] * x);
          db_p[i] += x * (v4[i] - eg_s[i] * ks_[m][i]);
          de_p[i] -= bet_s[i] * x * ks_[m][i];
        }
      }
      }
      __syncthreads();
      // dv rows of this block, 16 bytes a lane
#pragma unroll
      for (int m = 0; m < LP::NOP; ++m) {
        const int idx = tid + kThreads * m;
        const int r = idx / PB, cv = idx % PB;
        if (idx < 64 * PB && r < rows)
          *reinterpret_cast<uint4 *>(dvtile + r * v_rs + (uint32_t)((v0 + cv * VEC) * sizeof(E))) =
              *reinterpret_cast<const uint4 *>(sV + r * LDB + cv * VEC);
      }
      // ---- phase 6: dP += dO Vn^T, dA -= dR Vn^T, dk += (-beta e^g dR) S^T
      // (the dR rows scaled in registers for the last)
      const float dr_s = -sbet[ra] * seg[ra];
#pragma unroll
      for (int ks = 0; ks < NKB; ++ks) {
        const auto doa = M::ld(sDO + ra * LDB + ks * KS + EPL * lg);
        const auto dra = M::ld(sDR + ra * LDB + ks * KS + EPL * lg);
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
          if (pc0 + cc <= rt) {
            const auto vnb = M::ld(sVn + (16 * (pc0 + cc) + lr) * LDB + ks * KS + EPL * lg);
            dp[cc] = M::mma(doa, vnb, dp[cc]);
            da[cc] = M::mma(dra, vnb, da[cc]);
          }
        const auto drs = M::scaled(dra, dr_s);
#pragma unroll
        for (int m = 0; m < NCHK; ++m)
          dk[m] = M::mma(drs, M::ld_tr(sS + ks * KS * C::LDSK + 16 * (ch * NCHK + m), C::LDSK),
                         dk[m]);
      }
    }
    __syncthreads();  // the block buffers are free: dP*E and dKK reuse them
    if (hl + 1 == Gq && has_next) load_qk(item_of(it_next));
    // ---- phase 7: masks, dP*E, dKK, dgamma row/column terms
    float rs_p[4] = {0.f, 0.f, 0.f, 0.f};
    f32x4 qk[2], kk[2];
    qk_tiles(qk, kk);
    const f32x4 gam_s = row4(sgam), bet_s = row4(sbet);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int t = 16 * (pc0 + cc) + lr;
      const float gt = sgam[t];
      float pe[4], kkv[4], cs = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 16 * rt + 4 * lg + i;
        const float e = (t <= s) ? __builtin_amdgcn_exp2f(gam_s[i] - gt) : 0.f;
        const float dpm = (t <= s) ? scale * dp[cc][i] : 0.f;
        const float dam = (t < s) ? -da[cc][i] : 0.f;
        pe[i] = dpm * e;
        kkv[i] = bet_s[i] * dam * e;
        // P_st = QK_st E_st,  A_st = beta_s KK_st E_st
        const float term = dpm * qk[cc][i] * e + dam * bet_s[i] * kk[cc][i] * e;
        rs_p[i] += term;
        cs += term;
        db_p[i] += dam * kk[cc][i] * e;
      }
      // stored transposed (row t): 4 consecutive elements a lane
      st4(sPE + t * C::LDC + 16 * rt + 4 * lg, pe[0], pe[1], pe[2], pe[3]);
      st4(sKK + t * C::LDC + 16 * rt + 4 * lg, kkv[0], kkv[1], kkv[2], kkv[3]);
      cs += __shfl_xor(cs, 16, 64);
      cs += __shfl_xor(cs, 32, 64);
      if (lg == 0) colp[rt][t] = cs;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float de = sum16(de_p[i]), db = sum16(db_p[i]), rs = sum16(rs_p[i]);
      const float cr = sum16(c_p[i]);
      if (lr == 0) {
        const int s = 16 * rt + 4 * lg + i;
        rowp[0][ch][s] = de;
        rowp[1][ch][s] = db;
        rowp[2][ch][s] = rs;
        rowp[3][ch][s] = cr;
      }
    }
    {
      const float gsum = wave_sum(gl_p);
      if (lane == 0) glp[w] = gsum;
    }
    __syncthreads();
    // ---- phase 8: dq += (dP*E) K;  dk += (dP*E)^T Q + (dKK + dKK^T) K
    // (sPE holds (dP*E)^T, sKK dKK^T: the symmetric sum is the same)
#pragma unroll
    for (int ks = 0; ks < NKC; ++ks) {
      const auto pea = M::ld_tr(sPE + ks * KS * C::LDC + 16 * rt, C::LDC);
      const auto peta = M::ld(sPE + ra * C::LDC + ks * KS + EPL * lg);
      const auto ma = M::ld_sym_tr(sKK + ra * C::LDC + ks * KS + EPL * lg,
                                   sKK + ks * KS * C::LDC + 16 * rt, C::LDC);
#pragma unroll
      for (int m = 0; m < NCHK; ++m) {
        const auto kb = M::ld_tr(sK + ks * KS * C::LDK + 16 * (ch * NCHK + m), C::LDK);
        const auto qb = M::ld_tr(sQ + ks * KS * C::LDK + 16 * (ch * NCHK + m), C::LDK);
        dq[m] = M::mma(pea, kb, dq[m]);
        dk[m] = M::mma(peta, qb, dk[m]);
        dk[m] = M::mma(ma, kb, dk[m]);
        __builtin_amdgcn_sched_barrier(0);  // bound the gathers in flight
      }
    }
    // ---- phase 9: dbeta, dgamma -> dg (reverse cumsum inside the chunk):
    // lane l takes row 63 - l, so the reverse sum is a prefix sum over lanes
    if (w == 0) {
      const int r = 63 - lane;
      const float cr = rowp[3][0][r] + rowp[3][1][r];
      const float csum = wave_sum(cr);
      float gl = 0.f;
#pragma unroll
      for (int i = 0; i < kNW; ++i) gl += glp[i];
      const float de = rowp[0][0][r] + rowp[0][1][r];
      const float db = rowp[1][0][r] + rowp[1][1][r];
      const float rs = rowp[2][0][r] + rowp[2][1][r];
      const float cs = colp[0][r] + colp[1][r] + colp[2][r] + colp[3][r];
      float dgam = seg[r] * de + rs - cs - cr;
      if (r == rows - 1) dgam += csum + seg[63] * gl;
      if (r >= rows) dgam = 0.f;
      const float x = wave_incl_scan(dgam);  // dg_r = sum_{r' >= r} dgam_r'
      if (r < rows) {
        const int64_t gi = (tok0 + r) * p.Hv + h;
        a.dg[gi] = x;
        dbp[gi] = from_f32<E>(db);
      }
    }
    __syncthreads();
  }
#undef QA
#undef KA
  // ---- in-library L2 normalisation: dq, dk so far are with respect to the
  // normalised rows x_hat = x r (held in sQ, sK); back to the raw rows,
  // dx = r (dx_hat - x_hat <x_hat, dx_hat>), the row dot taken over K (this
  // wave's columns, then both column halves through LDS)
  if (p.l2 || a.rq) {
    relane();
    f32x4 xq[NCHK], xk[NCHK];
    float pq[4] = {0.f, 0.f, 0.f, 0.f}, pk[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NCHK; ++m) {
      xq[m] = M::ld_acc(sQ + 16 * rt * C::LDK + 16 * (ch * NCHK + m), C::LDK, lane);
      xk[m] = M::ld_acc(sK + 16 * rt * C::LDK + 16 * (ch * NCHK + m), C::LDK, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pq[i] += xq[m][i] * dq[m][i];
        pk[i] += xk[m][i] * dk[m][i];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float tq = sum16(pq[i]), tk = sum16(pk[i]);
      if (lr == 0) {
        rowp[0][ch][16 * rt + 4 * lg + i] = tq;
        rowp[1][ch][16 * rt + 4 * lg + i] = tk;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 16 * rt + 4 * lg + i;
      const float tq = rowp[0][0][s] + rowp[0][1][s];
      const float tk = rowp[1][0][s] + rowp[1][1][s];
      float fq = 0.f, fk = 0.f;
      if (s < rows) {
        fq = p.l2 ? ls.rq[s] : a.rq[(tok0 + s) * p.Hq + hq];
        fk = p.l2 ? ls.rk[s] : a.rk[(tok0 + s) * p.Hq + hq];
      }
#pragma unroll
      for (int m = 0; m < NCHK; ++m) {
        dq[m][i] = fq * (dq[m][i] - xq[m][i] * tq);
        dk[m][i] = fk * (dk[m][i] - xk[m][i] * tk);
      }
    }
  }
  // ---- dq, dk of the q/k head (sum over its v-heads in order): each lane
  // puts its own elements in place of the q, k elements it alone still
  // reads, then the rows leave 16 bytes a lane
#pragma unroll
  for (int m = 0; m < NCHK; ++m) {
    const int ic = 16 * (ch * NCHK + m) + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 16 * rt + 4 * lg + i;
      sQ[s * C::LDK + ic] = from_f32<E>(dq[m][i]);
      sK[s * C::LDK + ic] = from_f32<E>(dk[m][i]);
    }
  }
  __syncthreads();
  {
    constexpr int PK = K / VEC;
    char *dqtile = reinterpret_cast<char *>(dqp + (tok0 * p.Hq + hq) * K);
    char *dktile = reinterpret_cast<char *>(dkp + (tok0 * p.Hq + hq) * K);
#pragma unroll
    for (int m = 0; m < (64 * PK + kThreads - 1) / kThreads; ++m) {
      const int idx = tid + kThreads * m;
      const int r = idx / PK, cv = idx % PK;
      if (idx < 64 * PK && r < rows) {
        const uint32_t off = r * qk_rs + cv * 16u;
        *reinterpret_cast<uint4 *>(dqtile + off) =
            *reinterpret_cast<const uint4 *>(sQ + r * C::LDK + cv * VEC);
        *reinterpret_cast<uint4 *>(dktile + off) =
            *reinterpret_cast<const uint4 *>(sK + r * C::LDK + cv * VEC);
      }
    }
  }
  __syncthreads();  // sQ, sK read out before the next item's tiles land
  if (has_next) cur = item_of(it_next);
  }
}

// ---------------------------------------------------------------- launch
// GDN_REV_SLICE=0 in the environment runs reverse pass 1 on the general
// segment kernel even where the register-resident one applies (comparisons).
static bool rev_slice_disabled() {
  static const bool off = [] {
    const char *e = getenv("GDN_REV_SLICE");
    return e && e[0] == '0';
  }();
  return off;
}

// GDN_GRAD_SLICE=0 runs the local gradients on local_grad_kernel where the
// 32x32-tile kernel applies (comparisons).
static bool grad_slice_disabled() {
  static const bool off = [] {
    const char *e = getenv("GDN_GRAD_SLICE");
    return e && e[0] == '0';
  }();
  return off;
}

template <typename E, int K, int V>
static hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t st) {
  const Problem &p = a.p;
  const Plan &pl = a.plan;
  FwdArgs fa;
  fa.p = p;
  fa.plan = pl;
  fa.q = a.q;
  fa.k = a.k;
  fa.v = a.v;
  fa.beta = a.beta;
  fa.g = a.g;
  fa.h0 = a.h0;
  fa.o = nullptr;
  fa.ht = nullptr;
  fa.g_cum = nullptr;
  fa.A = nullptr;
  fa.h = nullptr;
  fa.h_e = a.ws + a.wl.hstates;
  fa.tm_ext = const_cast<void *>(a.tm_ext);
  fa.ws = a.ws;
  fa.wl = a.wl.fwd;
  // plan and T; then the per-chunk states, unless the forward left them
  hipError_t e = launch_bwd_prep(fa, a.A, st);
  if (e != hipSuccess) return e;
  if (!a.hcache) {
    e = launch_fwd_states(fa, st);
    if (e != hipSuccess) return e;
  }
  if (pl.total_chunks > 0) {
    if (rev_slice_supported(a) && !rev_slice_disabled()) {
      e = launch_rev_slice_main(a, st);
      if (e != hipSuccess) return e;
    } else {
      KernelTimer kt("rev_main", st);
      rev_segment_kernel<E, K, V, kRMain>
          <<<dim3((unsigned)(pl.total_segs * p.Hv)), kThreads, 0, st>>>(a);
    }
    if (pl.max_segs_per_seq > 1) {
      KernelTimer kt("rev_fix", st);
      rev_segment_kernel<E, K, V, kRFix>
          <<<dim3((unsigned)(pl.total_segs * p.Hv)), kThreads, 0, st>>>(a);
    }
  }
  if (pl.max_segs_per_seq > 1 || pl.has_empty) {
    KernelTimer kt("rev_serial", st);
    rev_serial_kernel<E, K, V><<<dim3((unsigned)(p.N * p.Hv)), kThreads, 0, st>>>(a);
  }
  if (pl.total_chunks > 0 && grad_slice_supported(a) && !grad_slice_disabled()) {
    e = launch_grad_slice(a, st);
    if (e != hipSuccess) return e;
  } else if (pl.total_chunks > 0) {
    KernelTimer kt("local_grad", st);
    // persistent: one workgroup per compute unit (its LDS use leaves room
    // for one), each looping over items
    const int64_t items = pl.total_chunks * p.Hq;
    const int64_t grid = std::min<int64_t>(items, pl.cus > 0 ? pl.cus : 256);
    local_grad_kernel<E, K, V><<<dim3((unsigned)grid), kThreads, 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs &a, hipStream_t st) {
  const int K = a.p.K, V = a.p.V;
#define GDN_KV(E, KK, VV) \
  if (K == KK && V == VV) return launch_bwd_t<E, KK, VV>(a, st);
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

}  // namespace gdn
