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
//          the resulting output corrections; it stops as soon as every
//          element of D is zero or denormal (the gates decay it
//          geometrically; what is dropped then is below 2^-126 per element),
//          recording the leftover E_j otherwise.
//   pass 3 (serial_kernel): per (sequence, head), carries the remaining
//          residual rho_{j+1} = E_j + Phi_j(rho_j) through the segments and
//          writes the final state H_last + rho.  Every step is exact by
//          linearity of the recurrence in the state, up to the dropped
//          denormal remainders.
#include <stdlib.h>

#include "gdn_seg.hpp"

namespace gdn {

// ------------------------------------------------------------------- plan
// Chunk and segment prefix sums over packed sequences (one thread; only
// launched with cu_seqlens).
__global__ void plan_kernel(Problem p, int seg_chunks, int32_t *chunk_prefix,
                            int32_t *seg_prefix) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  int32_t c = 0, s = 0;
  chunk_prefix[0] = 0;
  seg_prefix[0] = 0;
  for (int n = 0; n < p.N; ++n) {
    const int len = p.cu[n + 1] - p.cu[n];
    const int nc = (len + kChunk - 1) / kChunk;
    c += nc;
    s += (nc + seg_chunks - 1) / seg_chunks;
    chunk_prefix[n + 1] = c;
    seg_prefix[n + 1] = s;
  }
}

// ------------------------------------------------------------------- prep
// One workgroup per (chunk, q/k head); its waves take the group's v-heads.
// K K^T is formed once on MFMA.  Per v-head: gate cumsum, the strictly lower
// A = beta_r exp(gamma_r - gamma_j) (k_r . k_j), and T = (I + A)^-1 by a
// blocked inversion on 16 x 16 blocks, all in fp32:
//   diagonal blocks  T_bb = (I + A_bb)^-1  by forward substitution (one lane
//                    per column, the four blocks side by side in one wave);
//   off-diagonal     T_ij = -T_ii (sum_{j<=k<i} A_ik T_kj), level by level
//                    (i - j = 1, 2, 3) as 16x16x16 fp32 MFMA products.
template <typename E, int K>
struct PrepCfg {
  static constexpr int PAD = 32 / (int)sizeof(E);  // conflict-free 16-byte fragment reads
  static constexpr int LDK = K + PAD;
  static constexpr int LDA = 68;                          // fp32 64x64 rows
  static constexpr int bytesK = 64 * LDK * (int)sizeof(E);
  // per wave, 16x16 fp32 blocks with row stride 17 (the MFMA operand reads
  // of 16 rows x 4 columns then hit distinct banks): the 6 off-diagonal A
  // blocks, the 10 lower blocks of T (the 4 diagonal ones first), one
  // product.  The 4 diagonal A blocks, transposed with row stride 20 (float4
  // reads), share the space of T's off-diagonal blocks: they are dead once
  // the diagonal blocks are inverted, before any off-diagonal block is
  // written.  (19 KB a wave: four 2-wave workgroups fit a compute unit.)
  static constexpr int BS = 16 * 17;
  static constexpr int fA = 0, fT = 6 * BS, fM = 16 * BS, fAd = fT + 4 * BS;
  static_assert(4 * 16 * 20 <= 6 * BS, "diagonal A blocks fit the off-diagonal T space");
  // gamma log2(e) and beta of the chunk rows
  static constexpr int fG = fM + BS, fB = fG + 64;
  static constexpr int floatsW = fB + 64;
  static constexpr int bytesW = floatsW * 4;
};

// acc += X * Y for 16x16 fp32 blocks stored row-major with stride ld
__device__ __forceinline__ f32x4 mm16(f32x4 acc, const float *X, const float *Y, int ld) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[lr * ld + 4 * s + lg],
                                               Y[(4 * s + lg) * ld + lr], acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 16x16 accumulator tile -> row-major block (stride ld), optionally negated
__device__ __forceinline__ void put16(float *dst, int ld, f32x4 c, float sgn) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[(4 * lg + i) * ld + lr] = sgn * c[i];
}

// Two waves a workgroup, each taking every other v-head of the item's q/k
// head (the second wave idles when there is one v-head per q/k head).
constexpr int kPrepThreads = 128;

// WN: the normalised q and k rows of every item, and their factors, are
// written out (in-library L2 normalisation with a state cache): the passes
// after this one and the backward read those rows.
template <typename E, int K, bool WN>
__global__ __launch_bounds__(kPrepThreads) __attribute__((amdgpu_waves_per_eu(2))) void prep_kernel(
    FwdArgs a) {
  using C = PrepCfg<E, K>;
  using M = Mma<E>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  E *sK = reinterpret_cast<E *>(smem);
  const Problem &p = a.p;
  const int tid = threadIdx.x, w = wave_of(tid), lane = tid & 63;
  constexpr int nw = kPrepThreads / 64;
  const int G = p.Hv / p.Hq;
  const int lr = lane & 15, lg = lane >> 4;
  // Work items are (chunk, q/k head) pairs; a workgroup takes items
  // blockIdx.x, + gridDim.x, ... and loads the next item's k tile, gates and
  // beta while it computes the current one.
  const int64_t n_items = a.plan.total_chunks * p.Hq;
  struct Item {
    int hq, rows;
    int64_t gid, tok0;
  };
  auto item_of = [&](int64_t it) {
    Item x;
    x.hq = (int)(it % p.Hq);
    x.gid = it / p.Hq;
    const ChunkLoc cl =
        locate_chunk(p, reinterpret_cast<const int32_t *>(a.ws + a.wl.chunk_prefix), x.gid);
    x.tok0 = cl.si.tok0 + (int64_t)cl.c * kChunk;
    x.rows = min(kChunk, cl.si.len - cl.c * kChunk);
    // wave-uniform (scalar registers), so that the buffer descriptors built
    // on it are scalar too (no per-load loop over distinct descriptors)
    x.hq = __builtin_amdgcn_readfirstlane(x.hq);
    x.rows = __builtin_amdgcn_readfirstlane(x.rows);
    x.gid = (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x.gid >> 32)) << 32) |
                      __builtin_amdgcn_readfirstlane((uint32_t)x.gid));
    x.tok0 = (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x.tok0 >> 32)) << 32) |
                       __builtin_amdgcn_readfirstlane((uint32_t)x.tok0));
    return x;
  };
  // raw gate and beta of a v-head of an item (beta stays in the element
  // type until used, so nothing waits for the load); the loads are
  // unconditional, with on = false their range is empty
  auto load_gb = [&](float &gv, E &bv, const Item &x, int hl, bool on) {
    const int64_t g0 = x.tok0 * p.Hv + x.hq * G + hl;
    const uint32_t rs = (uint32_t)p.Hv;
    const uint32_t n = on && hl < G ? (uint32_t)x.rows * rs : 0u;
    const auto rg = raw_buffer(a.g + g0, n * 4u);
    const auto rb = raw_buffer(reinterpret_cast<const E *>(a.beta) + g0, n * (uint32_t)sizeof(E));
    gv = buf_load_elem<float>(rg, (uint32_t)lane * rs * 4u);
    bv = buf_load_elem<E>(rb, (uint32_t)lane * rs * (uint32_t)sizeof(E));
  };
  // this wave's first v-head of the current item (loaded with its k tile, a
  // whole item ahead) and of the next one; the wave's later v-heads of an
  // item (more than two v-heads per q/k head) one v-head ahead
  float gv_f = 0.f, gv_x = 0.f, gv_n = 0.f;
  E bv_f = from_f32<E>(0.f), bv_x = bv_f, bv_n = bv_f;
  const E *kp = reinterpret_cast<const E *>(a.k);
  const E *qp = reinterpret_cast<const E *>(a.q);
  constexpr int VEC = 16 / (int)sizeof(E);
  constexpr int PR = K / VEC;
  constexpr int NP = (64 * PR + kPrepThreads - 1) / kPrepThreads;  // 16-byte pieces a thread
  static_assert(64 * PR % kPrepThreads == 0, "whole rows a thread");
  constexpr int NQV = WN ? NP : 1;
  uint4 kv[NP], qv[NQV];
  const uint32_t qk_rs = (uint32_t)(p.Hq * K * sizeof(E));  // bytes between token rows
  // (the loads are unconditional: with on = false their range is empty)
  auto load_k = [&](const Item &x, bool on) {
    const int64_t e0 = (x.tok0 * p.Hq + x.hq) * K;
    const uint32_t n = on ? (uint32_t)x.rows * qk_rs : 0u;  // rows past the chunk read 0
    const auto rk = raw_buffer(kp + e0, n), rq = raw_buffer(qp + e0, n);
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      const int idx = tid + kPrepThreads * m;
      const uint32_t off = (uint32_t)(idx / PR) * qk_rs + (uint32_t)(idx % PR) * 16u;
      kv[m] = buf_load16(rk, off);
      if (WN) qv[m] = buf_load16(rq, off);
    }
  };
  if (blockIdx.x >= n_items) return;
  Item cur = item_of(blockIdx.x);
  load_gb(gv_f, bv_f, cur, w, true);
  load_k(cur, true);
  E *tmat = reinterpret_cast<E *>(a.tm_ext ? a.tm_ext : a.ws + a.wl.tmat);
  constexpr int LD = 17, BS = C::BS;
  float *W = reinterpret_cast<float *>(smem) + w * C::floatsW;
  float *sA = W + C::fA, *sT = W + C::fT, *sAd = W + C::fAd;
  // lower block (i >= j) of T (diagonal blocks first), off-diagonal block
  // (i > j) of A
#define TB(i, j) (sT + ((i) == (j) ? (i) : 4 + ((i) * ((i) - 1)) / 2 + (j)) * BS)
#define AB(i, j) (sA + (((i) * ((i) - 1)) / 2 + (j)) * BS)

  for (int64_t it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int64_t it_next = it + gridDim.x;
    const bool has_next = it_next < n_items;
    const int hq = cur.hq, rows = cur.rows;
    const int64_t gid = cur.gid, tok0 = cur.tok0;
    // the k tile into LDS (the per-wave buffers that alias it are free);
    // normalised rows out through buffers that end with the chunk's rows
    const int64_t e0 = (tok0 * p.Hq + hq) * K;
    const uint32_t nb = (uint32_t)rows * qk_rs;
    const auto wq = raw_buffer(reinterpret_cast<E *>(a.qn_out) + e0, WN ? nb : 0u);
    const auto wk = raw_buffer(reinterpret_cast<E *>(a.kn_out) + e0, WN ? nb : 0u);
    const auto wrq = raw_buffer(a.rq_out + tok0 * p.Hq + hq, WN ? (uint32_t)rows * p.Hq * 4u : 0u);
    const auto wrk = raw_buffer(a.rk_out + tok0 * p.Hq + hq, WN ? (uint32_t)rows * p.Hq * 4u : 0u);
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      const int idx = tid + kPrepThreads * m;
      const int r = idx / PR, cv = idx % PR;
      float fk = 0.f;
      const uint4 x = (WN || p.l2) ? l2n_piece<E, PR>(kv[m], fk) : kv[m];
      *reinterpret_cast<uint4 *>(sK + r * C::LDK + cv * VEC) = x;
      if (WN) {
        buf_store16(x, wk, (uint32_t)r * qk_rs + (uint32_t)cv * 16u);
        if (cv == 0)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, fk), wrk,
                                                (int)((uint32_t)r * p.Hq * 4u), 0, 0);
      }
    }
    __syncthreads();
    f32x4 kk[10];
    {
      int t = 0;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct <= rt; ++ct) kk[t++] = zero4();
#pragma unroll
      for (int ks = 0; ks < K / M::KS; ++ks) {
        typename M::frag x[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          x[rt] = M::ld(sK + (16 * rt + lr) * C::LDK + ks * M::KS + M::EPL * lg);
        t = 0;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int ct = 0; ct <= rt; ++ct, ++t) kk[t] = M::mma(x[rt], x[ct], kk[t]);
      }
    }
    if (WN) {
      // the q rows (their work overlaps the products above)
#pragma unroll
      for (int m = 0; m < NQV; ++m) {
        const int idx = tid + kPrepThreads * m;
        const int r = idx / PR, cv = idx % PR;
        float fq;
        const uint4 y = l2n_piece<E, PR>(qv[m], fq);
        buf_store16(y, wq, (uint32_t)r * qk_rs + (uint32_t)cv * 16u);
        if (cv == 0)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, fq), wrq,
                                                (int)((uint32_t)r * p.Hq * 4u), 0, 0);
      }
    }
    __syncthreads();  // the per-wave buffers alias sK
    const Item nxt = has_next ? item_of(it_next) : cur;
    load_k(nxt, has_next);
    load_gb(gv_x, bv_x, nxt, w, has_next);
    for (int hl = w; hl < G; hl += nw) {
      const int h = hq * G + hl;
      const int64_t gi = (tok0 + lane) * p.Hv + h;
      const bool first = hl == w;
      const float gv = first ? gv_f : gv_n, bv = to_f32(first ? bv_f : bv_n);
      if (hl + nw < G) load_gb(gv_n, bv_n, cur, hl + nw, true);
      const float gam = wave_incl_scan(gv);
      float *sG = W + C::fG, *sB = W + C::fB;
      sG[lane] = gam * kLog2e;
      sB[lane] = bv;
      wave_sync();
      // A = strict_lower(beta_r exp(gamma_r - gamma_j) KK): off-diagonal
      // blocks row-major, diagonal blocks transposed
      {
        int t = 0;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int ct = 0; ct <= rt; ++ct, ++t) {
            const int j = 16 * ct + lr;
            const float gj = sG[j];
            const f32x4 gr4 = *reinterpret_cast<const f32x4 *>(sG + 16 * rt + 4 * lg);
            const f32x4 br4 = *reinterpret_cast<const f32x4 *>(sB + 16 * rt + 4 * lg);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 16 * rt + 4 * lg + i;
              const float val =
                  (j < r) ? br4[i] * __builtin_amdgcn_exp2f(gr4[i] - gj) * kk[t][i] : 0.f;
              if (ct == rt)
                sAd[(rt * 16 + lr) * 20 + 4 * lg + i] = val;
              else
                AB(rt, ct)[(4 * lg + i) * LD + lr] = val;
            }
          }
      }
      wave_sync();
      // diagonal blocks: lane = (block b, column c)
      {
        const int b = lane >> 4, c = lane & 15;
        const float *at = sAd + b * 16 * 20;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          x[j] = (j == c ? 1.f : 0.f) - x[j];
#pragma unroll
          for (int r0 = (j + 1) & ~3; r0 < 16; r0 += 4) {
            const float4 a4 = *reinterpret_cast<const float4 *>(at + j * 20 + r0);
            if (r0 + 0 > j) x[r0 + 0] += a4.x * x[j];
            if (r0 + 1 > j) x[r0 + 1] += a4.y * x[j];
            if (r0 + 2 > j) x[r0 + 2] += a4.z * x[j];
            if (r0 + 3 > j) x[r0 + 3] += a4.w * x[j];
          }
        }
        float *tb = TB(b, b);
#pragma unroll
        for (int r = 0; r < 16; ++r) tb[r * LD + c] = x[r];
      }
      wave_sync();
      // level 1: T_{b+1,b} = -T_{b+1,b+1} A_{b+1,b} T_bb, the three blocks
      // side by side (each inner product waits in T_{b+1,b}'s own place)
      {
        f32x4 m[3];
#pragma unroll
        for (int b = 0; b < 3; ++b) m[b] = mm16(zero4(), AB(b + 1, b), TB(b, b), LD);
#pragma unroll
        for (int b = 0; b < 3; ++b) put16(TB(b + 1, b), LD, m[b], 1.f);
        wave_sync();
#pragma unroll
        for (int b = 0; b < 3; ++b) m[b] = mm16(zero4(), TB(b + 1, b + 1), TB(b + 1, b), LD);
        wave_sync();
#pragma unroll
        for (int b = 0; b < 3; ++b) put16(TB(b + 1, b), LD, m[b], -1.f);
      }
      wave_sync();
      // level 2: T_{b+2,b} = -T_{b+2,b+2} (A_{b+2,b} T_bb + A_{b+2,b+1} T_{b+1,b})
      {
        f32x4 m[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          m[b] = mm16(zero4(), AB(b + 2, b), TB(b, b), LD);
          m[b] = mm16(m[b], AB(b + 2, b + 1), TB(b + 1, b), LD);
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) put16(TB(b + 2, b), LD, m[b], 1.f);
        wave_sync();
#pragma unroll
        for (int b = 0; b < 2; ++b) m[b] = mm16(zero4(), TB(b + 2, b + 2), TB(b + 2, b), LD);
        wave_sync();
#pragma unroll
        for (int b = 0; b < 2; ++b) put16(TB(b + 2, b), LD, m[b], -1.f);
      }
      wave_sync();
      // level 3: T_30 = -T_33 (A_30 T_00 + A_31 T_10 + A_32 T_20)
      {
        f32x4 m = mm16(zero4(), AB(3, 0), TB(0, 0), LD);
        m = mm16(m, AB(3, 1), TB(1, 0), LD);
        m = mm16(m, AB(3, 2), TB(2, 0), LD);
        put16(TB(3, 0), LD, m, 1.f);
        wave_sync();
        m = mm16(zero4(), TB(3, 3), TB(3, 0), LD);
        wave_sync();
        put16(TB(3, 0), LD, m, -1.f);
      }
      wave_sync();
      // T out (element type, chunk-contiguous rows), 16 bytes a lane, in two
      // halves: each half's values are read from the blocks before its first
      // store.  Pieces of upper blocks read some other block and store 0.
      {
        E *tm = tmat + (gid * p.Hv + h) * 64 * 64;
        constexpr int TPR = 64 / VEC;  // pieces per row
        constexpr int TNP = TPR / 2;   // pieces per lane and half
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint4 tv[TNP];
#pragma unroll
          for (int q = 0; q < TNP; ++q) {
            const int idx = lane + 64 * (q + TNP * half);
            const int r = idx / TPR, c0 = (idx % TPR) * VEC;
            const int rb = r >> 4, cb = c0 >> 4;
            const float *src = TB(rb, cb) + (r & 15) * LD + (c0 & 15);
            E *o = reinterpret_cast<E *>(&tv[q]);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              const float v = src[e];
              o[e] = from_f32<E>(cb <= rb ? v : 0.f);
            }
          }
#pragma unroll
          for (int q = 0; q < TNP; ++q) {
            const int idx = lane + 64 * (q + TNP * half);
            const int r = idx / TPR, c0 = (idx % TPR) * VEC;
            *reinterpret_cast<uint4 *>(tm + r * 64 + c0) = tv[q];
          }
        }
      }
      // fp32 A (rows at their tokens) and the gate cumsum, when asked for
      if (a.A) {
        float *arow = a.A + (tok0 * p.Hv + h) * 64;
#pragma unroll 1
        for (int q = 0; q < 16; ++q) {
          const int idx = lane + 64 * q;
          const int r = idx >> 4, c0 = (idx & 15) * 4;
          const int rb = r >> 4, cb = c0 >> 4;
          float x[4] = {0.f, 0.f, 0.f, 0.f};
          if (cb <= rb) {
            const float *src = TB(rb, cb) + (r & 15) * LD + (c0 & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = src[e];
          }
          if (r < rows) st4(arow + (uint32_t)(r * p.Hv * 64 + c0), x[0], x[1], x[2], x[3]);
        }
      }
      if (a.g_cum && lane < rows) a.g_cum[gi] = gam;
      wave_sync();
    }
    __syncthreads();  // the per-wave buffers are read out before the next k tile lands
    cur = nxt;
    gv_f = gv_x;
    bv_f = bv_x;
  }
#undef TB
#undef AB
}

// T from a caller-supplied A ([B,T,Hv,64] fp32, chunk rows at their tokens);
// padded rows of a last partial chunk become identity rows.
template <typename E>
__global__ __launch_bounds__(256) void tmat_from_a_kernel(FwdArgs a, const float *Ain) {
  const Problem &p = a.p;
  const int h = (int)(blockIdx.x % p.Hv);
  const int64_t gid = blockIdx.x / p.Hv;
  const ChunkLoc cl =
      locate_chunk(p, reinterpret_cast<const int32_t *>(a.ws + a.wl.chunk_prefix), gid);
  const int64_t tok0 = cl.si.tok0 + (int64_t)cl.c * kChunk;
  const int rows = min(kChunk, cl.si.len - cl.c * kChunk);
  E *tm = reinterpret_cast<E *>(a.tm_ext ? a.tm_ext : a.ws + a.wl.tmat) +
          (gid * p.Hv + h) * 64 * 64;
  const float *ab = Ain + (tok0 * p.Hv + h) * 64;  // row r of the chunk at ab + r*Hv*64
  // 4 consecutive columns per thread (16-byte load, one store); rows past
  // the chunk end are rows of the identity
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = threadIdx.x + 256 * it;
    const int r = idx >> 4, c0 = (idx & 15) * 4;
    f32x4 x;
    if (r < rows) {
      x = *reinterpret_cast<const f32x4 *>(ab + (uint32_t)(r * p.Hv * 64 + c0));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (r == c0 + e) ? 1.f : 0.f;
    }
    st4(tm + r * 64 + c0, x[0], x[1], x[2], x[3]);
  }
}

// ------------------------------------------------------ segment machinery
enum { kMain = 0, kFix = 1 };

template <typename E, int K, int V>
struct FwdLds {
  using G = Geo<E, K, V>;
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + 64 * G::LDK;
  static constexpr int oV = oK + 64 * G::LDK;
  static constexpr int oSt = oV + 64 * G::LDV;
  static constexpr int oT = oSt + V * G::LDK;
  static constexpr int oPt = oT + 64 * G::LDC;  // P^T [64][64]
  static constexpr int oRt = oPt + 64 * G::LDC;
  static constexpr int oVnt = oRt + V * G::LDC;
  static constexpr int nE = oVnt + V * G::LDC;
  static constexpr int bytes = nE * (int)sizeof(E);
};

struct Smem {
  char *base;
  GateLds gate;
  int *flag;
};

template <typename E, int K, int V, bool WANT_V>
__device__ __forceinline__ void fwd_commit(const Pref<E, K, V> &pf, const Smem &S, bool l2,
                                           int tid = threadIdx.x) {
  using G = Geo<E, K, V>;
  using L = FwdLds<E, K, V>;
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
  if (WANT_V) {
#pragma unroll
    for (int m = 0; m < G::NV; ++m) {
      const int idx = tid + kThreads * m;
      if (idx < G::PV) {
        const int r = idx / PVr, cv = idx % PVr;
        *reinterpret_cast<uint4 *>(sm + L::oV + r * G::LDV + cv * G::VEC) = pf.v[m];
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
  gate_commit(pf.g, pf.beta(), S.gate, tid);
}

// Runs chunks [c_begin, c_end) of one (sequence, v-head) starting from the
// state in `st`.  kMain: normal recurrence, O written.  kFix: homogeneous
// recurrence (v = 0), O incremented, stops early once the state is zero or
// denormal in every element.  h (optional) receives (kMain) or accumulates
// (kFix) the state entering each chunk.  Returns true when a kFix run ended
// that way.
template <typename E, int K, int V, int MODE, bool WRITE_O>
__device__ __forceinline__ bool run_chunks(const FwdArgs &a, const Smem &S,
                                           Tiles<Geo<E, K, V>::NTS> &st, const SeqInfo &si,
                                           int64_t chunk_gid0, int c_begin, int c_end, int h) {
  using G = Geo<E, K, V>;
  using L = FwdLds<E, K, V>;
  using M = Mma<E>;
  constexpr int KS = M::KS, EPL = M::EPL;
  constexpr int NKK = K / KS;   // k-steps over the key dimension
  constexpr int NKC = 64 / KS;  // k-steps over the chunk dimension
  constexpr int NCH = G::NCH;
  constexpr bool WANT_V = MODE == kMain;
  const Problem &p = a.p;
  E *sm = reinterpret_cast<E *>(S.base);
  const E *sQ = sm + L::oQ;
  const E *sK = sm + L::oK;
  const E *sV = sm + L::oV;
  E *sSt = sm + L::oSt;
  const E *sT = sm + L::oT;
  E *sPt = sm + L::oPt;
  E *sRt = sm + L::oRt;
  E *sVnt = sm + L::oVnt;
  const int w = wave_of(threadIdx.x);
  const int rt = w & 3;            // chunk-row tile of this wave
  const int ct0 = (w >> 2) * NCH;  // first V column tile of this wave
  const float scale = p.scale;
  E *op = reinterpret_cast<E *>(a.o);
  const E *qp = reinterpret_cast<const E *>(a.q);
  const E *kp = reinterpret_cast<const E *>(a.k);
  const E *vp = reinterpret_cast<const E *>(a.v);
  const E *bp = reinterpret_cast<const E *>(a.beta);
  const E *tmat = reinterpret_cast<const E *>(a.tm_ext ? a.tm_ext : a.ws + a.wl.tmat);
  // pass-1 output rows are staged in the R^T buffer when they fit there
  constexpr bool STAGE_O = WRITE_O && MODE == kMain && 64 * G::LDV <= V * G::LDC;

  if (c_begin >= c_end)
    return MODE == kFix ? !block_any(tiles_significant<E, K, V>(st), S.flag) : false;
  const float thr = MODE == kFix ? fix_threshold<E, K, V>(st, S.flag) : 0.f;
  Pref<E, K, V> pf;
  {
    const int rows = min(kChunk, si.len - c_begin * kChunk);
    pref_load<E, K, V, WANT_V>(pf, p, qp, kp, vp, tmat, a.g, bp,
                               si.tok0 + (int64_t)c_begin * kChunk, rows, h,
                               chunk_gid0 + c_begin);
    fwd_commit<E, K, V, WANT_V>(pf, S, p.l2);
    tiles_to_lds_t<E, K, V>(st, sSt);
  }
  __syncthreads();
  bool zero_exit = false;
  for (int c = c_begin; c < c_end && !zero_exit; ++c) {
    const int tid = opaque_tid(), lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int64_t tok0 = si.tok0 + (int64_t)c * kChunk;
    const int rows = pf.rows;
    if (a.h) {
      float *hs = a.h + ((chunk_gid0 + c) * p.Hv + h) * (int64_t)K * V;
      tiles_store<E, K, V>(st, hs, nullptr, MODE == kFix, tid);
    }
    // per-chunk states (lane layout): pass 1 stores the LDS mirror written
    // last step; the fix-up pass adds its correction, reading the stored
    // values here and writing the sums after phase A
    E *hs = a.h_e ? reinterpret_cast<E *>(a.h_e) + ((chunk_gid0 + c) * p.Hv + h) * (int64_t)K * V
                  : nullptr;
    // fix-up pass: this lane's output elements (row 16 rt + (l & 15) of the
    // chunk, the 4-column pieces of its wave's V half), read here and
    // incremented in phase C
    typename E4<E>::type o_old[NCH];
    if (MODE == kFix && WRITE_O) {
      const int r = 16 * rt + lr;
      const char *orow = reinterpret_cast<const char *>(op + (tok0 * p.Hv + h) * V) +
                         (uint32_t)r * (uint32_t)(p.Hv * V * sizeof(E));
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2) {
        o_old[c2] = typename E4<E>::type{};
        if (r < rows)
          o_old[c2] = *reinterpret_cast<const typename E4<E>::type *>(
              orow + (uint32_t)((16 * (ct0 + c2) + 4 * lg) * sizeof(E)));
      }
    }
    TilesOld<E, K, V> hold;
    if (hs) {
      if (MODE == kFix)
        tiles_old_l<E, K, V>(hold, hs, tid);
      else
        mirror_store_l<E, K, V>(sSt, hs, tid);
    }
    // the next chunk's inputs travel while this whole chunk is computed (this
    // chunk's inputs were committed to LDS at the end of the previous one)
    if (c + 1 < c_end) {
      const int rows1 = min(kChunk, si.len - (c + 1) * kChunk);
      pref_load<E, K, V, WANT_V>(pf, p, qp, kp, vp, tmat, a.g, bp, tok0 + kChunk, rows1, h,
                                 chunk_gid0 + c + 1, tid);
    }
    // ---- phase A: (Q S)^T, K S (this wave's row tile, its half of V), Q K^T
    const int pc0 = 2 * (w >> 2);  // P column tiles of this wave: pc0, pc0 + 1
    f32x4 qs[NCH], kss[NCH];
    f32x4 qk[2] = {zero4(), zero4()};
#pragma unroll
    for (int c2 = 0; c2 < NCH; ++c2) {
      qs[c2] = zero4();
      kss[c2] = zero4();
    }
    // Fragments are double-buffered over the k-steps (the reads of step
    // ks + 1 are issued before the products of step ks).  The two Q K^T tiles
    // are formed whether or not they lie below the diagonal (P masks them),
    // which keeps the step free of branches.
    {
      typename M::frag fq[2], fk[2], fb[2][NCH], fkb[2][2];
      auto load_step = [&](int ks, int sl) {
        fq[sl] = M::ld(sQ + (16 * rt + lr) * G::LDK + ks * KS + EPL * lg);
        fk[sl] = M::ld(sK + (16 * rt + lr) * G::LDK + ks * KS + EPL * lg);
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2)
          fb[sl][c2] = M::ld(sSt + (16 * (ct0 + c2) + lr) * G::LDK + ks * KS + EPL * lg);
        if (WRITE_O) {
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
        for (int c2 = 0; c2 < NCH; ++c2) {
          // the output is built transposed (rows v, columns r): each lane
          // then holds 4 consecutive values of one output row
          if (WRITE_O) qs[c2] = M::mma(fb[sl][c2], fq[sl], qs[c2]);
          kss[c2] = M::mma(fk[sl], fb[sl][c2], kss[c2]);
        }
        if (WRITE_O) {
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) qk[cc] = M::mma(fq[sl], fkb[sl][cc], qk[cc]);
        }
      }
    }
    if (MODE == kFix && hs) tiles_accumulate_l<E, K, V>(st, hold, hs, tid);
    float eg_r[4], b_r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rt + 4 * lg + i;
      eg_r[i] = S.gate.eg[r];
      b_r[i] = S.gate.bet[r];
    }
    if (WRITE_O) {
      // P = lower_incl(Q K^T * E), stored transposed: this wave does column
      // tiles pc0, pc0 + 1 of its row tile
      float gam_r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) gam_r[i] = S.gate.gam[16 * rt + 4 * lg + i];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int j = 16 * (pc0 + cc) + lr;
        const float gj = S.gate.gam[j];
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * lg + i;
          pv[i] = (j <= r) ? qk[cc][i] * __builtin_amdgcn_exp2f(gam_r[i] - gj) : 0.f;
        }
        st4(sPt + j * G::LDC + 16 * rt + 4 * lg, pv[0], pv[1], pv[2], pv[3]);
      }
    }
    // V at this lane's accumulator positions (all reads issued first)
    f32x4 vv[NCH];
#pragma unroll
    for (int c2 = 0; c2 < NCH; ++c2)
      vv[c2] =
          WANT_V ? M::ld_acc(sV + 16 * rt * G::LDV + 16 * (ct0 + c2), G::LDV, lane) : zero4();
#pragma unroll
    for (int c2 = 0; c2 < NCH; ++c2) {
      const int vc = 16 * (ct0 + c2) + lr;
      float rr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) rr[i] = b_r[i] * (vv[c2][i] - eg_r[i] * kss[c2][i]);
      st4(sRt + vc * G::LDC + 16 * rt + 4 * lg, rr[0], rr[1], rr[2], rr[3]);
    }
    __syncthreads();
    // ---- phase B: Vn = T R (row tile rt, this wave's half of V)
    {
      typename M::frag ta[NKC];
#pragma unroll
      for (int ks = 0; ks < NKC; ++ks)
        ta[ks] = M::ld(sT + (16 * rt + lr) * G::LDC + ks * KS + EPL * lg);
      f32x4 vn[NCH];
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2) vn[c2] = zero4();
#pragma unroll
      for (int ks = 0; ks < NKC; ++ks)
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2)
          vn[c2] = M::mma(
              ta[ks], M::ld(sRt + (16 * (ct0 + c2) + lr) * G::LDC + ks * KS + EPL * lg),
              vn[c2]);
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2)
        st4(sVnt + (16 * (ct0 + c2) + lr) * G::LDC + 16 * rt + 4 * lg, vn[c2][0], vn[c2][1],
            vn[c2][2], vn[c2][3]);
    }
    __syncthreads();
    // ---- phase C: output rows of this wave, state update of its tiles
    if (WRITE_O) {
      // O^T = diag-scaled (Q S)^T + Vn^T P^T: P as the B operand (column r,
      // contraction over j) comes from P^T by transpose reads
      typename M::frag pb[NKC];
#pragma unroll
      for (int ks = 0; ks < NKC; ++ks) pb[ks] = M::ld_tr(sPt + ks * KS * G::LDC + 16 * rt, G::LDC, lane);
      const int r = 16 * rt + lr;  // the output row this lane holds
      const float eg_c = S.gate.eg[r];
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2)
#pragma unroll
        for (int i = 0; i < 4; ++i) qs[c2][i] *= eg_c;
#pragma unroll
      for (int ks = 0; ks < NKC; ++ks)
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2)
          qs[c2] = M::mma(M::ld(sVnt + (16 * (ct0 + c2) + lr) * G::LDC + ks * KS + EPL * lg),
                          pb[ks], qs[c2]);
      if (STAGE_O) {
        // this lane's row piece into the R^T buffer (free since phase B);
        // the rows leave as whole rows after the next barrier
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2) {
          const f32x4 val = qs[c2] * scale;
          st4(sRt + r * G::LDV + 16 * (ct0 + c2) + 4 * lg, val[0], val[1], val[2], val[3]);
        }
      } else if (r < rows) {
        char *orow = reinterpret_cast<char *>(op + (tok0 * p.Hv + h) * V) +
                     (uint32_t)r * (uint32_t)(p.Hv * V * sizeof(E));
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2) {
          E *dst = reinterpret_cast<E *>(orow + (uint32_t)((16 * (ct0 + c2) + 4 * lg) * sizeof(E)));
          f32x4 val = qs[c2] * scale;
          if (MODE == kFix) {
#pragma unroll
            for (int i = 0; i < 4; ++i) val[i] += to_f32(o_old[c2][i]);
          }
          st4(dst, val[0], val[1], val[2], val[3]);
        }
      }
    }
    if (G::owns(w)) {
      const float egL = S.gate.eg[63];
      const int srt = G::srt(w), sct = G::sct(w);
      typename M::frag kt[NKC];
#pragma unroll
      for (int ks = 0; ks < NKC; ++ks) {
        kt[ks] = M::ld_tr_scaled(sK + ks * KS * G::LDK + 16 * srt, G::LDK, S.gate.dec + ks * KS,
                                 lane);
      }
#pragma unroll
      for (int m = 0; m < G::NTS; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[m][i] *= egL;
#pragma unroll
      for (int ks = 0; ks < NKC; ++ks)
#pragma unroll
        for (int m = 0; m < G::NTS; ++m)
          st[m] = M::mma(kt[ks],
                         M::ld(sVnt + (16 * (sct + m) + lr) * G::LDC + ks * KS + EPL * lg),
                         st[m]);
    }
    tiles_to_lds_t<E, K, V>(st, sSt, tid);
    if (MODE == kFix) {
      zero_exit = !block_any(tiles_significant<E, K, V>(st, thr), S.flag);
    } else {
      __syncthreads();
    }
    if (STAGE_O) {
      // the staged output rows, 16 bytes a lane; rows past the chunk's end
      // fall outside the buffer's range and are dropped (no branch, so the
      // commit's wait for the prefetch does not wait for these stores)
      constexpr int PR = V / G::VEC;
      const uint32_t o_rs = (uint32_t)(p.Hv * V * sizeof(E));
      const auto ob = raw_buffer(op + (tok0 * p.Hv + h) * V, (uint32_t)rows * o_rs);
#pragma unroll
      for (int m = 0; m < (64 * PR + kThreads - 1) / kThreads; ++m) {
        const int idx = tid + kThreads * m;
        const int rr = idx / PR, cv = idx % PR;
        if (64 * PR % kThreads == 0 || idx < 64 * PR)
          buf_store16(*reinterpret_cast<const uint4 *>(sRt + rr * G::LDV + cv * G::VEC), ob,
                      (uint32_t)rr * o_rs + (uint32_t)(cv * 16));
      }
    }
    if (c + 1 < c_end && !zero_exit) {
      fwd_commit<E, K, V, WANT_V>(pf, S, p.l2, tid);
      __syncthreads();
    }
  }
  return zero_exit;
}

#define GDN_FWD_LDS(E, K, V)                                                   \
  __shared__ __attribute__((aligned(16))) char smem_[FwdLds<E, K, V>::bytes]; \
  __shared__ float sg_[4][64];                                                 \
  __shared__ int sflag_[kNW];                                                  \
  Smem S;                                                                      \
  S.base = smem_;                                                              \
  S.gate.gam = sg_[0];                                                         \
  S.gate.eg = sg_[1];                                                          \
  S.gate.dec = sg_[2];                                                         \
  S.gate.bet = sg_[3];                                                         \
  S.flag = sflag_;

// pass 1 (kMain) and pass 2 (kFix) over (segment, v-head) work items.
template <typename E, int K, int V, int MODE, bool WRITE_O>
__global__ __launch_bounds__(kThreads) void segment_kernel(FwdArgs a) {
  using G = Geo<E, K, V>;
  GDN_FWD_LDS(E, K, V)
  const Problem &p = a.p;
  const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
  const int h = (int)(wid % p.Hv);
  const int64_t sg = wid / p.Hv;
  const SegLoc sl =
      locate_segment(p, a.plan.seg_chunks,
                     reinterpret_cast<const int32_t *>(a.ws + a.wl.chunk_prefix),
                     reinterpret_cast<const int32_t *>(a.ws + a.wl.seg_prefix), sg);
  if (MODE == kFix && sl.j == 0) return;
  const int64_t KV = (int64_t)K * V;
  float *hseg = reinterpret_cast<float *>(a.ws + a.wl.hseg);
  float *eseg = reinterpret_cast<float *>(a.ws + a.wl.eseg);
  int32_t *flags = reinterpret_cast<int32_t *>(a.ws + a.wl.flags);

  Tiles<G::NTS> st;
  if (MODE == kMain) {
    const float *src =
        (sl.j == 0 && a.h0) ? a.h0 + ((int64_t)sl.n * p.Hv + h) * KV : nullptr;
    tiles_load<E, K, V>(st, src);
  } else {
    tiles_load<E, K, V>(st, hseg + ((sg - 1) * p.Hv + h) * KV);
  }
  const bool zero =
      run_chunks<E, K, V, MODE, WRITE_O>(a, S, st, sl.si, sl.chunk0, sl.c_begin, sl.c_end, h);
  if (MODE == kMain) {
    if (sl.nseg > 1) tiles_store<E, K, V>(st, hseg + (sg * p.Hv + h) * KV, nullptr, false);
    if (sl.nseg == 1 && a.ht)
      tiles_store<E, K, V>(st, a.ht + ((int64_t)sl.n * p.Hv + h) * KV, nullptr, false);
  } else {
    if (!zero) tiles_store<E, K, V>(st, eseg + (sg * p.Hv + h) * KV, nullptr, false);
    if (threadIdx.x == 0) flags[sg * p.Hv + h] = zero ? 0 : 1;
  }
}

// pass 3: per (sequence, v-head), serial residual carry across segments.
template <typename E, int K, int V, bool WRITE_O>
__global__ __launch_bounds__(kThreads) void serial_kernel(FwdArgs a) {
  using G = Geo<E, K, V>;
  GDN_FWD_LDS(E, K, V)
  const Problem &p = a.p;
  const int h = (int)(blockIdx.x % p.Hv);
  const int n = (int)(blockIdx.x / p.Hv);
  const SegLoc sl =
      locate_sequence(p, a.plan.seg_chunks,
                      reinterpret_cast<const int32_t *>(a.ws + a.wl.chunk_prefix),
                      reinterpret_cast<const int32_t *>(a.ws + a.wl.seg_prefix), n);
  const int64_t KV = (int64_t)K * V;
  if (sl.nseg == 0) {  // empty sequence: the final state is the initial one
    if (a.ht) {
      float *dst = a.ht + ((int64_t)n * p.Hv + h) * KV;
      const float *src = a.h0 ? a.h0 + ((int64_t)n * p.Hv + h) * KV : nullptr;
      copy_state<K, V>(dst, src);
    }
    return;
  }
  if (sl.nseg == 1) return;
  const float *hseg = reinterpret_cast<const float *>(a.ws + a.wl.hseg);
  const float *eseg = reinterpret_cast<const float *>(a.ws + a.wl.eseg);
  const int32_t *flags = reinterpret_cast<const int32_t *>(a.ws + a.wl.flags);
  const int64_t last = sl.seg0 + sl.nseg - 1;
  // common case: every pass-2 propagation died out inside its segment
  bool any_flag = false;
  for (int j = 1 + (int)threadIdx.x; j < sl.nseg; j += blockDim.x)
    any_flag |= flags[(sl.seg0 + j) * p.Hv + h] != 0;
  if (!block_any(any_flag, S.flag)) {
    if (a.ht) {
      float *dst = a.ht + ((int64_t)n * p.Hv + h) * KV;
      const float *src = hseg + (last * p.Hv + h) * KV;
      copy_state<K, V>(dst, src);
    }
    return;
  }
  Tiles<G::NTS> st;
  tiles_zero<E, K, V>(st);
  bool nonzero = false;
  for (int j = 1; j < sl.nseg; ++j) {
    const int64_t sg = sl.seg0 + j;
    if (nonzero) {
      const int c_begin = j * a.plan.seg_chunks;
      const int c_end = min(c_begin + a.plan.seg_chunks, sl.si.nchunks);
      run_chunks<E, K, V, kFix, WRITE_O>(a, S, st, sl.si, sl.chunk0, c_begin, c_end, h);
      __syncthreads();
    }
    if (flags[sg * p.Hv + h]) {
      Tiles<G::NTS> e;
      tiles_load<E, K, V>(e, eseg + (sg * p.Hv + h) * KV);
#pragma unroll
      for (int m = 0; m < G::NTS; ++m) st[m] += e[m];
    }
    nonzero = block_any(tiles_significant<E, K, V>(st), S.flag);
  }
  if (a.ht)
    tiles_store<E, K, V>(st, a.ht + ((int64_t)n * p.Hv + h) * KV,
                         hseg + (last * p.Hv + h) * KV, false);
}

// ---------------------------------------------------------------- launch
template <typename E, int K>
static void launch_prep(const FwdArgs &a, const float *Ain, hipStream_t st) {
  const Problem &p = a.p;
  const Plan &pl = a.plan;
  if (Ain) {
    KernelTimer kt("tmat_from_a", st);
    tmat_from_a_kernel<E><<<dim3((unsigned)(pl.total_chunks * p.Hv)), 256, 0, st>>>(a, Ain);
    return;
  }
  using C = PrepCfg<E, K>;
  constexpr int nw = kPrepThreads / 64;
  const size_t lds = (size_t)(C::bytesK > nw * C::bytesW ? C::bytesK : nw * C::bytesW);
  // persistent: as many workgroups as the LDS lets the compute units hold
  const int64_t items = pl.total_chunks * p.Hq;
  const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(8, (160 * 1024) / (int64_t)lds));
  const int64_t grid = std::min<int64_t>(items, per_cu * (pl.cus > 0 ? pl.cus : 256));
  KernelTimer kt("prep", st);
  if (p.l2 && a.qn_out)
    prep_kernel<E, K, true><<<dim3((unsigned)grid), kPrepThreads, lds, st>>>(a);
  else
    prep_kernel<E, K, false><<<dim3((unsigned)grid), kPrepThreads, lds, st>>>(a);
}

// GDN_FWD_SLICE=0 in the environment runs pass 1 on the general segment
// kernel even where the register-resident one applies (for comparisons).
static bool slice_disabled() {
  static const bool off = [] {
    const char *e = getenv("GDN_FWD_SLICE");
    return e && e[0] == '0';
  }();
  return off;
}

// Stage bits of launch_fwd_t: the plan prefix sums and prep (T from k or
// from a given A), then the segment passes.
constexpr int kStagePlan = 1, kStageT = 2, kStageSegs = 4;

template <typename E, int K, int V, bool WRITE_O>
static hipError_t launch_fwd_t(const FwdArgs &a, const float *Ain, hipStream_t st, int stages) {
  const Problem &p = a.p;
  const Plan &pl = a.plan;
  if ((stages & kStagePlan) && p.cu) {
    KernelTimer kt("plan", st);
    plan_kernel<<<1, 64, 0, st>>>(p, pl.seg_chunks,
                                  reinterpret_cast<int32_t *>(a.ws + a.wl.chunk_prefix),
                                  reinterpret_cast<int32_t *>(a.ws + a.wl.seg_prefix));
  }
  if ((stages & kStageT) && pl.total_chunks > 0) launch_prep<E, K>(a, Ain, st);
  if (!(stages & kStageSegs)) return hipGetLastError();
  if (a.qn_out && a.p.l2 && (stages & kStageT)) {
    // prep has written the normalised rows: the passes read those
    FwdArgs b = a;
    b.q = a.qn_out;
    b.k = a.kn_out;
    b.p.l2 = 0;
    return launch_fwd_t<E, K, V, WRITE_O>(b, Ain, st, stages & kStageSegs);
  }
  if (pl.total_chunks > 0) {
    if (WRITE_O && fwd_slice_supported(a) && !slice_disabled()) {
      const hipError_t e = launch_fwd_slice_main(a, st);
      if (e != hipSuccess) return e;
    } else {
      KernelTimer kt(WRITE_O ? "fwd_main" : "state_main", st);
      segment_kernel<E, K, V, kMain, WRITE_O>
          <<<dim3((unsigned)(pl.total_segs * p.Hv)), kThreads, 0, st>>>(a);
    }
    if (pl.max_segs_per_seq > 1) {
      KernelTimer kt(WRITE_O ? "fwd_fix" : "state_fix", st);
      segment_kernel<E, K, V, kFix, WRITE_O>
          <<<dim3((unsigned)(pl.total_segs * p.Hv)), kThreads, 0, st>>>(a);
    }
  }
  if (pl.max_segs_per_seq > 1 || pl.has_empty) {
    KernelTimer kt(WRITE_O ? "fwd_serial" : "state_serial", st);
    serial_kernel<E, K, V, WRITE_O><<<dim3((unsigned)(p.N * p.Hv)), kThreads, 0, st>>>(a);
  }
  return hipGetLastError();
}

template <bool WRITE_O>
static hipError_t dispatch_kv(const FwdArgs &a, const float *Ain, hipStream_t st, int stages) {
  const int K = a.p.K, V = a.p.V;
#define GDN_KV(E, KK, VV) \
  if (K == KK && V == VV) return launch_fwd_t<E, KK, VV, WRITE_O>(a, Ain, st, stages);
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

hipError_t launch_fwd(const FwdArgs &a, hipStream_t st) {
  return dispatch_kv<true>(a, nullptr, st, kStagePlan | kStageT | kStageSegs);
}

// The backward's prep: plan prefix sums and, unless a state cache holds it,
// T (from the forward's A if given).
hipError_t launch_bwd_prep(const FwdArgs &a, const float *Ain, hipStream_t st) {
  return dispatch_kv<false>(a, Ain, st, kStagePlan | (a.tm_ext ? 0 : kStageT));
}

// Forward state recompute for the backward: states only (a.h_e), no output.
hipError_t launch_fwd_states(const FwdArgs &a, hipStream_t st) {
  return dispatch_kv<false>(a, nullptr, st, kStageSegs);
}

}  // namespace gdn
