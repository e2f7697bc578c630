// Reverse pass 1 of the backward (the state-gradient recurrence) with the
// gradient held in registers, for bf16 problems with K = V = 128 (other
// shapes take rev_segment_kernel of gdn_bwd.hip).
//
// Per 64-token chunk, visited from the last to the first, with D the
// gradient of the state leaving the chunk (the same reverse step as
// rev_segment_kernel):
//   dVn = diag(e^(gamma_L - gamma)) K D + scale P^T dO
//   X   = -diag(beta e^gamma) T^T dVn
//   D  <- e^gamma_L D + K^T X + Q^T diag(scale e^gamma) dO
// D's V columns are independent; the wave roles, buffer sets and operand
// layouts are those of gdn_slice.hpp.  Chain wave j keeps columns
// [32 j, 32 j + 32) of D and stores the gradient leaving every chunk into the
// backward's per-chunk gradients in the lane layout (gdn_seg.hpp), as whole
// 1 KB pieces.  Helper waves stage the previous chunk: q, k, dO, T, the
// gates, and P^T (P = lower_incl(Q K^T * E)) on MFMA.
#include "gdn_slice.hpp"

namespace gdn {
namespace rslice {

using namespace slice;

// One buffer set (element offsets) and its gates (float offsets).
constexpr int oQ = 0, oK = oQ + 64 * PITCH, oDO = oK + 64 * PITCH, oT = oDO + 64 * PITCH,
              oPt = oT + 64 * PITCH_C, SET_ELEMS = oPt + 64 * PITCH_C;
// gam (gamma log2 e), eg = e^gamma, dec = e^(gamma_L - gamma),
// wq = scale e^gamma, wk = -beta e^gamma
constexpr int gGam = 0, gEg = 64, gDec = 128, gWq = 192, gWk = 256, GATE_FLOATS = 320;
constexpr int SET_BYTES = SET_ELEMS * 2;
constexpr int LDS_BYTES = 2 * SET_BYTES + 2 * GATE_FLOATS * 4 + 3 * 64 * 4;
static_assert(SET_BYTES % 16 == 0, "sets stay 16-byte aligned");
static_assert(LDS_BYTES <= 160 * 1024, "two buffer sets fit the LDS of a compute unit");

// ------------------------------------------------------------------ helpers
// Roles (HW = wave - 4):
//   0  q, k and T rows 0..31; P^T tile (rows 0..31, columns 0..31)
//   1  dO rows
//   2  q, k and T rows 32..63; P^T tile (rows 32..63, columns 32..63)
//   3  the gates; P^T tile (rows 0..31, columns 32..63), from q rows 32..63
//      and k rows 0..31 that it writes itself (the same bytes roles 2 and 0
//      write there)
// (P^T is upper triangular: its tile (rows 32..63, columns 0..31) is zero
// and never read.)
template <int HW>
struct HelperRegs {
  // roles 0, 2, 3: q rows (buf[0..7]) and k rows (buf[8..15]) of one half,
  // 16-byte piece lane & 15 of row 4 m + (lane >> 4); roles 0, 2 also 4
  // pieces of T (buf[16..19]); role 1: dO rows (buf[0..15])
  static constexpr int NB = (HW == 0 || HW == 2) ? 20 : 16;
  uint4 buf[NB];
  float g;
  float b;
};
// q rows of role HW: 0..31 (role 0) or 32..63; k rows: 32..63 (role 2) or 0..31
__device__ __forceinline__ constexpr int q_half(int hw) { return hw == 0 ? 0 : 1; }
__device__ __forceinline__ constexpr int k_half(int hw) { return hw == 2 ? 1 : 0; }

template <int HW>
// (parts: 1 = everything but the k rows, 2 = the k rows, 3 = all)
__device__ __forceinline__ void helper_load(HelperRegs<HW> &R, const BwdArgs &a, const Item &it,
                                            int c, int lane, int part = 3) {
  const Problem &p = a.p;
  const int64_t tok0 = it.sl.si.tok0 + (int64_t)c * kChunk;
  const int rows = min(kChunk, it.sl.si.len - c * kChunk);
  const int r16 = lane >> 4, pc = lane & 15;
  if (HW != 1) {
    const uint32_t rs = (uint32_t)(p.Hq * K * 2);
    const bf16 *qb = reinterpret_cast<const bf16 *>(a.q) + (tok0 * p.Hq + it.hq) * K;
    const bf16 *kb = reinterpret_cast<const bf16 *>(a.k) + (tok0 * p.Hq + it.hq) * K;
    const auto rq = rsrc_of(qb, (uint32_t)rows * rs), rk = rsrc_of(kb, (uint32_t)rows * rs);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint32_t rq0 = (uint32_t)(32 * q_half(HW) + 4 * m + r16);
      const uint32_t rk0 = (uint32_t)(32 * k_half(HW) + 4 * m + r16);
      if (part & 1) R.buf[m] = bload16(rq, rq0 * rs + 16u * pc);
      if (part & 2) R.buf[8 + m] = bload16(rk, rk0 * rs + 16u * pc);
    }
    if (!(part & 1)) return;
  } else {
    const uint32_t rs = (uint32_t)(p.Hv * V * 2);
    const bf16 *ob = reinterpret_cast<const bf16 *>(a.dout) + (tok0 * p.Hv + it.h) * V;
    const auto ro = rsrc_of(ob, (uint32_t)rows * rs);
#pragma unroll
    for (int m = 0; m < 16; ++m) R.buf[m] = bload16(ro, (uint32_t)(4 * m + r16) * rs + 16u * pc);
  }
  if (HW == 0 || HW == 2) {
    const int64_t cgid = it.sl.chunk0 + c;
    const uint4 *tb = reinterpret_cast<const uint4 *>(
        reinterpret_cast<const bf16 *>(a.tm_ext ? a.tm_ext : a.ws + a.wl.fwd.tmat) +
        (cgid * p.Hv + it.h) * 64 * 64);
#pragma unroll
    for (int m = 0; m < 4; ++m) R.buf[16 + m] = tb[lane + 64 * (m + 2 * HW)];
  }
  const uint32_t gs = (uint32_t)(p.Hv * 4);
  const auto rg = rsrc_of(a.g + tok0 * p.Hv + it.h, (uint32_t)rows * gs);
  R.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, (int)(lane * gs), 0, 0));
  const uint32_t bs = (uint32_t)(p.Hv * 2);
  const auto rb = rsrc_of(reinterpret_cast<const bf16 *>(a.beta) + tok0 * p.Hv + it.h,
                          (uint32_t)rows * bs);
  const unsigned short braw = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)(lane * bs), 0, 0);
  R.b = (float)__builtin_bit_cast(bf16, braw);
}

template <int HW>
__device__ __forceinline__ void helper_commit(const HelperRegs<HW> &R, bf16 *set, float *gates,
                                              float *scratch, float scale, bool l2, int lane) {
  const int h = lane >> 5, r32 = lane & 31, r16 = lane >> 4, pc = lane & 15;
  const float gam = wave_incl_scan(R.g) * kLog2e;
  if (HW != 1) {
    constexpr int rbq = q_half(HW), rbk = k_half(HW);
    float *sg = scratch + 64 * (HW == 3 ? 1 : HW);
    sg[lane] = gam;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint4 xq = l2 ? l2n_piece<bf16, 16>(R.buf[m]) : R.buf[m];
      const uint4 xk = l2 ? l2n_piece<bf16, 16>(R.buf[8 + m]) : R.buf[8 + m];
      put_pi(set + oQ + (32 * rbq + 4 * m + r16) * PITCH, pc, xq);
      put_pi(set + oK + (32 * rbk + 4 * m + r16) * PITCH, pc, xk);
    }
    if (HW != 3) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int idx = lane + 64 * (m + 2 * HW);
        put_pi(set + oT + (idx >> 3) * PITCH_C, idx & 7, R.buf[16 + m]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // P tile (rows r: q rows 32 rbq.., columns j: k rows 32 rbk..), built so
    // that lane = j: the lane then writes row j of P^T, 4 consecutive r
    const bf16 *qa = set + oQ + (32 * rbq + r32) * PITCH + 8 * h;
    const bf16 *ka = set + oK + (32 * rbk + r32) * PITCH + 8 * h;
    f32x16 acc = zero16();
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = mma32(lds16(qa + 16 * s), lds16(ka + 16 * s), acc);
    const int jr = 32 * rbk + r32;  // this lane's row of P^T (column j of P)
    const float gj = sg[jr];
    bf16 *prow = set + oPt + jr * PITCH_C;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int r0 = 32 * rbq + 8 * b + 4 * h;  // 4 consecutive r
      const f32x4 gr = *reinterpret_cast<const f32x4 *>(sg + r0);
      float pv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        pv[u] = (jr <= r0 + u) ? acc[4 * b + u] * __builtin_amdgcn_exp2f(gr[u] - gj) : 0.f;
      st4(prow + pi_pos(r0), pv[0], pv[1], pv[2], pv[3]);
    }
  } else {
#pragma unroll
    for (int m = 0; m < 16; ++m)
      *reinterpret_cast<uint4 *>(set + oDO + (4 * m + r16) * PITCH + 8 * pc) = R.buf[m];
  }
  if (HW == 3) {
    const float gL = lane63(gam);
    const float eg = __builtin_amdgcn_exp2f(gam);
    gates[gGam + lane] = gam;
    gates[gEg + lane] = eg;
    gates[gDec + lane] = __builtin_amdgcn_exp2f(gL - gam);
    gates[gWq + lane] = scale * eg;
    gates[gWk + lane] = -R.b * eg;
  }
}

// Helper step during chain step c (chunks descend): loads of chunk c - 2
// into Rl, chunk c - 1 from Rc into its set.  Chunk indices below the
// segment are clamped to its first chunk (a repeated load and a commit to the
// set nobody reads any more).
template <int HW>
__device__ __forceinline__ void helper_step(HelperRegs<HW> &Rc, HelperRegs<HW> &Rl,
                                            const BwdArgs &a, const Item &it, int c, char *smem,
                                            float *scratch, int lane) {
  const int c0 = it.sl.c_begin;
  // the P-tile roles issue their k rows after the commit the next barrier
  // waits for, so that the loads issued ahead of it queue less
  helper_load<HW>(Rl, a, it, max(c - 2, c0), lane, HW == 1 ? 3 : 1);
  const int cn = c - 1;
  helper_commit<HW>(Rc, reinterpret_cast<bf16 *>(smem + (cn & 1) * SET_BYTES),
                    reinterpret_cast<float *>(smem + 2 * SET_BYTES) + (cn & 1) * GATE_FLOATS,
                    scratch, a.p.scale, a.p.l2, lane);
  if (HW != 1) helper_load<HW>(Rl, a, it, max(c - 2, c0), lane, 2);
}

template <int HW>
__device__ __forceinline__ void helper_loop(const BwdArgs &a, const Item &it, char *smem,
                                            float *scratch, int lane) {
  const int c0 = it.sl.c_begin, c1 = it.sl.c_end;
  HelperRegs<HW> R0, R1;
  if (c0 < c1) {
    const int cl = c1 - 1;
    helper_load<HW>(R0, a, it, cl, lane);
    helper_load<HW>(R1, a, it, max(cl - 1, c0), lane);
    helper_commit<HW>(R0, reinterpret_cast<bf16 *>(smem + (cl & 1) * SET_BYTES),
                      reinterpret_cast<float *>(smem + 2 * SET_BYTES) + (cl & 1) * GATE_FLOATS,
                      scratch, a.p.scale, a.p.l2, lane);
  }
  __syncthreads();
  // R1 holds chunk c - 1 at even steps (from c1 - 1), R0 at odd ones
  for (int c = c1 - 1; c >= c0; c -= 2) {
    helper_step<HW>(R1, R0, a, it, c, smem, scratch, lane);
    __syncthreads();
    if (c - 1 >= c0) {
      helper_step<HW>(R0, R1, a, it, c - 1, smem, scratch, lane);
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------- chain waves
#define GDN_FENCE() __builtin_amdgcn_sched_barrier(0)
// One reverse chunk of chain wave j on buffer set `set` (gates `gt`): D (4
// tiles, rows 32 m .. of K, columns 32 j .. of V) steps from the gradient
// leaving the chunk to the one entering it; `dcache` (nullable) receives the
// leaving gradient (bf16, lane layout).
__device__ __forceinline__ void chain_step(f32x16 (&D)[4], const bf16 *set, const float *gt,
                                           const ChainCtx &x, bf16 *dcache, float scale) {
  const int lane = x.lane, h = x.h, r32 = x.r32, j = x.j;
  const bf16 *sQ = set + oQ, *sK = set + oK, *sDO = set + oDO, *sT = set + oT, *sPt = set + oPt;
  // dO at the accumulator positions (rows r), as operand slots: plain (for
  // P^T dO) and scaled by scale e^gamma_r (for Q^T diag(scale e^gamma) dO)
  bf16x8 dob[4], yb[4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    bf16x4 xv[4];
    acc_rows(xv, sDO, t, j, lane);
    f32x16 dv, yv;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const f32x4 wq = *reinterpret_cast<const f32x4 *>(gt + gWq + 32 * t + 8 * b + 4 * h);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        dv[4 * b + u] = (float)xv[b][u];
        yv[4 * b + u] = wq[u] * (float)xv[b][u];
      }
    }
    dob[2 * t] = slots(dv, 0);
    dob[2 * t + 1] = slots(dv, 1);
    yb[2 * t] = slots(yv, 0);
    yb[2 * t + 1] = slots(yv, 1);
  }
  // a, b. K D over the key dimension, and D <- e^gamma_L D + Q^T Y
  //    interleaved with it (the leaving gradient's slots are stored to the
  //    per-chunk gradients at the end of the step: at its start the helpers'
  //    loads fill the memory queue, and the stores would wait behind them)
  const float egL = gt[gEg + 63];
  bf16x8 Db[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) Db[s] = slots(D[s >> 1], s & 1);
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) D[m][i] *= egL;
  const TrA qt(sQ, PITCH, lane), kt(sK, PITCH, lane);
  f32x16 KD[2] = {zero16(), zero16()};
  const bf16 *k0 = sK + r32 * PITCH + 8 * h;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const bf16x8 fk0 = lds16(k0 + 16 * s), fk1 = lds16(k0 + 32 * PITCH + 16 * s);
    // Q^T Y: k-step s >> 1 of the token dimension, m tiles 2 (s & 1), +1
    const int sr = s >> 1, m0 = 2 * (s & 1);
    const bf16x8 qa0 = qt.at(sr, m0, PITCH), qa1 = qt.at(sr, m0 + 1, PITCH);
    GDN_FENCE();
    KD[0] = mma32(fk0, Db[s], KD[0]);
    KD[1] = mma32(fk1, Db[s], KD[1]);
    D[m0] = mma32(qa0, yb[sr], D[m0]);
    D[m0 + 1] = mma32(qa1, yb[sr], D[m0 + 1]);
    GDN_FENCE();
  }
  // c. dVn = dec (K D) + scale P^T dO (P^T upper triangular: its row tile 1
  //    needs k-steps 2, 3 only)
  f32x16 PD[2] = {zero16(), zero16()};
  {
    const bf16 *p0 = sPt + r32 * PITCH_C + 8 * h, *p1 = p0 + 32 * PITCH_C;
#pragma unroll
    for (int s = 0; s < 4; ++s) PD[0] = mma32(lds16(p0 + 16 * s), dob[s], PD[0]);
#pragma unroll
    for (int s = 2; s < 4; ++s) PD[1] = mma32(lds16(p1 + 16 * s), dob[s], PD[1]);
  }
  bf16x8 dvb[4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x16 dvn;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const f32x4 dc = *reinterpret_cast<const f32x4 *>(gt + gDec + 32 * t + 8 * b + 4 * h);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        dvn[4 * b + u] = dc[u] * KD[t][4 * b + u] + scale * PD[t][4 * b + u];
    }
    dvb[2 * t] = slots(dvn, 0);
    dvb[2 * t + 1] = slots(dvn, 1);
  }
  GDN_FENCE();
  // d. X = -beta e^gamma (T^T dVn): T^T's slots from transpose reads of the
  //    pi-layout T rows (T^T upper triangular: row tile 1 needs k-steps 2, 3)
  f32x16 X[2] = {zero16(), zero16()};
  {
    const TrA tt(sT, PITCH_C, lane);
#pragma unroll
    for (int s = 0; s < 4; ++s) X[0] = mma32(tt.at(s, 0, PITCH_C), dvb[s], X[0]);
#pragma unroll
    for (int s = 2; s < 4; ++s) X[1] = mma32(tt.at(s, 1, PITCH_C), dvb[s], X[1]);
  }
  bf16x8 xb[4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const f32x4 wk = *reinterpret_cast<const f32x4 *>(gt + gWk + 32 * t + 8 * b + 4 * h);
#pragma unroll
      for (int u = 0; u < 4; ++u) X[t][4 * b + u] *= wk[u];
    }
    xb[2 * t] = slots(X[t], 0);
    xb[2 * t + 1] = slots(X[t], 1);
  }
  GDN_FENCE();
  // e. D += K^T X over the token dimension
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bf16x8 ka[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) ka[m] = kt.at(s, m, PITCH);
    GDN_FENCE();
#pragma unroll
    for (int m = 0; m < 4; ++m) D[m] = mma32(ka[m], xb[s], D[m]);
    GDN_FENCE();
  }
  if (dcache) {
#pragma unroll
    for (int s = 0; s < 8; ++s)
      *reinterpret_cast<bf16x8 *>(dcache + ((j * 8 + s) * 64 + lane) * 8) = Db[s];
  }
}
#undef GDN_FENCE

__global__ __launch_bounds__(kThreadsS) void rev_slice_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  float *scratch = reinterpret_cast<float *>(smem + 2 * SET_BYTES) + 2 * GATE_FLOATS;
  const Problem &p = a.p;
  const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
  Item it;
  it.h = (int)(wid % p.Hv);
  it.hq = it.h / (p.Hv / p.Hq);
  const int64_t sg = wid / p.Hv;
  it.sl = locate_segment(p, a.plan.seg_chunks,
                         reinterpret_cast<const int32_t *>(a.ws + a.wl.fwd.chunk_prefix),
                         reinterpret_cast<const int32_t *>(a.ws + a.wl.fwd.seg_prefix), sg);
  const int w = wave_of(threadIdx.x), lane = threadIdx.x & 63;
  const int c0 = it.sl.c_begin, c1 = it.sl.c_end;
  const int64_t KV = (int64_t)K * V;

  if (w < 4) {
    ChainCtx x{w, lane, lane >> 5, lane & 31};
    f32x16 D[4];
    const float *src = (it.sl.j == it.sl.nseg - 1 && a.dht)
                           ? a.dht + ((int64_t)it.sl.n * p.Hv + it.h) * KV : nullptr;
    state_load(D, src, x);
    bf16 *dstates = reinterpret_cast<bf16 *>(a.ws + a.wl.dstates);
    __syncthreads();  // set of chunk c1 - 1 committed
    for (int c = c1 - 1; c >= c0; --c) {
      chain_step(D, reinterpret_cast<const bf16 *>(smem + (c & 1) * SET_BYTES),
                 reinterpret_cast<const float *>(smem + 2 * SET_BYTES) + (c & 1) * GATE_FLOATS,
                 x, dstates + ((it.sl.chunk0 + c) * p.Hv + it.h) * KV, p.scale);
      __syncthreads();
    }
    if (it.sl.nseg > 1)
      state_store(D, reinterpret_cast<float *>(a.ws + a.wl.dseg) + (sg * p.Hv + it.h) * KV, x);
    if (it.sl.nseg == 1 && a.dh0)
      state_store(D, a.dh0 + ((int64_t)it.sl.n * p.Hv + it.h) * KV, x);
  } else if (w == 4) {
    helper_loop<0>(a, it, smem, scratch, lane);
  } else if (w == 5) {
    helper_loop<1>(a, it, smem, scratch, lane);
  } else if (w == 6) {
    helper_loop<2>(a, it, smem, scratch, lane);
  } else {
    helper_loop<3>(a, it, smem, scratch, lane);
  }
}

}  // namespace rslice

bool rev_slice_supported(const BwdArgs &a) {
  return a.p.dtype == 1 && a.p.K == slice::K && a.p.V == slice::V;
}

hipError_t launch_rev_slice_main(const BwdArgs &a, hipStream_t st) {
  if (a.plan.total_segs * a.p.Hv <= 0) return hipSuccess;
  KernelTimer kt("rev_main", st);
  rslice::rev_slice_kernel<<<dim3((unsigned)(a.plan.total_segs * a.p.Hv)), slice::kThreadsS, 0,
                             st>>>(a);
  return hipGetLastError();
}

}  // namespace gdn
