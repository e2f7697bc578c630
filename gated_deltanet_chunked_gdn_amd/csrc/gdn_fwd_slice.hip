// Forward segment pass 1 with the state recurrence held in registers, for
// bf16 problems with K = V = 128 (the pages' head shape; other shapes take the
// general segment kernel of gdn_fwd.hip).
//
// Same arithmetic as the general pass 1 (per 64-token chunk, entering state S):
//   R  = diag(beta) (V - diag(e^gamma) K S),   Vn = T R
//   O  = scale (diag(e^gamma) Q S + P Vn),     P = lower_incl(Q K^T * E)
//   S' = e^gamma_L S + K^T diag(e^(gamma_L - gamma)) Vn
// but organised around one fact: the V columns of the recurrence are
// independent.  A workgroup owns one (segment, v-head) item and has two
// kinds of waves (the pages' wave-role split, FlashQLA article "FlashQLA
// 架构图" and aiwebcool "flashqla-resource" section 三, third feature, redone
// for CDNA4):
//
//   chain waves 0..3  wave j owns V columns [32 j, 32 j + 32): its slice of S
//                     (128 x 32 fp32) lives in 32x32 MFMA accumulator tiles
//                     for the whole segment, and every S-dependent product of
//                     a chunk (K S, Q S, T R, P Vn, K^T Vn) runs on the
//                     slice without talking to the other chain waves;
//   helper waves 4..7 stage the next chunk: q, k, v, T and the gates into
//                     the other LDS buffer set, P = Q K^T * E on MFMA, and
//                     the previous chunk's output rows out of LDS to HBM.
//
// A 32x32x16 MFMA accumulator holds, in lane l, column l & 31 and rows
// 8 (i >> 2) + 4 (l >> 5) + (i & 3) of its tile (register i).  Read as
// operand slots, registers 8 s .. 8 s + 7 of a tile are rows 16 s + [0..15]
// in the order rho(h, e) = 8 (e >> 2) + 4 h + (e & 3) (h = l >> 5): so an
// accumulator is, without any data movement, the B operand of A X or the A
// operand of X^T B with the contraction over its rows, provided the other
// operand supplies its k-slots in the same rho order.  The LDS copies of
// q, k, T and P therefore store each row with the 4-element groups 1 and 2
// of every 16-element block swapped ("pi" layout): one 16-byte read at
// position 16 s + 8 h then yields exactly the rho-ordered slots.
//
// One workgroup barrier per chunk: chain waves read buffer set c & 1 while
// the helpers fill set (c + 1) & 1, from registers loaded one chunk earlier.
#include "gdn_slice.hpp"

namespace gdn {
namespace slice {

// One buffer set (element offsets), and the gates (float offsets after it).
constexpr int oQ = 0, oK = oQ + 64 * PITCH, oV = oK + 64 * PITCH, oT = oV + 64 * PITCH,
              oP = oT + 64 * PITCH_C, SET_ELEMS = oP + 64 * PITCH_C;
// gates per set: gam (gamma log2 e), eg = e^gamma, dec = e^(gamma_L - gamma),
// beta, beta e^gamma
constexpr int gGam = 0, gEg = 64, gDec = 128, gBeta = 192, gBeg = 256, GATE_FLOATS = 320;
constexpr int SET_BYTES = SET_ELEMS * 2;
constexpr int LDS_BYTES = 2 * SET_BYTES + 2 * GATE_FLOATS * 4 + 3 * 64 * 4;
static_assert(SET_BYTES % 16 == 0, "sets stay 16-byte aligned");
static_assert(LDS_BYTES <= 160 * 1024, "two buffer sets fit the LDS of a compute unit");

// ------------------------------------------------------------------ helpers
// Helper wave roles (HW = wave - 4):
//   0  q, k rows 0..31 into LDS; P tile (rows 0..31, columns 0..31)
//   1  the previous chunk's output rows out of LDS, then v rows into the
//      same LDS rows (one wave, so the reads come before the writes); T
//   2  q, k rows 32..63 into LDS; P tile (rows 32..63, columns 32..63)
//   3  the gates; P tile (rows 32..63, columns 0..31)
// (P is lower triangular: its tile (rows 0..31, columns 32..63) is zero and
// never read.)  Rows are loaded whole (16 consecutive lanes cover one
// 256-byte row) and each P tile reads its operands back from the LDS rows
// its own wave has just written: role 3 writes the q rows 32..63 and k rows
// 0..31 it needs itself, the same bytes roles 2 and 0 write there, so no
// helper ever waits for another.  Loads are issued a chunk and a half before
// their data is committed: the registers hold two chunks, and loads past the
// end of a sequence return zeros (buffer range), so no load is conditional.
template <int HW>
struct HelperRegs {
  // roles 0, 2, 3: q rows (buf[0..7]) and k rows (buf[8..15]) of one half of
  // the chunk, 16-byte piece lane & 15 of row 4 m + (lane >> 4); role 1: v
  // rows (buf[0..15]) and T (buf[16..23], 16-byte piece lane + 64 m)
  static constexpr int NB = HW == 1 ? 24 : 16;
  uint4 buf[NB];
  float g;
  float b;
};
// q rows of role HW: 0..31 (role 0) or 32..63; k rows: 32..63 (role 2) or 0..31
__device__ __forceinline__ constexpr int q_half(int hw) { return hw == 0 ? 0 : 1; }
__device__ __forceinline__ constexpr int k_half(int hw) { return hw == 2 ? 1 : 0; }


// Loads chunk c of the item into the registers of helper role HW.
template <int HW>
// (parts: 1 = everything but the k rows, 2 = the k rows, 3 = all)
__device__ __forceinline__ void helper_load(HelperRegs<HW> &R, const FwdArgs &a, const Item &it,
                                            int c, int lane, int part = 3) {
  const Problem &p = a.p;
  const int64_t tok0 = it.sl.si.tok0 + (int64_t)c * kChunk;
  const int rows = min(kChunk, it.sl.si.len - c * kChunk);
  const int r16 = lane >> 4, pc = lane & 15;
  if (HW != 1) {
    const uint32_t rs = (uint32_t)(p.Hq * K * 2);  // bytes between token rows
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
    const bf16 *vb = reinterpret_cast<const bf16 *>(a.v) + (tok0 * p.Hv + it.h) * V;
    const auto rv = rsrc_of(vb, (uint32_t)rows * rs);
#pragma unroll
    for (int m = 0; m < 16; ++m) R.buf[m] = bload16(rv, (uint32_t)(4 * m + r16) * rs + 16u * pc);
  }
  if (HW == 1) {
    // T (role 1, which has the shortest step): 8 16-byte pieces a row
    const int64_t cgid = it.sl.chunk0 + c;
    const uint4 *tb = reinterpret_cast<const uint4 *>(
        reinterpret_cast<const bf16 *>(a.tm_ext ? a.tm_ext : a.ws + a.wl.tmat) +
        (cgid * p.Hv + it.h) * 64 * 64);
#pragma unroll
    for (int m = 0; m < 8; ++m) R.buf[16 + m] = tb[lane + 64 * m];
  }
  // every role keeps the chunk's gates (P needs gamma); rows past the end: 0
  const uint32_t gs = (uint32_t)(p.Hv * 4);
  const auto rg = rsrc_of(a.g + tok0 * p.Hv + it.h, (uint32_t)rows * gs);
  R.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, (int)(lane * gs), 0, 0));
  const uint32_t bs = (uint32_t)(p.Hv * 2);
  const auto rb = rsrc_of(reinterpret_cast<const bf16 *>(a.beta) + tok0 * p.Hv + it.h,
                          (uint32_t)rows * bs);
  const unsigned short braw = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)(lane * bs), 0, 0);
  R.b = (float)__builtin_bit_cast(bf16, braw);
}


// Writes the chunk held in R into buffer set `set` (role HW's share).
template <int HW>
__device__ __forceinline__ void helper_commit(const HelperRegs<HW> &R, bf16 *set, float *gates,
                                              float *scratch, bool l2, int lane) {
  const int h = lane >> 5, r32 = lane & 31, r16 = lane >> 4, pc = lane & 15;
  const float gam = wave_incl_scan(R.g) * kLog2e;  // gate cumsum, times log2(e)
  if (HW != 1) {
    constexpr int rbq = q_half(HW), rbk = k_half(HW);
    float *sg = scratch + 64 * (HW == 3 ? 1 : HW);  // this wave's own copy of gamma
    sg[lane] = gam;
    // q and k rows of this half into the pi layout
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint4 xq = l2 ? l2n_piece<bf16, 16>(R.buf[m]) : R.buf[m];
      const uint4 xk = l2 ? l2n_piece<bf16, 16>(R.buf[8 + m]) : R.buf[8 + m];
      put_pi(set + oQ + (32 * rbq + 4 * m + r16) * PITCH, pc, xq);
      put_pi(set + oK + (32 * rbk + 4 * m + r16) * PITCH, pc, xk);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // P^T tile: rows j (k rows 32 rbk..), columns r (q rows 32 rbq..), from
    // the rows just written (rho-ordered slots of both operands)
    const bf16 *ka = set + oK + (32 * rbk + r32) * PITCH + 8 * h;
    const bf16 *qa = set + oQ + (32 * rbq + r32) * PITCH + 8 * h;
    f32x16 acc = zero16();
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = mma32(lds16(ka + 16 * s), lds16(qa + 16 * s), acc);
    const int r = 32 * rbq + r32;  // this lane's output row (token) of P
    const float gr = sg[r];
    bf16 *prow = set + oP + r * PITCH_C;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int j0 = 32 * rbk + 8 * b + 4 * h;  // 4 consecutive columns j0 .. j0 + 3
      const f32x4 gj = *reinterpret_cast<const f32x4 *>(sg + j0);
      float pv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        pv[u] = (j0 + u <= r) ? acc[4 * b + u] * __builtin_amdgcn_exp2f(gr - gj[u]) : 0.f;
      st4(prow + pi_pos(j0), pv[0], pv[1], pv[2], pv[3]);
    }
  } else {
    // v rows (natural layout), T rows (pi layout)
#pragma unroll
    for (int m = 0; m < 16; ++m)
      *reinterpret_cast<uint4 *>(set + oV + (4 * m + r16) * PITCH + 8 * pc) = R.buf[m];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int idx = lane + 64 * m;  // 16-byte piece of T
      put_pi(set + oT + (idx >> 3) * PITCH_C, idx & 7, R.buf[16 + m]);
    }
  }
  if (HW == 3) {
    // the gates
    const float gL = lane63(gam);
    const float eg = __builtin_amdgcn_exp2f(gam);
    gates[gGam + lane] = gam;
    gates[gEg + lane] = eg;
    gates[gDec + lane] = __builtin_amdgcn_exp2f(gL - gam);
    gates[gBeta + lane] = R.b;
    gates[gBeg + lane] = R.b * eg;
  }
}

// Output rows of chunk c (staged in the v rows of `set`) to HBM, 16 bytes a
// lane, whole rows; rows past the chunk's end are dropped by the buffer
// range (`rows` = 0 drops every store).
__device__ __forceinline__ void helper_store_o(const FwdArgs &a, const Item &it, int c, int rows,
                                               const bf16 *set, int lane) {
  const Problem &p = a.p;
  const int64_t tok0 = it.sl.si.tok0 + (int64_t)c * kChunk;
  const uint32_t o_rs = (uint32_t)(p.Hv * V * 2);
  const auto ob = raw_buffer(reinterpret_cast<bf16 *>(a.o) + (tok0 * p.Hv + it.h) * V,
                             (uint32_t)rows * o_rs);
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int idx = lane + 64 * m, r = idx >> 4, pc = idx & 15;
    buf_store16(*reinterpret_cast<const uint4 *>(set + oV + r * PITCH + 8 * pc), ob,
                (uint32_t)r * o_rs + (uint32_t)pc * 16u);
  }
}

// One helper step during chain step c: loads of chunk c + 2 into Rl, the
// output rows of chunk c - 1 (role 1), and chunk c + 1 from Rc into its set.
// Chunk indices past the segment are clamped to its last chunk (a repeated
// load and a commit to the set nobody reads any more), so nothing branches.
template <int HW>
__device__ __forceinline__ void helper_step(HelperRegs<HW> &Rc, HelperRegs<HW> &Rl,
                                            const FwdArgs &a, const Item &it, int c, char *smem,
                                            float *scratch, int lane) {
  const int c0 = it.sl.c_begin, c1 = it.sl.c_end;
  // role 1 has the shortest step: its loads go last, so that the roles whose
  // commit and P tile the next barrier waits for are not queued behind them;
  // those roles issue their k rows after the commit
  if (HW != 1) helper_load<HW>(Rl, a, it, min(c + 2, c1 - 1), lane, 1);
  if (HW == 1) {
    const int cp = max(c - 1, c0);
    const int rows = c > c0 ? min(kChunk, it.sl.si.len - cp * kChunk) : 0;
    helper_store_o(a, it, cp, rows, reinterpret_cast<bf16 *>(smem + (cp & 1) * SET_BYTES), lane);
  }
  const int cn = c + 1;
  helper_commit<HW>(Rc, reinterpret_cast<bf16 *>(smem + (cn & 1) * SET_BYTES),
                    reinterpret_cast<float *>(smem + 2 * SET_BYTES) + (cn & 1) * GATE_FLOATS,
                    scratch, a.p.l2, lane);
  if (HW == 1) helper_load<HW>(Rl, a, it, min(c + 2, c1 - 1), lane);
  if (HW != 1) helper_load<HW>(Rl, a, it, min(c + 2, c1 - 1), lane, 2);
}

template <int HW>
__device__ __forceinline__ void helper_loop(const FwdArgs &a, const Item &it, char *smem,
                                            float *scratch, int lane) {
  const int c0 = it.sl.c_begin, c1 = it.sl.c_end;
  HelperRegs<HW> R0, R1;
  if (c0 < c1) {
    helper_load<HW>(R0, a, it, c0, lane);
    helper_load<HW>(R1, a, it, min(c0 + 1, c1 - 1), lane);
    helper_commit<HW>(R0, reinterpret_cast<bf16 *>(smem + (c0 & 1) * SET_BYTES),
                      reinterpret_cast<float *>(smem + 2 * SET_BYTES) + (c0 & 1) * GATE_FLOATS,
                      scratch, a.p.l2, lane);
  }
  __syncthreads();
  // R1 holds chunk c + 1 at even steps (from c0), R0 at odd ones
  for (int c = c0; c < c1; c += 2) {
    helper_step<HW>(R1, R0, a, it, c, smem, scratch, lane);
    __syncthreads();
    if (c + 1 < c1) {
      helper_step<HW>(R0, R1, a, it, c + 1, smem, scratch, lane);
      __syncthreads();
    }
  }
  if (HW == 1 && c1 > c0)
    helper_store_o(a, it, c1 - 1, min(kChunk, it.sl.si.len - (c1 - 1) * kChunk),
                   reinterpret_cast<bf16 *>(smem + ((c1 - 1) & 1) * SET_BYTES), lane);
}

// ------------------------------------------------------------- chain waves

// One chunk of chain wave j on buffer set `set` (gates `gt`): S (4 tiles,
// rows 32 m .. of K, columns 32 j .. of V) advances by one chunk and the
// chunk's output slice is staged (scaled, bf16) in the v rows of the set.
// `hcache` (nullable) receives the entering state, bf16, in the lane layout
// of the state cache (gdn_seg.hpp).
//
// With one chain wave per SIMD the wave's own instruction stream has to hide
// the LDS latency: every operand fragment is read one or two product groups
// before the products that use it, and scheduling fences (sched_barrier)
// keep the compiler from sinking those reads back next to their use.
#define GDN_FENCE() __builtin_amdgcn_sched_barrier(0)
__device__ __forceinline__ void chain_step(f32x16 (&S)[4], bf16 *set, const float *gt,
                                           float scale, const ChainCtx &x, bf16 *hcache) {
  const int lane = x.lane, h = x.h, r32 = x.r32, j = x.j;
  const bf16 *sQ = set + oQ, *sK = set + oK, *sT = set + oT, *sP = set + oP;
  bf16 *sV = set + oV;
  // b. K S (rows r, columns of the slice) and O^T = S^T Q^T (rows of the
  //    slice, columns r), over the 8 k-steps of the key dimension; the
  //    state's operand slots (k-step s: rows 16 s .. of S) are rounded to
  //    bf16 as they are used
  f32x16 KS[2] = {zero16(), zero16()}, OT[2] = {zero16(), zero16()};
  const bf16 *k0 = sK + r32 * PITCH + 8 * h, *q0 = sQ + r32 * PITCH + 8 * h;
  bf16x8 F[3][4];
  auto load_b = [&](int s, bf16x8 (&f)[4]) {
    f[0] = lds16(k0 + 16 * s);
    f[1] = lds16(k0 + 32 * PITCH + 16 * s);
    f[2] = lds16(q0 + 16 * s);
    f[3] = lds16(q0 + 32 * PITCH + 16 * s);
  };
  load_b(0, F[0]);
  load_b(1, F[1]);
  bf16x4 vx[2][4];
  // the entering state's slots for the state cache, stored at the end of
  // the step (at its start the helpers' loads fill the memory queue)
  bf16x8 Sb[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if (s + 2 < 8) load_b(s + 2, F[(s + 2) % 3]);
    if (s == 5) {
      // phase c's V at the accumulator positions
#pragma unroll
      for (int t = 0; t < 2; ++t) acc_rows(vx[t], sV, t, j, lane);
    }
    GDN_FENCE();
    const bf16x8 sb = slots(S[s >> 1], s & 1);
    if (hcache) Sb[s] = sb;
    const bf16x8(&f)[4] = F[s % 3];
    KS[0] = mma32(f[0], sb, KS[0]);
    KS[1] = mma32(f[1], sb, KS[1]);
    OT[0] = mma32(sb, f[2], OT[0]);
    OT[1] = mma32(sb, f[3], OT[1]);
    GDN_FENCE();
  }
  // d's operands: T rows (lower triangular: row tile 0 needs k-steps 0, 1)
  bf16x8 tf[6];
  {
    const bf16 *t0 = sT + r32 * PITCH_C + 8 * h, *t1 = t0 + 32 * PITCH_C;
    tf[0] = lds16(t0);
    tf[1] = lds16(t0 + 16);
#pragma unroll
    for (int s = 0; s < 4; ++s) tf[2 + s] = lds16(t1 + 16 * s);
  }
  GDN_FENCE();
  // c. R = beta V - beta e^gamma (K S) at the accumulator positions
  bf16x8 Rb[4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x16 R;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int r0 = 32 * t + 8 * b + 4 * h;
      const f32x4 be = *reinterpret_cast<const f32x4 *>(gt + gBeta + r0);
      const f32x4 bg = *reinterpret_cast<const f32x4 *>(gt + gBeg + r0);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        R[4 * b + u] = be[u] * (float)vx[t][b][u] - bg[u] * KS[t][4 * b + u];
    }
    Rb[2 * t] = slots(R, 0);
    Rb[2 * t + 1] = slots(R, 1);
  }
  GDN_FENCE();
  // f's operands (P rows), read while d runs
  bf16x8 pf[6];
  float egr[2];
  {
    const bf16 *p0 = sP + r32 * PITCH_C + 8 * h, *p1 = p0 + 32 * PITCH_C;
    pf[0] = lds16(p0);
    pf[1] = lds16(p0 + 16);
#pragma unroll
    for (int s = 0; s < 4; ++s) pf[2 + s] = lds16(p1 + 16 * s);
#pragma unroll
    for (int t = 0; t < 2; ++t) egr[t] = gt[gEg + 32 * t + r32];
  }
  // d. Vn = T R
  f32x16 Vn[2] = {zero16(), zero16()};
  Vn[0] = mma32(tf[0], Rb[0], Vn[0]);
  Vn[1] = mma32(tf[2], Rb[0], Vn[1]);
  Vn[0] = mma32(tf[1], Rb[1], Vn[0]);
  Vn[1] = mma32(tf[3], Rb[1], Vn[1]);
  Vn[1] = mma32(tf[4], Rb[2], Vn[1]);
  Vn[1] = mma32(tf[5], Rb[3], Vn[1]);
  GDN_FENCE();
  // g's first operands: K^T slots from transpose reads of the pi-layout k rows
  const TrA kt(sK, PITCH, lane);
  auto load_kt = [&](int s, int m) { return kt.at(s, m, PITCH); };
  bf16x8 ka[2][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) ka[0][m] = load_kt(0, m);
#pragma unroll
  for (int m = 0; m < 4; ++m) ka[1][m] = load_kt(1, m);
  const float egL = gt[gEg + 63];
  GDN_FENCE();
  // e. Vn as operand slots, plain and scaled by e^(gamma_L - gamma_r)
  bf16x8 Vnb[4], Vnd[4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x16 d;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const f32x4 dc = *reinterpret_cast<const f32x4 *>(gt + gDec + 32 * t + 8 * b + 4 * h);
#pragma unroll
      for (int u = 0; u < 4; ++u) d[4 * b + u] = dc[u] * Vn[t][4 * b + u];
    }
    Vnb[2 * t] = slots(Vn[t], 0);
    Vnb[2 * t + 1] = slots(Vn[t], 1);
    Vnd[2 * t] = slots(d, 0);
    Vnd[2 * t + 1] = slots(d, 1);
  }
  // f. O^T = e^gamma_r (S^T Q^T) + Vn^T P^T (P lower triangular)
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) OT[t][i] *= egr[t];
  OT[0] = mma32(Vnb[0], pf[0], OT[0]);
  OT[1] = mma32(Vnb[0], pf[2], OT[1]);
  OT[0] = mma32(Vnb[1], pf[1], OT[0]);
  OT[1] = mma32(Vnb[1], pf[3], OT[1]);
  OT[1] = mma32(Vnb[2], pf[4], OT[1]);
  OT[1] = mma32(Vnb[3], pf[5], OT[1]);
  GDN_FENCE();
  // g. S' = e^gamma_L S + K^T (dec Vn), k-step by k-step, the K^T slots read
  //    two k-steps ahead; h. the output slice, scaled, into the v rows (own
  //    columns only: this wave has read them already; lane = row r, 4
  //    consecutive columns), placed between g's products so that its VALU
  //    and LDS work overlaps them
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) S[m][i] *= egL;
  bf16x8 kb3[4];
  auto g_step = [&](const bf16x8(&kf)[4], int st) {
#pragma unroll
    for (int m = 0; m < 4; ++m) S[m] = mma32(kf[m], Vnd[st], S[m]);
  };
#pragma unroll
  for (int m = 0; m < 4; ++m) kb3[m] = load_kt(2, m);
  GDN_FENCE();
  g_step(ka[0], 0);
  GDN_FENCE();
#pragma unroll
  for (int m = 0; m < 4; ++m) ka[0][m] = load_kt(3, m);
  GDN_FENCE();
  g_step(ka[1], 1);
  GDN_FENCE();
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    bf16 *orow = sV + (32 * t + r32) * PITCH + 32 * j + 4 * h;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      st4(orow + 8 * b, OT[t][4 * b] * scale, OT[t][4 * b + 1] * scale,
          OT[t][4 * b + 2] * scale, OT[t][4 * b + 3] * scale);
  }
  GDN_FENCE();
  g_step(kb3, 2);
  GDN_FENCE();
  g_step(ka[0], 3);
  if (hcache) {
    // the lane layout of the state cache is these very slots: one whole 1 KB
    // piece per k-step and wave
#pragma unroll
    for (int s = 0; s < 8; ++s)
      *reinterpret_cast<bf16x8 *>(hcache + ((j * 8 + s) * 64 + lane) * 8) = Sb[s];
  }
}
#undef GDN_FENCE

__global__ __launch_bounds__(kThreadsS) void slice_main_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  auto set_of = [&](int c) { return reinterpret_cast<bf16 *>(smem + (c & 1) * SET_BYTES); };
  auto gates_of = [&](int c) {
    return reinterpret_cast<float *>(smem + 2 * SET_BYTES) + (c & 1) * GATE_FLOATS;
  };
  float *scratch = reinterpret_cast<float *>(smem + 2 * SET_BYTES) + 2 * GATE_FLOATS;
  const Problem &p = a.p;
  const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
  Item it;
  it.h = (int)(wid % p.Hv);
  it.hq = it.h / (p.Hv / p.Hq);
  const int64_t sg = wid / p.Hv;
  it.sl = locate_segment(p, a.plan.seg_chunks,
                         reinterpret_cast<const int32_t *>(a.ws + a.wl.chunk_prefix),
                         reinterpret_cast<const int32_t *>(a.ws + a.wl.seg_prefix), sg);
  const int w = wave_of(threadIdx.x), lane = threadIdx.x & 63;
  const int c0 = it.sl.c_begin, c1 = it.sl.c_end;
  const int64_t KV = (int64_t)K * V;

  if (w < 4) {
    ChainCtx x{w, lane, lane >> 5, lane & 31};
    f32x16 S[4];
    const float *src = (it.sl.j == 0 && a.h0) ? a.h0 + ((int64_t)it.sl.n * p.Hv + it.h) * KV
                                              : nullptr;
    state_load(S, src, x);
    __syncthreads();  // set c0 committed
    for (int c = c0; c < c1; ++c) {
      bf16 *hc = a.h_e ? reinterpret_cast<bf16 *>(a.h_e) +
                             ((it.sl.chunk0 + c) * p.Hv + it.h) * KV
                       : nullptr;
      // fp32 state entering the chunk, when the caller asks for it
      if (a.h) state_store(S, a.h + ((it.sl.chunk0 + c) * p.Hv + it.h) * KV, x);
      chain_step(S, set_of(c), gates_of(c), p.scale, x, hc);
      __syncthreads();
    }
    if (it.sl.nseg > 1)
      state_store(S, reinterpret_cast<float *>(a.ws + a.wl.hseg) + (sg * p.Hv + it.h) * KV, x);
    if (it.sl.nseg == 1 && a.ht) state_store(S, a.ht + ((int64_t)it.sl.n * p.Hv + it.h) * KV, x);
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

}  // namespace slice

bool fwd_slice_supported(const FwdArgs &a) {
  return a.p.dtype == 1 && a.p.K == slice::K && a.p.V == slice::V;
}

hipError_t launch_fwd_slice_main(const FwdArgs &a, hipStream_t st) {
  if (a.plan.total_segs * a.p.Hv <= 0) return hipSuccess;
  KernelTimer kt("fwd_main", st);
  slice::slice_main_kernel<<<dim3((unsigned)(a.plan.total_segs * a.p.Hv)), slice::kThreadsS, 0,
                             st>>>(a);
  return hipGetLastError();
}

}  // namespace gdn
