// Local gradients of the GDN chunked backward for bf16, K = V = 128, on the
// 32x32x16 matrix-core tiles of the register-resident passes (gdn_slice.hpp).
//
// The products are those of gdn_bwd.hip's local_grad (the reverse mode of the
// chunked forward of the FlashQLA article's low-level API, "底层 API"):
// per chunk and v-head, with S the entering state and D the gradient of the
// leaving state (both bf16, in the lane layout of the register-resident
// passes), the forward's T and gates recomputed,
//   KS = K S, R = diag(beta)(V - diag(e^gamma) KS), Vn = T R, KD = K D,
//   dVn = diag(dec) KD + scale P^T dO, dR = T^T dVn, dv = diag(beta) dR,
//   dq += diag(scale e^gamma) dO S^T + (dP * E) K,
//   dk += diag(dec) Vn D^T - diag(beta e^gamma) dR S^T + (dP * E)^T Q
//         + (dKK + dKK^T) K,
//   dP = dO Vn^T, dA = dR Vn^T (lower parts), dKK = diag(beta)(-dA) * E,
// and the row terms of dbeta and dgamma.  Three row dots over V are taken
// over K instead, from products that are formed anyway:
//   sum_v dO QS = sum_k Q (dO S^T),  sum_v Vn KD = sum_k K (Vn D^T),
//   sum_v dR KS = sum_k K (dR S^T),
// so Q S is never computed.
//
// Work item: (chunk, q/k head); its v-heads in turn, each over two 64-column
// blocks of V.  Per block, after the block's S, D, dO, V are in LDS:
//   phase V  waves 0, 1: KS -> R -> Vn for V columns 32 c .. 32 c + 31
//            (c = wave), Vn^T into LDS;
//            waves 2, 3: KD, P^T dO -> dVn -> dR for their 32 columns, dR^T
//            into LDS;
//            waves 4..7: dO S^T for two 32x32 tiles of dq each;
//   phase K  waves 4..7: Vn D^T and dR S^T for the same tiles of dk;
//            waves 0..3: dP, dA tiles; every wave: its share of the dv rows.
// At the end of a v-head the dP, dA holders form (dP * E)^T and dKK^T in LDS
// and waves 4..7 add their products with K and Q to dq, dk.  Accumulators
// feed the next product as operands without leaving registers wherever the
// contraction runs over their rows (T R, T^T dVn); the LDS copies of operands
// are in the pi layout, so 16-byte reads give slots in the accumulator order.
// One workgroup per compute unit, looping over items; the next block's inputs
// are loaded into registers while the current one is computed.
#include "gdn_slice.hpp"

namespace gdn {
namespace gslice {

using slice::f32x16;
using slice::K;
using slice::lds16;
using slice::mma32;
using slice::pi4;
using slice::put_pi;
using slice::slots;
using slice::tr4;
using slice::TrA;
using slice::zero16;

constexpr int VB = 64;                  // V columns per block
constexpr int NVB = slice::V / VB;      // blocks per v-head
constexpr int P128 = slice::PITCH;      // LDS pitch of 128-wide rows (elements)
constexpr int P64 = slice::PITCH_C;     // LDS pitch of 64-wide rows
constexpr int kThr = slice::kThreadsS;  // 512

// LDS regions (bytes).  Row-major, bf16, all in the pi layout along the row:
//   Q, K      [64 rows r][128 k]
//   S, D      [64 rows v of the block][128 k]
//   dO, V     [64 rows r][64 v of the block]
//   T         [64 rows r][64 t]
//   Pt        [64 rows t][64 s]   P^T
//   VnT, dRT  [64 rows v of the block][64 r]
//   PEt, Ut   [64 rows t][64 s]   (dP * E)^T and the strict part of dKK^T
//             of the previous v-head
constexpr int B_QK = 64 * P128 * 2;
constexpr int B_SD = VB * P128 * 2;
constexpr int B_C = 64 * P64 * 2;
constexpr int oQ = 0, oK = oQ + B_QK, oS = oK + B_QK, oD = oS + B_SD, oO = oD + B_SD,
              oV = oO + B_C, oT = oV + B_C, oPt = oT + B_C, oVnT = oPt + B_C,
              oDRT = oVnT + B_C, oPEt = oDRT + B_C, oUt = oPEt + B_C, oF = oUt + B_C;

// per-row values: gates (two sets, alternating over v-heads) and the partial
// row and column sums of dbeta and dgamma, each with its own contributor slot
// so that every sum is taken in a fixed order
struct Small {
  float gam[2][64];  // gamma * log2(e)
  float eg[2][64];   // exp(gamma)
  float dec[2][64];  // exp(gamma_L - gamma)
  float bet[2][64];
  float pq[2][64];   // sum_k Q (dO S^T)      [contributor][row]
  float pc[2][64];   // sum_k K (Vn D^T)
  float pa2[2][64];  // sum_k K (dR S^T)
  float pa1[2][64];  // sum_v dR V
  float rsP[3][32], csP[3][32];  // row / column sums of scale dP E QK  [E tile]
  float rsA[3][32], csA[3][32];  // of beta (-dA) E KK
  float dbA[3][32];              // row sums of (-dA) E KK
  float gl[8];                   // <D, S> per wave
  // in-library q/k L2 normalisation: the item's row factors
  float rq[64], rk[64];
};
constexpr int LDS_BYTES = oF + (int)sizeof(Small);
static_assert(LDS_BYTES <= 160 * 1024, "LDS");

// E tiles (32x32 tiles of the lower 64x64 chunk matrices): p = 0: rows 0..31
// x columns 0..31, p = 1: rows 32..63 x 0..31, p = 2: rows 32..63 x 32..63
__device__ __forceinline__ constexpr int e_st(int p) { return p == 0 ? 0 : 1; }
__device__ __forceinline__ constexpr int e_tt(int p) { return p == 2 ? 1 : 0; }

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

struct GItem {
  int hq;
  int64_t gid;   // global chunk id
  int64_t tok0;  // first token of the chunk
  int rows;      // valid rows (< 64 only in a sequence's last chunk)
};

__device__ __forceinline__ GItem item_at(const BwdArgs &a, int64_t it) {
  const Problem &p = a.p;
  GItem x;
  x.hq = (int)(it % p.Hq);
  x.gid = it / p.Hq;
  const ChunkLoc cl =
      locate_chunk(p, reinterpret_cast<const int32_t *>(a.ws + a.wl.fwd.chunk_prefix), x.gid);
  x.tok0 = cl.si.tok0 + (int64_t)cl.c * kChunk;
  x.rows = min(kChunk, cl.si.len - cl.c * kChunk);
  // the same for every lane: held in scalar registers, so that the buffer
  // descriptors built on it are scalar too
  x.hq = __builtin_amdgcn_readfirstlane(x.hq);
  x.rows = __builtin_amdgcn_readfirstlane(x.rows);
  x.gid = uniform64(x.gid);
  x.tok0 = uniform64(x.tok0);
  return x;
}
__device__ __forceinline__ GItem pick(bool first, const GItem &x, const GItem &y) {
  GItem r;
  r.hq = first ? x.hq : y.hq;
  r.gid = first ? x.gid : y.gid;
  r.tok0 = first ? x.tok0 : y.tok0;
  r.rows = first ? x.rows : y.rows;
  return r;
}

// Registers carrying the next block's inputs (and at a v-head or item
// boundary its T, gates, q and k) while the current block is computed.
struct Pref {
  uint4 s[2], d[2], o, v, t, q[2], k[2];
  float g, b;
  float fr;  // waves 5, 6: the q (k) row factor of lane's row (rows normalised upstream)
};

struct Ctx {
  char *smem;
  int tid, w, lane, h, r32;
  // lane quantities re-derived from an opaque copy of the thread index, so
  // that the per-lane addresses built on them are recomputed inside each
  // loop iteration rather than hoisted out and held (or spilled) across it
  __device__ void relane() {
    tid = opaque_tid();
    lane = tid & 63;
    h = lane >> 5;
    r32 = lane & 31;
  }
  __device__ bf16 *bf(int off) const { return reinterpret_cast<bf16 *>(smem + off); }
  __device__ Small &sm() const { return *reinterpret_cast<Small *>(smem + oF); }
};

__device__ __forceinline__ const bf16 *states_of(const BwdArgs &a) {
  return reinterpret_cast<const bf16 *>(a.hcache ? a.hcache : a.ws + a.wl.hstates);
}

// The loads below are issued unconditionally; with on = false their buffer
// ranges are empty (no memory access; the registers read 0).  Loads in
// branches would leave the compiler copying the results between registers
// where the branches join, which waits for the loads right after their issue.
//
// S, D, dO and V of block vb of v-head hl (rows past the chunk read 0)
// (parts: 1 = S and D, 2 = dO and V, 3 = all)
__device__ __forceinline__ void load_block(Pref &pf, const BwdArgs &a, const GItem &x, int hl,
                                           int vb, bool on, const Ctx &c, int part = 3) {
  const Problem &p = a.p;
  const int h = x.hq * (p.Hv / p.Hq) + hl;
  const int64_t cg = x.gid * p.Hv + h;
  const uint32_t kv_bytes = on ? (uint32_t)(K * slice::V * 2) : 0u;
  const auto rs = slice::rsrc_of(states_of(a) + cg * (K * slice::V), kv_bytes);
  const auto rd = slice::rsrc_of(reinterpret_cast<const bf16 *>(a.ws + a.wl.dstates) +
                                     cg * (K * slice::V),
                                 kv_bytes);
  if (part & 1) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint32_t off = (uint32_t)(vb * 1024 + c.tid + kThr * m) * 16u;
      pf.s[m] = slice::bload16(rs, off);
      pf.d[m] = slice::bload16(rd, off);
    }
  }
  if (!(part & 2)) return;
  const uint32_t v_rs = (uint32_t)(p.Hv * slice::V * 2);
  const int64_t e0 = (x.tok0 * p.Hv + h) * slice::V + vb * VB;
  const uint32_t vbytes = on ? x.rows * v_rs : 0u;
  const auto ro = slice::rsrc_of(reinterpret_cast<const bf16 *>(a.dout) + e0, vbytes);
  const auto rv = slice::rsrc_of(reinterpret_cast<const bf16 *>(a.v) + e0, vbytes);
  const uint32_t off = (uint32_t)(c.tid >> 3) * v_rs + (uint32_t)(c.tid & 7) * 16u;
  pf.o = slice::bload16(ro, off);
  pf.v = slice::bload16(rv, off);
}

// T and (wave 7) the raw gates of v-head hl
__device__ __forceinline__ void load_head(Pref &pf, const BwdArgs &a, const GItem &x, int hl,
                                          bool on, const Ctx &c) {
  const Problem &p = a.p;
  const int h = x.hq * (p.Hv / p.Hq) + hl;
  const int64_t cg = x.gid * p.Hv + h;
  const bf16 *tm = reinterpret_cast<const bf16 *>(a.tm_ext ? a.tm_ext : a.ws + a.wl.fwd.tmat);
  pf.t = slice::bload16(slice::rsrc_of(tm + cg * 4096, on ? 8192u : 0u), (uint32_t)c.tid * 16u);
  if (c.w == 7) {
    const int64_t gi = x.tok0 * p.Hv + h;
    const int rows = on ? x.rows : 0;
    const auto rg = slice::rsrc_of(a.g + gi, (uint32_t)(rows * p.Hv * 4));
    const auto rb = slice::rsrc_of(reinterpret_cast<const bf16 *>(a.beta) + gi,
                                   (uint32_t)(rows * p.Hv * 2));
    pf.g = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rg, (int)(c.lane * p.Hv * 4), 0, 0));
    const unsigned short bb =
        __builtin_amdgcn_raw_buffer_load_b16(rb, (int)(c.lane * p.Hv * 2), 0, 0);
    pf.b = __builtin_bit_cast(float, (unsigned)bb << 16);
  }
}

__device__ __forceinline__ void load_qk(Pref &pf, const BwdArgs &a, const GItem &x, bool on,
                                        const Ctx &c) {
  const Problem &p = a.p;
  const uint32_t qk_rs = (uint32_t)(p.Hq * K * 2);
  const int64_t e0 = (x.tok0 * p.Hq + x.hq) * K;
  const uint32_t bytes = on ? x.rows * qk_rs : 0u;
  const auto rq = slice::rsrc_of(reinterpret_cast<const bf16 *>(a.q) + e0, bytes);
  const auto rk = slice::rsrc_of(reinterpret_cast<const bf16 *>(a.k) + e0, bytes);
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int ci = c.tid + kThr * m;
    const uint32_t off = (uint32_t)(ci >> 4) * qk_rs + (uint32_t)(ci & 15) * 16u;
    pf.q[m] = slice::bload16(rq, off);
    pf.k[m] = slice::bload16(rk, off);
  }
  // rows normalised upstream: their factors (wave 5 for q, wave 6 for k;
  // empty ranges elsewhere)
  const bool fw = a.rq && (c.w == 5 || c.w == 6) && on;
  const float *fb = (c.w == 5 ? a.rq : a.rk);
  const auto rf = slice::rsrc_of(fb ? fb + x.tok0 * p.Hq + x.hq : nullptr,
                                 fw ? (uint32_t)(x.rows * p.Hq * 4) : 0u);
  pf.fr = __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(rf, (int)(c.lane * p.Hq * 4), 0, 0));
}

// The block's inputs into LDS.  A 16-byte piece of the states' lane layout
// holds k = 16 kb + rho(h, e) of one column v: stored at position 16 kb + 8 h
// of row v it is already in the pi layout.  Also <D, S> of the pieces.
__device__ __forceinline__ void commit_block(const Pref &pf, const Ctx &c, float &glp) {
  uint4 *sS = reinterpret_cast<uint4 *>(c.smem + oS), *sD = reinterpret_cast<uint4 *>(c.smem + oD);
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    // 16-byte units: rows of P128 / 8, piece 2 w + h
    const int u = (32 * m + c.r32) * (P128 / 8) + 2 * c.w + c.h;
    sS[u] = pf.s[m];
    sD[u] = pf.d[m];
    glp = dot_piece<bf16>(pf.s[m], pf.d[m], glp);
  }
  const int r = c.tid >> 3, pc = c.tid & 7;
  put_pi(c.bf(oO) + r * P64, pc, pf.o);
  put_pi(c.bf(oV) + r * P64, pc, pf.v);
}
__device__ __forceinline__ void commit_head(const Pref &pf, const Ctx &c) {
  put_pi(c.bf(oT) + (c.tid >> 3) * P64, c.tid & 7, pf.t);
}
// (with in-library L2 normalisation the rows are normalised on the way, and
// their factors kept for the chain rule of dq, dk; rows normalised upstream
// come with their factors)
__device__ __forceinline__ void commit_qk(const Pref &pf, const Ctx &c, bool l2) {
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int ci = c.tid + kThr * m;
    float fq = 0.f, fk = 0.f;
    const uint4 xq = l2 ? l2n_piece<bf16, 16>(pf.q[m], fq) : pf.q[m];
    const uint4 xk = l2 ? l2n_piece<bf16, 16>(pf.k[m], fk) : pf.k[m];
    put_pi(c.bf(oQ) + (ci >> 4) * P128, ci & 15, xq);
    put_pi(c.bf(oK) + (ci >> 4) * P128, ci & 15, xk);
    if (l2 && (ci & 15) == 0) {
      c.sm().rq[ci >> 4] = fq;
      c.sm().rk[ci >> 4] = fk;
    }
  }
  if (!l2 && (c.w == 5 || c.w == 6)) (c.w == 5 ? c.sm().rq : c.sm().rk)[c.lane] = pf.fr;
}
// one wave: cumulative gates of the chunk (lane = row) into gate set `set`
__device__ __forceinline__ void commit_gates(const Pref &pf, const Ctx &c, int set) {
  Small &sm = c.sm();
  const float gam = wave_incl_scan(pf.g) * kLog2e;
  const float gL = lane63(gam);
  sm.gam[set][c.lane] = gam;
  sm.eg[set][c.lane] = __builtin_amdgcn_exp2f(gam);
  sm.dec[set][c.lane] = __builtin_amdgcn_exp2f(gL - gam);
  sm.bet[set][c.lane] = pf.b;
}

// The 16 per-row values of arr at this lane's accumulator rows of row tile rt
// (rows 32 rt + 8 (i >> 2) + 4 h + (i & 3)).
__device__ __forceinline__ void rows16(float (&x)[16], const float *arr, int rt, int h) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(arr + 32 * rt + 8 * b + 4 * h);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * b + e] = v[e];
  }
}
// Values of a pi-layout matrix X (row pitch PITCH) at the accumulator
// positions of tile (row tile rt, column tile j), as floats.
template <int PITCH>
__device__ __forceinline__ void acc_vals(float (&x)[16], const TrA &tr, int rt, int j) {
  const bf16x8 a = tr.at(2 * rt, j, PITCH), b = tr.at(2 * rt + 1, j, PITCH);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = (float)a[e];
    x[8 + e] = (float)b[e];
  }
}
// Sum of x[i] over the 32 lanes that share l >> 5, by halving exchanges:
// lanes l and l ^ 1 end with the total of register index red_index(l).
__device__ __forceinline__ float reduce32(const float (&x)[16], int lane) {
  float y8[8], y4[4], y2[2];
  {
    const bool hi = lane & 16;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float keep = hi ? x[j + 8] : x[j], send = hi ? x[j] : x[j + 8];
      y8[j] = keep + __shfl_xor(send, 16, 64);
    }
  }
  {
    const bool hi = lane & 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float keep = hi ? y8[j + 4] : y8[j], send = hi ? y8[j] : y8[j + 4];
      y4[j] = keep + __shfl_xor(send, 8, 64);
    }
  }
  {
    const bool hi = lane & 4;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float keep = hi ? y4[j + 2] : y4[j], send = hi ? y4[j] : y4[j + 2];
      y2[j] = keep + __shfl_xor(send, 4, 64);
    }
  }
  const bool hi = lane & 2;
  float y = (hi ? y2[1] : y2[0]) + __shfl_xor(hi ? y2[0] : y2[1], 2, 64);
  return y + __shfl_xor(y, 1, 64);
}
__device__ __forceinline__ int red_index(int lane) {
  return ((lane >> 4) & 1) * 8 + ((lane >> 3) & 1) * 4 + ((lane >> 2) & 1) * 2 +
         ((lane >> 1) & 1);
}
// row (inside its 32-row tile) of register index j for this lane
__device__ __forceinline__ int acc_row(int j, int h) { return 8 * (j >> 2) + 4 * h + (j & 3); }
// reduce32 of x written to dst[row] (dst indexed by the row inside the tile)
__device__ __forceinline__ void reduce_rows_to(float *dst, const float (&x)[16], int lane) {
  const float y = reduce32(x, lane);
  if (!(lane & 1)) dst[acc_row(red_index(lane), lane >> 5)] = y;
}

// dv rows of the current block (all threads): wave w takes V columns
// 8 w .. 8 w + 7 of the block for all 64 rows, from dR^T by transpose reads.
__device__ __forceinline__ void store_dv(const BwdArgs &a, const GItem &x, int hl, int vb,
                                         int set, const Ctx &c) {
  const Problem &p = a.p;
  const int h = x.hq * (p.Hv / p.Hq) + hl;
  const int G = c.lane >> 4, sgm = c.lane & 15, i = c.lane & 15;
  const bf16 *src = c.bf(oDRT) + (8 * c.w + (sgm >> 2)) * P64 + 16 * G + 4 * (sgm & 3);
  const bf16x4 lo = tr4(src), hi = tr4(src + 4 * P64);
  const int r = 16 * G + 4 * pi4(i >> 2) + (i & 3);
  const float bt = c.sm().bet[set][r];
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = (bf16)(bt * (float)lo[e]);
    o[4 + e] = (bf16)(bt * (float)hi[e]);
  }
  const uint32_t v_rs = (uint32_t)(p.Hv * slice::V * 2);
  const auto rd = raw_buffer(reinterpret_cast<bf16 *>(a.dv) +
                                 (x.tok0 * p.Hv + h) * slice::V + vb * VB,
                             x.rows * v_rs);
  buf_store16(__builtin_bit_cast(uint4, o), rd, (uint32_t)r * v_rs + (uint32_t)c.w * 16u);
}

// dgamma -> dg (reverse cumulative sum inside the chunk) and dbeta of v-head
// hl from the partial sums (one wave; lane l takes row 63 - l)
__device__ __forceinline__ void store_gates(const BwdArgs &a, const GItem &x, int hl, int set,
                                            const Ctx &c) {
  const Problem &p = a.p;
  const Small &sm = c.sm();
  const int r = 63 - c.lane, rr = r & 31;
  float gl = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) gl += sm.gl[i];
  const float pq = sm.pq[0][r] + sm.pq[1][r];
  const float pc = sm.pc[0][r] + sm.pc[1][r];
  const float pa2 = sm.pa2[0][r] + sm.pa2[1][r];
  const float pa1 = sm.pa1[0][r] + sm.pa1[1][r];
  float rs, cs, dbk;
  if (r < 32) {
    rs = sm.rsP[0][rr] + sm.rsA[0][rr];
    dbk = sm.dbA[0][rr];
    cs = sm.csP[0][rr] + sm.csA[0][rr] + sm.csP[1][rr] + sm.csA[1][rr];
  } else {
    rs = sm.rsP[1][rr] + sm.rsA[1][rr] + sm.rsP[2][rr] + sm.rsA[2][rr];
    dbk = sm.dbA[1][rr] + sm.dbA[2][rr];
    cs = sm.csP[2][rr] + sm.csA[2][rr];
  }
  const float eg = sm.eg[set][r], bt = sm.bet[set][r];
  const float de = p.scale * pq - bt * pa2;
  const float cr = sm.dec[set][r] * pc;
  float dgam = eg * de + rs - cs - cr;
  const float csum = wave_sum(cr);
  if (r == x.rows - 1) dgam += csum + sm.eg[set][63] * gl;
  if (r >= x.rows) dgam = 0.f;
  const float xs = wave_incl_scan(dgam);
  if (r < x.rows) {
    const int h = x.hq * (p.Hv / p.Hq) + hl;
    const int64_t gi = (x.tok0 + r) * p.Hv + h;
    a.dg[gi] = xs;
    reinterpret_cast<bf16 *>(a.dbeta)[gi] = (bf16)(pa1 - eg * pa2 + dbk);
  }
}

// ---------------------------------------------------------------- roles
// ROLE 0..3: waves 0..3 (V-chain waves; 0, 1 form Vn, 2, 3 form dR, for
// V column tile c = ROLE & 1 of the block).  E tiles: wave 0 holds dP of
// tiles 0, 1 (with the raw Q K^T), wave 1 dA of tiles 0, 1 (with the raw
// K K^T), wave 2 dP of tile 2, wave 3 dA of tile 2.
// ROLE 4: waves 4..7, dq and dk tiles (row tile rt = (w - 4) >> 1, column
// tiles 2 kp, 2 kp + 1 with kp = (w - 4) & 1).
template <int ROLE>
struct Role {
  static constexpr bool kV = ROLE < 4;
  static constexpr bool kVn = ROLE == 0 || ROLE == 1;  // KS -> Vn chain
  static constexpr bool kDR = ROLE == 2 || ROLE == 3;  // KD -> dR chain
  static constexpr int c = ROLE & 1;
  static constexpr bool kHoldP = ROLE == 0 || ROLE == 2;  // dP + QK^T holder
  static constexpr int NE = ROLE < 2 ? 2 : (ROLE < 4 ? 1 : 0);
  static constexpr int E0 = ROLE < 2 ? 0 : 2;
};

// raw Q K^T (dP holders) or K K^T (dA holders) of the held E tiles
template <int ROLE>
__device__ __forceinline__ void raw_tiles(f32x16 (&raw)[2], const Ctx &c) {
  using R = Role<ROLE>;
  const bf16 *sA = c.bf(R::kHoldP ? oQ : oK), *sK = c.bf(oK);
#pragma unroll
  for (int j = 0; j < R::NE; ++j) {
    const int p = R::E0 + j;
    const bf16 *pa = sA + (32 * e_st(p) + c.r32) * P128 + 8 * c.h;
    const bf16 *pb = sK + (32 * e_tt(p) + c.r32) * P128 + 8 * c.h;
    f32x16 acc = zero16();
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = mma32(lds16(pa + 16 * s), lds16(pb + 16 * s), acc);
    raw[j] = acc;
  }
}
// P^T of the held tiles (dP holders) into LDS for gate set `set`
template <int ROLE>
__device__ __forceinline__ void write_pt(const f32x16 (&raw)[2], const Ctx &c, int set) {
  using R = Role<ROLE>;
  const Small &sm = c.sm();
#pragma unroll
  for (int j = 0; j < R::NE; ++j) {
    const int p = R::E0 + j, st = e_st(p), tt = e_tt(p);
    const int t = 32 * tt + c.r32;
    const float gt = sm.gam[set][t];
    float gs[16];
    rows16(gs, sm.gam[set], st, c.h);
    f32x16 pv;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int s = 32 * st + acc_row(i, c.h);
      pv[i] = (t <= s) ? raw[j][i] * __builtin_amdgcn_exp2f(gs[i] - gt) : 0.f;
    }
    bf16 *dst = c.bf(oPt) + t * P64 + 32 * st + 8 * c.h;
    *reinterpret_cast<bf16x8 *>(dst) = slots(pv, 0);
    *reinterpret_cast<bf16x8 *>(dst + 16) = slots(pv, 1);
  }
}

// End of a v-head, dP / dA holders: (dP * E)^T and dKK^T (strict part) of
// their tiles into LDS, with the row and column sums for dgamma, dbeta.
template <int ROLE>
__device__ __forceinline__ void e_tiles_out(const f32x16 (&eacc)[2], const f32x16 (&eraw)[2],
                                            const Ctx &c, int set, float scale) {
  using R = Role<ROLE>;
  Small &sm = c.sm();
#pragma unroll
  for (int j = 0; j < R::NE; ++j) {
    const int pt = R::E0 + j, st = e_st(pt), tt = e_tt(pt);
    const int t = 32 * tt + c.r32;
    const float gt = sm.gam[set][t];
    float gs[16], bs[16];
    rows16(gs, sm.gam[set], st, c.h);
    rows16(bs, sm.bet[set], st, c.h);
    f32x16 out;
    float rsum[16], dbk[16], csum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int s = 32 * st + acc_row(i, c.h);
      if constexpr (R::kHoldP) {
        const bool in = t <= s;
        const float e = in ? __builtin_amdgcn_exp2f(gs[i] - gt) : 0.f;
        const float pe = in ? scale * eacc[j][i] * e : 0.f;
        out[i] = pe;
        rsum[i] = pe * eraw[j][i];
      } else {
        const bool in = t < s;
        const float e = in ? __builtin_amdgcn_exp2f(gs[i] - gt) : 0.f;
        const float dam = in ? -eacc[j][i] : 0.f;
        const float kkv = in ? bs[i] * dam * e : 0.f;
        out[i] = kkv;
        rsum[i] = kkv * eraw[j][i];
        dbk[i] = dam * eraw[j][i] * e;
      }
      csum += rsum[i];
    }
    bf16 *dst = c.bf(R::kHoldP ? oPEt : oUt) + t * P64 + 32 * st + 8 * c.h;
    *reinterpret_cast<bf16x8 *>(dst) = slots(out, 0);
    *reinterpret_cast<bf16x8 *>(dst + 16) = slots(out, 1);
    reduce_rows_to(R::kHoldP ? sm.rsP[pt] : sm.rsA[pt], rsum, c.lane);
    if constexpr (!R::kHoldP) reduce_rows_to(sm.dbA[pt], dbk, c.lane);
    csum += __shfl_xor(csum, 32, 64);
    if (c.h == 0) (R::kHoldP ? sm.csP[pt] : sm.csA[pt])[c.r32] = csum;
  }
}

// In-library L2 normalisation: dq, dk so far are gradients with respect to
// the normalised rows x_hat = x r; back to the raw rows,
// dx = r (dx_hat - x_hat <x_hat, dx_hat>).  The dq, dk waves put dx_hat into
// LDS in fp32 (rows of pitch F32P floats, over regions that are free at the
// end of an item); then every thread takes one 8-column piece of a q row and
// of a k row, forms the row dot over the 16 lanes that hold the row, and
// writes dx.
constexpr int F32P = 132;
constexpr int oFQ = oS, oFK = oO;
// (dk reaches into P^T's first rows, which the next item rewrites whole; it
// stays clear of P^T's zero block, rows 32..63 of positions 0..31)
static_assert(oFQ + 64 * F32P * 4 <= oO && oFK + 64 * F32P * 4 <= oPt + 32 * P64 * 2,
              "fp32 staging");
__device__ __forceinline__ void stage_f32(const f32x16 (&x)[2], int off, int rt, int kp,
                                          const Ctx &c) {
  float *f = reinterpret_cast<float *>(c.smem + off);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = 32 * (2 * kp + j) + c.r32;
#pragma unroll
    for (int i = 0; i < 16; ++i) f[(32 * rt + acc_row(i, c.h)) * F32P + col] = x[j][i];
  }
}
// piece pc (columns 8 pc .. 8 pc + 7) of a pi-layout bf16 row, in natural order
__device__ __forceinline__ uint4 get_pi(const bf16 *row, int pc) {
  const int blk = (8 * pc) & ~15, q0 = 2 * (pc & 1);
  const uint2 lo = *reinterpret_cast<const uint2 *>(row + blk + 4 * slice::pi4(q0));
  const uint2 hi = *reinterpret_cast<const uint2 *>(row + blk + 4 * slice::pi4(q0 + 1));
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}
__device__ __forceinline__ uint4 l2_back(const bf16 *xrow, const float *drow, float r, int pc) {
  const uint4 xp = get_pi(xrow, pc);
  const bf16 *xh = reinterpret_cast<const bf16 *>(&xp);
  const f32x4 d0 = *reinterpret_cast<const f32x4 *>(drow + 8 * pc);
  const f32x4 d1 = *reinterpret_cast<const f32x4 *>(drow + 8 * pc + 4);
  float d[8], x[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    d[e] = d0[e];
    d[4 + e] = d1[e];
  }
  float t = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = (float)xh[e];
    t += x[e] * d[e];
  }
  t = group_sum<16>(t);
  uint4 out;
  bf16 *o = reinterpret_cast<bf16 *>(&out);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (bf16)(r * (d[e] - x[e] * t));
  return out;
}

// dq += (dP * E) K;  dk += (dP * E)^T Q + (dKK + dKK^T) K  (dq, dk waves)
__device__ __forceinline__ void e_products(f32x16 (&dq)[2], f32x16 (&dk)[2], int rt, int kp,
                                           const Ctx &c) {
  const TrA trPE(c.bf(oPEt), P64, c.lane), trU(c.bf(oUt), P64, c.lane);
  const TrA trK(c.bf(oK), P128, c.lane), trQ(c.bf(oQ), P128, c.lane);
  const bf16 *ppe = c.bf(oPEt) + (32 * rt + c.r32) * P64 + 8 * c.h;
  const bf16 *pu = c.bf(oUt) + (32 * rt + c.r32) * P64 + 8 * c.h;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const bf16x8 ape = trPE.at(s, rt, P64), apt = lds16(ppe + 16 * s);
    // dKK^T has its strict part only: the two reads never overlap
    const uint4 x1 = __builtin_bit_cast(uint4, lds16(pu + 16 * s));
    const uint4 x2 = __builtin_bit_cast(uint4, trU.at(s, rt, P64));
    const bf16x8 am = __builtin_bit_cast(
        bf16x8, make_uint4(x1.x | x2.x, x1.y | x2.y, x1.z | x2.z, x1.w | x2.w));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kt = 2 * kp + j;
      const bf16x8 kb = trK.at(s, kt, P128);
      dq[j] = mma32(ape, kb, dq[j]);
      dk[j] = mma32(apt, trQ.at(s, kt, P128), dk[j]);
      dk[j] = mma32(am, kb, dk[j]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int ROLE>
__device__ void run(const BwdArgs &a, const Ctx &c0) {
  using R = Role<ROLE>;
  const Problem &p = a.p;
  const int Gq = p.Hv / p.Hq;
  const int64_t n_items = a.plan.total_chunks * p.Hq;
  const float scale = p.scale;
  Ctx c = c0;
  Small &sm = c.sm();

  // role state
  f32x16 eacc[2], eraw[2];            // V waves: dP / dA tiles and raw products
  float pa1[2][16];                   // waves 2, 3: sum_v dR V of a block
  f32x16 dq[2], dk[2];                // waves 4..7
  float pq[16], pc[16], pa2[16];      // waves 4..7: row-dot partials
  const int rt = (c.w - 4) >> 1, kp = (c.w - 4) & 1;  // waves 4..7
  float glp = 0.f;

  Pref pf;
  GItem cur = item_at(a, blockIdx.x);
  load_qk(pf, a, cur, true, c);
  load_head(pf, a, cur, 0, true, c);
  load_block(pf, a, cur, 0, 0, true, c);
  int u = 0;  // v-heads done by this workgroup (gate set u & 1)

  for (int64_t it = blockIdx.x; it < n_items; it += gridDim.x) {
    const bool has_next = it + gridDim.x < n_items;
    const GItem nxt = has_next ? item_at(a, it + gridDim.x) : cur;
    c.relane();
    // ---- item start: q, k, the first v-head's T and gates
    __syncthreads();
    commit_qk(pf, c, p.l2);
    commit_head(pf, c);
    if (c.w == 7) commit_gates(pf, c, u & 1);
    __syncthreads();
    if constexpr (R::kV) {
      raw_tiles<ROLE>(eraw, c);
      if constexpr (R::kHoldP) write_pt<ROLE>(eraw, c, u & 1);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        dq[j] = zero16();
        dk[j] = zero16();
      }
    }

    for (int hl = 0; hl < Gq; ++hl) {
      const int set = u & 1;
      if constexpr (R::kV) {
#pragma unroll
        for (int j = 0; j < R::NE; ++j) eacc[j] = zero16();
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) pq[i] = pc[i] = pa2[i] = 0.f;
      }
      for (int vb = 0; vb < NVB; ++vb) {
        c.relane();
        __syncthreads();  // the previous block's readers are done
        commit_block(pf, c, glp);
        // the block after this one: the next V block, else the next v-head's
        // first block (with its T and gates: loaded in a v-head's last
        // block), else the next item's (with its q, k).  Waves 4..7 issue
        // their share of the loads at the start of phase V (theirs is the
        // shorter one), waves 0..3 theirs at its end and at the start of
        // phase K, so that the loads of the workgroup do not queue together.
        auto prefetch = [&](int part) {
          const bool in_head = vb + 1 < NVB, in_item = in_head || hl + 1 < Gq;
          const GItem x = pick(in_item, cur, nxt);
          const int nhl = in_head ? hl : (in_item ? hl + 1 : 0);
          const int nvb = in_head ? vb + 1 : 0;
          const bool any = in_item || has_next;
          load_block(pf, a, x, nhl, nvb, any, c, part);
          if ((part & 2) && vb + 1 == NVB) {
            load_head(pf, a, x, nhl, any, c);
            load_qk(pf, a, x, !in_item && has_next, c);
          }
        };
        if (vb == 0 && hl > 0) {
          // this v-head's P^T (its gates were committed at the end of the
          // previous v-head); the previous v-head's dg, dbeta
          if constexpr (R::kHoldP) write_pt<ROLE>(eraw, c, set);
          if constexpr (ROLE == 1) store_gates(a, cur, hl - 1, set ^ 1, c);
          if constexpr (!R::kV) e_products(dq, dk, rt, kp, c);
        }
        __syncthreads();
        // ---------------------------------------------------------- phase V
        if constexpr (R::kVn) {
          // KS for columns 32 c .., both row tiles
          f32x16 acc[2] = {zero16(), zero16()};
          {
            const bf16 *pb = c.bf(oS) + (32 * R::c + c.r32) * P128 + 8 * c.h;
            const bf16 *pa = c.bf(oK) + c.r32 * P128 + 8 * c.h;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              const bf16x8 b = lds16(pb + 16 * s);
              acc[0] = mma32(lds16(pa + 16 * s), b, acc[0]);
              acc[1] = mma32(lds16(pa + 32 * P128 + 16 * s), b, acc[1]);
            }
          }
          // R = beta (V - e^gamma KS) as operand slots over its rows
          bf16x8 rsl[4];
          {
            const TrA trV(c.bf(oV), P64, c.lane);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              float vv[16], eg[16], bt[16];
              acc_vals<P64>(vv, trV, t, R::c);
              rows16(eg, sm.eg[set], t, c.h);
              rows16(bt, sm.bet[set], t, c.h);
#pragma unroll
              for (int i = 0; i < 16; ++i)
                rsl[2 * t + (i >> 3)][i & 7] = (bf16)(bt[i] * (vv[i] - eg[i] * acc[t][i]));
            }
          }
          // Vn = T R; Vn^T rows into LDS
          f32x16 vn[2] = {zero16(), zero16()};
          {
            const bf16 *pa = c.bf(oT) + c.r32 * P64 + 8 * c.h;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              vn[0] = mma32(lds16(pa + 16 * s), rsl[s], vn[0]);
              vn[1] = mma32(lds16(pa + 32 * P64 + 16 * s), rsl[s], vn[1]);
            }
          }
          bf16 *dst = c.bf(oVnT) + (32 * R::c + c.r32) * P64 + 8 * c.h;
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            *reinterpret_cast<bf16x8 *>(dst + 32 * t) = slots(vn[t], 0);
            *reinterpret_cast<bf16x8 *>(dst + 32 * t + 16) = slots(vn[t], 1);
          }
        } else if constexpr (R::kDR) {
          // P^T dO and KD for columns 32 c .., both row tiles
          f32x16 kd[2] = {zero16(), zero16()}, y[2] = {zero16(), zero16()};
          {
            const TrA trO(c.bf(oO), P64, c.lane);
            const bf16 *pp = c.bf(oPt) + c.r32 * P64 + 8 * c.h;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const bf16x8 b = trO.at(s, R::c, P64);
              y[0] = mma32(lds16(pp + 16 * s), b, y[0]);
              y[1] = mma32(lds16(pp + 32 * P64 + 16 * s), b, y[1]);
            }
            const bf16 *pb = c.bf(oD) + (32 * R::c + c.r32) * P128 + 8 * c.h;
            const bf16 *pa = c.bf(oK) + c.r32 * P128 + 8 * c.h;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              const bf16x8 b = lds16(pb + 16 * s);
              kd[0] = mma32(lds16(pa + 16 * s), b, kd[0]);
              kd[1] = mma32(lds16(pa + 32 * P128 + 16 * s), b, kd[1]);
            }
          }
          // dVn = dec KD + scale P^T dO as operand slots over its rows
          bf16x8 dsl[4];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            float dc[16];
            rows16(dc, sm.dec[set], t, c.h);
#pragma unroll
            for (int i = 0; i < 16; ++i)
              dsl[2 * t + (i >> 3)][i & 7] = (bf16)(dc[i] * kd[t][i] + scale * y[t][i]);
          }
          // dR = T^T dVn; dR^T rows into LDS; sum_v dR V
          f32x16 dr[2] = {zero16(), zero16()};
          {
            const TrA trT(c.bf(oT), P64, c.lane);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              dr[0] = mma32(trT.at(s, 0, P64), dsl[s], dr[0]);
              dr[1] = mma32(trT.at(s, 1, P64), dsl[s], dr[1]);
            }
          }
          bf16 *dst = c.bf(oDRT) + (32 * R::c + c.r32) * P64 + 8 * c.h;
          const TrA trV(c.bf(oV), P64, c.lane);
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            *reinterpret_cast<bf16x8 *>(dst + 32 * t) = slots(dr[t], 0);
            *reinterpret_cast<bf16x8 *>(dst + 32 * t + 16) = slots(dr[t], 1);
            float vv[16];
            acc_vals<P64>(vv, trV, t, R::c);
#pragma unroll
            for (int i = 0; i < 16; ++i) pa1[t][i] = dr[t][i] * vv[i];
          }
        } else {
          prefetch(3);
          // X = dO S^T for dq tiles (rt, 2 kp + j); row dot with Q
          const bf16 *pa = c.bf(oO) + (32 * rt + c.r32) * P64 + 8 * c.h;
          bf16x8 ao[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) ao[s] = lds16(pa + 16 * s);
          const TrA trS(c.bf(oS), P128, c.lane), trQ(c.bf(oQ), P128, c.lane);
          float sce[16];
          rows16(sce, sm.eg[set], rt, c.h);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int kt = 2 * kp + j;
            f32x16 x = zero16();
#pragma unroll
            for (int s = 0; s < 4; ++s) x = mma32(ao[s], trS.at(s, kt, P128), x);
            float qv[16];
            acc_vals<P128>(qv, trQ, rt, kt);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              pq[i] += qv[i] * x[i];
              dq[j][i] += scale * sce[i] * x[i];
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if constexpr (R::kV) prefetch(2);
        __syncthreads();
        // ---------------------------------------------------------- phase K
        if constexpr (R::kV) prefetch(1);
        store_dv(a, cur, hl, vb, set, c);
        if constexpr (R::kV) {
          const TrA trVn(c.bf(oVnT), P64, c.lane);
#pragma unroll
          for (int j = 0; j < R::NE; ++j) {
            const int pt = R::E0 + j, st = e_st(pt), tt = e_tt(pt);
            if constexpr (R::kHoldP) {
              const bf16 *pa = c.bf(oO) + (32 * st + c.r32) * P64 + 8 * c.h;
#pragma unroll
              for (int s = 0; s < 4; ++s)
                eacc[j] = mma32(lds16(pa + 16 * s), trVn.at(s, tt, P64), eacc[j]);
            } else {
              const TrA trDR(c.bf(oDRT), P64, c.lane);
#pragma unroll
              for (int s = 0; s < 4; ++s)
                eacc[j] = mma32(trDR.at(s, st, P64), trVn.at(s, tt, P64), eacc[j]);
            }
          }
        } else {
          // Vn D^T and dR S^T for dk tiles (rt, 2 kp + j), one after the
          // other (row dots with K, then into dk with their row scales)
          const TrA trVn(c.bf(oVnT), P64, c.lane), trDR(c.bf(oDRT), P64, c.lane);
          const TrA trD(c.bf(oD), P128, c.lane), trS(c.bf(oS), P128, c.lane);
          const TrA trK(c.bf(oK), P128, c.lane);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int kt = 2 * kp + j;
            float kv[16];
            acc_vals<P128>(kv, trK, rt, kt);
            {
              f32x16 t1 = zero16();
#pragma unroll
              for (int s = 0; s < 4; ++s) t1 = mma32(trVn.at(s, rt, P64), trD.at(s, kt, P128), t1);
              float dc[16];
              rows16(dc, sm.dec[set], rt, c.h);
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                pc[i] += kv[i] * t1[i];
                dk[j][i] += dc[i] * t1[i];
              }
            }
            __builtin_amdgcn_sched_barrier(0);
            {
              f32x16 t2 = zero16();
#pragma unroll
              for (int s = 0; s < 4; ++s) t2 = mma32(trDR.at(s, rt, P64), trS.at(s, kt, P128), t2);
              float eg[16], bt[16];
              rows16(eg, sm.eg[set], rt, c.h);
              rows16(bt, sm.bet[set], rt, c.h);
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                pa2[i] += kv[i] * t2[i];
                dk[j][i] -= bt[i] * eg[i] * t2[i];
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if constexpr (R::kDR) {
          // sum_v dR V of this block, added to the rows' totals in LDS
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            float y[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) y[i] = pa1[t][i];
            const float r = reduce32(y, c.lane);
            float *dst = sm.pa1[R::c] + 32 * t + acc_row(red_index(c.lane), c.h);
            if (!(c.lane & 1)) *dst = vb == 0 ? r : *dst + r;
          }
        }
      }
      // ---- end of the v-head (no barrier needed: each wave works on its own
      // registers; the LDS it writes is not read before the next barrier)
      // the held dP, dA tiles are complete
      if constexpr (R::kV) {
        e_tiles_out<ROLE>(eacc, eraw, c, set, scale);
      } else {
        reduce_rows_to(sm.pq[kp] + 32 * rt, pq, c.lane);
        reduce_rows_to(sm.pc[kp] + 32 * rt, pc, c.lane);
        reduce_rows_to(sm.pa2[kp] + 32 * rt, pa2, c.lane);
      }
      const float gsum = wave_sum(glp);
      if (c.lane == 0) sm.gl[c.w] = gsum;
      glp = 0.f;
      if (hl + 1 < Gq) {
        // the next v-head's T (sT is no longer read) and gates
        commit_head(pf, c);
        if (c.w == 7) commit_gates(pf, c, set ^ 1);
      }
      ++u;
    }
    // ---- item end: the last v-head's chunk-matrix products and gates, then
    // dq, dk of the q/k head out through LDS
    c.relane();
    __syncthreads();
    if constexpr (!R::kV) e_products(dq, dk, rt, kp, c);
    if constexpr (ROLE == 1) store_gates(a, cur, Gq - 1, (u - 1) & 1, c);
    __syncthreads();
    const bool l2 = p.l2 || a.rq;
    if constexpr (!R::kV) {
      if (l2) {
        stage_f32(dq, oFQ, rt, kp, c);
        stage_f32(dk, oFK, rt, kp, c);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = 32 * (2 * kp + j) + c.r32;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = 32 * rt + acc_row(i, c.h);
            c.bf(oQ)[row * P128 + col] = (bf16)dq[j][i];
            c.bf(oK)[row * P128 + col] = (bf16)dk[j][i];
          }
        }
      }
    }
    __syncthreads();
    {
      const uint32_t qk_rs = (uint32_t)(p.Hq * K * 2);
      const int64_t e0 = (cur.tok0 * p.Hq + cur.hq) * K;
      const auto rq = raw_buffer(reinterpret_cast<bf16 *>(a.dq) + e0, cur.rows * qk_rs);
      const auto rk = raw_buffer(reinterpret_cast<bf16 *>(a.dk) + e0, cur.rows * qk_rs);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int ci = c.tid + kThr * m;
        const int r = ci >> 4, pc16 = ci & 15;
        const uint32_t off = (uint32_t)r * qk_rs + (uint32_t)pc16 * 16u;
        uint4 xq, xk;
        if (l2) {
          const float *fq = reinterpret_cast<const float *>(c.smem + oFQ) + r * F32P;
          const float *fk = reinterpret_cast<const float *>(c.smem + oFK) + r * F32P;
          xq = l2_back(c.bf(oQ) + r * P128, fq, c.sm().rq[r], pc16);
          xk = l2_back(c.bf(oK) + r * P128, fk, c.sm().rk[r], pc16);
        } else {
          xq = *reinterpret_cast<const uint4 *>(c.bf(oQ) + r * P128 + 8 * pc16);
          xk = *reinterpret_cast<const uint4 *>(c.bf(oK) + r * P128 + 8 * pc16);
        }
        buf_store16(xq, rq, off);
        buf_store16(xk, rk, off);
      }
    }
    cur = nxt;
  }
}

__global__ __launch_bounds__(kThr) void grad_slice_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  if ((int64_t)blockIdx.x >= a.plan.total_chunks * a.p.Hq) return;
  Ctx c;
  c.smem = smem;
  c.tid = threadIdx.x;
  c.w = wave_of(threadIdx.x);
  c.lane = threadIdx.x & 63;
  c.h = c.lane >> 5;
  c.r32 = c.lane & 31;
  // P^T, (dP * E)^T and dKK^T above the diagonal (rows t 32..63, positions
// 0..31) are 0 throughout
  if (c.tid < 128) {
    const int off = (32 + (c.tid >> 2)) * P64 + 8 * (c.tid & 3);
    *reinterpret_cast<uint4 *>(c.bf(oPt) + off) = make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4 *>(c.bf(oPEt) + off) = make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4 *>(c.bf(oUt) + off) = make_uint4(0u, 0u, 0u, 0u);
  }
  switch (c.w) {
    case 0: run<0>(a, c); break;
    case 1: run<1>(a, c); break;
    case 2: run<2>(a, c); break;
    case 3: run<3>(a, c); break;
    default: run<4>(a, c); break;
  }
}

}  // namespace gslice

bool grad_slice_supported(const BwdArgs &a) {
  return a.p.dtype == 1 && a.p.K == slice::K && a.p.V == slice::V;
}

hipError_t launch_grad_slice(const BwdArgs &a, hipStream_t st) {
  const int64_t items = a.plan.total_chunks * a.p.Hq;
  if (items <= 0) return hipSuccess;
  const int64_t grid = std::min<int64_t>(items, a.plan.cus > 0 ? a.plan.cus : 256);
  KernelTimer kt("local_grad", st);
  gslice::grad_slice_kernel<<<dim3((unsigned)grid), gslice::kThr, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace gdn
