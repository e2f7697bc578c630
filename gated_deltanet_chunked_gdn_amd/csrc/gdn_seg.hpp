// Machinery shared by the segment kernels of the forward and the backward:
// locating a chunk / segment of a (possibly packed) batch, the register
// prefetch of one chunk's inputs, and the K x V fp32 state held as 16x16
// accumulator tiles spread over the waves of a workgroup.
#pragma once

#include "gdn_common.hpp"
#include "gdn_internal.h"

namespace gdn {

constexpr int kNW = 8;              // waves per segment workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 64 * kNW;  // 512

struct SeqInfo {
  int64_t tok0;  // first token (flat index into the [B*T] token axis)
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

// Chunk `gid` (global, token order) -> sequence and chunk index inside it.
struct ChunkLoc {
  int n, c;
  SeqInfo si;
};

__device__ __forceinline__ ChunkLoc locate_chunk(const Problem &p, const int32_t *chunk_prefix,
                                                 int64_t gid) {
  ChunkLoc l;
  if (!p.cu) {
    const int nc = (p.T + kChunk - 1) / kChunk;
    l.n = (int)(gid / nc);
    l.c = (int)(gid % nc);
  } else {
    l.n = find_seq(chunk_prefix, p.N, gid);
    l.c = (int)(gid - chunk_prefix[l.n]);
  }
  l.si = seq_info(p, l.n);
  return l;
}

// Segment `sg` -> sequence, segment index j, chunk range, first chunk id.
struct SegLoc {
  int n, j, nseg;
  SeqInfo si;
  int64_t chunk0;  // global id of the sequence's first chunk
  int64_t seg0;    // global id of the sequence's first segment
  int c_begin, c_end;
};

__device__ __forceinline__ SegLoc locate_segment(const Problem &p, int seg_chunks,
                                                 const int32_t *chunk_prefix,
                                                 const int32_t *seg_prefix, int64_t sg) {
  SegLoc l;
  if (!p.cu) {
    const int nc = (p.T + kChunk - 1) / kChunk;
    l.nseg = (nc + seg_chunks - 1) / seg_chunks;
    l.n = (int)(sg / l.nseg);
    l.j = (int)(sg % l.nseg);
    l.chunk0 = (int64_t)l.n * nc;
    l.seg0 = (int64_t)l.n * l.nseg;
  } else {
    l.n = find_seq(seg_prefix, p.N, sg);
    l.j = (int)(sg - seg_prefix[l.n]);
    l.nseg = seg_prefix[l.n + 1] - seg_prefix[l.n];
    l.chunk0 = chunk_prefix[l.n];
    l.seg0 = seg_prefix[l.n];
  }
  l.si = seq_info(p, l.n);
  l.c_begin = l.j * seg_chunks;
  l.c_end = min(l.c_begin + seg_chunks, l.si.nchunks);
  return l;
}

// Same for a (sequence n) without a segment id (serial passes).
__device__ __forceinline__ SegLoc locate_sequence(const Problem &p, int seg_chunks,
                                                  const int32_t *chunk_prefix,
                                                  const int32_t *seg_prefix, int n) {
  SegLoc l;
  l.n = n;
  l.j = 0;
  l.si = seq_info(p, n);
  if (!p.cu) {
    const int nc = (p.T + kChunk - 1) / kChunk;
    l.nseg = (nc + seg_chunks - 1) / seg_chunks;
    l.chunk0 = (int64_t)n * nc;
    l.seg0 = (int64_t)n * l.nseg;
  } else {
    l.nseg = seg_prefix[n + 1] - seg_prefix[n];
    l.chunk0 = chunk_prefix[n];
    l.seg0 = seg_prefix[n];
  }
  l.c_begin = 0;
  l.c_end = l.si.nchunks;
  return l;
}

// Tile geometry of the segment kernels.
template <typename E, int K, int V>
struct Geo {
  // 32 bytes of row padding: 16-byte fragment reads of 16 consecutive rows
  // are then free of LDS bank conflicts (measured; 16 bytes of padding
  // leaves half of the LDS cycles to conflicts)
  static constexpr int PAD = 32 / (int)sizeof(E);
  static constexpr int LDK = K + PAD;   // rows of length K
  static constexpr int LDV = V + PAD;   // rows of length V
  static constexpr int LDC = 64 + PAD;  // rows of length 64 (chunk)
  static constexpr int NCT = V / 16;    // 16-wide column tiles over V
  static constexpr int NRT = K / 16;    // 16-high row tiles over K
  static constexpr int NCH = NCT / 2;   // column tiles per half
  // state tiles: wave w owns tiles w*NTS .. w*NTS+NTS-1 (row-major over
  // NRT x NCT); all of them share one row tile.
  static constexpr int NT = NRT * NCT;
  static constexpr int NTS = (NT + kNW - 1) / kNW;
  __device__ static bool owns(int w) { return w * NTS < NT; }
  __device__ static int srt(int w) { return (w * NTS) / NCT; }
  __device__ static int sct(int w) { return (w * NTS) % NCT; }
  // chunk-input prefetch: 16-byte pieces
  static constexpr int VEC = 16 / (int)sizeof(E);
  static constexpr int PQ = 64 * K / VEC;   // pieces of a 64 x K tile
  static constexpr int PV = 64 * V / VEC;   // pieces of a 64 x V tile
  static constexpr int PT = 64 * 64 / VEC;  // pieces of a 64 x 64 tile
  static constexpr int NQ = (PQ + kThreads - 1) / kThreads;
  static constexpr int NV = (PV + kThreads - 1) / kThreads;
  static constexpr int NTM = (PT + kThreads - 1) / kThreads;
};

template <typename E, int K, int V>
struct Pref {
  using G = Geo<E, K, V>;
  uint4 q[G::NQ], k[G::NQ], v[G::NV], t[G::NTM];
  float g;
  E b;  // raw beta: converted when committed, so its load is not waited on early
  int rows;
  __device__ float beta() const { return to_f32(b); }
};

// Load one chunk's q, k, (v-like tile), T, g, beta into registers.
// vsrc is v (forward) or do (backward); it is skipped when null-like (want_v).
// Every load goes through a buffer whose range ends with the chunk's valid
// rows (or the tile), so the guards need no branch and nothing waits for a
// load before its data is committed; the buffer bases are wave-uniform and
// lanes add 32-bit byte offsets.
template <typename E, int K, int V, bool WANT_V>
__device__ __forceinline__ void pref_load(Pref<E, K, V> &pf, const Problem &p, const E *qp,
                                          const E *kp, const E *vsrc, const E *tmat,
                                          const float *g, const E *beta, int64_t tok0,
                                          int rows, int h, int64_t cgid,
                                          int tid = threadIdx.x) {
  using G = Geo<E, K, V>;
  // the chunk's coordinates are the same for every lane: as scalars, the
  // buffer descriptors built on them are scalar (no per-load descriptor loop)
  tok0 = (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)tok0 >> 32)) << 32) |
                   __builtin_amdgcn_readfirstlane((uint32_t)tok0));
  cgid = (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)cgid >> 32)) << 32) |
                   __builtin_amdgcn_readfirstlane((uint32_t)cgid));
  rows = __builtin_amdgcn_readfirstlane(rows);
  h = __builtin_amdgcn_readfirstlane(h);
  const int hq = h / (p.Hv / p.Hq);
  constexpr int PK = K / G::VEC, PVr = V / G::VEC;
  pf.rows = rows;
  const uint32_t qrs = (uint32_t)(p.Hq * K * sizeof(E));  // bytes between token rows
  const auto rq = raw_buffer(qp + (tok0 * p.Hq + hq) * K, (uint32_t)rows * qrs);
  const auto rk = raw_buffer(kp + (tok0 * p.Hq + hq) * K, (uint32_t)rows * qrs);
#pragma unroll
  for (int m = 0; m < G::NQ; ++m) {
    // pieces past the tile (idx >= PQ) fall past the range: rows >= 64
    const int idx = tid + kThreads * m;
    const uint32_t off = (uint32_t)(idx / PK) * qrs + (uint32_t)(idx % PK) * 16u;
    pf.q[m] = buf_load16(rq, off);
    pf.k[m] = buf_load16(rk, off);
  }
  if (WANT_V) {
    const uint32_t vrs = (uint32_t)(p.Hv * V * sizeof(E));
    const auto rv = raw_buffer(vsrc + (tok0 * p.Hv + h) * V, (uint32_t)rows * vrs);
#pragma unroll
    for (int m = 0; m < G::NV; ++m) {
      const int idx = tid + kThreads * m;
      pf.v[m] = buf_load16(rv, (uint32_t)(idx / PVr) * vrs + (uint32_t)(idx % PVr) * 16u);
    }
  }
  const auto rt = raw_buffer(tmat + (cgid * p.Hv + h) * 64 * 64, (uint32_t)G::PT * 16u);
#pragma unroll
  for (int m = 0; m < G::NTM; ++m) pf.t[m] = buf_load16(rt, (uint32_t)(tid + kThreads * m) * 16u);
  // g and beta of row tid (threads 0..63; past the rows and above 63: 0)
  const int64_t gi0 = tok0 * p.Hv + h;
  const uint32_t gs = (uint32_t)p.Hv;
  const uint32_t gn = (uint32_t)rows * gs;
  pf.g = buf_load_elem<float>(raw_buffer(g + gi0, gn * 4u), (uint32_t)tid * gs * 4u);
  pf.b = buf_load_elem<E>(raw_buffer(beta + gi0, gn * (uint32_t)sizeof(E)),
                          (uint32_t)tid * gs * (uint32_t)sizeof(E));
}

// Per-chunk gate quantities in LDS.
struct GateLds {
  float *gam;  // inclusive cumsum gamma_r, times log2(e) (decays are exp2 of differences)
  float *eg;   // exp(gamma_r)
  float *dec;  // exp(gamma_L - gamma_r)
  float *bet;  // beta_r
};

// Wave 0 turns the prefetched g, beta into the gate quantities.
__device__ __forceinline__ void gate_commit(float g, float b, const GateLds &G,
                                            int tid = threadIdx.x) {
  if (tid < 64) {
    const float gam = wave_incl_scan(g) * kLog2e;
    const float gL = lane63(gam);
    G.gam[tid] = gam;
    G.eg[tid] = __builtin_amdgcn_exp2f(gam);
    G.dec[tid] = __builtin_amdgcn_exp2f(gL - gam);
    G.bet[tid] = b;
  }
}

// ----- fp32 K x V state as register tiles (owned tiles of Geo) -----
template <int N>
using Tiles = TileArr<N>;

template <typename E, int K, int V>
__device__ __forceinline__ void tiles_zero(Tiles<Geo<E, K, V>::NTS> &s) {
#pragma unroll
  for (int m = 0; m < Geo<E, K, V>::NTS; ++m) s[m] = zero4();
}

// Read a global fp32 [K][V] matrix (or zeros if src is null) into the tiles.
template <typename E, int K, int V>
__device__ __forceinline__ void tiles_load(Tiles<Geo<E, K, V>::NTS> &s, const float *src,
    int tid = threadIdx.x) {
  using G = Geo<E, K, V>;
  const int w = wave_of(tid), lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int m = 0; m < G::NTS; ++m) {
    f32x4 x = zero4();
    if (src && G::owns(w)) {
      const int rt = G::srt(w), ct = G::sct(w) + m;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = src[(16 * rt + 4 * lg + i) * V + 16 * ct + lr];
    }
    s[m] = x;
  }
}

// dst = tiles (+ add[] if given) (+ dst if accumulate).
template <typename E, int K, int V>
__device__ __forceinline__ void tiles_store(const Tiles<Geo<E, K, V>::NTS> &s, float *dst,
                                            const float *add, bool accumulate,
    int tid = threadIdx.x) {
  using G = Geo<E, K, V>;
  const int w = wave_of(tid), lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  if (!G::owns(w)) return;
  const int rt = G::srt(w);
#pragma unroll
  for (int m = 0; m < G::NTS; ++m) {
    const int ct = G::sct(w) + m;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // 32-bit element offset from the (wave-uniform) matrix base
      const uint32_t off = (uint32_t)((16 * rt + 4 * lg + i) * V + 16 * ct + lr);
      float x = s[m][i];
      if (add) x += add[off];
      if (accumulate) x += dst[off];
      dst[off] = x;
    }
  }
}

// The per-chunk states of the backward (element type) are stored
// transposed, dstT[v][k] = S[k][v]: a lane's 4 accumulator rows are then 4
// consecutive elements, and the LDS mirror (also transposed) leaves as whole
// rows.
//
// dstT += tiles (fp32 sum, rounded once to E), 4 elements a lane, in two
// halves so that the read's latency hides behind other work: the old values
// are read first (tiles_old_t), added and written back later
// (tiles_accumulate_t), before the tiles change.
template <typename E>
struct E4 {
  using type = bf16x4;
};
template <>
struct E4<float> {
  using type = f32x4;
};
template <typename E, int K, int V>
struct TilesOld {
  typename E4<E>::type x[Geo<E, K, V>::NTS];
};

template <typename E, int K, int V>
__device__ __forceinline__ void tiles_old_t(TilesOld<E, K, V> &o, const E *dstT,
                                            int tid = threadIdx.x) {
  using G = Geo<E, K, V>;
  const int w = wave_of(tid), lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  // (no branch where every wave owns tiles: loads under a branch are waited
  // for where it joins)
  if (G::NT < kNW * G::NTS && !G::owns(w)) return;
  const int rt = G::srt(w);
#pragma unroll
  for (int m = 0; m < G::NTS; ++m) {
    const int ct = G::sct(w) + m;
    o.x[m] = *reinterpret_cast<const typename E4<E>::type *>(
        dstT + (uint32_t)((16 * ct + lr) * K + 16 * rt + 4 * lg));
  }
}

template <typename E, int K, int V>
__device__ __forceinline__ void tiles_accumulate_t(const Tiles<Geo<E, K, V>::NTS> &s,
                                                   const TilesOld<E, K, V> &o, E *dstT,
                                                   int tid = threadIdx.x) {
  using G = Geo<E, K, V>;
  const int w = wave_of(tid), lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  if (!G::owns(w)) return;
  const int rt = G::srt(w);
#pragma unroll
  for (int m = 0; m < G::NTS; ++m) {
    const int ct = G::sct(w) + m;
    E *d = dstT + (uint32_t)((16 * ct + lr) * K + 16 * rt + 4 * lg);
    st4(d, s[m][0] + to_f32(o.x[m][0]), s[m][1] + to_f32(o.x[m][1]),
        s[m][2] + to_f32(o.x[m][2]), s[m][3] + to_f32(o.x[m][3]));
  }
}

// dstT = the transposed LDS mirror srcT ([V][G::LDK]), 16 bytes a lane.  The
// mirror holds the tiles rounded to E, so this equals storing the tiles.
template <typename E, int K, int V>
__device__ __forceinline__ void mirror_store_t(const E *srcT, E *dstT, int tid = threadIdx.x) {
  using G = Geo<E, K, V>;
  constexpr int PR = K / G::VEC;  // 16-byte pieces per row
  constexpr int NP = (V * PR + kThreads - 1) / kThreads;
#pragma unroll
  for (int m = 0; m < NP; ++m) {
    const int idx = tid + kThreads * m;
    if (idx < V * PR) {
      const int r = idx / PR, cv = idx % PR;
      *reinterpret_cast<uint4 *>(dstT + r * K + cv * G::VEC) =
          *reinterpret_cast<const uint4 *>(srcT + r * G::LDK + cv * G::VEC);
    }
  }
}

// ---- per-chunk states in the "lane layout" (state cache, backward's states)
// The forward's register-resident pass keeps S in 32x32 MFMA accumulators
// (gdn_fwd_slice.hip); the state cache stores S as those registers hold it,
// so that pass writes it as whole 1 KB pieces: element (k, v) of S sits at
//   ((v / 32 * (K / 16) + k / 16) * 64 + (v % 32) + 32 h) * 8 + e,
//   h = (k >> 2) & 1,  e = (k & 3) + 4 ((k >> 3) & 1).
// Four consecutive k from a multiple of 4 are four consecutive elements, and
// the 32 columns v0 .. v0 + 31 (v0 % 32 == 0) fill the contiguous range
// [v0 K, (v0 + 32) K), like 32 rows of S^T.
template <int K>
__device__ __forceinline__ uint32_t lane_off(int k, int v) {
  const int h = (k >> 2) & 1, e = (k & 3) + 4 * ((k >> 3) & 1);
  return (uint32_t)((((v >> 5) * (K / 16) + (k >> 4)) * 64 + (v & 31) + 32 * h) * 8 + e);
}
// The inverse for one 8-element unit u of the layout: its column v and the
// first k of its two 4-element groups (elements 0..3 and 4..7).
template <int K>
__device__ __forceinline__ void lane_unit(int u, int &v, int &k_lo, int &k_hi) {
  const int lane = u & 63, s = (u >> 6) % (K / 16), j = (u >> 6) / (K / 16);
  v = 32 * j + (lane & 31);
  k_lo = 16 * s + 4 * (lane >> 5);
  k_hi = k_lo + 8;
}

template <typename E, int K, int V>
__device__ __forceinline__ void tiles_old_l(TilesOld<E, K, V> &o, const E *dst,
                                            int tid = threadIdx.x) {
  using G = Geo<E, K, V>;
  const int w = wave_of(tid), lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  // (no branch where every wave owns tiles: loads under a branch are waited
  // for where it joins)
  if (G::NT < kNW * G::NTS && !G::owns(w)) return;
  const int rt = G::srt(w);
#pragma unroll
  for (int m = 0; m < G::NTS; ++m) {
    const int ct = G::sct(w) + m;
    o.x[m] = *reinterpret_cast<const typename E4<E>::type *>(
        dst + lane_off<K>(16 * rt + 4 * lg, 16 * ct + lr));
  }
}

template <typename E, int K, int V>
__device__ __forceinline__ void tiles_accumulate_l(const Tiles<Geo<E, K, V>::NTS> &s,
                                                   const TilesOld<E, K, V> &o, E *dst,
                                                   int tid = threadIdx.x) {
  using G = Geo<E, K, V>;
  const int w = wave_of(tid), lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  if (!G::owns(w)) return;
  const int rt = G::srt(w);
#pragma unroll
  for (int m = 0; m < G::NTS; ++m) {
    const int ct = G::sct(w) + m;
    E *d = dst + lane_off<K>(16 * rt + 4 * lg, 16 * ct + lr);
    st4(d, s[m][0] + to_f32(o.x[m][0]), s[m][1] + to_f32(o.x[m][1]),
        s[m][2] + to_f32(o.x[m][2]), s[m][3] + to_f32(o.x[m][3]));
  }
}

// dst (lane layout) = the transposed LDS mirror srcT ([V][G::LDK]); the
// stores are whole 16-byte pieces in address order.
template <typename E, int K, int V>
__device__ __forceinline__ void mirror_store_l(const E *srcT, E *dst, int tid = threadIdx.x) {
  using G = Geo<E, K, V>;
  constexpr int NPC = K * V / G::VEC;  // 16-byte pieces
  constexpr int NP = (NPC + kThreads - 1) / kThreads;
#pragma unroll
  for (int m = 0; m < NP; ++m) {
    const int idx = tid + kThreads * m;
    if (idx < NPC) {
      int v, k_lo, k_hi;
      if (sizeof(E) == 2) {
        lane_unit<K>(idx, v, k_lo, k_hi);
        const uint2 a = *reinterpret_cast<const uint2 *>(srcT + v * G::LDK + k_lo);
        const uint2 b = *reinterpret_cast<const uint2 *>(srcT + v * G::LDK + k_hi);
        *reinterpret_cast<uint4 *>(dst + idx * G::VEC) = make_uint4(a.x, a.y, b.x, b.y);
      } else {
        lane_unit<K>(idx >> 1, v, k_lo, k_hi);
        *reinterpret_cast<uint4 *>(dst + idx * G::VEC) =
            *reinterpret_cast<const uint4 *>(srcT + v * G::LDK + ((idx & 1) ? k_hi : k_lo));
      }
    }
  }
}

// dst[0 .. K V) = src[0 .. K V), or zeros when src is null (fp32 states;
// kThreads threads).  Every load is in flight before the first store: 16
// bytes a lane when both pointers allow it, else 4.
template <int K, int V>
__device__ __forceinline__ void copy_state(float *dst, const float *src) {
  constexpr int N4 = K * V / 4;
  constexpr int NP = (N4 + kThreads - 1) / kThreads;
  const int tid = threadIdx.x;
  if (((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 15) == 0) {
    f32x4 x[NP];
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      const int i = tid + kThreads * m;
      x[m] = (src && i < N4) ? reinterpret_cast<const f32x4 *>(src)[i] : zero4();
    }
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      const int i = tid + kThreads * m;
      if (i < N4) reinterpret_cast<f32x4 *>(dst)[i] = x[m];
    }
  } else {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      float x[NP];
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        const int i = tid + kThreads * (m + NP * b);
        x[m] = (src && i < K * V) ? src[i] : 0.f;
      }
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        const int i = tid + kThreads * (m + NP * b);
        if (i < K * V) dst[i] = x[m];
      }
    }
  }
}

// Transposed working copy (element type) in LDS: dstT[v][i] = S[i][v].
template <typename E, int K, int V>
__device__ __forceinline__ void tiles_to_lds_t(const Tiles<Geo<E, K, V>::NTS> &s, E *dstT,
    int tid = threadIdx.x) {
  using G = Geo<E, K, V>;
  const int w = wave_of(tid), lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  if (!G::owns(w)) return;
  const int rt = G::srt(w);
#pragma unroll
  for (int m = 0; m < G::NTS; ++m) {
    const int ct = G::sct(w) + m;
    st4(dstT + (16 * ct + lr) * G::LDK + 16 * rt + 4 * lg, s[m][0], s[m][1], s[m][2],
        s[m][3]);
  }
}

// True when some element of the (correction) state has magnitude at least
// thr (by default 2^-126, the smallest normal fp32).  The fix-up passes stop
// once it fails for fix_threshold(): what they drop is a correction below
// 2^-30 of the one they started with (or zero / denormal), whose further
// contributions to outputs and states lie below the fp32 resolution of the
// contributions already made.
template <typename E, int K, int V>
__device__ __forceinline__ bool tiles_significant(const Tiles<Geo<E, K, V>::NTS> &s,
                                                  float thr = 0x1p-126f) {
  bool nz = false;
#pragma unroll
  for (int m = 0; m < Geo<E, K, V>::NTS; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) nz |= (__builtin_fabsf(s[m][i]) >= thr);
  return nz;
}

// Exit threshold of a fix-up pass whose correction starts as s: 2^-30 of its
// largest magnitude over the workgroup, at least 2^-126 (uses 8 ints of LDS;
// every thread of the workgroup calls it).
template <typename E, int K, int V>
__device__ __forceinline__ float fix_threshold(const Tiles<Geo<E, K, V>::NTS> &s, int *sflag) {
  float x = 0.f;
#pragma unroll
  for (int m = 0; m < Geo<E, K, V>::NTS; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) x = __builtin_fmaxf(x, __builtin_fabsf(s[m][i]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = __builtin_fmaxf(x, __shfl_xor(x, o, 64));
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) sflag[w] = __builtin_bit_cast(int, x);
  __syncthreads();
  int r = 0;  // non-negative floats order as their bit patterns
#pragma unroll
  for (int i = 0; i < kNW; ++i) r = max(r, sflag[i]);
  __syncthreads();
  return __builtin_fmaxf(0x1p-126f, 0x1p-30f * __builtin_bit_cast(float, r));
}

// Workgroup-wide OR of a per-thread flag (uses 8 ints of LDS).
__device__ __forceinline__ bool block_any(bool x, int *sflag) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool wx = __any(x);
  if (lane == 0) sflag[w] = wx ? 1 : 0;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int i = 0; i < kNW; ++i) r |= sflag[i];
  __syncthreads();
  return r != 0;
}

}  // namespace gdn
