// Pieces shared by the register-resident segment passes (forward pass 1 in
// gdn_fwd_slice.hip, the backward's reverse pass 1 in gdn_rev_slice.hip), for
// bf16 problems with K = V = 128.
//
// Both passes carry a K x V state (S forward, its gradient D backward) whose
// V columns are independent.  A workgroup owns one (segment, v-head) item:
// chain waves 0..3 each hold columns [32 j, 32 j + 32) of the state in 32x32
// MFMA accumulator tiles for the whole segment; helper waves 4..7 stage the
// next chunk's inputs into the other of two LDS buffer sets.  One workgroup
// barrier per chunk.
//
// A 32x32x16 MFMA accumulator holds, in lane l, column l & 31 and rows
// 8 (i >> 2) + 4 (l >> 5) + (i & 3) of its tile (register i).  Read as
// operand slots, registers 8 s .. 8 s + 7 of a tile are rows 16 s + [0..15]
// in the order rho(h, e) = 8 (e >> 2) + 4 h + (e & 3) (h = l >> 5): so an
// accumulator is, without any data movement, the B operand of A X or the A
// operand of X^T B with the contraction over its rows, provided the other
// operand supplies its k-slots in the same rho order.  The LDS copies of the
// MFMA operands therefore store each row with the 4-element groups 1 and 2
// of every 16-element block swapped ("pi" layout): one 16-byte read at
// position 16 s + 8 h then yields exactly the rho-ordered slots, and the
// transpose reads of a pi-layout matrix point each source lane at the
// position of its column group.
#pragma once

#include "gdn_seg.hpp"

namespace gdn {
namespace slice {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int K = 128, V = 128;
constexpr int kWaves = 8, kThreadsS = 64 * kWaves;
// LDS row pitches (elements): rows of 128 are 288 bytes, rows of 64 are 160
// bytes (16-byte reads of 32 consecutive rows are then free of bank
// conflicts)
constexpr int PITCH = K + 16;
constexpr int PITCH_C = 64 + 16;

__device__ __forceinline__ f32x16 mma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}
// 4-element group q of a 16-element block -> its position group in the pi layout
__device__ __forceinline__ constexpr int pi4(int q) { return (q == 1 || q == 2) ? 3 - q : q; }
// pi-layout position of column c (c % 4 == 0) of a row
__device__ __forceinline__ constexpr int pi_pos(int c) { return (c & ~15) + 4 * pi4((c >> 2) & 3); }

__device__ __forceinline__ bf16x8 lds16(const bf16 *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
__device__ __forceinline__ bf16x4 tr4(const bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p);
}

// Operand slots 8 s .. 8 s + 7 of accumulator tile x, rounded to bf16.
__device__ __forceinline__ bf16x8 slots(const f32x16 &x, int s) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)x[8 * s + e];
  return r;
}

// A operand slots of X^T for a pi-layout row-major X in LDS (rows = the
// contraction index): lane l gets X[16 s + rho(h, e)][32 m + (l & 31)], from
// two transpose reads (16-lane group: 4 rows, 16 columns; source lane 4 e + q
// points at row e of the block and at the position of column group q).
struct TrA {
  const bf16 *base;
  __device__ __forceinline__ TrA(const bf16 *x, int pitch, int lane) {
    const int G = lane >> 4, sgm = lane & 15;
    base = x + (4 * (lane >> 5) + (sgm >> 2)) * pitch + 16 * (G & 1) + 4 * pi4(sgm & 3);
  }
  __device__ __forceinline__ bf16x8 at(int s, int m, int pitch) const {
    const bf16 *b = base + 16 * s * pitch + 32 * m;
    const bf16x4 lo = tr4(b), hi = tr4(b + 8 * pitch);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
};

// Values of a natural-layout row-major X (rows r, 128 columns) at this
// lane's accumulator positions: rows 32 t + 8 b + 4 h + [0..3] of column
// 32 j + (l & 31), for b = 0..3 (one transpose read each).
__device__ __forceinline__ void acc_rows(bf16x4 (&x)[4], const bf16 *X, int t, int j, int lane) {
  const int G = lane >> 4, sgm = lane & 15, h = lane >> 5;
  const int col = 32 * j + 16 * (G & 1) + 4 * (sgm & 3);
#pragma unroll
  for (int b = 0; b < 4; ++b) x[b] = tr4(X + (32 * t + 8 * b + 4 * h + (sgm >> 2)) * PITCH + col);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// A 16-byte piece holding columns 8 pc .. 8 pc + 7 of a row, written into a
// pi-layout row: its two 4-column groups go to their swapped positions.
__device__ __forceinline__ void put_pi(bf16 *row, int pc, const uint4 &x) {
  const int blk = (8 * pc) & ~15, q0 = 2 * (pc & 1);
  *reinterpret_cast<uint2 *>(row + blk + 4 * pi4(q0)) = make_uint2(x.x, x.y);
  *reinterpret_cast<uint2 *>(row + blk + 4 * pi4(q0 + 1)) = make_uint2(x.z, x.w);
}

struct Item {
  SegLoc sl;
  int h, hq;
};

struct ChainCtx {
  int j, lane, h, r32;
};

// State tiles <-> fp32 [K][V] matrix (row k, column v): lane holds column
// 32 j + r32 and rows 32 m + 8 (i >> 2) + 4 h + (i & 3).
__device__ __forceinline__ void state_load(f32x16 (&S)[4], const float *src, const ChainCtx &x) {
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = 32 * m + 8 * (i >> 2) + 4 * x.h + (i & 3);
      S[m][i] = src ? src[k * V + 32 * x.j + x.r32] : 0.f;
    }
}
__device__ __forceinline__ void state_store(const f32x16 (&S)[4], float *dst, const ChainCtx &x) {
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = 32 * m + 8 * (i >> 2) + 4 * x.h + (i & 3);
      dst[k * V + 32 * x.j + x.r32] = S[m][i];
    }
}

}  // namespace slice
}  // namespace gdn
