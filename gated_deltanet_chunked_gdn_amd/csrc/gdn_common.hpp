// Device helpers shared by the GDN kernels (gfx950 / CDNA4).
//
// Matrix products use the 16x16 MFMA family with a 64-lane wavefront:
//   bf16: v_mfma_f32_16x16x32_bf16  (8 bf16 of A and of B per lane)
//   fp32: v_mfma_f32_16x16x4_f32    (1 fp32 of A and of B per lane)
// Operand convention used everywhere here: for C = X * Y (M x N, contraction
// index k), X is stored in LDS as X[m][k] and Y as Yt[n][k], both contiguous
// along k.  Lane l supplies X[m0 + (l & 15)][k0 + EPL*(l >> 4) + e] and
// Yt[n0 + (l & 15)][k0 + EPL*(l >> 4) + e] for e < EPL; since A and B use the
// same (lane group, slot) -> k assignment, the instruction's internal k
// order does not matter.  The accumulator element i of lane l is
// C[m0 + 4*(l >> 4) + i][n0 + (l & 15)].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int N>
using TileArr = f32x4[N];  // N accumulator tiles held by one lane

constexpr int kChunk = 64;  // tokens per chunk
constexpr int kWave = 64;   // lanes per wavefront

template <typename E>
struct Mma;

template <>
struct Mma<bf16> {
  static constexpr int KS = 32;  // contraction length of one instruction
  static constexpr int EPL = 8;  // elements per lane per operand
  typedef bf16x8 frag;
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // 16-byte aligned LDS or global read of 8 contiguous elements
  __device__ static __forceinline__ frag ld(const bf16 *p) {
    return *reinterpret_cast<const frag *>(p);
  }
  // Operand fragment of a matrix stored k-major in LDS (X[k][c], contiguous
  // along c, row pitch `ld` elements, ld % 4 == 0): `tile` = &X[k0][c0] with
  // c0 % 4 == 0.  Lane l receives X[k0 + 8*(l >> 4) + e][c0 + (l & 15)] for
  // e < 8, from two LDS transpose reads (ds_read_b64_tr_b16).  That
  // instruction works on groups of 16 lanes: each lane reads 4 contiguous
  // 16-bit elements, and output lane j receives element j & 3 of the group's
  // lanes 4e + (j >> 2), e < 4.  Source lane s of a group therefore points at
  // row (s >> 2) and columns 4*(s & 3) .. +3 of a 4 x 16 block.
  // (l: lane index; callers in long loops pass a per-iteration copy)
  __device__ static __forceinline__ frag ld_tr(const bf16 *tile, int ld,
                                               int l = threadIdx.x & 63) {
    const bf16 *p = tile + (8 * (l >> 4) + ((l & 15) >> 2)) * ld + 4 * (l & 3);
    typedef __attribute__((address_space(3))) bf16x4 lds4;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4 *)p);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4 *)(p + 4 * ld));
    return frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  // The 4 values at this lane's accumulator positions, X[r0 + 4*(l >> 4) + e]
  // [c0 + (l & 15)] for e < 4, of a row-major tile (`tile` = &X[r0][c0],
  // c0 % 4 == 0, ld % 4 == 0), from one transpose read: source lane s of
  // each 16-lane group points at row 4*(l >> 4) + (s >> 2), columns
  // 4*(s & 3) .. +3.
  __device__ static __forceinline__ f32x4 ld_acc(const bf16 *tile, int ld,
                                                 int l = threadIdx.x & 63) {
    const bf16 *p = tile + (4 * (l >> 4) + ((l & 15) >> 2)) * ld + 4 * (l & 3);
    typedef __attribute__((address_space(3))) bf16x4 lds4;
    const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4 *)p);
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
  }
  // ld_tr with element e scaled by w[8*(l >> 4) + e] (a factor per row k)
  __device__ static __forceinline__ frag ld_tr_scaled(const bf16 *tile, int ld, const float *w,
                                                      int l = threadIdx.x & 63) {
    const frag x = ld_tr(tile, ld, l);
    const float *wl = w + 8 * (l >> 4);
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16)((float)x[e] * wl[e]);
    return f;
  }
  // a fragment with every element multiplied by s (rounded once)
  __device__ static __forceinline__ frag scaled(const frag &x, float s) {
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16)((float)x[e] * s);
    return f;
  }
  // X[m][k] + X[k][m]: 8 contiguous elements at p (as ld) plus the k-major
  // fragment of the same tile (rounded once)
  __device__ static __forceinline__ frag ld_sym_tr(const bf16 *p, const bf16 *tile, int pitch,
                                                   int l = threadIdx.x & 63) {
    const frag a = ld(p), b = ld_tr(tile, pitch, l);
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16)((float)a[e] + (float)b[e]);
    return f;
  }
};

template <>
struct Mma<float> {
  static constexpr int KS = 4;
  static constexpr int EPL = 1;
  typedef float frag;
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag ld(const float *p) { return *p; }
  __device__ static __forceinline__ f32x4 ld_acc(const float *tile, int ld,
                                                 int l = threadIdx.x & 63) {
    const float *p = tile + 4 * (l >> 4) * ld + (l & 15);
    return f32x4{p[0], p[ld], p[2 * ld], p[3 * ld]};
  }
  // k-major operand (see Mma<bf16>::ld_tr): lane l reads X[k0 + (l >> 4)][c0 + (l & 15)]
  __device__ static __forceinline__ frag ld_tr(const float *tile, int ld,
                                               int l = threadIdx.x & 63) {
    return tile[(l >> 4) * ld + (l & 15)];
  }
  __device__ static __forceinline__ frag ld_tr_scaled(const float *tile, int ld, const float *w,
                                                      int l = threadIdx.x & 63) {
    return ld_tr(tile, ld, l) * w[l >> 4];
  }
  __device__ static __forceinline__ frag scaled(frag x, float s) { return x * s; }
  __device__ static __forceinline__ frag ld_sym_tr(const float *p, const float *tile, int ld,
                                                   int l = threadIdx.x & 63) {
    return p[0] + ld_tr(tile, ld, l);
  }
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename E>
__device__ __forceinline__ E from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// c + the dot product of two 16-byte pieces of element type E (8 bf16 pairs
// through v_dot2 with fp32 accumulation, or 4 fp32 pairs).
template <typename E>
__device__ __forceinline__ float dot_piece(const uint4 &a, const uint4 &b, float c);
template <>
__device__ __forceinline__ float dot_piece<bf16>(const uint4 &a, const uint4 &b, float c) {
  typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 *x = reinterpret_cast<const bf16x2 *>(&a);
  const bf16x2 *y = reinterpret_cast<const bf16x2 *>(&b);
#pragma unroll
  for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_fdot2_f32_bf16(x[e], y[e], c, false);
  return c;
}
template <>
__device__ __forceinline__ float dot_piece<float>(const uint4 &a, const uint4 &b, float c) {
  const float *x = reinterpret_cast<const float *>(&a);
  const float *y = reinterpret_cast<const float *>(&b);
#pragma unroll
  for (int e = 0; e < 4; ++e) c += x[e] * y[e];
  return c;
}

// A 16-byte piece of element type E with every element times s (rounded once).
template <typename E>
__device__ __forceinline__ uint4 scale_piece(const uint4 &x, float s) {
  uint4 r;
  const E *a = reinterpret_cast<const E *>(&x);
  E *b = reinterpret_cast<E *>(&r);
#pragma unroll
  for (int e = 0; e < 16 / (int)sizeof(E); ++e) b[e] = from_f32<E>(to_f32(a[e]) * s);
  return r;
}

// Store 4 consecutive elements (8 bytes for bf16, 16 for fp32).
__device__ __forceinline__ void st4(bf16 *p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  v[2] = (bf16)c;
  v[3] = (bf16)d;
  *reinterpret_cast<bf16x4 *>(p) = v;
}
__device__ __forceinline__ void st4(float *p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4 *>(p) = f32x4{a, b, c, d};
}

// A raw buffer over [base, base + bytes): a store whose byte offset falls
// outside the range is dropped by the hardware, so row guards need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void buf_store16(const uint4 &x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{x.x, x.y, x.z, x.w}, r, (int)off, 0, 0);
}
// Loads through such a buffer: past the range they read 0 without touching
// memory, so guarded loads need no branch (a load under a branch makes the
// compiler wait for it where the branches join, right after its issue).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void *base, uint32_t bytes) {
  return raw_buffer(const_cast<void *>(base), bytes);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(x[0], x[1], x[2], x[3]);
}
template <typename E>
__device__ __forceinline__ E buf_load_elem(__amdgpu_buffer_rsrc_t r, uint32_t off);
template <>
__device__ __forceinline__ float buf_load_elem<float>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
template <>
__device__ __forceinline__ bf16 buf_load_elem<bf16>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16, __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// The thread index as an opaque value.  Long loops take a copy at the top of
// each iteration: address arithmetic derived from it is then recomputed inside
// the iteration instead of being hoisted out of the loop, where the many
// per-lane LDS addresses (regions past the 64 KB reach of the LDS immediate
// offset each need their own register) would otherwise be spilled.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}
// Wave index of a thread index, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_of(int tid) {
  return __builtin_amdgcn_readfirstlane(tid >> 6);
}

// x moved across lanes by a DPP control; lanes that the control gives no
// source lane, and lanes of rows (16 lanes each) outside ROWS, read 0.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xF, false));
}

// Inclusive prefix sum across the 64 lanes of a wavefront, in registers:
// shifts by 1, 2, 4 and 8 lanes inside each row of 16, then lane 15's row
// total broadcast into rows 1 and 3 and lane 31's total into rows 2 and 3.
__device__ __forceinline__ float wave_incl_scan(float x) {
  x += dpp_mov<0x111>(x);       // row_shr:1
  x += dpp_mov<0x112>(x);       // row_shr:2
  x += dpp_mov<0x114>(x);       // row_shr:4
  x += dpp_mov<0x118>(x);       // row_shr:8
  x += dpp_mov<0x142, 0xA>(x);  // row_bcast:15
  x += dpp_mov<0x143, 0xC>(x);  // row_bcast:31
  return x;
}

// Sum over the 16 lanes of each row (the lanes that share l >> 4): swap
// neighbours and pairs inside quads, then rotate the row by 4 and by 8.
__device__ __forceinline__ float sum16(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x124>(x);  // row_ror:4
  x += dpp_mov<0x128>(x);  // row_ror:8
  return x;
}

// Sum over aligned groups of LPR lanes (LPR = 2, 4, 8 or 16, inside a row):
// swap neighbours, then pairs inside quads, then quads (mirror inside each
// half row), then halves (row mirror).  The two partners of every exchange
// hold equal partial sums, so every lane of a group ends with the same value.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPR == 2 || LPR == 4 || LPR == 8 || LPR == 16, "lanes per group");
  x += dpp_mov<0xB1>(x);                   // quad_perm [1,0,3,2]
  if (LPR >= 4) x += dpp_mov<0x4E>(x);     // quad_perm [2,3,0,1]
  if (LPR >= 8) x += dpp_mov<0x141>(x);    // row_half_mirror
  if (LPR >= 16) x += dpp_mov<0x140>(x);   // row_mirror
  return x;
}

// The optional in-library L2 normalisation of q and k rows, applied where a
// kernel moves the rows it has loaded into LDS: x is one 16-byte piece of a
// row whose LPR pieces are held by LPR consecutive lanes.  Returns the piece
// times r = (sum of the row's squares + 1e-6)^(-1/2), rounded once; r is
// also returned (the same in every lane of the row).
template <typename E, int LPR>
__device__ __forceinline__ uint4 l2n_piece(const uint4 &x, float &r) {
  const float ss = group_sum<LPR>(dot_piece<E>(x, x, 0.f));
  r = 1.0f / __builtin_sqrtf(ss + 1e-6f);
  return scale_piece<E>(x, r);
}
template <typename E, int LPR>
__device__ __forceinline__ uint4 l2n_piece(const uint4 &x) {
  float r;
  return l2n_piece<E, LPR>(x, r);
}

// Lane 63's value of x, as a wave-uniform float.
__device__ __forceinline__ float lane63(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
// Sum over all 64 lanes (wave-uniform).
__device__ __forceinline__ float wave_sum(float x) { return lane63(wave_incl_scan(x)); }

// Locate sequence n with prefix[n] <= x < prefix[n+1] (prefix non-decreasing,
// prefix[0] = 0, x < prefix[N]).  Skips empty sequences.
__device__ __forceinline__ int find_seq(const int32_t *prefix, int N, int64_t x) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)prefix[mid] <= x)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Map a linear workgroup id so that ids dispatched to the same XCD (the
// hardware deals workgroups round-robin over the 8 XCDs) cover a contiguous
// range of work items; neighbouring work items (e.g. the v-heads that share a
// q/k head) then share one XCD's L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nblocks) {
  constexpr int kXcd = 8;
  if (nblocks % kXcd != 0) return bid;
  const int64_t per = nblocks / kXcd;
  return (bid % kXcd) * per + bid / kXcd;
}

}  // namespace gdn
