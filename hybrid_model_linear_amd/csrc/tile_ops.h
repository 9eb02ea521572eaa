// MFMA operand and LDS tile helpers shared by the chunked kernels (gfx950, wave64):
// operand conversions between fp32 accumulators and 16-bit MFMA operands, the
// swizzled and padded row-major LDS tile layouts with their 16-byte and transpose
// reads, the DPP wave scan, and the LDS-only workgroup barrier.
//
// MFMA layouts used throughout (lane l, g16 = l / 16, j16 = l % 16):
//   16x16x32: A operand lane l supplies A[j16][8 g16 .. 8 g16 + 7], B operand
//             B[8 g16 .. 8 g16 + 7][j16]; accumulator element r of lane l is
//             D[4 g16 + r][j16].
//   32x32x16: A lane l supplies A[l % 32][8 (l / 32) .. + 7], B likewise by column;
//             accumulator element r of lane l is D[acc_row(r, l / 32)][l % 32].
#pragma once
#include "gdn_common.h"

namespace gdn {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
// Buffer resource word 3 for untyped dword accesses on gfx9 (32-bit data format)
constexpr int kBufWord3 = 0x00020000;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma1632(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x4 mfma1632h(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16h(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
// fp32 -> fp16 bits (round to nearest even)
__device__ __forceinline__ u16 f32_to_f16(float f) { return __builtin_bit_cast(u16, (_Float16)f); }
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x8 join(uint2 lo, uint2 hi) {
  return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}
// LDS transpose read of 4 bf16 at p (8-byte aligned).
__device__ __forceinline__ uint2 tr_read(const u16* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p)));
}

// Row-major bf16 tiles of 64 rows x D columns are padded by one 16-byte segment per
// row (D + 8 elements) so that MFMA operand reads of consecutive rows spread over
// the LDS banks while every address stays an affine function of the lane.
template <int D>
__device__ __forceinline__ int pidx(int r, int c) { return r * (D + 8) + c; }
// Q and K tiles: rows of D bf16 in natural column order without padding (the
// state's accumulator rows are ordered to match, see Sacc); the 16-byte chunk j of
// row r is stored at chunk position j ^ qswz(r).  This keeps the state waves' operand reads
// (16 rows x 4 chunks per instruction) and their transpose reads free of LDS bank
// conflicts (the producers' 32-row reads see two-way conflicts).
__device__ __forceinline__ int qswz(int r) { return (((r & 3) << 2) ^ r) & 15; }
template <int D>
__device__ __forceinline__ int qidx(int r, int c) { return r * D + ((((c >> 3) ^ qswz(r)) << 3) | (c & 7)); }
// 8 consecutive bf16 (16 B), c % 8 == 0.
template <int D>
__device__ __forceinline__ bf16x8 ld8(const u16* t, int r, int c) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(t + pidx<D>(r, c)));
}
template <int D>
__device__ __forceinline__ bf16x8 ldq8(const u16* t, int r, int c) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(t + qidx<D>(r, c)));
}
// 8 consecutive bf16 at an 8-byte aligned address (rows of the C x C tiles)
__device__ __forceinline__ bf16x8 ld8u(const u16* p) {
  return join(*reinterpret_cast<const uint2*>(p), *reinterpret_cast<const uint2*>(p + 4));
}
// Transpose read: lane j of a 16-lane group receives elements (rows[e], c0 + j),
// e = 0..3, when lane i of the group passes (rows[i / 4], c0 + 4 (i % 4)).
template <int D>
__device__ __forceinline__ uint2 ldtr(const u16* t, int r, int c) {
  return tr_read(t + pidx<D>(r, c));
}
template <int D>
__device__ __forceinline__ uint2 ldqtr(const u16* t, int r, int c) {
  return tr_read(t + qidx<D>(r, c));
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
// two fp32 -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
// two fp32 -> packed fp16 pair (one v_cvt_pk_f16_f32, round to nearest even)
__device__ __forceinline__ uint32_t cvt2h(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}
__device__ __forceinline__ bf16x8 acc_to_op(const f32x16& a, int half) {
  const int o = 8 * half;
  return as_bf16x8(make_uint4(cvt2(a[o], a[o + 1]), cvt2(a[o + 2], a[o + 3]), cvt2(a[o + 4], a[o + 5]),
                              cvt2(a[o + 6], a[o + 7])));
}
// Two 16x16 accumulator tiles (rows 4 g + r of tile t0 and of tile t1) as one B
// operand of a 16x16x32 MFMA whose 32 k slots are (g, e): e < 4 -> tile t0 row
// 4 g + e, e >= 4 -> tile t1 row 4 g + e - 4.
__device__ __forceinline__ bf16x8 pair_to_op(const f32x4& a, const f32x4& b) {
  return as_bf16x8(make_uint4(cvt2(a[0], a[1]), cvt2(a[2], a[3]), cvt2(b[0], b[1]), cvt2(b[2], b[3])));
}
__device__ __forceinline__ f16x8 acc_to_op_h(const f32x16& a, int half) {
  const int o = 8 * half;
  return __builtin_bit_cast(f16x8, make_uint4(cvt2h(a[o], a[o + 1]), cvt2h(a[o + 2], a[o + 3]),
                                              cvt2h(a[o + 4], a[o + 5]), cvt2h(a[o + 6], a[o + 7])));
}
__device__ __forceinline__ f16x8 pair_to_op_h(const f32x4& a, const f32x4& b) {
  return __builtin_bit_cast(f16x8, make_uint4(cvt2h(a[0], a[1]), cvt2h(a[2], a[3]), cvt2h(b[0], b[1]), cvt2h(b[2], b[3])));
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// x minus the low / high bf16 of the packed pair w (exact: a float minus its own
// bf16 rounding is representable)
__device__ __forceinline__ float sub_bf_lo(uint32_t w, float x) { return x - bf_lo(w); }
__device__ __forceinline__ float sub_bf_hi(uint32_t w, float x) { return x - bf_hi(w); }
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi), for the pair layout above
__device__ __forceinline__ void pair_split(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = cvt2(x[2 * e], x[2 * e + 1]);
    l[e] = cvt2(sub_bf_lo(h[e], x[2 * e]), sub_bf_hi(h[e], x[2 * e + 1]));
  }
  hi = as_bf16x8(make_uint4(h[0], h[1], h[2], h[3]));
  lo = as_bf16x8(make_uint4(l[0], l[1], l[2], l[3]));
}
// 8 fp16 values as hi + lo bf16 operands (exact: fp16's 11-bit significand splits into
// a bf16 and a bf16 remainder)
__device__ __forceinline__ void h8_split(const uint4 w, bf16x8& hi, bf16x8& lo) {
  const f16x8 h = __builtin_bit_cast(f16x8, w);
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = (float)h[2 * e], b = (float)h[2 * e + 1];
    hw[e] = cvt2(a, b);
    lw[e] = cvt2(sub_bf_lo(hw[e], a), sub_bf_hi(hw[e], b));
  }
  hi = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
  lo = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
}
// Row (token / d_k index) of accumulator element r held by lane half hh.
__device__ __forceinline__ int acc_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }
__device__ __forceinline__ float4 ld_f4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float f4get(const float4& v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}
// a + lo(w)^2 + hi(w)^2 for a packed bf16 pair w (v_dot2_f32_bf16; the squares of
// bf16 values are exact in fp32)
__device__ __forceinline__ float dot2sq(uint32_t w, float a) {
  const bf16x2 x = __builtin_bit_cast(bf16x2, w);
  return __builtin_amdgcn_fdot2_f32_bf16(x, x, a, false);
}
// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and row
// broadcasts (no LDS round trip): four shift-and-add steps within each row of 16
// lanes, then the last lane of row 0 (2) is added to row 1 (3), and the last lane of
// row 1 to rows 2 and 3.
template <int CTRL, int ROW_MASK, bool BOUND>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, BOUND));
}
__device__ __forceinline__ float wave_inclusive_scan(float v) {
  v += dpp_mov<0x111, 0xf, true>(v);    // row_shr:1 (lanes shifted in from outside the row read 0)
  v += dpp_mov<0x112, 0xf, true>(v);    // row_shr:2
  v += dpp_mov<0x114, 0xf, true>(v);    // row_shr:4
  v += dpp_mov<0x118, 0xf, true>(v);    // row_shr:8
  v += dpp_mov<0x142, 0xa, false>(v);   // row_bcast:15 into rows 1 and 3 (others add 0)
  v += dpp_mov<0x143, 0xc, false>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}
// Sum over each row of 16 lanes, in every lane of the row (DPP: swaps within pairs
// and quads, then the half-row and row mirrors).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1, 0xf, true>(v);    // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4E, 0xf, true>(v);    // quad_perm [2, 3, 0, 1]
  v += dpp_mov<0x141, 0xf, true>(v);   // row_half_mirror (lane i <- 7 - i within 8)
  v += dpp_mov<0x140, 0xf, true>(v);   // row_mirror (lane i <- 15 - i)
  return v;
}
__device__ __forceinline__ float sumsq8(const bf16x8& v, float a) {
  const uint4 u = __builtin_bit_cast(uint4, v);
  return dot2sq(u.w, dot2sq(u.z, dot2sq(u.y, dot2sq(u.x, a))));
}

// Workgroup barrier for LDS traffic only.  __syncthreads() is a workgroup-scope
// fence and would also wait for the staged global loads in flight; here the wave's
// own LDS accesses are drained (lgkmcnt(0)) and the compiler is kept from moving
// memory accesses across the barrier.
__device__ __forceinline__ void lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// Order this wave's earlier LDS writes before its later LDS reads (the LDS executes
// one wave's accesses in order; this keeps the compiler from reordering them).
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

template <int I> struct Par { static constexpr int value = I; };

}  // namespace gdn
