// Chunked delta-off kernel (Mamba2 SSD scan of flashinfer.mamba.ssd_combined_fwd),
// chunk 128, bf16 inputs, fp32 state, fp16 MFMA operands, gfx950.
//
// Per sequence and head h (group j = h / (H / G)), state S in R^{P x N} (P = headdim
// 64, N = dstate 128).  Within a chunk of C = 128 tokens, with dt'_i and
// log g_i = dt'_i A from the gate, G_i = sum_{m <= i} log g_m and the chunk's entry
// state S0 (Mamba2 SSD, the structured state-space dual form):
//
//   y_i  = e^{G_i} C_i S0^T + sum_{m <= i} e^{G_i - G_m} (C_i . B_m) dt'_m x_m
//   out_i = (y_i + D x_i) silu(z_i)
//   S1   = e^{G_C} S0 + sum_m e^{G_C - G_m} dt'_m x_m B_m^T
//
// Only the last line carries a dependency from chunk to chunk, and it is a single
// accumulate into the state; everything else of a chunk is independent of the scan.
// Because the decay is a scalar per (token, head), the state map of a run of chunks
// is S_out = e^{Lambda} S_in + R with R the run's state from zero: a sequence is cut
// into segments, a state-only pass computes every segment's (R, Lambda) in parallel,
// and the full pass of segment s starts from S_in(s), folded from the segments before
// it (S <- e^{Lambda_s'} S + R_s', s' < s).  The grid is (head, sequence x segment).
//
// Work split inside a workgroup (8 waves): wave w owns the state columns of P-tile
// pt = w % 4 (p = 16 pt .. 16 pt + 15) and the N-half nh = w / 4 (n = 64 nh .. + 63),
// four 16x16 accumulator tiles of S^T held in registers.  Per chunk:
//   * landing: the chunk's fp16 C and B rows (converted once per call into the
//     workspace, shared by every head) and U = diag(dt') X (fp16) into LDS; each wave
//     posts its half of S0 as fp16 operands for its partner (same pt, other nh);
//   * P = (C B^T) masked and decayed, fp16, by 32x32x16 MFMA tiles spread over the
//     waves; one wave prepares the next chunk's gate, decay cumsum and coefficients;
//   * Y^T = S0 C^T diag(e^G) for four 16-token tiles per wave, with S0's two N-halves
//     from registers and from the partner;
//   * S^T <- e^{G_C} S^T + B^T diag(e^{G_C - G}) U on the wave's own tiles;
//   * Y^T += U^T P^T, then D x and silu(z) and the output rows.
// The chunk's C, B and x rows are staged from memory through registers one chunk
// ahead.  Operand precision: C, B exact in fp16 (bf16 values in fp16's normal range);
// U, P, S0 and the state update's U carry fp16's 11-bit significand (2^-12 relative
// rounding, well below the bf16 output's); every product accumulates in fp32.  fp16's
// range bounds the magnitudes: |C.B|, |dt' x| and |S| must stay below 65504 (beyond
// it the results turn inf / NaN, visibly).
#include "gdn_common.h"
#include "gdn_launch.h"
#include "tile_ops.h"

namespace gdn {

namespace {

constexpr int CS = 128;             // chunk length
constexpr int NS = 128;             // dstate (d_k)
constexpr int PH = 64;              // headdim (d_v)
constexpr int kW = 8;               // waves per workgroup
constexpr int kThreads = kW * kWave;
constexpr int kPP = CS + 8;         // row length (fp16) of the P tile: 272 B rows
constexpr float kLog2e = 1.4426950408889634f;

typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ f16x8 join_h(uint2 lo, uint2 hi) {
  return as_f16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}
// Two packed fp16 pairs multiplied lane-wise (v_pk_mul_f16).
__device__ __forceinline__ uint32_t pk_mul_h(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2v, a) * __builtin_bit_cast(f16x2v, b));
}
__device__ __forceinline__ f16x8 scale_h(const f16x8& v, uint4 f) {
  const uint4 u = __builtin_bit_cast(uint4, v);
  return as_f16x8(make_uint4(pk_mul_h(u.x, f.x), pk_mul_h(u.y, f.y), pk_mul_h(u.z, f.z), pk_mul_h(u.w, f.w)));
}
// silu(y) = y / (1 + e^-y) (the reciprocal's argument is >= 1, or +inf for y < -88,
// where the result is -0: the limit)
__device__ __forceinline__ float silu_f(float y) {
  return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y));
}

// The C x C tile P keeps each 32-column block with its 4-column groups in the order
// 0, 4, 1, 5, 2, 6, 3, 7, so that the 8 k slots of a 16x16x32 operand (tokens 4g ..
// 4g+3 and 16+4g .. 16+4g+3 of a block, the order of the state's token k slots) are
// 16 contiguous bytes.  Logical column -> stored column:
__device__ __forceinline__ int pperm(int c) {
  const int q = (c >> 2) & 7;
  return (c & ~31) | ((2 * (q & 3) + (q >> 2)) << 2) | (c & 3);
}

// The ten 32x32 tiles of the lower block triangle of P, as (i-tile, m-tile): the
// diagonal tiles (one exp per element) on waves 0-3, the off-diagonal ones (factored
// decays) on waves 4-7, and the last two on waves 5 and 6 (so each SIMD -- waves w and
// w + 4 -- gets two or three tiles; wave 7 also prepares the next chunk's vectors).
__device__ __forceinline__ int ptile_i(int k) {
  constexpr int ti[10] = {0, 1, 2, 3, 1, 2, 3, 3, 2, 3};
  return ti[k];
}
__device__ __forceinline__ int ptile_m(int k) {
  constexpr int tm[10] = {0, 1, 2, 3, 0, 1, 2, 1, 0, 0};
  return tm[k];
}

// Per-chunk coefficient vectors (token m of the chunk), double-buffered by chunk parity.
struct SsdVec {
  float G2[CS];      // G_m log2 e (G: in-chunk cumulative log decay)
  float eG[CS];      // e^{G_m}
  float cu[CS];      // dt'_m (0 past the sequence end)
  float bcol[CS];    // e^{G_r - G_m}, r the last token of m's 32-token block
  u16 ecol[CS];      // e^{G_C - G_m} in fp16 (the state update's token weights)
  float gC[4];       // e^{G_C}, G_C (natural log), -, -
};

template <bool kFull>
struct SsdSmem;
template <>
struct SsdSmem<true> {
  u16 C[CS * NS];                 // fp16 C rows, swizzled 16-byte chunks (qidx)
  u16 B[CS * NS];                 // fp16 B rows, same layout
  u16 U[CS * (PH + 8)];           // fp16 dt' x rows, padded (pidx)
  u16 P[CS * kPP];                // fp16 P, pperm columns
  uint4 S[kW][2][kWave];          // S0 halves as fp16 operands, per wave
  SsdVec vec[2];
};
template <>
struct SsdSmem<false> {
  u16 B[CS * NS];
  u16 U[CS * (PH + 8)];
  SsdVec vec[2];
};

// kFull: the whole chunk (outputs, final state); else the state-only pass that
// produces the segment states R and log decays Lambda.
template <typename OutT, bool kGate, bool kFull, bool kCk>
__global__ void __launch_bounds__(kThreads, 1) ssd_kernel(SeqLaunch p) {
  __shared__ __attribute__((aligned(16))) SsdSmem<kFull> sm;

  const int h = blockIdx.x;
  const int gsegs = kFull ? p.ssd_segs : p.ssd_segs - 1;
  const int nseq = blockIdx.y / gsegs, seg = blockIdx.y % gsegs;
  const int sl = p.slot[nseq];
  if (sl < 0) return;                                      // uniform over the block
  const int tbeg = p.cu_seqlens[nseq], tend = p.cu_seqlens[nseq + 1];
  const int nch = (tend - tbeg + CS - 1) / CS;
  const bool last_seg = seg == p.ssd_segs - 1;
  int c0 = min(seg * p.ssd_seg_chunks, nch);
  const int c1 = last_seg ? nch : min(c0 + p.ssd_seg_chunks, nch);
  const int j = h / (p.H_v / p.H_qk);

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wu = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int pt = wu & 3, nh = wu >> 2;
  const int g16 = lane >> 4, j16 = lane & 15;

  // gate parameters of the head (gate folded in)
  float gA = 0.f, gBias = 0.f;
  if constexpr (kGate) {
    gA = p.gA[h];
    gBias = p.gdt_bias ? p.gdt_bias[h] : 0.f;
  }

  // ---------------------------------------------------------------- state tiles
  // Sacc[q] (q = 0..3, tile tk = 4 nh + q) in 16x16 accumulator layout: element r of
  // lane (g16, j16) is S[p = 16 pt + j16][n = 32 (tk / 2) + 4 (tk % 2) + 8 g16 + r], so
  // that tiles 2u, 2u + 1 hold n = 64 nh + 32 u + 8 g16 + 0..7: the natural order of a
  // 16-byte read of a C / B row (k step s2 = 2 nh + u).
  const int64_t hstride = (int64_t)PH * NS;
  auto tile_off = [&](int q) __attribute__((always_inline)) {
    const int tk = 4 * nh + q;
    return (int64_t)(16 * pt + j16) * NS + 32 * (tk >> 1) + 4 * (tk & 1) + 8 * g16;
  };
  f32x4 Sacc[4];
  auto load_state = [&](const float* src, f32x4* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(src + tile_off(q));
      dst[q] = f32x4{v.x, v.y, v.z, v.w};
    }
  };
  auto store_state = [&](float* dst, const f32x4* src) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(dst + tile_off(q)) = make_float4(src[q][0], src[q][1], src[q][2], src[q][3]);
  };
  const int64_t segbase = ((int64_t)nseq * (p.ssd_segs - 1)) * p.H_v;   // (n, s'=0, h=0) in segR / segL
#pragma unroll
  for (int q = 0; q < 4; ++q) Sacc[q] = f32x4{};
  if constexpr (kFull) {
    const bool init = p.has_init ? (p.has_init[nseq] != 0) : true;
    if (init) load_state(p.pool + ((int64_t)sl * p.H_v + h) * hstride, Sacc);
    // entry state of the segment: S <- e^{Lambda_s'} S + R_s' over the segments before it
    for (int s2 = 0; s2 < seg; ++s2) {
      const int64_t row = segbase + (int64_t)s2 * p.H_v + h;
      const float e = __expf(p.segL[row]);
      f32x4 R[4];
      load_state(p.segR + row * hstride, R);
#pragma unroll
      for (int q = 0; q < 4; ++q) Sacc[q] = Sacc[q] * e + R[q];
    }
  }
  float lam = 0.f;                           // (state-only pass) segment log decay

  // checkpoint: the state after ck_b tokens of the sequence, captured by the segment
  // that owns the boundary (its chunk, or the last segment for the sequence's end)
  int ck_b = -1;
  float* ck_st = nullptr;
  if constexpr (kCk) {
    const int tok = p.ck_token[nseq], cks = p.ck_slot[nseq];
    const int b = p.ck_relative ? tok : tok - tbeg;
    const int len = tend - tbeg;
    if (tok >= 0 && cks >= 0 && b >= 0 && b <= len) {
      const bool mine = b == len ? last_seg : (b / CS >= c0 && b / CS < c1);
      if (mine) {
        ck_b = b;
        ck_st = p.ck_states + ((int64_t)cks * p.H_v + h) * hstride;
      }
    }
  }

  // ---------------------------------------------------------------- staging
  // Chunk rows through registers: 512 threads x 16-byte segments.  C, B: 128 rows x 16
  // segments each (4 per thread); x: 128 rows x 8 segments (2 per thread).  Rows past
  // the sequence end re-read the chunk's first row (valid memory; their coefficients
  // are zero and their output rows are not stored).
  const u16* Cg = p.ssd_Ch + (int64_t)j * NS;
  const u16* Bg = p.ssd_Bh + (int64_t)j * NS;
  const int64_t bc_stride = (int64_t)p.H_qk * NS;         // fp16 copies: [T, G, N]
  const u16* xg = reinterpret_cast<const u16*>(p.v) + (int64_t)h * PH;
  // (named registers, not arrays: arrays captured by the lambdas below would be kept
  // in scratch memory)
  uint4 rC0, rC1, rC2, rC3, rB0, rB1, rB2, rB3, rX0, rX1;
  auto ld_cb = [&](const u16* g, int t0, int n, int i) __attribute__((always_inline)) {
    const int sidx = tid + i * kThreads, r = sidx >> 4, c = sidx & 15;
    const int64_t row = (int64_t)t0 + (r < n ? r : 0);
    return *reinterpret_cast<const uint4*>(g + row * bc_stride + 8 * c);
  };
  auto ld_x = [&](int t0, int n, int i) __attribute__((always_inline)) {
    const int sidx = tid + i * kThreads, r = sidx >> 3, c = sidx & 7;
    const int64_t row = (int64_t)t0 + (r < n ? r : 0);
    return *reinterpret_cast<const uint4*>(xg + row * p.v_stride + 8 * c);
  };
  auto stage = [&](int cc) __attribute__((always_inline)) {
    const int t0 = tbeg + cc * CS, n = min(CS, tend - t0);
    if constexpr (kFull) {
      rC0 = ld_cb(Cg, t0, n, 0);
      rC1 = ld_cb(Cg, t0, n, 1);
      rC2 = ld_cb(Cg, t0, n, 2);
      rC3 = ld_cb(Cg, t0, n, 3);
    }
    rB0 = ld_cb(Bg, t0, n, 0);
    rB1 = ld_cb(Bg, t0, n, 1);
    rB2 = ld_cb(Bg, t0, n, 2);
    rB3 = ld_cb(Bg, t0, n, 3);
    rX0 = ld_x(t0, n, 0);
    rX1 = ld_x(t0, n, 1);
  };
  // raw gate inputs of one chunk for the vector wave (lane l: tokens 2 l, 2 l + 1),
  // kept as loaded until their use a step later (an instruction on a loaded value makes
  // the wave wait for the load there)
  uint32_t ra0 = 0u, ra1 = 0u, rb0 = 0u, rb1 = 0u;
  auto stage_gate = [&](int cc) __attribute__((always_inline)) {
    const int t0 = tbeg + cc * CS, n = min(CS, tend - t0);
    const int i0 = 2 * lane, i1 = 2 * lane + 1;
    const int64_t t_0 = t0 + (i0 < n ? i0 : 0), t_1 = t0 + (i1 < n ? i1 : 0);
    if constexpr (kGate) {
      const u16* ga = reinterpret_cast<const u16*>(p.ga);
      ra0 = ga[t_0 * p.ga_stride + h];
      ra1 = ga[t_1 * p.ga_stride + h];
    } else {
      const uint32_t* lg = reinterpret_cast<const uint32_t*>(p.log_g);
      const uint32_t* bt = reinterpret_cast<const uint32_t*>(p.beta);
      ra0 = lg[t_0 * p.H_v + h];
      ra1 = lg[t_1 * p.H_v + h];
      rb0 = bt[t_0 * p.H_v + h];
      rb1 = bt[t_1 * p.H_v + h];
    }
  };
  // the chunk's vectors from the staged gate inputs (vector wave, lane = token pair)
  auto make_vectors = [&](int cc, SsdVec& V) __attribute__((always_inline)) {
    const int t0 = tbeg + cc * CS, n = min(CS, tend - t0);
    const int i0 = 2 * lane, i1 = 2 * lane + 1;
    float lg0, lg1, d0, d1;
    if constexpr (kGate) {
      gate_ssd(__uint_as_float(ra0 << 16), gA, gBias, p.g_softplus, p.g_lo, p.g_hi, lg0, d0);
      gate_ssd(__uint_as_float(ra1 << 16), gA, gBias, p.g_softplus, p.g_lo, p.g_hi, lg1, d1);
    } else {
      lg0 = __uint_as_float(ra0);
      lg1 = __uint_as_float(ra1);
      d0 = __uint_as_float(rb0);
      d1 = __uint_as_float(rb1);
    }
    if (i0 >= n) { lg0 = 0.f; d0 = 0.f; }
    if (i1 >= n) { lg1 = 0.f; d1 = 0.f; }
    const float incl = wave_inclusive_scan(lg0 + lg1);      // G at token 2 l + 1
    const float G1 = incl, G0 = incl - lg1;
    const float GC = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), kWave - 1));
    // G at the last token of this lane's 32-token block (token 32 q + 31: lane 16 q + 15)
    const int blk_lane = (lane & ~15) | 15;
    const float Gr = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * blk_lane, __builtin_bit_cast(int, incl)));
    V.G2[i0] = G0 * kLog2e;
    V.G2[i1] = G1 * kLog2e;
    V.eG[i0] = __expf(G0);
    V.eG[i1] = __expf(G1);
    V.cu[i0] = d0;
    V.cu[i1] = d1;
    V.bcol[i0] = __expf(Gr - G0);
    V.bcol[i1] = __expf(Gr - G1);
    V.ecol[i0] = __builtin_bit_cast(u16, (_Float16)__expf(GC - G0));
    V.ecol[i1] = __builtin_bit_cast(u16, (_Float16)__expf(GC - G1));
    if (lane == 0) {
      V.gC[0] = __expf(GC);
      V.gC[1] = GC;
    }
  };

  // ---------------------------------------------------------------- per-chunk pieces
  // U operand (16x16x32, A as U^T or B as U): lane (g16, j16) holds U[m][16 pt + j16]
  // for the k slots m = 32 s2 + 4 g16 + e (e < 4) and 32 s2 + 16 + 4 g16 + e - 4.
  auto u_op = [&](int s2) __attribute__((always_inline)) {
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int rb = 4 * (lane_o >> 4) + ((lane_o & 15) >> 2), cp = 16 * pt + 4 * (lane_o & 3);
    return join_h(ldtr<PH>(sm.U, 32 * s2 + rb, cp), ldtr<PH>(sm.U, 32 * s2 + 16 + rb, cp));
  };
  // B^T operand for state tile tk (rows n of the tile's order, k slots as u_op)
  auto bt_op = [&](int tk, int s2) __attribute__((always_inline)) {
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int rb = 4 * (lane_o >> 4) + ((lane_o & 15) >> 2);
    const int ca = 32 * (tk >> 1) + 8 * (lane_o & 3) + 4 * (tk & 1);
    return join_h(ldqtr<NS>(sm.B, 32 * s2 + rb, ca), ldqtr<NS>(sm.B, 32 * s2 + 16 + rb, ca));
  };
  // token weights of the k slots of step s2 as fp16 pairs
  auto ecol_op = [&](const SsdVec& V, int s2) __attribute__((always_inline)) {
    const uint2 a = *reinterpret_cast<const uint2*>(&V.ecol[32 * s2 + 4 * g16]);
    const uint2 b = *reinterpret_cast<const uint2*>(&V.ecol[32 * s2 + 16 + 4 * g16]);
    return make_uint4(a.x, a.y, b.x, b.y);
  };
  // S^T <- gamma S^T + B^T diag(w) U with w the fp16 weights (state update, or the
  // masked update of a checkpoint inside the chunk)
  auto update = [&](f32x4* acc, float gamma, auto wfun) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = acc[q] * gamma;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const f16x8 w = scale_h(u_op(s2), wfun(s2));
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = mfma1632h(bt_op(4 * nh + q, s2), w, acc[q]);
    }
  };

  // landing of the staged rows of chunk cc (parity vector V): C, B as they are, x as
  // U = dt' x in fp16
  auto land = [&](const SsdVec& V) __attribute__((always_inline)) {
    auto st_cb = [&](u16* tile, int i, uint4 v) __attribute__((always_inline)) {
      const int sidx = tid + i * kThreads, r = sidx >> 4, c = sidx & 15;
      *reinterpret_cast<uint4*>(tile + qidx<NS>(r, 8 * c)) = v;
    };
    auto st_u = [&](int i, uint4 w) __attribute__((always_inline)) {
      const int sidx = tid + i * kThreads, r = sidx >> 3, c = sidx & 7;
      const float d = V.cu[r];
      *reinterpret_cast<uint4*>(sm.U + pidx<PH>(r, 8 * c)) =
          make_uint4(cvt2h(bf_lo(w.x) * d, bf_hi(w.x) * d), cvt2h(bf_lo(w.y) * d, bf_hi(w.y) * d),
                     cvt2h(bf_lo(w.z) * d, bf_hi(w.z) * d), cvt2h(bf_lo(w.w) * d, bf_hi(w.w) * d));
    };
    if constexpr (kFull) {
      st_cb(sm.C, 0, rC0);
      st_cb(sm.C, 1, rC1);
      st_cb(sm.C, 2, rC2);
      st_cb(sm.C, 3, rC3);
    }
    st_cb(sm.B, 0, rB0);
    st_cb(sm.B, 1, rB1);
    st_cb(sm.B, 2, rB2);
    st_cb(sm.B, 3, rB3);
    st_u(0, rX0);
    st_u(1, rX1);
  };

  // tiles of P = mask(e^{G_i - G_m}) (C B^T) for this wave (see ptile_*): lane holds
  // query row i = 32 ti + l32 and keys m = 32 tm + 8 q4 + 4 hh + e
  auto make_p = [&](const SsdVec& V, int k) __attribute__((always_inline)) {
   if constexpr (kFull) {
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int l32 = lane_o & 31, hh = lane_o >> 5;
    const int ti = ptile_i(k), tm = ptile_m(k);
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < NS / 16; ++s) {
      const f16x8 a = as_f16x8(__builtin_bit_cast(uint4, ldq8<NS>(sm.B, 32 * tm + l32, 16 * s + 8 * hh)));
      const f16x8 b = as_f16x8(__builtin_bit_cast(uint4, ldq8<NS>(sm.C, 32 * ti + l32, 16 * s + 8 * hh)));
      acc = mfma32h(a, b, acc);
    }
    const int i = 32 * ti + l32;
    const float gi = V.G2[i];
    const bool diag = ti == tm;
    // off-diagonal tiles: e^{G_i - G_m} = e^{G_i - G_r} e^{G_r - G_m}, r = 32 tm + 31,
    // both factors <= 1
    const float fi = diag ? 0.f : __builtin_amdgcn_exp2f(gi - V.G2[32 * tm + 31]);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int mb = 32 * tm + 8 * q4 + 4 * hh;
      float pv[4];
      if (diag) {
        const float4 gm = ld_f4(&V.G2[mb]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pv[e] = __builtin_amdgcn_exp2f(mb + e <= i ? gi - f4get(gm, e) : -INFINITY) * acc[4 * q4 + e];
      } else {
        const float4 bc = ld_f4(&V.bcol[mb]);
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = (fi * f4get(bc, e)) * acc[4 * q4 + e];
      }
      *reinterpret_cast<uint2*>(&sm.P[i * kPP + pperm(mb)]) = make_uint2(cvt2h(pv[0], pv[1]), cvt2h(pv[2], pv[3]));
    }
   }
  };

  // output token tiles of this wave: {0, 3, 4, 7} (nh = 0) or {1, 2, 5, 6} (nh = 1),
  // which splits the triangular P U work evenly
  auto out_tile = [&](int k) __attribute__((always_inline)) {
    return nh == 0 ? (k == 0 ? 0 : k == 1 ? 3 : k == 2 ? 4 : 7) : (k == 0 ? 1 : k == 1 ? 2 : k == 2 ? 5 : 6);
  };
  // per-lane output columns 16 pt + 4 g16 + e
  float4 Dc = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (kFull) {
    if (p.D) {
      const u16* Db = reinterpret_cast<const u16*>(p.D);
      float d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        d[e] = bf16_to_f32(Db[p.D_per_dim ? (int64_t)h * PH + 16 * pt + 4 * g16 + e : (int64_t)h]);
      Dc = make_float4(d[0], d[1], d[2], d[3]);
    }
  }
  const u16* zg = reinterpret_cast<const u16*>(p.z);
  const uint32_t ostride_b = (uint32_t)p.out_stride * (uint32_t)sizeof(OutT);

  // ---------------------------------------------------------------- chunk loop
  const bool vwave = wu == kW - 1;           // prepares the next chunk's vectors
  if (c0 < c1) {
    stage(c0);
    if (vwave) stage_gate(c0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0)
  if (vwave && c0 < c1) {
    make_vectors(c0, sm.vec[c0 & 1]);
    stage_gate(min(c0 + 1, c1 - 1));
  }
  if (kCk && ck_b >= 0 && ck_b == CS * c0 && ck_b < tend - tbeg) store_state(ck_st, Sacc);

  for (int c = c0; c < c1; ++c) {
    const int par = c & 1;
    const SsdVec& V = sm.vec[par];
    const int t0 = tbeg + c * CS, n = min(CS, tend - t0);
    lds_sync();                              // the previous chunk's LDS reads are done
    land(V);
    if constexpr (kFull) {
#pragma unroll
      for (int u = 0; u < 2; ++u) sm.S[wu][u][lane] = __builtin_bit_cast(uint4, pair_to_op_h(Sacc[2 * u], Sacc[2 * u + 1]));
    }
    // the epilogue's x and z of this chunk (token 16 it + j16, columns 16 pt + 4 g16 ..),
    // issued before the next chunk's staging so that their use waits for them only
    uint2 ex[4], ez[4];
    if constexpr (kFull) {
      const u16* zrow = zg ? zg + (int64_t)h * PH : xg;   // (without z: re-read x, unused)
      const int64_t zs = zg ? p.z_stride : p.v_stride;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = 16 * out_tile(k) + j16;
        const int64_t t = t0 + (i < n ? i : 0);
        ex[k] = *reinterpret_cast<const uint2*>(xg + t * p.v_stride + 16 * pt + 4 * g16);
        ez[k] = *reinterpret_cast<const uint2*>(zrow + t * zs + 16 * pt + 4 * g16);
      }
    }
    stage(min(c + 1, c1 - 1));               // (unconditional: past the last chunk it re-reads it)
    lds_sync();                              // landing visible
    const float gamma = V.gC[0];
    if constexpr (kFull) {
      make_p(V, wu);
      if (wu == 5 || wu == 6) make_p(V, wu + 3);
    }
    if (vwave) {
      if (c + 1 < c1) make_vectors(c + 1, sm.vec[par ^ 1]);
      stage_gate(min(c + 2, c1 - 1));
    }
    if constexpr (kFull) {
      // Y^T = S0 C^T diag(e^G): k steps 2 nh + u from this wave's registers, the
      // other two from the partner's posted operands
      f32x4 Y[4];
      f16x8 Sown[2], Sprt[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        Sown[u] = pair_to_op_h(Sacc[2 * u], Sacc[2 * u + 1]);
        Sprt[u] = __builtin_bit_cast(f16x8, sm.S[wu ^ 4][u][lane]);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int row = 16 * out_tile(k) + j16;
        Y[k] = f32x4{};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const f16x8 cb = as_f16x8(__builtin_bit_cast(uint4, ldq8<NS>(sm.C, row, 32 * s2 + 8 * g16)));
          const bool own = (s2 >> 1) == nh;
          Y[k] = mfma1632h(own ? Sown[s2 & 1] : Sprt[s2 & 1], cb, Y[k]);
        }
        Y[k] = Y[k] * V.eG[row];
      }
      // checkpoint inside the chunk, after its first m tokens:
      //   S_m^T = e^{G_{m-1}} S0^T + B^T diag(e^{G_{m-1} - G_i} [i < m]) U
      if (kCk && ck_b > CS * c && ck_b < CS * c + n) {
        const int m = ck_b - CS * c;
        const float Gm2 = V.G2[m - 1];
        f32x4 Sc[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) Sc[q] = Sacc[q];
        update(Sc, __builtin_amdgcn_exp2f(Gm2), [&](int s2) {
          uint32_t w[4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            float f[2];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
              const int e = 2 * e2 + x;
              const int i = 32 * s2 + (e < 4 ? 4 * g16 + e : 16 + 4 * g16 + e - 4);
              f[x] = i < m ? __builtin_amdgcn_exp2f(Gm2 - V.G2[i]) : 0.f;
            }
            w[e2] = cvt2h(f[0], f[1]);
          }
          return make_uint4(w[0], w[1], w[2], w[3]);
        });
        store_state(ck_st, Sc);
      }
      update(Sacc, gamma, [&](int s2) { return ecol_op(V, s2); });
      lds_sync();                            // P complete
      // Y^T += U^T P^T over the key steps s2 <= it / 2 (P is zero above the diagonal)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int it = out_tile(k);
        const int row = 16 * it + j16;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          if (s2 > (it >> 1)) continue;
          const f16x8 pb = as_f16x8(*reinterpret_cast<const uint4*>(&sm.P[row * kPP + 32 * s2 + 8 * g16]));
          Y[k] = mfma1632h(u_op(s2), pb, Y[k]);
        }
      }
      // epilogue: (y + D x) silu(z), rows past the sequence end dropped by the bounded
      // buffer stores (record = the chunk's n rows)
      char* obase = reinterpret_cast<char*>(p.out) +
                    ((int64_t)t0 * p.out_stride + (int64_t)h * PH + 16 * pt) * (int64_t)sizeof(OutT);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(obase, (short)0, (int)((uint32_t)n * ostride_b), kBufWord3);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int it = out_tile(k);
        const float xv[4] = {bf_lo(ex[k].x), bf_hi(ex[k].x), bf_lo(ex[k].y), bf_hi(ex[k].y)};
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Y[k][e] + f4get(Dc, e) * xv[e];
        if (zg) {
          const float zv[4] = {bf_lo(ez[k].x), bf_hi(ez[k].x), bf_lo(ez[k].y), bf_hi(ez[k].y)};
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] *= silu_f(zv[e]);
        }
        const int off = (int)((uint32_t)(16 * it + j16) * ostride_b + (uint32_t)(4 * g16 * sizeof(OutT)));
        if constexpr (sizeof(OutT) == 2) {
          const u32x2 w = {cvt2(y[0], y[1]), cvt2(y[2], y[3])};
          __builtin_amdgcn_raw_buffer_store_b64(w, rs, off, 0, 0);
        } else {
          const u32x4 w = {__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
                           __float_as_uint(y[3])};
          __builtin_amdgcn_raw_buffer_store_b128(w, rs, off, 0, 0);
        }
      }
      if (kCk && ck_b >= 0 && ck_b == CS * (c + 1) && ck_b < tend - tbeg) store_state(ck_st, Sacc);
    } else {
      update(Sacc, gamma, [&](int s2) { return ecol_op(V, s2); });
      lam += V.gC[1];
    }
  }

  if constexpr (kFull) {
    if (last_seg) {
      if (kCk && ck_b >= 0 && ck_b == tend - tbeg) store_state(ck_st, Sacc);
      if (!p.keep_pool) store_state(p.pool + ((int64_t)sl * p.H_v + h) * hstride, Sacc);
    }
  } else {
    const int64_t row = segbase + (int64_t)seg * p.H_v + h;
    store_state(p.segR + row * hstride, Sacc);
    if (tid == 0) p.segL[row] = lam;
  }
}

// fp16 copies of B and C ([T, G, N] contiguous) for the chunked delta-off kernels:
// every head of a group reads them, so they are converted once per call.  One thread
// per 8 elements.
__global__ void __launch_bounds__(256) ssd_prep_kernel(SeqLaunch p) {
  const int64_t seg = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 16-byte output segment
  const int per_tok = p.H_qk * NS / 8;
  const int64_t t = seg / per_tok;
  if (t >= p.T) return;
  const int r = (int)(seg % per_tok);
  const int g = r / (NS / 8), c = r % (NS / 8);
  const u16* src[2] = {reinterpret_cast<const u16*>(p.k), reinterpret_cast<const u16*>(p.q)};
  const int64_t str[2] = {p.k_stride, p.q_stride};
  u16* dst[2] = {const_cast<u16*>(p.ssd_Bh), const_cast<u16*>(p.ssd_Ch)};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint4 w = *reinterpret_cast<const uint4*>(src[k] + t * str[k] + (int64_t)g * NS + 8 * c);
    *reinterpret_cast<uint4*>(dst[k] + (t * p.H_qk + g) * NS + 8 * c) =
        make_uint4(cvt2h(bf_lo(w.x), bf_hi(w.x)), cvt2h(bf_lo(w.y), bf_hi(w.y)),
                   cvt2h(bf_lo(w.z), bf_hi(w.z)), cvt2h(bf_lo(w.w), bf_hi(w.w)));
  }
}

template <typename OutT, bool kGate, bool kCk>
hipError_t launch_ssd_typed(const SeqLaunch& p, hipStream_t stream) {
  const int64_t segs16 = p.T * p.H_qk * (NS / 8);
  if (segs16 > 0) {
    hipLaunchKernelGGL(ssd_prep_kernel, dim3((unsigned)((segs16 + 255) / 256)), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.ssd_segs > 1) {
    hipLaunchKernelGGL((ssd_kernel<OutT, kGate, false, false>), dim3(p.H_v, p.N * (p.ssd_segs - 1)),
                       dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((ssd_kernel<OutT, kGate, true, kCk>), dim3(p.H_v, p.N * p.ssd_segs), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename OutT, bool kGate>
hipError_t launch_ssd_ck(const SeqLaunch& p, hipStream_t stream) {
  return p.ck_token ? launch_ssd_typed<OutT, kGate, true>(p, stream)
                    : launch_ssd_typed<OutT, kGate, false>(p, stream);
}

}  // namespace

// Workspace of a chunk-128 delta-off call with `segs` segments per sequence: the fp16
// copies of B and C, then the segment states and log decays (segs - 1 per sequence).
int64_t ssd_workspace_bytes(int64_t T, int N, int H_qk, int H_v, int segs) {
  auto up = [](int64_t b) { return (b + 255) & ~int64_t(255); };
  const int64_t bc = up(T * H_qk * NS * 2);
  const int64_t r = up((int64_t)N * (segs - 1) * H_v * PH * NS * 4);
  const int64_t l = up((int64_t)N * (segs - 1) * H_v * 4);
  return 2 * bc + r + l;
}

void ssd_bind_workspace(SeqLaunch& p, void* ws) {
  auto up = [](int64_t b) { return (b + 255) & ~int64_t(255); };
  char* base = static_cast<char*>(ws);
  const int64_t bc = up(p.T * p.H_qk * NS * 2);
  p.ssd_Bh = reinterpret_cast<const u16*>(base);
  p.ssd_Ch = reinterpret_cast<const u16*>(base + bc);
  p.segR = reinterpret_cast<float*>(base + 2 * bc);
  p.segL = reinterpret_cast<float*>(base + 2 * bc + up((int64_t)p.N * (p.ssd_segs - 1) * p.H_v * PH * NS * 4));
}

bool ssd_chunked_shape(const SeqLaunch& p) { return p.ssd && p.d_k == NS && p.d_v == PH; }

int ssd_obstacles(const SeqLaunch& p) {
  int why = 0;
  if (!p.in_bf16) why |= GDN_WHY_FP32;
  if (!ssd_chunked_shape(p)) why |= GDN_WHY_HEAD_DIMS;
  if (p.N > 65535) why |= GDN_WHY_BATCH;
  // B, C (prep kernel) and x rows are read as 16-byte segments
  const uintptr_t ptrs = reinterpret_cast<uintptr_t>(p.q) | reinterpret_cast<uintptr_t>(p.k) |
                         reinterpret_cast<uintptr_t>(p.v);
  if (ptrs % 16 != 0 || (p.q_stride | p.k_stride | p.v_stride) % 8 != 0) why |= GDN_WHY_ALIGN;
  // 32-bit offsets of the output rows of a chunk (bounded buffer stores)
  if (p.out_stride > (int64_t(1) << 31) / (CS * 4)) why |= GDN_WHY_STRIDE;
  return why;
}

hipError_t launch_ssd(const SeqLaunch& p, hipStream_t stream) {
  if (p.N == 0) return hipSuccess;
  if (p.out_bf16) return p.gate_fused ? launch_ssd_ck<u16, true>(p, stream) : launch_ssd_ck<u16, false>(p, stream);
  return p.gate_fused ? launch_ssd_ck<float, true>(p, stream) : launch_ssd_ck<float, false>(p, stream);
}

}  // namespace gdn
