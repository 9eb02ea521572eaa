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
// it (S <- e^{Lambda_s'} S + R_s', s' < s).
//
// Once per call, per chunk and group (every head of the group shares them), a prep
// kernel converts the chunk's B and C rows to fp16 and computes the chunk's raw C B^T
// tiles on and below the diagonal (32x32x16 MFMA), both kept in the workspace.
//
// A workgroup takes two heads of one group for one segment of one sequence: grid
// (group x head pair, sequence x segment).  Wave w owns the state columns
// p = 16 pt .. 16 pt + 15 (pt = w % 4) of head slot w / 4 over all of N: eight 16x16
// accumulator tiles of S^T in registers.  Per chunk:
//   * landing: the chunk's fp16 C and B rows and both heads' x rows (as fp16) into LDS,
//     with the chunk's z rows and this wave's raw C B^T tiles loaded alongside; two
//     waves prepare the next chunk's gate, decay cumsum and per-token factors, one
//     head each;
//   * Y^T = S0 C^T diag(e^G) for the 128 tokens, then S^T <- e^{G_C} S^T +
//     B^T diag(e^{G_C - G} dt') X;
//   * the LDS tiles from the raw ones: each wave the diagonal 32x32 tile pt of its
//     head's P (masked, decayed), waves 0-5 one off-diagonal tile each (shared by both
//     heads);
//   * the intra-chunk term: the diagonal 32-token blocks from the head's P, every
//     earlier block from the raw C B^T tile with the decay factored at the block's last
//     token r, e^{G_i - G_m} = e^{G_i - G_r} e^{G_r - G_m} (both <= 1: the key factor
//     scales X, the query factor the block's partial sum);
//   * the epilogue: the y tiles go through LDS (over the C and B rows, read by then), so
//     that each thread finishes (y + D x) silu(z) for 8 columns of a token row, with z
//     read and the output written in whole 128-byte rows.
// The chunk's C, B and x rows are staged from memory through registers one chunk
// ahead.  The state-only pass (segment states from zero) runs the same loop with B, x
// and the update alone.  Operand precision: C, B, x exact in fp16 (bf16 values in fp16's normal
// range); S0, P and the scaled X carry fp16's 11-bit significand (2^-12 relative
// rounding, well below the bf16 output's); every product accumulates in fp32.  fp16's
// range bounds the magnitudes: |C.B|, |x|, |dt' x| and |S| must stay below 65504
// (beyond it the results turn inf / NaN, visibly).
#include "gdn_common.h"
#include "gdn_launch.h"
#include "tile_ops.h"

namespace gdn {

namespace {

constexpr int CS = 128;             // chunk length
constexpr int NS = 128;             // dstate (d_k)
constexpr int PH = 64;              // headdim (d_v)
constexpr int kW = 8;               // waves per workgroup (two head slots x four column tiles)
constexpr int kThreads = kW * kWave;
constexpr int kTP = 40;             // row length (fp16) of the 32x32 P and C B^T tiles: 80 B rows
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
__device__ __forceinline__ float h_lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2v, w)[0]; }
__device__ __forceinline__ float h_hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2v, w)[1]; }
// bf16 pair -> fp16 pair (exact for bf16 values in fp16's normal range)
__device__ __forceinline__ uint32_t bf2h(uint32_t w) { return cvt2h(bf_lo(w), bf_hi(w)); }
// silu(y) = y / (1 + e^-y) (the reciprocal's argument is >= 1, or +inf for y < -88,
// where the result is -0: the limit)
__device__ __forceinline__ float silu_f(float y) {
  return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y));
}

// The 32x32 tiles keep their 4-column groups in the order 0, 4, 1, 5, 2, 6, 3, 7, so
// that the 8 k slots of a 16x16x32 operand (tokens 4g .. 4g+3 and 16+4g .. 16+4g+3 of
// the block, the order of the state update's token k slots) are 16 contiguous bytes.
// Column within the block -> stored column:
__device__ __forceinline__ int pperm(int c) {
  const int q = c >> 2;
  return ((2 * (q & 3) + (q >> 2)) << 2) | (c & 3);
}
// y row buffer of the epilogue: token row r, 16-byte chunk q (p = 4 q .. 4 q + 3) at
// chunk q ^ (r % 16) of the row, so that both the owner waves' 16-byte writes (16 rows
// x 4 chunks) and the epilogue's reads (8 rows x 8 chunk pairs) spread over the banks.
__device__ __forceinline__ int yidx(int r, int q) { return r * PH + 4 * (q ^ (r & 15)); }

// Off-diagonal 32x32 tiles of C B^T (i-block d > m-block s2), in the order
// (1,0), (2,0), (2,1), (3,0), (3,1), (3,2): index d (d - 1) / 2 + s2.
__device__ __forceinline__ int offdiag_i(int o) { return o == 0 ? 1 : o < 3 ? 2 : 3; }
__device__ __forceinline__ int offdiag_m(int o) { return o == 0 ? 0 : o < 3 ? o - 1 : o - 3; }

// The raw C B^T tiles of every chunk (computed once per call for all heads of a group):
// chunk c of sequence s, starting at token tbeg_s + 128 c, has the slot
// floor(tbeg_s / 128) + s + c -- consecutive within a sequence, increasing from one
// sequence to the next, all below floor(T / 128) + N.  A slot holds per group the ten
// 32x32 tiles (the six off-diagonal ones in offdiag order, then the four diagonal
// ones), each as fp16 in 32x32 accumulator order: lane l32 + 32 hh holds query row l32
// and keys 8 q4 + 4 hh + e at position 4 q4 + e (32 bytes per lane).
constexpr int kCBTiles = 10;
constexpr int kCBTileElems = 32 * 32;
__device__ __forceinline__ int64_t cb_slot_base(int tbeg, int s) { return (int64_t)(tbeg / CS) + s; }

// One head's per-token coefficients of one chunk (token m of the chunk).
struct SsdVec {
  float G2[CS];      // G_m log2 e (G: in-chunk cumulative log decay)
  float eG[CS];      // e^{G_m}
  u16 dtp[CS];       // dt'_m in fp16 (0 past the sequence end)
  u16 wfac[CS];      // e^{G_C - G_m} dt'_m in fp16: the state update's token weights
  u16 ufac[CS];      // e^{G_r - G_m} dt'_m in fp16, r the last token of m's 32-token block
  float gC[2];       // e^{G_C}, G_C (natural log)
};

// One chunk's staged rows in registers (16-byte segments; named members, no arrays,
// so that they stay in registers): C, B and both heads' x.
struct SsdStage {
  uint4 c0, c1, c2, c3, b0, b1, b2, b3, x0, x1, x2, x3;
};

template <bool kFull>
struct SsdSmem;
template <>
struct SsdSmem<true> {
  union {
    struct {
      u16 C[CS * NS];             // fp16 C rows, swizzled 16-byte chunks (qidx)
      u16 B[CS * NS];             // fp16 B rows, same layout
    };
    // (epilogue, once C and B are read) both head slots' y rows, [token][p] in fp32
    // with the 16-byte chunks of a row swizzled (yidx)
    float Yx[2][CS * PH];
  };
  float Dv[2][PH];                // D per output column of each head slot (0 without D)
  u16 X[2][CS * (PH + 8)];        // fp16 x rows per head slot, padded (pidx)
  u16 CB[6][32 * kTP];            // off-diagonal 32x32 tiles of C B^T, pperm columns
  u16 Pd[2][4][32 * kTP];         // per head slot: the diagonal tiles of P (masked, decayed)
  SsdVec vec[2][2];               // [chunk parity][head slot]
};
template <>
struct SsdSmem<false> {
  u16 B[CS * NS];
  u16 X[2][CS * (PH + 8)];
  SsdVec vec[2][2];
};

// kFull: the whole chunk (outputs, final state); else the state-only pass that
// produces the segment states R and log decays Lambda.
template <typename OutT, bool kGate, bool kFull, bool kCk>
__global__ void __launch_bounds__(kThreads, 1) ssd_kernel(SeqLaunch p) {
  __shared__ __attribute__((aligned(16))) SsdSmem<kFull> sm;

  // ---------------------------------------------------------------- work item
  const int hpg = p.H_v / p.H_qk;                  // heads per group
  const int ppg = (hpg + 1) / 2;                   // head pairs per group
  const int j = blockIdx.x / ppg, pq = blockIdx.x % ppg;
  const int hA = j * hpg + 2 * pq;
  const bool two = 2 * pq + 1 < hpg;               // (an odd group's last pair has one head)
  const int hB = two ? hA + 1 : hA;
  // full pass: segment seg of sequence nseq; state-only pass: piece sub of segment seg
  // (segments 0 .. segs - 2, each cut into ssd_sub pieces of about equal length)
  const int nsub = kFull ? 1 : p.ssd_sub;
  const int gsegs = kFull ? p.ssd_segs : (p.ssd_segs - 1) * nsub;
  const int nseq = blockIdx.y / gsegs, gi = blockIdx.y % gsegs;
  const int seg = gi / nsub, sub = gi % nsub;
  const int sl = p.slot[nseq];
  if (sl < 0) return;                              // uniform over the block
  const int tbeg = p.cu_seqlens[nseq], tend = p.cu_seqlens[nseq + 1];
  const int nch = (tend - tbeg + CS - 1) / CS;
  const bool last_seg = seg == p.ssd_segs - 1;
  int c0, c1;
  if constexpr (kFull) {
    c0 = min(seg * p.ssd_seg_chunks, nch);
    c1 = last_seg ? nch : min(c0 + p.ssd_seg_chunks, nch);
  } else {
    const int sb = seg * p.ssd_seg_chunks;
    c0 = min(sb + sub * p.ssd_seg_chunks / nsub, nch);
    c1 = min(sb + (sub + 1) * p.ssd_seg_chunks / nsub, nch);
  }

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wu = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int hs = wu >> 2, pt = wu & 3;             // head slot, column tile
  const int h = hs ? hB : hA;                      // this wave's head
  const bool owner = hs == 0 || two;               // (a lone head's second slot only mirrors it)
  const int g16 = lane >> 4, j16 = lane & 15;
  const bool vwave = wu >= kW - 2;                 // waves 6, 7: vectors of head slot wu - 6
  const int vh = wu == kW - 1 ? hB : hA;

  // gate parameters of the vector wave's head (gate folded in)
  float gA = 0.f, gBias = 0.f;
  if constexpr (kGate) {
    gA = p.gA[vh];
    gBias = p.gdt_bias ? p.gdt_bias[vh] : 0.f;
  }

  // ---------------------------------------------------------------- state tiles
  // Sacc[tk] (tk = 0..7) in 16x16 accumulator layout: element r of lane (g16, j16) is
  // S[p = 16 pt + j16][n = 32 (tk / 2) + 4 (tk % 2) + 8 g16 + r], so that tiles 2 s2,
  // 2 s2 + 1 hold n = 32 s2 + 8 g16 + 0..7: the natural order of a 16-byte read of a
  // C / B row (k step s2 of the products over N).
  const int64_t hstride = (int64_t)PH * NS;
  auto tile_off = [&](int tk) __attribute__((always_inline)) {
    return (int64_t)(16 * pt + j16) * NS + 32 * (tk >> 1) + 4 * (tk & 1) + 8 * g16;
  };
  f32x4 Sacc[8];
  auto load_state = [&](const float* src, f32x4* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int tk = 0; tk < 8; ++tk) {
      const float4 v = *reinterpret_cast<const float4*>(src + tile_off(tk));
      dst[tk] = f32x4{v.x, v.y, v.z, v.w};
    }
  };
  auto store_state = [&](float* dst, const f32x4* src) __attribute__((always_inline)) {
#pragma unroll
    for (int tk = 0; tk < 8; ++tk)
      *reinterpret_cast<float4*>(dst + tile_off(tk)) = make_float4(src[tk][0], src[tk][1], src[tk][2], src[tk][3]);
  };
  // (n, piece 0, h = 0) in segR / segL: the pieces of the first segs - 1 segments in token order
  const int64_t segbase = ((int64_t)nseq * (p.ssd_segs - 1) * p.ssd_sub) * p.H_v;
#pragma unroll
  for (int tk = 0; tk < 8; ++tk) Sacc[tk] = f32x4{};
  if constexpr (kFull) {
    const bool init = p.has_init ? (p.has_init[nseq] != 0) : true;
    if (init) load_state(p.pool + ((int64_t)sl * p.H_v + h) * hstride, Sacc);
    // entry state of the segment: S <- e^{Lambda_s'} S + R_s' over the state-only pass's
    // pieces before it, in order, two pieces' loads in flight at a time (the staging
    // registers are free here)
    const int nfold = seg * p.ssd_sub;
    int s2 = 0;
    for (; s2 + 1 < nfold; s2 += 2) {
      const int64_t row = segbase + (int64_t)s2 * p.H_v + h;
      const float e0 = __expf(p.segL[row]), e1 = __expf(p.segL[row + p.H_v]);
      f32x4 R0[8], R1[8];
      load_state(p.segR + row * hstride, R0);
      load_state(p.segR + (row + p.H_v) * hstride, R1);
#pragma unroll
      for (int tk = 0; tk < 8; ++tk) Sacc[tk] = (Sacc[tk] * e0 + R0[tk]) * e1 + R1[tk];
    }
    if (s2 < nfold) {
      const int64_t row = segbase + (int64_t)s2 * p.H_v + h;
      const float e = __expf(p.segL[row]);
      f32x4 R[8];
      load_state(p.segR + row * hstride, R);
#pragma unroll
      for (int tk = 0; tk < 8; ++tk) Sacc[tk] = Sacc[tk] * e + R[tk];
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
    if (owner && tok >= 0 && cks >= 0 && b >= 0 && b <= len) {
      const bool mine = b == len ? last_seg : (b / CS >= c0 && b / CS < c1);
      if (mine) {
        ck_b = b;
        ck_st = p.ck_states + ((int64_t)cks * p.H_v + h) * hstride;
      }
    }
  }

  // ---------------------------------------------------------------- staging
  // Chunk rows through registers, 16-byte segments from a wave-uniform row base plus
  // 32-bit lane offsets: C, B 128 rows x 16 segments (4 per thread each), x of both
  // heads 2 x 128 rows x 8 segments (4 per thread: the first two of head slot 0).  Rows
  // past the sequence end re-read the chunk's first row (valid memory; their
  // coefficients are zero and their output rows are not stored).  Named registers, not
  // arrays: arrays captured by the lambdas below would be kept in scratch memory.
  const int64_t bcs = (int64_t)p.H_qk * NS;        // fp16 copies: [T, G, N]
  const u16* Cg = p.ssd_Ch + (int64_t)j * NS;
  const u16* Bg = p.ssd_Bh + (int64_t)j * NS;
  const u16* xg = reinterpret_cast<const u16*>(p.v);
  SsdStage rs0;
  auto ld_cb = [&](const u16* g, int t0, int n, int i) __attribute__((always_inline)) {
    const int sidx = tid + i * kThreads, r = sidx >> 4, c = sidx & 15;
    const char* base = reinterpret_cast<const char*>(g + (int64_t)t0 * bcs);
    const uint32_t off = ((uint32_t)(r < n ? r : 0) * (uint32_t)bcs + 8u * (uint32_t)c) * 2u;
    return *reinterpret_cast<const uint4*>(base + off);
  };
  auto ld_x = [&](int t0, int n, int i) __attribute__((always_inline)) {
    const int sidx = (tid + i * kThreads) & 1023, r = sidx >> 3, c = sidx & 7;
    const char* base = reinterpret_cast<const char*>(xg + (int64_t)t0 * p.v_stride + (int64_t)(i < 2 ? hA : hB) * PH);
    const uint32_t off = ((uint32_t)(r < n ? r : 0) * (uint32_t)p.v_stride + 8u * (uint32_t)c) * 2u;
    return *reinterpret_cast<const uint4*>(base + off);
  };
  // parts: kStC | kStB | kStX (a constant at every call)
  enum { kStC = 1, kStB = 2, kStX = 4, kStAll = 7 };
  auto stage = [&](SsdStage& r, int cc, int parts) __attribute__((always_inline)) {
    const int t0 = tbeg + cc * CS, n = min(CS, tend - t0);
    if (kFull && (parts & kStC)) {
      r.c0 = ld_cb(Cg, t0, n, 0);
      r.c1 = ld_cb(Cg, t0, n, 1);
      r.c2 = ld_cb(Cg, t0, n, 2);
      r.c3 = ld_cb(Cg, t0, n, 3);
    }
    if (parts & kStB) {
      r.b0 = ld_cb(Bg, t0, n, 0);
      r.b1 = ld_cb(Bg, t0, n, 1);
      r.b2 = ld_cb(Bg, t0, n, 2);
      r.b3 = ld_cb(Bg, t0, n, 3);
    }
    if (parts & kStX) {
      r.x0 = ld_x(t0, n, 0);
      r.x1 = ld_x(t0, n, 1);
      r.x2 = ld_x(t0, n, 2);
      r.x3 = ld_x(t0, n, 3);
    }
  };
  // raw gate inputs of one chunk for a vector wave (lane l: tokens 2 l, 2 l + 1), kept
  // as loaded until their use a step later (an instruction on a loaded value makes the
  // wave wait for the load there)
  uint32_t ra0 = 0u, ra1 = 0u, rb0 = 0u, rb1 = 0u;
  auto stage_gate = [&](int cc) __attribute__((always_inline)) {
    const int t0 = tbeg + cc * CS, n = min(CS, tend - t0);
    const int i0 = 2 * lane, i1 = 2 * lane + 1;
    const int t_0 = i0 < n ? i0 : 0, t_1 = i1 < n ? i1 : 0;
    if constexpr (kGate) {
      const char* ga = reinterpret_cast<const char*>(reinterpret_cast<const u16*>(p.ga) + (int64_t)t0 * p.ga_stride + vh);
      ra0 = *reinterpret_cast<const u16*>(ga + (uint32_t)t_0 * (uint32_t)p.ga_stride * 2u);
      ra1 = *reinterpret_cast<const u16*>(ga + (uint32_t)t_1 * (uint32_t)p.ga_stride * 2u);
    } else {
      const char* lg = reinterpret_cast<const char*>(p.log_g + (int64_t)t0 * p.H_v + vh);
      const char* bt = reinterpret_cast<const char*>(p.beta + (int64_t)t0 * p.H_v + vh);
      const uint32_t s4 = (uint32_t)p.H_v * 4u;
      ra0 = *reinterpret_cast<const uint32_t*>(lg + (uint32_t)t_0 * s4);
      ra1 = *reinterpret_cast<const uint32_t*>(lg + (uint32_t)t_1 * s4);
      rb0 = *reinterpret_cast<const uint32_t*>(bt + (uint32_t)t_0 * s4);
      rb1 = *reinterpret_cast<const uint32_t*>(bt + (uint32_t)t_1 * s4);
    }
  };
  // a chunk's vectors of the vector wave's head from its staged gate inputs
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
    *reinterpret_cast<uint32_t*>(&V.wfac[i0]) = cvt2h(__expf(GC - G0) * d0, __expf(GC - G1) * d1);
    if constexpr (kFull) {   // (the state-only pass needs the update's weights and e^{G_C} only)
      // G at the last token of this lane's 32-token block (token 32 q + 31: lane 16 q + 15)
      const int blk_lane = (lane & ~15) | 15;
      const float Gr = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * blk_lane, __builtin_bit_cast(int, incl)));
      V.G2[i0] = G0 * kLog2e;
      V.G2[i1] = G1 * kLog2e;
      V.eG[i0] = __expf(G0);
      V.eG[i1] = __expf(G1);
      *reinterpret_cast<uint32_t*>(&V.dtp[i0]) = cvt2h(d0, d1);
      *reinterpret_cast<uint32_t*>(&V.ufac[i0]) = cvt2h(__expf(Gr - G0) * d0, __expf(Gr - G1) * d1);
    }
    if (lane == 0) {
      V.gC[0] = __expf(GC);
      V.gC[1] = GC;
    }
  };

  // ---------------------------------------------------------------- per-chunk pieces
  // Lane-derived LDS addresses are recomputed once per chunk step from an opaque copy of
  // the lane id, lane_s, set at the top of every step: the reads of one step share them
  // (one computation per step), and they are not kept live across the chunk loop.
  int lane_s = lane;
  // X operand (16x16x32, as A = X^T or B = X): lane (g16, j16) holds x[m][16 pt + j16] of
  // this wave's head for the k slots m = 32 s2 + 4 g16 + e (e < 4), 32 s2 + 16 + 4 g16 + e - 4
  auto x_op = [&](int s2) __attribute__((always_inline)) {
    const int lane_o = lane_s;
    const int rb = 4 * (lane_o >> 4) + ((lane_o & 15) >> 2), cp = 16 * pt + 4 * (lane_o & 3);
    return join_h(ldtr<PH>(sm.X[hs], 32 * s2 + rb, cp), ldtr<PH>(sm.X[hs], 32 * s2 + 16 + rb, cp));
  };
  // B^T operand for state tile tk (rows n in the tile's order, k slots as x_op)
  auto bt_op = [&](int tk, int s2) __attribute__((always_inline)) {
    const int lane_o = lane_s;
    const int rb = 4 * (lane_o >> 4) + ((lane_o & 15) >> 2);
    const int ca = 32 * (tk >> 1) + 8 * (lane_o & 3) + 4 * (tk & 1);
    return join_h(ldqtr<NS>(sm.B, 32 * s2 + rb, ca), ldqtr<NS>(sm.B, 32 * s2 + 16 + rb, ca));
  };
  // per-token fp16 factors of the k slots of step s2, as the pairs of x_op's order
  auto fac_op = [&](const u16* f, int s2) __attribute__((always_inline)) {
    const uint2 a = *reinterpret_cast<const uint2*>(&f[32 * s2 + 4 * g16]);
    const uint2 b = *reinterpret_cast<const uint2*>(&f[32 * s2 + 16 + 4 * g16]);
    return make_uint4(a.x, a.y, b.x, b.y);
  };
  // S^T <- gamma S^T + B^T W with the update's X operands W[s2]
  auto update = [&](f32x4* acc, float gamma, const f16x8* W) __attribute__((always_inline)) {
#pragma unroll
    for (int tk = 0; tk < 8; ++tk) acc[tk] = acc[tk] * gamma;
    if constexpr (!kFull) {
      // state-only pass (registers to spare): one k step's eight B^T operands are read
      // while the previous step's MFMAs run (sched_barrier keeps the compiler from
      // pairing each read with its MFMA)
      f16x8 a[2][8];
#pragma unroll
      for (int tk = 0; tk < 8; ++tk) a[0][tk] = bt_op(tk, 0);
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        if (s2 < 3) {
#pragma unroll
          for (int tk = 0; tk < 8; ++tk) a[(s2 + 1) & 1][tk] = bt_op(tk, s2 + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tk = 0; tk < 8; ++tk) acc[tk] = mfma1632h(a[s2 & 1][tk], W[s2], acc[tk]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
        for (int tk = 0; tk < 8; ++tk) acc[tk] = mfma1632h(bt_op(tk, s2), W[s2], acc[tk]);
    }
  };

  // landing of the staged rows: C, B as they are, x converted to fp16
  auto land = [&](const SsdStage& r) __attribute__((always_inline)) {
    auto st_cb = [&](u16* tile, int i, uint4 v) __attribute__((always_inline)) {
      const int sidx = tid + i * kThreads, r = sidx >> 4, c = sidx & 15;
      *reinterpret_cast<uint4*>(tile + qidx<NS>(r, 8 * c)) = v;
    };
    auto st_x = [&](int i, uint4 w) __attribute__((always_inline)) {
      const int sidx = (tid + i * kThreads) & 1023, r = sidx >> 3, c = sidx & 7;
      *reinterpret_cast<uint4*>(sm.X[i >> 1] + pidx<PH>(r, 8 * c)) = make_uint4(bf2h(w.x), bf2h(w.y), bf2h(w.z), bf2h(w.w));
    };
    if constexpr (kFull) {
      st_cb(sm.C, 0, r.c0);
      st_cb(sm.C, 1, r.c1);
      st_cb(sm.C, 2, r.c2);
      st_cb(sm.C, 3, r.c3);
    }
    st_cb(sm.B, 0, r.b0);
    st_cb(sm.B, 1, r.b1);
    st_cb(sm.B, 2, r.b2);
    st_cb(sm.B, 3, r.b3);
    st_x(0, r.x0);
    st_x(1, r.x1);
    st_x(2, r.x2);
    st_x(3, r.x3);
  };

  // This wave's raw C B^T tiles of the chunk, loaded at the top of its step: the
  // diagonal tile pt, and for waves 0-5 the off-diagonal tile wu (16 fp16 per lane).
  auto load_tiles = [&](int cc, uint4& d0, uint4& d1, uint4& o0, uint4& o1) __attribute__((always_inline)) {
    if constexpr (kFull) {
      const u16* base = p.ssd_CB + ((cb_slot_base(tbeg, nseq) + cc) * p.H_qk + j) * (int64_t)(kCBTiles * kCBTileElems) +
                        16 * lane;
      d0 = *reinterpret_cast<const uint4*>(base + (6 + pt) * kCBTileElems);
      d1 = *reinterpret_cast<const uint4*>(base + (6 + pt) * kCBTileElems + 8);
      if (wu < 6) {
        o0 = *reinterpret_cast<const uint4*>(base + wu * kCBTileElems);
        o1 = *reinterpret_cast<const uint4*>(base + wu * kCBTileElems + 8);
      }
    }
  };
  // ... and from them this wave's head's diagonal tile pt of P (masked, decayed) and,
  // waves 0-5, the raw off-diagonal tile wu in LDS
  auto make_tiles = [&](const SsdVec& V, uint4 d0, uint4 d1, uint4 o0, uint4 o1) __attribute__((always_inline)) {
    if constexpr (kFull) {
      int lane_o = lane;
      asm volatile("" : "+v"(lane_o));
      const int l32 = lane_o & 31, hh = lane_o >> 5;
      {
        const uint32_t w[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
        const int i = 32 * pt + l32;
        const float gi = V.G2[i];
        u16* dst = sm.Pd[hs][pt] + l32 * kTP;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int mb = 32 * pt + 8 * q4 + 4 * hh;
          const float4 gm = ld_f4(&V.G2[mb]);
          float pv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t we = w[2 * q4 + (e >> 1)];
            pv[e] = __builtin_amdgcn_exp2f(mb + e <= i ? gi - f4get(gm, e) : -INFINITY) * (e & 1 ? h_hi(we) : h_lo(we));
          }
          *reinterpret_cast<uint2*>(dst + pperm(8 * q4 + 4 * hh)) = make_uint2(cvt2h(pv[0], pv[1]), cvt2h(pv[2], pv[3]));
        }
      }
      if (wu < 6) {
        const uint32_t w[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
        u16* dst = sm.CB[wu] + l32 * kTP;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<uint2*>(dst + pperm(8 * q4 + 4 * hh)) = make_uint2(w[2 * q4], w[2 * q4 + 1]);
      }
    }
  };

  // The epilogue's work split: thread tid finishes output columns 8 (tid % 8) .. + 7
  // of token rows tid / 8 and tid / 8 + 64 of both head slots (slice i = 0..3: head
  // slot i / 2, row tid / 8 + 64 (i % 2)) -- 8 threads per 128-byte row of a head, so
  // that z is read and the output written in whole rows.
  const int ek = tid & 7, er = tid >> 3;
  if constexpr (kFull) {   // D of the two head slots (visible after the first barrier)
    if (tid < 2 * PH) {
      const int hsl = tid / PH, col = tid % PH, hd = hsl ? hB : hA;
      const u16* Db = reinterpret_cast<const u16*>(p.D);
      sm.Dv[hsl][col] = Db ? bf16_to_f32(Db[p.D_per_dim ? (int64_t)hd * PH + col : (int64_t)hd]) : 0.f;
    }
  }
  const uint32_t ostride_b = (uint32_t)p.out_stride * (uint32_t)sizeof(OutT);
  // z rows (x again when there is no z: valid memory, unused)
  const u16* zg = p.z ? reinterpret_cast<const u16*>(p.z) : xg;
  const uint32_t zs_b = (uint32_t)(p.z ? p.z_stride : p.v_stride) * 2u;

  // ---------------------------------------------------------------- chunk loop
  if (c0 < c1) {
    stage(rs0, c0, kStAll);
    if (vwave) stage_gate(c0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0)
  if (vwave && c0 < c1) {
    make_vectors(c0, sm.vec[c0 & 1][wu - 6]);
    stage_gate(min(c0 + 1, c1 - 1));
  }
  if (kCk && ck_b >= 0 && ck_b == CS * c0 && ck_b < tend - tbeg) store_state(ck_st, Sacc);

  for (int c = c0; c < c1; ++c) {
    lane_s = lane;
    asm volatile("" : "+v"(lane_s));
    const int par = c & 1;
    const SsdVec& V = sm.vec[par][hs];
    const int t0 = tbeg + c * CS, n = min(CS, tend - t0);
    lds_sync();                              // the previous chunk's LDS reads are done
    land(rs0);
    // the epilogue's z of this chunk (its four slices), loaded after Y (the update, the
    // tiles and the intra-chunk term cover their latency)
    uint4 ez0, ez1, ez2, ez3;
    auto load_z = [&]() __attribute__((always_inline)) {
      const char* zb = reinterpret_cast<const char*>(zg + (int64_t)t0 * (zs_b / 2));
      auto ldz = [&](int i) __attribute__((always_inline)) {
        const int r = er + 64 * (i & 1);
        const uint32_t col = (uint32_t)((i >> 1 ? hB : hA) * PH + 8 * ek);
        return *reinterpret_cast<const uint4*>(zb + (uint32_t)(r < n ? r : 0) * zs_b + 2u * col);
      };
      ez0 = ldz(0); ez1 = ldz(1); ez2 = ldz(2); ez3 = ldz(3);
    };
    // this chunk's raw C B^T tiles (made into LDS tiles after the update; with
    // checkpoints, loaded after the in-chunk checkpoint, whose registers they would add to)
    uint4 td0, td1, to0 = {}, to1 = {};
    if constexpr (!kCk) load_tiles(c, td0, td1, to0, to1);
    // The next chunk's rows (staging loads are unconditional: past the last chunk they
    // re-read it).  The full pass spreads them over the step -- C rows after Y, B rows
    // after the tiles, x rows after the intra-chunk term -- so that the vector memory
    // pipeline streams them while the waves compute: issued in one burst here they
    // stalled every wave for ~3k cycles per chunk (about a seventh of the step).
    const int cn = min(c + 1, c1 - 1);
    if constexpr (!kFull) stage(rs0, cn, kStAll);
    lds_sync();                              // landing visible
    const float gamma = V.gC[0];
    if (vwave) {
      if (c + 1 < c1) make_vectors(c + 1, sm.vec[par ^ 1][wu - 6]);
      stage_gate(min(c + 2, c1 - 1));
    }
    if constexpr (kFull) {
      // Y^T = S0 C^T diag(e^G) over the chunk's 8 token tiles (k steps outermost: one
      // k step's S0 operand is live at a time)
      f32x4 Y[8];
#pragma unroll
      for (int it = 0; it < 8; ++it) Y[it] = f32x4{};
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const f16x8 sop = pair_to_op_h(Sacc[2 * s2], Sacc[2 * s2 + 1]);
#pragma unroll
        for (int it = 0; it < 8; ++it)
          Y[it] = mfma1632h(sop, as_f16x8(__builtin_bit_cast(uint4, ldq8<NS>(sm.C, 16 * it + j16, 32 * s2 + 8 * g16))), Y[it]);
      }
#pragma unroll
      for (int it = 0; it < 8; ++it) Y[it] = Y[it] * V.eG[16 * it + j16];
      load_z();
      stage(rs0, cn, kStC);
      // checkpoint inside the chunk, after its first m tokens:
      //   S_m^T = e^{G_{m-1}} S0^T + B^T diag(e^{G_{m-1} - G_i} dt'_i [i < m]) X
      if (kCk && ck_b > CS * c && ck_b < CS * c + n) {
        const int m = ck_b - CS * c;
        const float Gm2 = V.G2[m - 1];
        f32x4 Sc[8];
        f16x8 Wc[4];
#pragma unroll
        for (int tk = 0; tk < 8; ++tk) Sc[tk] = Sacc[tk];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          uint32_t w[4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            float f[2];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
              const int e = 2 * e2 + x;
              const int i = 32 * s2 + (e < 4 ? 4 * g16 + e : 16 + 4 * g16 + e - 4);
              f[x] = i < m ? __builtin_amdgcn_exp2f(Gm2 - V.G2[i]) * (float)__builtin_bit_cast(_Float16, V.dtp[i]) : 0.f;
            }
            w[e2] = cvt2h(f[0], f[1]);
          }
          Wc[s2] = scale_h(x_op(s2), make_uint4(w[0], w[1], w[2], w[3]));
        }
        update(Sc, __builtin_amdgcn_exp2f(Gm2), Wc);
        store_state(ck_st, Sc);
      }
      if constexpr (kCk) load_tiles(c, td0, td1, to0, to1);
      {
        f16x8 W[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) W[s2] = scale_h(x_op(s2), fac_op(V.wfac, s2));
        update(Sacc, gamma, W);
      }
      make_tiles(V, td0, td1, to0, to1);
      stage(rs0, cn, kStB);
      lds_sync();                            // P and C B^T tiles complete
      f16x8 xo[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) xo[s2] = x_op(s2);
      // Y^T += the intra-chunk term: diagonal block d = it / 2 from the head's P, the
      // blocks s2 < d from the raw C B^T tile with the decay factored at token 32 s2 + 31
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int d = it >> 1, row = 16 * it + j16, trow = 16 * (it & 1) + j16;
        const f16x8 ud = scale_h(xo[d], fac_op(V.dtp, d));
        Y[it] = mfma1632h(ud, as_f16x8(*reinterpret_cast<const uint4*>(sm.Pd[hs][d] + trow * kTP + 8 * g16)), Y[it]);
#pragma unroll
        for (int s2 = 0; s2 < d; ++s2) {
          const f16x8 uq = scale_h(xo[s2], fac_op(V.ufac, s2));
          const f32x4 t = mfma1632h(uq, as_f16x8(*reinterpret_cast<const uint4*>(sm.CB[d * (d - 1) / 2 + s2] + trow * kTP + 8 * g16)), f32x4{});
          Y[it] += t * __builtin_amdgcn_exp2f(V.G2[row] - V.G2[32 * s2 + 31]);
        }
      }
      // epilogue: every wave's y tiles into Yx (C and B are no longer read in this
      // chunk), then per slice (y + D x) silu(z) in whole rows; rows past the sequence
      // end are dropped by the bounded buffer stores (record = the chunk's n rows)
      stage(rs0, cn, kStX);
#pragma unroll
      for (int it = 0; it < 8; ++it)
        *reinterpret_cast<f32x4*>(&sm.Yx[hs][yidx(16 * it + j16, 4 * pt + g16)]) = Y[it];
      lds_sync();
      {
        char* obase = reinterpret_cast<char*>(p.out) + (int64_t)t0 * p.out_stride * (int64_t)sizeof(OutT);
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(obase, (short)0, (int)((uint32_t)n * ostride_b), kBufWord3);
        const uint4 ez[4] = {ez0, ez1, ez2, ez3};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int hsl = i >> 1, r = er + 64 * (i & 1);
          if (hsl == 1 && !two) continue;   // (a lone head: its mirror slot stores nothing)
          const f32x4 ya = *reinterpret_cast<const f32x4*>(&sm.Yx[hsl][yidx(r, 2 * ek)]);
          const f32x4 yb = *reinterpret_cast<const f32x4*>(&sm.Yx[hsl][yidx(r, 2 * ek + 1)]);
          const f32x4 da = *reinterpret_cast<const f32x4*>(&sm.Dv[hsl][8 * ek]);
          const f32x4 db = *reinterpret_cast<const f32x4*>(&sm.Dv[hsl][8 * ek + 4]);
          const uint4 xw = *reinterpret_cast<const uint4*>(sm.X[hsl] + pidx<PH>(r, 8 * ek));
          const uint32_t xs[4] = {xw.x, xw.y, xw.z, xw.w};
          const uint32_t zs[4] = {ez[i].x, ez[i].y, ez[i].z, ez[i].w};
          float y[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            y[e] = ya[e] + da[e] * (e & 1 ? h_hi(xs[e >> 1]) : h_lo(xs[e >> 1]));
            y[4 + e] = yb[e] + db[e] * (e & 1 ? h_hi(xs[2 + (e >> 1)]) : h_lo(xs[2 + (e >> 1)]));
          }
          if (p.z) {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] *= silu_f(e & 1 ? bf_hi(zs[e >> 1]) : bf_lo(zs[e >> 1]));
          }
          const int off = (int)((uint32_t)r * ostride_b + (uint32_t)(((hsl ? hB : hA) * PH + 8 * ek) * sizeof(OutT)));
          if constexpr (sizeof(OutT) == 2) {
            const u32x4 w = {cvt2(y[0], y[1]), cvt2(y[2], y[3]), cvt2(y[4], y[5]), cvt2(y[6], y[7])};
            __builtin_amdgcn_raw_buffer_store_b128(w, rs, off, 0, 0);
          } else {
            const u32x4 w0 = {__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])};
            const u32x4 w1 = {__float_as_uint(y[4]), __float_as_uint(y[5]), __float_as_uint(y[6]), __float_as_uint(y[7])};
            __builtin_amdgcn_raw_buffer_store_b128(w0, rs, off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(w1, rs, off + 16, 0, 0);
          }
        }
      }
      if (kCk && ck_b >= 0 && ck_b == CS * (c + 1) && ck_b < tend - tbeg) store_state(ck_st, Sacc);
    } else {
      f16x8 W[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) W[s2] = scale_h(x_op(s2), fac_op(V.wfac, s2));
      update(Sacc, gamma, W);
      lam += V.gC[1];
    }
  }

  if (!owner) return;
  if constexpr (kFull) {
    if (last_seg) {
      if (kCk && ck_b >= 0 && ck_b == tend - tbeg) store_state(ck_st, Sacc);
      if (!p.keep_pool) store_state(p.pool + ((int64_t)sl * p.H_v + h) * hstride, Sacc);
    }
  } else {
    const int64_t row = segbase + (int64_t)(seg * nsub + sub) * p.H_v + h;
    store_state(p.segR + row * hstride, Sacc);
    if (pt == 0 && lane == 0) p.segL[row] = lam;
  }
}

// Per chunk, once per call (every head of a group shares it): the fp16 copies of the
// chunk's B and C rows ([T, G, N] contiguous) and its raw C B^T tiles.  Workgroup =
// (chunk slot, group): the rows land converted in LDS and go out as the copies, then
// wave w computes the tiles w, w + 4, w + 8 from LDS.  Rows past the sequence end take
// the chunk's first row, as the chunk kernel's landing does (and are not copied out).
__global__ void __launch_bounds__(256) ssd_prep_kernel(SeqLaunch p) {
  __shared__ __attribute__((aligned(16))) u16 sC[CS * NS], sB[CS * NS];
  const int q = blockIdx.x, g = blockIdx.y;
  // the sequence whose chunk has slot q: the last s with cb_slot_base(tbeg_s, s) <= q
  int lo = 0, hi = p.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cb_slot_base(p.cu_seqlens[mid], mid) <= q) lo = mid; else hi = mid - 1;
  }
  const int s = lo, tbeg = p.cu_seqlens[s], len = p.cu_seqlens[s + 1] - tbeg;
  const int64_t c = q - cb_slot_base(tbeg, s);
  if (p.slot[s] < 0 || c < 0 || c * CS >= len) return;   // a slot no chunk has, or a skipped sequence
  const int t0 = tbeg + (int)c * CS, n = min(CS, len - (int)c * CS);
  const int tid = threadIdx.x;
  const u16* kin = reinterpret_cast<const u16*>(p.k) + (int64_t)g * NS;
  const u16* qin = reinterpret_cast<const u16*>(p.q) + (int64_t)g * NS;
  u16* bout = const_cast<u16*>(p.ssd_Bh) + (int64_t)g * NS;
  u16* cout = const_cast<u16*>(p.ssd_Ch) + (int64_t)g * NS;
  const int64_t rs = (int64_t)p.H_qk * NS;
  // 128 rows x 16 segments of 16 bytes per tile: 8 per thread and tile
  uint4 wb[8], wc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int sidx = tid + 256 * i, r = sidx >> 4, cs = sidx & 15;
    const int64_t t = t0 + (r < n ? r : 0);
    wb[i] = *reinterpret_cast<const uint4*>(kin + t * p.k_stride + 8 * cs);
    wc[i] = *reinterpret_cast<const uint4*>(qin + t * p.q_stride + 8 * cs);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int sidx = tid + 256 * i, r = sidx >> 4, cs = sidx & 15;
    const uint4 hb = make_uint4(bf2h(wb[i].x), bf2h(wb[i].y), bf2h(wb[i].z), bf2h(wb[i].w));
    const uint4 hc = make_uint4(bf2h(wc[i].x), bf2h(wc[i].y), bf2h(wc[i].z), bf2h(wc[i].w));
    *reinterpret_cast<uint4*>(sB + qidx<NS>(r, 8 * cs)) = hb;
    *reinterpret_cast<uint4*>(sC + qidx<NS>(r, 8 * cs)) = hc;
    if (r < n) {
      *reinterpret_cast<uint4*>(bout + (int64_t)(t0 + r) * rs + 8 * cs) = hb;
      *reinterpret_cast<uint4*>(cout + (int64_t)(t0 + r) * rs + 8 * cs) = hc;
    }
  }
  __syncthreads();
  const int lane = tid % kWave, w = tid / kWave;
  const int l32 = lane & 31, hh = lane >> 5;
  u16* dst = const_cast<u16*>(p.ssd_CB) + ((int64_t)q * p.H_qk + g) * (int64_t)(kCBTiles * kCBTileElems) + 16 * lane;
  for (int t = w; t < kCBTiles; t += 4) {
    const int ti = t < 6 ? offdiag_i(t) : t - 6, tm = t < 6 ? offdiag_m(t) : t - 6;
    f32x16 acc = {};
#pragma unroll
    for (int k = 0; k < NS / 16; ++k) {
      const f16x8 a = as_f16x8(__builtin_bit_cast(uint4, ldq8<NS>(sB, 32 * tm + l32, 16 * k + 8 * hh)));
      const f16x8 b = as_f16x8(__builtin_bit_cast(uint4, ldq8<NS>(sC, 32 * ti + l32, 16 * k + 8 * hh)));
      acc = mfma32h(a, b, acc);
    }
    uint32_t o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = cvt2h(acc[2 * k], acc[2 * k + 1]);
    *reinterpret_cast<uint4*>(dst + t * kCBTileElems) = make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4*>(dst + t * kCBTileElems + 8) = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

template <typename OutT, bool kGate, bool kCk>
hipError_t launch_ssd_typed(const SeqLaunch& p, hipStream_t stream) {
  if (p.T > 0) {
    hipLaunchKernelGGL(ssd_prep_kernel, dim3((unsigned)(p.T / CS + p.N), (unsigned)p.H_qk), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const unsigned gx = (unsigned)ssd_units_per_seq(p);
  if (p.ssd_segs > 1) {
    hipLaunchKernelGGL((ssd_kernel<OutT, kGate, false, false>), dim3(gx, p.N * (p.ssd_segs - 1) * p.ssd_sub),
                       dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((ssd_kernel<OutT, kGate, true, kCk>), dim3(gx, p.N * p.ssd_segs), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename OutT, bool kGate>
hipError_t launch_ssd_ck(const SeqLaunch& p, hipStream_t stream) {
  return p.ck_token ? launch_ssd_typed<OutT, kGate, true>(p, stream)
                    : launch_ssd_typed<OutT, kGate, false>(p, stream);
}

}  // namespace

// Workspace of a chunk-128 delta-off call with `states` state-only pieces per sequence
// ((segments - 1) x pieces per segment; 0 for one segment): the fp16 copies of B and C,
// the raw C B^T tiles of every chunk slot, then the pieces' states and log decays.
int64_t ssd_workspace_bytes(int64_t T, int N, int H_qk, int H_v, int states) {
  auto up = [](int64_t b) { return (b + 255) & ~int64_t(255); };
  const int64_t bc = up(T * H_qk * NS * 2);
  const int64_t cb = up((T / CS + N) * H_qk * kCBTiles * kCBTileElems * 2);
  const int64_t r = up((int64_t)N * states * H_v * PH * NS * 4);
  const int64_t l = up((int64_t)N * states * H_v * 4);
  return 2 * bc + cb + r + l;
}

void ssd_bind_workspace(SeqLaunch& p, void* ws) {
  auto up = [](int64_t b) { return (b + 255) & ~int64_t(255); };
  char* base = static_cast<char*>(ws);
  const int64_t bc = up(p.T * p.H_qk * NS * 2);
  const int64_t cb = up((p.T / CS + p.N) * p.H_qk * kCBTiles * kCBTileElems * 2);
  p.ssd_Bh = reinterpret_cast<const u16*>(base);
  p.ssd_Ch = reinterpret_cast<const u16*>(base + bc);
  p.ssd_CB = reinterpret_cast<const u16*>(base + 2 * bc);
  p.segR = reinterpret_cast<float*>(base + 2 * bc + cb);
  p.segL = reinterpret_cast<float*>(base + 2 * bc + cb + up((int64_t)p.N * (p.ssd_segs - 1) * p.ssd_sub * p.H_v * PH * NS * 4));
}

bool ssd_chunked_shape(const SeqLaunch& p) { return p.ssd && p.d_k == NS && p.d_v == PH; }

// Workgroups per sequence and segment: the head pairs of every group.
int ssd_units_per_seq(const SeqLaunch& p) { return p.H_qk * ((p.H_v / p.H_qk + 1) / 2); }

int ssd_obstacles(const SeqLaunch& p) {
  int why = 0;
  if (!p.in_bf16) why |= GDN_WHY_FP32;
  if (!ssd_chunked_shape(p)) why |= GDN_WHY_HEAD_DIMS;
  if (p.N > 65535) why |= GDN_WHY_BATCH;
  // B, C (prep kernel), x and z rows are read, and the output rows written, as 16-byte
  // segments
  const uintptr_t ptrs = reinterpret_cast<uintptr_t>(p.q) | reinterpret_cast<uintptr_t>(p.k) |
                         reinterpret_cast<uintptr_t>(p.v) | reinterpret_cast<uintptr_t>(p.z) |
                         reinterpret_cast<uintptr_t>(p.out);
  const int64_t out_elems16 = p.out_bf16 ? 8 : 4;   // output elements per 16 bytes
  if (ptrs % 16 != 0 || (p.q_stride | p.k_stride | p.v_stride | (p.z ? p.z_stride : 0)) % 8 != 0 ||
      p.out_stride % out_elems16 != 0)
    why |= GDN_WHY_ALIGN;
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
