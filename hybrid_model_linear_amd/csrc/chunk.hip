// Chunked GDN extend kernel (bf16 inputs, fp32 state), MFMA bf16 -> fp32 on gfx950.
//
// Chunked form of the gated delta rule (Gated DeltaNet, ICLR 2025; the WY / UT
// representation of products of generalised Householder transitions).  Within a
// chunk of C = 64 tokens, with raw bf16 rows q_i, k_i, v_i, row norms
// r_q,i = 1/|q_i|, r_k,i = 1/|k_i|, G_i = sum_{m<=i} log g_m, gamma_i = exp(G_i),
// Gam_im = exp(G_i - G_m) (m <= i, masked before the exp) and the chunk's entry state S0:
//
//   A  = strict_lower( beta_i r_k,i r_k,m Gam_im (K K^T)_im ),   T = (I + A)^{-1}
//   X  = K S0^T,   R = diag(beta) V - diag(beta gamma r_k) X      (first-order innovations)
//   U  = T R = R + (T - I) R                                       (delta-rule corrected values)
//   O  = diag(scale gamma r_q) Q S0^T + P U,  P = lower( scale r_q,i r_k,m Gam_im (Q K^T)_im )
//   S1 = gamma_C S0 + U^T diag(exp(G_C - G_i) r_k,i) K
//
// Delta-off mode (Mamba2 SSD, flashinfer.mamba.ssd_combined_fwd): no norms, T = I,
// U = diag(dt') X, scale 1, then O += D x and O *= silu(z).
//
// Precision layout: q, k, v enter the MFMAs as their exact bf16 values; norms,
// beta and decays are fp32 row/column scalings applied after the products; S0 and
// (T - I) R are single bf16 operands; P U and the state update use two-term
// (hi + lo) bf16 splits of P, U and the scaled U.
//
// Work split: one workgroup per (sequence, v-head) walks the sequence's chunks in
// order; the state never leaves registers.  Phase A (all waves, independent of
// the state) stages Q, K, K^T, V^T in LDS and builds P and T - I; phase B gives
// each wave 32 of the d_v columns: state rows are independent given the chunk's
// keys, so the waves never exchange data there.  The state is held as S^T tiles in
// MFMA accumulator layout and fed back as B operands without any data movement:
// the reduction index of a 32x32x16 MFMA may be permuted freely as long as both
// operands agree, so A operands are read from LDS in the accumulator's row order.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int C = 64;            // chunk length
constexpr int kQS = 8;           // row padding (bf16 elements) of row-major tiles
constexpr int kTS = C + 8;       // row length of transposed tiles [d][token]
constexpr int kPS = C + 8;       // row length of C x C bf16 tiles

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 consecutive bf16 (16 B) from LDS: operand in natural k order.
__device__ __forceinline__ bf16x8 lds_nat(const u16* p) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(p));
}
// Operand in accumulator row order: k slots e = 0..3 at p[0..3], e = 4..7 at p[8..11]
// (p already offset by 16 s + 4 hh).
__device__ __forceinline__ bf16x8 lds_perm(const u16* p) {
  const uint2 lo = *reinterpret_cast<const uint2*>(p);
  const uint2 hi = *reinterpret_cast<const uint2*>(p + 8);
  return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}
// Accumulator half (elements 8 half .. 8 half + 7) as a bf16 operand.
__device__ __forceinline__ bf16x8 acc_to_op(const f32x16& a, int half) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)a[8 * half + e];
  return r;
}
__device__ __forceinline__ void acc_split(const f32x16& a, int half, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = a[8 * half + e];
    const __bf16 h = (__bf16)x;
    hi[e] = h;
    lo[e] = (__bf16)(x - (float)h);
  }
}
// Row (token / d_k index) of accumulator element r held by lane half hh, tile origin 0.
__device__ __forceinline__ int acc_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x4 lds4(const u16* p) {
  return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(p));
}

template <int DK, int DV, bool kSSD>
struct Smem {
  u16 Q[C][DK + kQS];          // raw q rows (bf16)
  u16 K[C][DK + kQS];          // raw k rows
  u16 KT[DK][kTS];             // k transposed [d_k][token]
  u16 VT[DV][kTS];             // v transposed [d_v][token]
  u16 Ph[C][kPS];              // P = hi + lo
  u16 Pl[C][kPS];
  u16 AB[kSSD ? 1 : C][kPS];   // bf16(A), strictly lower
  u16 Tb[kSSD ? 1 : C][kPS];   // bf16(T), unit lower, row-major
  u16 TT[kSSD ? 1 : C][kPS];   // bf16(T) transposed (column access)
  float Ad[kSSD ? 1 : 4][16][17];  // fp32 diagonal 16x16 blocks of A
  float G[C];
  float beta[C];
  float rk[C];
  float rq[C];
  float coefR[C];
  float coefO[C];
  float coefS[C];
};

// ------------------------------------------------------------------ phase A pieces
// Raw chunk data held in registers between its global load (issued one chunk
// ahead, so that it is in flight during the previous chunk's phase B) and its
// store into LDS.
template <int DK, int DV, int NT>
struct ChunkRegs {
  static constexpr int QK_IT = (C / 2) * (DK / 8) / NT;
  static constexpr int V_IT = (C / 2) * (DV / 8) / NT;
  static_assert(QK_IT * NT == (C / 2) * (DK / 8) && V_IT * NT == (C / 2) * (DV / 8), "split");
  uint4 q[QK_IT][2], k[QK_IT][2], v[V_IT][2];
  float lg, bt;
};

template <int DK, int DV, int NT>
__device__ __forceinline__ void load_chunk(ChunkRegs<DK, DV, NT>& R, const SeqLaunch& p, int h, int j,
                                           int t0, int n) {
  const int tid = threadIdx.x;
  const u16* qb = reinterpret_cast<const u16*>(p.q);
  const u16* kb = reinterpret_cast<const u16*>(p.k);
  const u16* vb = reinterpret_cast<const u16*>(p.v);
  const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int it = 0; it < R.QK_IT; ++it) {
    const int idx = tid + it * NT;
    const int pr = idx % (C / 2), cg = idx / (C / 2);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 2 * pr + u;
      const int64_t t = t0 + i;
      R.q[it][u] = i < n ? *reinterpret_cast<const uint4*>(qb + t * p.q_stride + (int64_t)j * DK + 8 * cg) : z;
      R.k[it][u] = i < n ? *reinterpret_cast<const uint4*>(kb + t * p.k_stride + (int64_t)j * DK + 8 * cg) : z;
    }
  }
#pragma unroll
  for (int it = 0; it < R.V_IT; ++it) {
    const int idx = tid + it * NT;
    const int pr = idx % (C / 2), cg = idx / (C / 2);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 2 * pr + u;
      R.v[it][u] = i < n ? *reinterpret_cast<const uint4*>(vb + (int64_t)(t0 + i) * p.v_stride + (int64_t)h * DV + 8 * cg) : z;
    }
  }
  R.lg = 0.f;
  R.bt = 0.f;
  if (tid < n) {                     // padded tokens: log g = 0, beta = 0 (no effect)
    const int64_t gi = (int64_t)(t0 + tid) * p.H_v + h;
    R.lg = p.log_g[gi];
    R.bt = p.beta[gi];
  }
}

template <int DK, int DV, bool kSSD, int NT>
__device__ __forceinline__ void store_chunk(Smem<DK, DV, kSSD>& sm, const ChunkRegs<DK, DV, NT>& R) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < R.QK_IT; ++it) {
    const int idx = tid + it * NT;
    const int pr = idx % (C / 2), cg = idx / (C / 2);
    const int i0 = 2 * pr;
    *reinterpret_cast<uint4*>(&sm.Q[i0][8 * cg]) = R.q[it][0];
    *reinterpret_cast<uint4*>(&sm.Q[i0 + 1][8 * cg]) = R.q[it][1];
    *reinterpret_cast<uint4*>(&sm.K[i0][8 * cg]) = R.k[it][0];
    *reinterpret_cast<uint4*>(&sm.K[i0 + 1][8 * cg]) = R.k[it][1];
    const uint32_t a0[4] = {R.k[it][0].x, R.k[it][0].y, R.k[it][0].z, R.k[it][0].w};
    const uint32_t a1[4] = {R.k[it][1].x, R.k[it][1].y, R.k[it][1].z, R.k[it][1].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {   // two tokens per 32-bit write of the transposed tile
      *reinterpret_cast<uint32_t*>(&sm.KT[8 * cg + 2 * e][i0]) = (a0[e] & 0xffffu) | (a1[e] << 16);
      *reinterpret_cast<uint32_t*>(&sm.KT[8 * cg + 2 * e + 1][i0]) = (a0[e] >> 16) | (a1[e] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int it = 0; it < R.V_IT; ++it) {
    const int idx = tid + it * NT;
    const int pr = idx % (C / 2), cg = idx / (C / 2);
    const int i0 = 2 * pr;
    const uint32_t a0[4] = {R.v[it][0].x, R.v[it][0].y, R.v[it][0].z, R.v[it][0].w};
    const uint32_t a1[4] = {R.v[it][1].x, R.v[it][1].y, R.v[it][1].z, R.v[it][1].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      *reinterpret_cast<uint32_t*>(&sm.VT[8 * cg + 2 * e][i0]) = (a0[e] & 0xffffu) | (a1[e] << 16);
      *reinterpret_cast<uint32_t*>(&sm.VT[8 * cg + 2 * e + 1][i0]) = (a0[e] >> 16) | (a1[e] & 0xffff0000u);
    }
  }
  if (tid < C) {
    sm.G[tid] = R.lg;
    sm.beta[tid] = R.bt;
  }
}

// Row norms (GDN), in-chunk cumulative decay and the per-token coefficients.
template <int DK, int DV, bool kSSD, int NT>
__device__ __forceinline__ void chunk_scalars(Smem<DK, DV, kSSD>& sm, float scale, int n,
                                              float& gL) {
  const int tid = threadIdx.x;
  if constexpr (!kSSD) {
    // 2 C rows (q and k), NT / (2C) threads per row.
    constexpr int TPR = NT / (2 * C);
    static_assert(TPR >= 1 && (TPR & (TPR - 1)) == 0, "threads per row");
    const int row = tid / TPR, part = tid % TPR;
    const u16* src = row < C ? &sm.Q[row][0] : &sm.K[row - C][0];
    float ss = 0.f;
#pragma unroll
    for (int c8 = part; c8 < DK / 8; c8 += TPR) {
      const uint4 w = *reinterpret_cast<const uint4*>(src + 8 * c8);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(ws[e] << 16), hi = __uint_as_float(ws[e] & 0xffff0000u);
        ss += lo * lo + hi * hi;
      }
    }
    ss = group_sum<TPR>(ss);
    if (part == 0) {
      const int i = row % C;
      const float r = i < n ? 1.0f / sqrtf(ss + 1e-6f) : 0.f;
      if (row < C) sm.rq[i] = r; else sm.rk[i] = r;
    }
  } else {
    if (tid < C) {
      const float r = tid < n ? 1.f : 0.f;
      sm.rq[tid] = r;
      sm.rk[tid] = r;
    }
  }
  __syncthreads();
  // inclusive prefix sum of log g over the chunk (wave 0, lane = token)
  if (tid < C) {
    float Gi = sm.G[tid];
#pragma unroll
    for (int off = 1; off < C; off <<= 1) {
      const float o = __shfl_up(Gi, off, kWave);
      if (tid >= off) Gi += o;
    }
    const float GL = __shfl(Gi, C - 1, kWave);
    const float gam = __expf(Gi);
    const float bt = sm.beta[tid], rk = sm.rk[tid], rq = sm.rq[tid];
    sm.G[tid] = Gi;
    sm.coefR[tid] = bt * gam * rk;
    sm.coefO[tid] = scale * gam * rq;
    sm.coefS[tid] = __expf(GL - Gi) * rk;
  }
  __syncthreads();
  gL = sm.G[C - 1];
}

// Q K^T and K K^T tiles of the lower block triangle (32x32 tiles (0,0), (1,0), (1,1));
// one wave per tile computes both products and shares the decay factors:
//   P_im = scale r_q,i r_k,m Gam_im (Q K^T)_im  (m <= i)      -> Ph + Pl (bf16 split)
//   A_im = beta_i r_k,i r_k,m Gam_im (K K^T)_im (m <  i)      -> AB (bf16), Ad (fp32 diag blocks)
template <int DK, int DV, bool kSSD, int NW>
__device__ __forceinline__ void build_A_P(Smem<DK, DV, kSSD>& sm, float scale) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int l32 = lane & 31, hh = lane >> 5;
  for (int tt = w; tt < 3; tt += NW) {
    const int ti = tt == 0 ? 0 : 1, tj = tt == 2 ? 1 : 0;
    const u16* qrow = &sm.Q[32 * ti + l32][8 * hh];
    const u16* krow = &sm.K[32 * ti + l32][8 * hh];
    const u16* brow = &sm.K[32 * tj + l32][8 * hh];
    f32x16 qk = {}, kk = {};
#pragma unroll
    for (int s = 0; s < DK / 16; ++s) {
      const bf16x8 b = lds_nat(brow + 16 * s);
      qk = mfma32(lds_nat(qrow + 16 * s), b, qk);
      if constexpr (!kSSD) kk = mfma32(lds_nat(krow + 16 * s), b, kk);
    }
    const int m = 32 * tj + l32;                 // key token (column)
    const float Gm = sm.G[m], rkm = sm.rk[m];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int ib = 32 * ti + 8 * q4 + 4 * hh;
      const float4 Gi = *reinterpret_cast<const float4*>(&sm.G[ib]);
      const float4 rqi = *reinterpret_cast<const float4*>(&sm.rq[ib]);
      const float4 rki = *reinterpret_cast<const float4*>(&sm.rk[ib]);
      const float4 bi = *reinterpret_cast<const float4*>(&sm.beta[ib]);
      const float Gv[4] = {Gi.x, Gi.y, Gi.z, Gi.w}, rqv[4] = {rqi.x, rqi.y, rqi.z, rqi.w};
      const float rkv[4] = {rki.x, rki.y, rki.z, rki.w}, bv[4] = {bi.x, bi.y, bi.z, bi.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * q4 + e, i = ib + e;
        const float gam = m <= i ? __expf(Gv[e] - Gm) : 0.f;    // masked before the exp
        const float pv = kSSD ? gam * qk[r] : scale * rqv[e] * rkm * gam * qk[r];
        const __bf16 ph = (__bf16)pv;
        sm.Ph[i][m] = __builtin_bit_cast(u16, ph);
        sm.Pl[i][m] = f32_to_bf16(pv - (float)ph);
        if constexpr (!kSSD) {
          const float av = m < i ? bv[e] * rkv[e] * rkm * gam * kk[r] : 0.f;
          sm.AB[i][m] = f32_to_bf16(av);
          if ((i >> 4) == (m >> 4)) sm.Ad[i >> 4][i & 15][m & 15] = av;
        }
      }
    }
  }
  if constexpr (!kSSD) {
    if (w == NW - 1) {
      // zero the upper 16x16 blocks inside the two diagonal 32x32 tiles of T and T^T
      const int blk = lane >> 4, row = lane & 15;
      u16* dst = blk == 0 ? &sm.Tb[row][16] : blk == 1 ? &sm.Tb[32 + row][48]
               : blk == 2 ? &sm.TT[16 + row][0] : &sm.TT[48 + row][32];
      *reinterpret_cast<uint4*>(dst) = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(dst + 8) = make_uint4(0, 0, 0, 0);
    }
  }
}

// T = (I + A)^{-1} for strictly lower A, in bf16 (unit diagonal), by 16 -> 32 -> 64
// block doubling: diagonal 16x16 blocks by fp32 forward substitution, then
// T_ab = -T_bb^{-1}... merged as T21 = -T22 (A21 T11) with MFMAs.  T - I only
// enters the chunk as a correction term whose operand is bf16 already.
template <int DK, int DV, int NW>
__device__ __forceinline__ void invert_unit_lower(Smem<DK, DV, false>& sm) {
  static_assert(NW >= 2, "needs two waves");
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  // (1) diagonal blocks: wave w < 4 solves block w; lane c < 16 owns column c
  for (int b = w; b < 4; b += NW) {
    if (lane < 16) {
      const int c = lane;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (i == c) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int mm = i + 1; mm < 16; ++mm) x[mm] -= sm.Ad[b][mm][i] * x[i];
      }
      uint32_t pk[8];
#pragma unroll
      for (int i = 0; i < 16; ++i) sm.Tb[16 * b + i][16 * b + c] = f32_to_bf16(x[i]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pk[i] = uint32_t(f32_to_bf16(x[2 * i])) | (uint32_t(f32_to_bf16(x[2 * i + 1])) << 16);
      *reinterpret_cast<uint4*>(&sm.TT[16 * b + c][16 * b]) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      *reinterpret_cast<uint4*>(&sm.TT[16 * b + c][16 * b + 8]) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
    }
  }
  __syncthreads();
  // (2) 16 -> 32: inside diagonal 32x32 tile pp, T[16..31][0..15] = -D1^{-1} (A10 D0^{-1})
  if (w < 2) {
    const int pp = w, c = lane & 15, g = lane >> 4;
    const int r0 = 32 * pp;
    f32x4 y = {};
    y = mfma16(lds4(&sm.AB[r0 + 16 + c][r0 + 4 * g]), lds4(&sm.TT[r0 + c][r0 + 4 * g]), y);
    bf16x4 yb;
#pragma unroll
    for (int e = 0; e < 4; ++e) yb[e] = (__bf16)y[e];
    f32x4 zz = {};
    zz = mfma16(lds4(&sm.Tb[r0 + 16 + c][r0 + 16 + 4 * g]), yb, zz);
    // zz: lane holds rows 4g .. 4g+3 of column c
    uint32_t pk[2];
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.Tb[r0 + 16 + 4 * g + e][r0 + c] = f32_to_bf16(-zz[e]);
    pk[0] = uint32_t(f32_to_bf16(-zz[0])) | (uint32_t(f32_to_bf16(-zz[1])) << 16);
    pk[1] = uint32_t(f32_to_bf16(-zz[2])) | (uint32_t(f32_to_bf16(-zz[3])) << 16);
    *reinterpret_cast<uint2*>(&sm.TT[r0 + c][r0 + 16 + 4 * g]) = make_uint2(pk[0], pk[1]);
  }
  __syncthreads();
  // (3) 32 -> 64: T[32..63][0..31] = -T22 (A21 T11)
  if (w == 0) {
    const int l32 = lane & 31, hh = lane >> 5;
    f32x16 y = {};
#pragma unroll
    for (int s = 0; s < 2; ++s)
      y = mfma32(lds_nat(&sm.AB[32 + l32][16 * s + 8 * hh]), lds_nat(&sm.TT[l32][16 * s + 8 * hh]), y);
    f32x16 zz = {};
#pragma unroll
    for (int s = 0; s < 2; ++s)
      zz = mfma32(lds_perm(&sm.Tb[32 + l32][32 + 16 * s + 4 * hh]), acc_to_op(y, s), zz);
#pragma unroll
    for (int r = 0; r < 16; ++r) sm.Tb[32 + acc_row(r, hh)][l32] = f32_to_bf16(-zz[r]);
  }
}

template <int DK, int DV, bool kSSD, typename OutT>
__global__ void __launch_bounds__((DV / 32) * kWave, 1) chunk_kernel(SeqLaunch p) {
  constexpr int NW = DV / 32;
  constexpr int NT = NW * kWave;
  constexpr int NKS = DK / 16;     // k-steps over d_k
  constexpr int NTK = DK / 32;     // S^T row tiles
  __shared__ Smem<DK, DV, kSSD> sm;

  const int h = blockIdx.x;
  const int nseq = blockIdx.y;
  const int sl = p.slot[nseq];
  if (sl < 0) return;                                      // uniform over the block
  const int tbeg = p.cu_seqlens[nseq], tend = p.cu_seqlens[nseq + 1];
  const bool init = p.has_init ? (p.has_init[nseq] != 0) : true;
  const int j = h / (p.H_v / p.H_qk);

  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int l32 = lane & 31, hh = lane >> 5;
  const int col = 32 * w + l32;                            // this lane's d_v column

  float* state = p.pool + ((int64_t)sl * p.H_v + h) * (int64_t)(DV * DK);
  f32x16 Sacc[NTK];
#pragma unroll
  for (int tk = 0; tk < NTK; ++tk) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (init) v = *reinterpret_cast<const float4*>(state + (int64_t)col * DK + 32 * tk + 8 * q4 + 4 * hh);
      Sacc[tk][4 * q4 + 0] = v.x;
      Sacc[tk][4 * q4 + 1] = v.y;
      Sacc[tk][4 * q4 + 2] = v.z;
      Sacc[tk][4 * q4 + 3] = v.w;
    }
  }

  OutT* ob = reinterpret_cast<OutT*>(p.out);

  ChunkRegs<DK, DV, NT> pre;
  if (tbeg < tend) load_chunk<DK, DV, NT>(pre, p, h, j, tbeg, min(C, tend - tbeg));

  for (int t0 = tbeg; t0 < tend; t0 += C) {
    const int n = min(C, tend - t0);
    __syncthreads();                                       // previous chunk's readers done
    store_chunk<DK, DV, kSSD, NT>(sm, pre);
    __syncthreads();
    float gL;
    chunk_scalars<DK, DV, kSSD, NT>(sm, p.scale, n, gL);
    build_A_P<DK, DV, kSSD, NW>(sm, p.scale);
    __syncthreads();
    if constexpr (!kSSD) {
      invert_unit_lower<DK, DV, NW>(sm);
      __syncthreads();
    }
    // next chunk's raw data: in flight while this chunk's phase B runs
    if (t0 + C < tend) load_chunk<DK, DV, NT>(pre, p, h, j, t0 + C, min(C, tend - t0 - C));

    // ---------------- phase B: this wave's 32 d_v columns
    bf16x8 Sb[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) Sb[s] = acc_to_op(Sacc[s >> 1], s & 1);

    f32x16 Y[2], U[2];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      Y[ti] = f32x16{};
      U[ti] = f32x16{};
      const u16* qrow = &sm.Q[32 * ti + l32][4 * hh];
      const u16* krow = &sm.K[32 * ti + l32][4 * hh];
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        Y[ti] = mfma32(lds_perm(qrow + 16 * s), Sb[s], Y[ti]);
        if constexpr (!kSSD) U[ti] = mfma32(lds_perm(krow + 16 * s), Sb[s], U[ti]);   // X = K S0^T
      }
    }
    // R = beta V - coefR X  (GDN),  U = beta V (delta-off); kept in U
    float vkeep[kSSD ? 2 : 1][kSSD ? 16 : 1];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int i0 = 32 * ti + 8 * q4 + 4 * hh;
        const uint2 vw = *reinterpret_cast<const uint2*>(&sm.VT[col][i0]);
        const float vv[4] = {__uint_as_float(vw.x << 16), __uint_as_float(vw.x & 0xffff0000u),
                             __uint_as_float(vw.y << 16), __uint_as_float(vw.y & 0xffff0000u)};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q4 + e, i = i0 + e;
          if constexpr (kSSD) {
            U[ti][r] = sm.beta[i] * vv[e];
            vkeep[ti][r] = vv[e];
          } else {
            U[ti][r] = sm.beta[i] * vv[e] - sm.coefR[i] * U[ti][r];
          }
        }
      }
    }
    if constexpr (!kSSD) {
      // U = R + (T - I) bf16(R) = (R - bf16(R)) + T bf16(R); T is unit lower, so row
      // tile 0 needs k-steps 0..1 only
      bf16x8 Rb[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) Rb[s] = acc_to_op(U[s >> 1], s & 1);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int e = 0; e < 8; ++e) U[s >> 1][8 * (s & 1) + e] -= (float)Rb[s][e];
      }
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        const u16* trow = &sm.Tb[32 * ti + l32][4 * hh];
#pragma unroll
        for (int s = 0; s < 2 * (ti + 1); ++s) U[ti] = mfma32(lds_perm(trow + 16 * s), Rb[s], U[ti]);
      }
    }
    // O = coefO Y + P U with two-term splits of P and U
    {
      bf16x8 Uh[4], Ul[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) acc_split(U[s >> 1], s & 1, Uh[s], Ul[s]);
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
#pragma unroll
        for (int r = 0; r < 16; ++r) Y[ti][r] *= sm.coefO[32 * ti + acc_row(r, hh)];
        const u16* phrow = &sm.Ph[32 * ti + l32][4 * hh];
        const u16* plrow = &sm.Pl[32 * ti + l32][4 * hh];
#pragma unroll
        for (int s = 0; s < 2 * (ti + 1); ++s) {
          const bf16x8 ph = lds_perm(phrow + 16 * s), pl = lds_perm(plrow + 16 * s);
          Y[ti] = mfma32(ph, Uh[s], Y[ti]);
          Y[ti] = mfma32(pl, Uh[s], Y[ti]);
          Y[ti] = mfma32(ph, Ul[s], Y[ti]);
        }
      }
    }
    // epilogue and store of this chunk's outputs
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 32 * ti + acc_row(r, hh);
        if (i < n) {
          float o = Y[ti][r];
          const int64_t tok = t0 + i;
          if constexpr (kSSD) {
            const u16* Db = reinterpret_cast<const u16*>(p.D);
            if (Db) o += bf16_to_f32(Db[p.D_per_dim ? (int64_t)h * DV + col : (int64_t)h]) * vkeep[ti][r];
            if (p.z) {
              const float zz = bf16_to_f32(reinterpret_cast<const u16*>(p.z)[tok * p.z_stride + (int64_t)h * DV + col]);
              o *= zz * sigmoid_f(zz);
            }
          }
          Elem<OutT>::store(ob, tok * p.out_stride + (int64_t)h * DV + col, o);
        }
      }
    }
    // state update: S^T = gamma_C S^T + K^T diag(coefS) U  (split hi + lo)
    {
      bf16x8 Wh[4], Wl[4];
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
#pragma unroll
        for (int r = 0; r < 16; ++r) U[ti][r] *= sm.coefS[32 * ti + acc_row(r, hh)];
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) acc_split(U[s >> 1], s & 1, Wh[s], Wl[s]);
      const float gC = __expf(gL);
#pragma unroll
      for (int tk = 0; tk < NTK; ++tk) {
        Sacc[tk] *= gC;
        const u16* krow = &sm.KT[32 * tk + l32][4 * hh];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 kt = lds_perm(krow + 16 * s);
          Sacc[tk] = mfma32(kt, Wh[s], Sacc[tk]);
          Sacc[tk] = mfma32(kt, Wl[s], Sacc[tk]);
        }
      }
    }
  }

#pragma unroll
  for (int tk = 0; tk < NTK; ++tk) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 v = make_float4(Sacc[tk][4 * q4 + 0], Sacc[tk][4 * q4 + 1], Sacc[tk][4 * q4 + 2],
                                   Sacc[tk][4 * q4 + 3]);
      *reinterpret_cast<float4*>(state + (int64_t)col * DK + 32 * tk + 8 * q4 + 4 * hh) = v;
    }
  }
}

template <int DK, int DV, bool kSSD, typename OutT>
hipError_t launch_typed(const SeqLaunch& p, hipStream_t stream) {
  dim3 grid(p.H_v, p.N), block((DV / 32) * kWave);
  hipLaunchKernelGGL((chunk_kernel<DK, DV, kSSD, OutT>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_dims(const SeqLaunch& p, hipStream_t stream) {
  if (p.ssd) return p.out_bf16 ? launch_typed<DK, DV, true, u16>(p, stream)
                               : launch_typed<DK, DV, true, float>(p, stream);
  return p.out_bf16 ? launch_typed<DK, DV, false, u16>(p, stream)
                    : launch_typed<DK, DV, false, float>(p, stream);
}

}  // namespace

bool chunked_supported(const SeqLaunch& p) {
  return p.in_bf16 && p.d_k == 128 && (p.d_v == 128 || p.d_v == 64) && p.N <= 65535;
}

hipError_t launch_chunked(const SeqLaunch& p, hipStream_t stream) {
  if (p.N == 0) return hipSuccess;
  if (p.d_k == 128 && p.d_v == 128) return launch_dims<128, 128>(p, stream);
  if (p.d_k == 128 && p.d_v == 64) return launch_dims<128, 64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
