// Chunked GDN extend kernel (bf16 inputs, fp32 state), MFMA bf16/fp16 -> fp32 on gfx950.
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
// Precision.  T = (I + A)^{-1} is built and kept in fp16 in both (A and T entries
// are bounded by one in magnitude: decays <= 1, beta <= 1, unit keys), with its
// diagonal blocks solved in fp32 and the merges on fp16 MFMAs.  bf16 output: q and k
// land in LDS normalised, Q^ = diag(r_q) Q and K^ = diag(r_k) K in fp16, and every
// product takes them, S0, R, P, U and the scaled U of the state update as single
// fp16 operands (each bounded by construction or by the values; fp16's 11-bit
// significand keeps every product's rounding below the output's bf16 rounding).  fp32
// output: q, k, v enter the MFMAs as their exact bf16 values, norms, beta and decays
// are fp32 scalings around the products, and S0, T - I, R, P, U and the state update
// use two-term (hi + lo) bf16 splits.  The delta-off mode (no T) takes S0 as a single
// bf16 operand.
//
// Work split: one workgroup per (sequence, v-head) walks the sequence's chunks in
// order.  Two kinds of waves run side by side:
//  * state waves own 32 d_v columns each (16 in delta-off mode; state rows are
//    independent given the chunk's keys); the state never leaves their registers,
//    held as S^T tiles in 16x16 MFMA accumulator layout and fed back as B operands
//    directly (the reduction index of an MFMA may be permuted freely when both
//    operands agree, so the accumulator's rows are ordered to match the A operands'
//    reads from LDS).  In the step for chunk c they compute X, Y, R, U, O and the new
//    state: only the state-dependent part, with no barrier inside.
//  * four producer waves run meanwhile on chunk c + 1: the Q K^T and K K^T tiles,
//    decay cumsum and the per-token coefficient vectors, P and A, the diagonal
//    blocks of T = (I + A)^{-1}; and, early in step c, the merges that finish chunk
//    c's T.
// The raw rows of q, k, v (z) are staged from HBM through registers into LDS one
// step ahead; the row norms of q and k are taken from the registers as they land.
// Each step has one workgroup barrier, which ends the previous step; the landing of
// the staged rows that follows, like every other hand-off, is announced on an LDS
// arrival counter, so the state waves start on chunk c (its Q and K landed a step
// earlier) while it is under way.  P, T and the coefficients are double-buffered,
// and so are Q and K (chunk c for the state waves, c + 1 for the producers).
//
// Data layout in LDS: tiles are row-major; V, Z and the C x C tiles padded per row,
// Q and K unpadded with swizzled 16-byte chunks.  K^T and V^T operands come from the
// row-major tiles through the LDS transpose read (ds_read_b64_tr_b16): lane j of each
// 16-lane group receives column c0 + j of the four rows addressed by the group's
// lanes 4e + j/4.
#include "gdn_common.h"
#include "gdn_launch.h"
#include "tile_ops.h"

namespace gdn {

namespace {

constexpr int C = 64;            // chunk length
constexpr int kPS = C + 4;       // row length (bf16) of the padded C x C tiles: 34 dwords,
                                 // so 16 consecutive rows hit distinct bank pairs
constexpr int kNP = 4;           // producer waves

// The C x C operand tiles keep each 32-column block with its 4-column groups in the
// order 0, 4, 1, 5, 2, 6, 3, 7, so that the 8 k slots of a 16x16x32 MFMA operand
// (columns 4g .. 4g+3 and 16+4g .. 16+4g+3 of a block, the order of the accumulator
// rows) are 16 contiguous bytes.  Logical column -> stored column:
__device__ __forceinline__ int kperm(int c) {
  const int q = (c >> 2) & 7;
  return (c & ~31) | ((2 * (q & 3) + (q >> 2)) << 2) | (c & 3);
}

// ------------------------------------------------------------------ chunk staging
// The waves of one role (NST threads, staging index si) load a chunk's q, k or v
// (and z) rows into registers one step before they store them into LDS, so the HBM
// latency hides behind a whole step.  Consecutive threads read consecutive 16-byte
// segments of a row (coalesced); rows past the sequence end re-read row t0 (always
// valid): their values are finite and every coefficient that touches them is zero.
template <int D, int NST>
struct TileRegs {
  static constexpr int NSEG = D / 8;                  // 16-byte segments per row
  static constexpr int N = 64 * NSEG / NST;           // segments per thread
  static_assert(N * NST == 64 * NSEG && (N == 1 || N == 2 || N == 4), "segments split evenly");
  // named registers, no array, and native vectors rather than uint4 structs (whose
  // copies can go through scratch)
  u32x4 s0, s1, s2, s3;
  // (a uniform base at row t0 plus a 32-bit lane offset: the scalar-base address form)
  __device__ __forceinline__ static u32x4 ld(const u16* g, int64_t gs, int t0, int n, int si, int i) {
    const int sidx = si + i * NST, r = sidx / NSEG, c = sidx % NSEG;
    const char* base = reinterpret_cast<const char*>(g + (int64_t)t0 * gs);
    const uint32_t off = ((uint32_t)(r < n ? r : 0) * (uint32_t)gs + 8u * (uint32_t)c) * 2u;
    return *reinterpret_cast<const u32x4*>(base + off);
  }
  template <bool kSwz>
  __device__ __forceinline__ static void st(u16* tile, int si, int i, u32x4 v) {
    const int sidx = si + i * NST, r = sidx / NSEG, c = sidx % NSEG;
    if constexpr (kSwz) {   // Q and K tiles: unpadded rows, swizzled 16-byte chunks
      *reinterpret_cast<u32x4*>(tile + qidx<D>(r, 8 * c)) = v;
    } else {
      *reinterpret_cast<u32x4*>(tile + r * (D + 8) + 8 * c) = v;
    }
  }
  __device__ __forceinline__ void load(const u16* g, int64_t gs, int t0, int n, int si) {
    s0 = ld(g, gs, t0, n, si, 0);
    if constexpr (N >= 2) s1 = ld(g, gs, t0, n, si, 1);
    if constexpr (N == 4) {
      s2 = ld(g, gs, t0, n, si, 2);
      s3 = ld(g, gs, t0, n, si, 3);
    }
  }
  // 1 / sqrt(|row|^2 + 1e-6) of the row that segment v (staging slot i) belongs to, 0
  // for rows >= n.  The 16 segments of a row (D = 128) are held by 16 consecutive lanes,
  // so its squared norm is a sum over a row of 16 lanes.
  __device__ __forceinline__ static float rnorm(u32x4 v, int si, int i, int n) {
    static_assert(NSEG == 16 && NST % 16 == 0, "a row's segments in one row of 16 lanes");
    const float a = row16_sum(dot2sq(v[3], dot2sq(v[2], dot2sq(v[1], dot2sq(v[0], 0.f)))));
    return (si + i * NST) / NSEG < n ? __builtin_amdgcn_rsqf(a + 1e-6f) : 0.f;   // 1 ulp
  }
  // the 8 bf16 of v times f, as fp16
  __device__ __forceinline__ static u32x4 scale_h(u32x4 v, float f) {
    return u32x4{cvt2h(bf_lo(v[0]) * f, bf_hi(v[0]) * f), cvt2h(bf_lo(v[1]) * f, bf_hi(v[1]) * f),
                 cvt2h(bf_lo(v[2]) * f, bf_hi(v[2]) * f), cvt2h(bf_lo(v[3]) * f, bf_hi(v[3]) * f)};
  }
  template <bool kPerm>   // Q and K tiles: permuted column groups, swizzled chunks
  __device__ __forceinline__ void store(u16* tile, int si) const {
    st<kPerm>(tile, si, 0, s0);
    if constexpr (N >= 2) st<kPerm>(tile, si, 1, s1);
    if constexpr (N == 4) {
      st<kPerm>(tile, si, 2, s2);
      st<kPerm>(tile, si, 3, s3);
    }
  }
};


template <int DK, int DV, bool kSSD, typename OutT, int CT, bool kGate, bool kCk>
__global__ void __launch_bounds__((DV / (16 * CT) + kNP) * kWave, 1) chunk_kernel(SeqLaunch p) {
  constexpr int CW = 16 * CT;      // d_v columns per state wave (CT tiles of 16)
  constexpr int NSW = DV / CW;     // state waves
  constexpr int NKS = DK / 32;     // 32-wide k-steps over d_k
  constexpr int NTK = DK / 16;     // S^T row tiles (16 d_k rows each)
  static_assert(DK == 128 && (DV == 128 || DV == 64) && NSW * CW == DV, "tile shapes");
  // fp16 operands (GDN with bf16 output): Q^ = diag(r_q) Q and K^ = diag(r_k) K land
  // in fp16 (normalised as they land), and the products take them, S0, R, the scaled
  // U of the state update and P U as single fp16 operands.  Every operand is bounded
  // by construction or by the values (|Q^|, |K^| <= 1, |P| <= scale, decays <= 1), and
  // fp16's 11-bit significand keeps each product's error well below the output's bf16
  // rounding.  fp32 output keeps raw bf16 Q, K with two-term bf16 splits of the rest;
  // the delta-off mode, raw bf16 Q, K with a bf16 S0.
  constexpr bool kF16 = !kSSD && sizeof(OutT) == 2;

  // chunk data: Q and K of chunk c (state waves) and c + 1 (producers); V, Z of chunk c
  __shared__ __attribute__((aligned(16))) u16 sQ[2][C * DK], sK[2][C * DK];
  __shared__ __attribute__((aligned(16))) u16 sV[C * (DV + 8)], sZ[kSSD ? C * (DV + 8) : 8];
  // producer outputs for the state waves, double-buffered
  __shared__ __attribute__((aligned(16))) u16 sPh[2][C][kPS];                 // P (hi, or fp16)
  __shared__ __attribute__((aligned(16))) u16 sPl[kF16 ? 1 : 2][kF16 ? 1 : C][kPS];   // P lo
  __shared__ __attribute__((aligned(16))) u16 sTb[kSSD ? 1 : 2][C][kPS];
  __shared__ __attribute__((aligned(16))) float sCR[2][C], sCO[2][C], sCS[2][C], sBeta[2][C], sGC[2][4];
  __shared__ __attribute__((aligned(16))) float sGr[2][C], sBr[2][C];    // raw log g, beta (staged)
  // 1 / |q_i|, 1 / |k_i| from the landing (raw bf16 operands only: the fp16 operands
  // land normalised)
  __shared__ __attribute__((aligned(16))) float sRq[kF16 ? 1 : 2][kF16 ? 1 : C], sRk[kF16 ? 1 : 2][kF16 ? 1 : C];
  __shared__ __attribute__((aligned(16))) float sGc[2][C];   // G_i, the in-chunk decay cumsum (checkpoints)
  // producer working set (per producer wave where private)
  // fp32 diagonal 16x16 blocks of A, rows of 20 floats, double-buffered; the block
  // stride of 336 floats puts the four blocks on different banks (the solve reads all
  // four at once)
  __shared__ __attribute__((aligned(16))) float sAd[kSSD ? 1 : 2][4][16 * 20 + 16];
  // vectors of the chunk being prepared, per token (see the producer roles)
  __shared__ __attribute__((aligned(16))) float sEG[C], sEB[C], sERp[C], sERa[C], sEF[C], sEFa[C];
  // arrival counters: chunk vectors ready (0), T ready (1), state waves' landing
  // done (2), producers' landing done (3); and
  // (entry kFailFlag) the flag of a bounded wait that ran out
  __shared__ uint32_t sSync[8];
  constexpr int kFailFlag = 7;

  // Work item (v-head h, sequence position yr).  Workgroups go to the 8 XCDs in turn
  // (linear id % 8), each XCD with its own L2, and the r = H_v / H_qk v-heads of a
  // qk-head read the same q, k rows: they take the linear ids i, i + 8, .., i + 8 (r - 1)
  // -- one XCD, dispatched together, so all but one read q, k from that XCD's L2.
  // (With (sequences x qk-heads) not a multiple of 8, the plain order is kept.)
  int h, yr;
  {
    const int r = p.H_v / p.H_qk;
    const int lin = blockIdx.x + gridDim.x * blockIdx.y;
    if ((gridDim.y * p.H_qk) % 8 == 0) {
      const int blk = lin / (8 * r), o = lin % (8 * r);
      const int u = 8 * blk + (o & 7);             // (sequence position, qk-head) unit
      yr = u / p.H_qk;
      h = (u % p.H_qk) * r + (o >> 3);
    } else {
      h = blockIdx.x;
      yr = blockIdx.y;
    }
  }
  // Workgroups are dispatched sequence by sequence.  With lpt set, the sequence
  // position yr is a rank in descending length (ties by index), so the longest
  // sequences start first and a ragged batch ends without a long tail (longest-
  // processing-time first).  Thread m ranks sequence m in O(N); the host sets lpt only
  // for small N.
  int nseq = yr;
  if (p.lpt) {
    __shared__ int sSel;
    const int m = threadIdx.x;
    if (m < p.N) {
      const int lm = p.cu_seqlens[m + 1] - p.cu_seqlens[m];
      int rank = 0;
      for (int q = 0; q < p.N; ++q) {
        const int lq = p.cu_seqlens[q + 1] - p.cu_seqlens[q];
        rank += (lq > lm) | ((lq == lm) & (q < m));
      }
      if (rank == yr) sSel = m;
    }
    __syncthreads();
    nseq = __builtin_amdgcn_readfirstlane(sSel);
  }
  const int sl = p.slot[nseq];
  if (sl < 0) return;                                      // uniform over the block
  const int tbeg = p.cu_seqlens[nseq], tend = p.cu_seqlens[nseq + 1];
  const int nch = (tend - tbeg + C - 1) / C;
  const bool init = p.has_init ? (p.has_init[nseq] != 0) : true;
  const int j = h / (p.H_v / p.H_qk);
  // gate folded in: the head's gate parameters (the raw a, b / dt are staged per token)
  float gA = 0.f, gBias = 0.f;   // GDN: exp(A_log); delta-off: A
  if constexpr (kGate) {
    gA = kSSD ? p.gA[h] : expf(p.gA[h]);
    gBias = p.gdt_bias ? p.gdt_bias[h] : 0.f;
  }

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wu = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave index, uniform
  const bool isP = wu >= NSW;                                   // producer wave (uniform)
  // Producers issue first where both roles are ready: what they prepare (P, T and the
  // vectors of the next chunk) gates the state waves' next step, and the state waves'
  // chain has stalls enough to absorb the delay (measured: ~4-7% faster than equal
  // priorities or the state waves first).
  if (isP) __builtin_amdgcn_s_setprio(3);
  const int g16 = lane >> 4, j16 = lane & 15;

  const u16* qg = reinterpret_cast<const u16*>(p.q) + (int64_t)j * DK;
  const u16* kg = reinterpret_cast<const u16*>(p.k) + (int64_t)j * DK;
  const u16* vg = reinterpret_cast<const u16*>(p.v) + (int64_t)h * DV;
  // (without z, its staging re-reads v, unused: the loads stay unconditional)
  const u16* zg = reinterpret_cast<const u16*>(p.z ? p.z : p.v) + (int64_t)h * DV;
  const int64_t z_stride = p.z ? p.z_stride : p.v_stride;

  // ================================================================ state waves
  // Wave wu owns d_v columns CW wu .. CW wu + CW - 1 (CT tiles of 16).
  // Output rows: a wave-uniform base (a chunk's first row, this wave's columns) plus
  // 32-bit lane offsets, so that the stores use the scalar-base address form.
  auto out_base = [&](int t0) {
    return reinterpret_cast<char*>(p.out) + ((int64_t)t0 * p.out_stride + (int64_t)h * DV + CW * wu) * (int64_t)sizeof(OutT);
  };
  const uint32_t ostride_b = (uint32_t)p.out_stride * (uint32_t)sizeof(OutT);

  // S^T tiles in 16x16 accumulator layout: Sacc[ct][tk][r] = S[col_ct][dk(tk) + 8 g16 + r]
  // with dk(tk) = 32 (tk / 2) + 4 (tk % 2): the two tiles 2 s2, 2 s2 + 1 together hold
  // d_k 32 s2 + 8 g16 + 0..7 in a lane, the natural column order of the Q, K tiles.
  float* state = p.pool + ((int64_t)sl * p.H_v + h) * (int64_t)(DV * DK);
  f32x4 Sacc[CT][NTK];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int tk = 0; tk < NTK; ++tk) {
      Sacc[ct][tk] = f32x4{};
      if (!isP && init) {
        const int col = CW * wu + 16 * ct + j16;
        const float4 v = *reinterpret_cast<const float4*>(state + (int64_t)col * DK + 32 * (tk >> 1) + 4 * (tk & 1) + 8 * g16);
        Sacc[ct][tk] = f32x4{v.x, v.y, v.z, v.w};
      }
    }
  // One S^T tile of this lane in the pool's [d_v, d_k] layout at `dst` (a pool slot
  // or a checkpoint row of this head).
  // (an opaque copy of the lane id: the addresses are computed where they are used,
  // not hoisted out of the step loop and kept live through it)
  auto store_tile = [&](float* dst, int ct, int tk, const f32x4& v) __attribute__((always_inline)) {
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int col = CW * wu + 16 * ct + (lane_o & 15);
    *reinterpret_cast<float4*>(dst + (int64_t)col * DK + 32 * (tk >> 1) + 4 * (tk & 1) + 8 * (lane_o >> 4)) =
        make_float4(v[0], v[1], v[2], v[3]);
  };
  auto store_state = [&](float* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int tk = 0; tk < NTK; ++tk) store_tile(dst, ct, tk, Sacc[ct][tk]);
  };
  // State checkpoint (state waves): the state after ck_b tokens of the sequence goes
  // to ck_st; ck_b = -1 when none is requested.
  int ck_b = -1;
  float* ck_st = nullptr;
  // delta-off D skip coefficients of this lane's output columns (16 ct + 4 g16 + e)
  float4 Dc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    Dc[ct] = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (kSSD) {
      const u16* Db = reinterpret_cast<const u16*>(p.D);
      if (!isP && Db) {
        float d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = CW * wu + 16 * ct + 4 * g16 + e;
          d[e] = bf16_to_f32(Db[p.D_per_dim ? (int64_t)h * DV + col : (int64_t)h]);
        }
        Dc[ct] = make_float4(d[0], d[1], d[2], d[3]);
      }
    }
  }

  // ================================================================ staging
  // Each role stages the raw rows it consumes: the producers Q, K (and the gate
  // inputs) of chunk c + 2, issued right after the landing of step c (producer 2 right
  // after its merge of T); the state waves V (z) of chunk c + 1, issued in the middle
  // of their step.  Both stay in flight in
  // registers during step c.  Each role lands its rows right after the step's barrier
  // and announces them on its own arrival counter, so neither waits for the other's
  // landing: the producers wait for theirs before their first products, the state
  // waves for theirs before they first read V.
  constexpr int NSTQ = kNP * kWave, NSTV = NSW * kWave;
  const int siq = tid - NSW * kWave;          // staging index of a producer thread
  const int siv = tid;                        // staging index of a state-wave thread
  TileRegs<DK, NSTQ> rq_, rk_;                // (producers)
  TileRegs<DV, NSTV> rv_, rz_;                // (state waves; z: delta-off only)
  float rg_ = 0.f, rb_ = 0.f;                 // log g, beta of chunk c + 2 (lane = token), for the producers
  // (gate folded in: the aligned 32-bit words holding the raw bf16 a, b / dt, kept
  // exactly as loaded -- any instruction on the loaded value, even a zero-extension
  // of a 16-bit load, would make the producers wait for these loads at the step's end)
  uint32_t ra_ = 0u, rbr_ = 0u;
  // Gate folded in: producer 2, idle once T is done, turns its staged raw inputs of
  // chunk c + 2 into log g, beta at the end of step c and stores them at once into the
  // gate buffer of that chunk's parity (free during step c: its previous chunk was
  // prepared in step c - 1), so the arithmetic stays off every wave's path.
  auto gate_store = [&](int par) __attribute__((always_inline)) {
    if constexpr (kGate) {
      float lg, bt;
      // head h's bf16 is the low (h even) or high (h odd) half of the word
      const float ga = __uint_as_float((h & 1) ? (ra_ & 0xffff0000u) : (ra_ << 16));
      if constexpr (kSSD) {
        gate_ssd(ga, gA, gBias, p.g_softplus, p.g_lo, p.g_hi, lg, bt);
      } else {
        const float gb = __uint_as_float((h & 1) ? (rbr_ & 0xffff0000u) : (rbr_ << 16));
        gate_gdn(ga, gb, gA, gBias, lg, bt);
      }
      sGr[par][lane] = lg;
      sBr[par][lane] = bt;
    }
  };
  // Landing of a chunk's Q and K rows (delta rule; n rows in the sequence): every
  // thread holds two 16-byte segments of each, of rows r and r + 32, and takes their
  // row norms from the staged values.  fp16 operands: the rows land normalised,
  // q / |q| and k / |k| (|entries| <= 1) in fp16, zero past the end; raw bf16
  // operands: the rows land as they are and 1 / |row| goes to sRq, sRk.
  auto land_qk = [&](auto parq, int n) __attribute__((always_inline)) {
    constexpr int PQ = decltype(parq)::value;
    using Reg = TileRegs<DK, NSTQ>;
    static_assert(Reg::N == 4, "four segments of each tile per thread");
    constexpr int RS = NSTQ / Reg::NSEG;      // rows between a thread's segments
    const float q0 = Reg::rnorm(rq_.s0, siq, 0, n), q1 = Reg::rnorm(rq_.s1, siq, 1, n);
    const float q2 = Reg::rnorm(rq_.s2, siq, 2, n), q3 = Reg::rnorm(rq_.s3, siq, 3, n);
    const float k0 = Reg::rnorm(rk_.s0, siq, 0, n), k1 = Reg::rnorm(rk_.s1, siq, 1, n);
    const float k2 = Reg::rnorm(rk_.s2, siq, 2, n), k3 = Reg::rnorm(rk_.s3, siq, 3, n);
    if constexpr (kF16) {
      Reg::template st<true>(sQ[PQ], siq, 0, Reg::scale_h(rq_.s0, q0));
      Reg::template st<true>(sQ[PQ], siq, 1, Reg::scale_h(rq_.s1, q1));
      Reg::template st<true>(sQ[PQ], siq, 2, Reg::scale_h(rq_.s2, q2));
      Reg::template st<true>(sQ[PQ], siq, 3, Reg::scale_h(rq_.s3, q3));
      Reg::template st<true>(sK[PQ], siq, 0, Reg::scale_h(rk_.s0, k0));
      Reg::template st<true>(sK[PQ], siq, 1, Reg::scale_h(rk_.s1, k1));
      Reg::template st<true>(sK[PQ], siq, 2, Reg::scale_h(rk_.s2, k2));
      Reg::template st<true>(sK[PQ], siq, 3, Reg::scale_h(rk_.s3, k3));
    } else {
      rq_.template store<true>(sQ[PQ], siq);
      rk_.template store<true>(sK[PQ], siq);
      if ((siq & 15) == 0) {
        const int r = siq / Reg::NSEG;
        sRq[PQ][r] = q0;
        sRq[PQ][r + RS] = q1;
        sRq[PQ][r + 2 * RS] = q2;
        sRq[PQ][r + 3 * RS] = q3;
        sRk[PQ][r] = k0;
        sRk[PQ][r + RS] = k1;
        sRk[PQ][r + 2 * RS] = k2;
        sRk[PQ][r + 3 * RS] = k3;
      }
    }
  };
  auto stage_qk = [&](int cc) __attribute__((always_inline)) {
    const int t0 = tbeg + cc * C, n = min(C, tend - t0);
    rq_.load(qg, p.q_stride, t0, n, siq);
    rk_.load(kg, p.k_stride, t0, n, siq);
    const int64_t tt = (int64_t)(t0 + (lane < n ? lane : 0));
    if constexpr (kGate) {   // raw gate inputs (bf16)
      ra_ = reinterpret_cast<const uint32_t*>(p.ga)[tt * (p.ga_stride >> 1) + (h >> 1)];
      if constexpr (!kSSD) rbr_ = reinterpret_cast<const uint32_t*>(p.gb)[tt * (p.gb_stride >> 1) + (h >> 1)];
    } else {
      rg_ = p.log_g[tt * p.H_v + h];
      rb_ = p.beta[tt * p.H_v + h];
    }
  };
  auto stage_v = [&](int cc) __attribute__((always_inline)) {
    const int t0 = tbeg + cc * C, n = min(C, tend - t0);
    rv_.load(vg, p.v_stride, t0, n, siv);
    if constexpr (kSSD) rz_.load(zg, z_stride, t0, n, siv);
  };

  // Hand-off between waves inside a step: arrival counters in LDS.  A wave's LDS
  // writes are performed before its later increment (the LDS executes one wave's
  // accesses in order); the waiting wave reads the data only after seeing the count.
  // Waits are bounded: every counted arrival happens unconditionally.  A wait that
  // runs out (~0.1 s; an arrival was lost) raises the fail flag and goes on; at the
  // end the workgroup then overwrites its output rows and final state with NaN, so
  // the failure shows in the results instead of passing as plausible numbers.
  auto arrive = [&](uint32_t* ctr) __attribute__((always_inline)) {
    lds_order();
    if (lane == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  auto wait_count = [&](uint32_t* ctr, uint32_t target) __attribute__((always_inline)) {
    for (int it = 0;; ++it) {
      if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
      if (it == (1 << 22)) {
        if (lane == 0) __hip_atomic_store(&sSync[kFailFlag], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    lds_order();
  };

  // State-dependent part of chunk c (buffers of parity PAR).  A operands (rows of Q,
  // K, T, P and K^T) are read once and shared by the wave's CT column tiles.
  auto consume = [&](int c, auto parc) __attribute__((always_inline)) {
    constexpr int PAR = decltype(parc)::value;
    const int t0 = tbeg + c * C, n = min(C, tend - t0);
    // Lane-derived indices are recomputed in every step (an opaque copy of the lane
    // id): hoisting the many per-lane LDS addresses out of the loop would keep them
    // all live at once and spill them.
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int g16 = lane_o >> 4, j16 = lane_o & 15;
    const u16* Q = sQ[PAR];
    const u16* K = sK[PAR];
    const float gC = sGC[PAR][0];
    if constexpr (kCk) {
      if (c > 0 && ck_b == C * c) store_state(ck_st);   // checkpoint at this chunk's start
    }

    // U: tiles of 16 tokens (rows 16 rt + 4 g16 + r) x 16 d_v columns (lane j16).
    // Y: the output in transposed tiles (O^T: rows = d_v 16 ct + 4 g16 + r, lane j16 =
    // token 16 rt + j16), from the same operands with A and B swapped, so that a lane
    // holds 4 consecutive output columns of one token (8-byte stores).
    f32x4 Y[CT][4], U[CT][4];
    if constexpr (kF16) {   // Y = Q^ S0^T, X = K^ S0^T (Q^, K^ the normalised rows)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          Y[ct][rt] = f32x4{};
          U[ct][rt] = f32x4{};
        }
      // k-steps outermost: one k-step's S0 operand is live at a time
#pragma unroll
      for (int s2 = 0; s2 < NKS; ++s2) {
        f16x8 Sb[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) Sb[ct] = pair_to_op_h(Sacc[ct][2 * s2], Sacc[ct][2 * s2 + 1]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const int row = 16 * rt + j16;
          const f16x8 aq = __builtin_bit_cast(f16x8, ldq8<DK>(Q, row, 32 * s2 + 8 * g16));
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) Y[ct][rt] = mfma1632h(Sb[ct], aq, Y[ct][rt]);
          const f16x8 ak = __builtin_bit_cast(f16x8, ldq8<DK>(K, row, 32 * s2 + 8 * g16));
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) U[ct][rt] = mfma1632h(ak, Sb[ct], U[ct][rt]);
        }
      }
    } else if constexpr (kSSD) {
      bf16x8 Sb[CT][NKS];      // S0^T as B operand: k = d_k 32 s2 + 8 g16 + e
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int s2 = 0; s2 < NKS; ++s2) Sb[ct][s2] = pair_to_op(Sacc[ct][2 * s2], Sacc[ct][2 * s2 + 1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          Y[ct][rt] = f32x4{};
          U[ct][rt] = f32x4{};
        }
        const int row = 16 * rt + j16;
#pragma unroll
        for (int s2 = 0; s2 < NKS; ++s2) {
          const bf16x8 aq = ldq8<DK>(Q, row, 32 * s2 + 8 * g16);   // stored columns: k slots in order
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) Y[ct][rt] = mfma1632(Sb[ct][s2], aq, Y[ct][rt]);   // (Q S0^T)^T
        }
      }
    } else {   // raw operands, delta rule: S0 as hi + lo bf16, k-steps outermost
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          Y[ct][rt] = f32x4{};
          U[ct][rt] = f32x4{};
        }
#pragma unroll
      for (int s2 = 0; s2 < NKS; ++s2) {
        bf16x8 Sh[CT], Sl[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) pair_split(Sacc[ct][2 * s2], Sacc[ct][2 * s2 + 1], Sh[ct], Sl[ct]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const int row = 16 * rt + j16;
          const bf16x8 aq = ldq8<DK>(Q, row, 32 * s2 + 8 * g16);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {   // (Q S0^T)^T
            Y[ct][rt] = mfma1632(Sh[ct], aq, Y[ct][rt]);
            Y[ct][rt] = mfma1632(Sl[ct], aq, Y[ct][rt]);
          }
          const bf16x8 ak = ldq8<DK>(K, row, 32 * s2 + 8 * g16);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {   // X = K S0^T
            U[ct][rt] = mfma1632(ak, Sh[ct], U[ct][rt]);
            U[ct][rt] = mfma1632(ak, Sl[ct], U[ct][rt]);
          }
        }
      }
    }
    // This wave's share of the next staged rows (V, z of chunk c + 1): issued before
    // this step's output stores, so that the next landing's wait for these loads never
    // includes the stores (the memory counter retires in order).
    stage_v(min(c + 1, nch - 1));
    wait_count(&sSync[2], (uint32_t)NSW * (uint32_t)(c + 2));   // this step's landing (V of chunk c) done
    // R = beta V - CR X (GDN); U = beta V (delta-off).  V through transpose reads.
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int ib = 16 * rt + 4 * g16;
      const float4 bi = ld_f4(&sBeta[PAR][ib]);
      float4 cr = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (!kSSD) cr = ld_f4(&sCR[PAR][ib]);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const uint2 t = ldtr<DV>(sV, ib + (j16 >> 2), CW * wu + 16 * ct + 4 * (j16 & 3));
        const float vv[4] = {bf_lo(t.x), bf_hi(t.x), bf_lo(t.y), bf_hi(t.y)};
        if constexpr (kSSD) {
#pragma unroll
          for (int e = 0; e < 4; ++e) U[ct][rt][e] = f4get(bi, e) * vv[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) U[ct][rt][e] = f4get(bi, e) * vv[e] - f4get(cr, e) * U[ct][rt][e];
        }
      }
    }
    if constexpr (!kSSD) {
      wait_count(&sSync[1], (uint32_t)(c + 1));   // T of chunk c (finished in this step)
      // U = T R = R + L R with L = T - I (fp16, stored with a zero diagonal): R stays
      // exact in the accumulator; L is strictly lower, so row tile rt needs k-steps <= rt / 2.
      // fp16 operands: R in fp16; raw operands: L and R each as hi + lo bf16, three products.
      if constexpr (kF16) {
        f16x8 Rh[CT][2];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) Rh[ct][s2] = pair_to_op_h(U[ct][2 * s2], U[ct][2 * s2 + 1]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const u16* trow = &sTb[PAR][16 * rt + j16][8 * g16];
#pragma unroll
          for (int s2 = 0; s2 <= (rt >> 1); ++s2) {
            const f16x8 ta = __builtin_bit_cast(f16x8, ld8u(trow + 32 * s2));
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) U[ct][rt] = mfma1632h(ta, Rh[ct][s2], U[ct][rt]);
          }
        }
      } else {
        bf16x8 Rh[CT][2], Rl[CT][2];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) pair_split(U[ct][2 * s2], U[ct][2 * s2 + 1], Rh[ct][s2], Rl[ct][s2]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const u16* trow = &sTb[PAR][16 * rt + j16][8 * g16];
#pragma unroll
          for (int s2 = 0; s2 <= (rt >> 1); ++s2) {
            bf16x8 th, tl;
            h8_split(__builtin_bit_cast(uint4, ld8u(trow + 32 * s2)), th, tl);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              U[ct][rt] = mfma1632(th, Rh[ct][s2], U[ct][rt]);
              U[ct][rt] = mfma1632(th, Rl[ct][s2], U[ct][rt]);
              U[ct][rt] = mfma1632(tl, Rh[ct][s2], U[ct][rt]);
            }
          }
        }
      }
    }
    // O = CO (Q S0^T) + P U (fp16 operands, or two-term bf16 splits of P and U)
    if constexpr (kF16) {
      f16x8 Uf[CT][2];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) Uf[ct][s2] = pair_to_op_h(U[ct][2 * s2], U[ct][2 * s2 + 1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const float co = sCO[PAR][16 * rt + j16];    // this lane's token
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) Y[ct][rt] *= co;
        const u16* prow = &sPh[PAR][16 * rt + j16][8 * g16];
#pragma unroll
        for (int s2 = 0; s2 <= (rt >> 1); ++s2) {
          const f16x8 pf = __builtin_bit_cast(f16x8, ld8u(prow + 32 * s2));
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) Y[ct][rt] = mfma1632h(Uf[ct][s2], pf, Y[ct][rt]);   // (P U)^T = U^T P^T
        }
      }
    } else {
      bf16x8 Uh[CT][2], Ul[CT][2];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) pair_split(U[ct][2 * s2], U[ct][2 * s2 + 1], Uh[ct][s2], Ul[ct][s2]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const float co = sCO[PAR][16 * rt + j16];    // this lane's token
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) Y[ct][rt] *= co;
        const u16* phrow = &sPh[PAR][16 * rt + j16][8 * g16];
        const u16* plrow = &sPl[PAR][16 * rt + j16][8 * g16];
#pragma unroll
        for (int s2 = 0; s2 <= (rt >> 1); ++s2) {
          const bf16x8 ph = ld8u(phrow + 32 * s2);
          const bf16x8 pl = ld8u(plrow + 32 * s2);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {   // (P U)^T = U^T P^T
            Y[ct][rt] = mfma1632(Uh[ct][s2], ph, Y[ct][rt]);
            Y[ct][rt] = mfma1632(Uh[ct][s2], pl, Y[ct][rt]);
            Y[ct][rt] = mfma1632(Ul[ct][s2], ph, Y[ct][rt]);
          }
        }
      }
    }
    // epilogue (delta-off: D skip and silu(z) gate; x and z re-read from LDS)
    if constexpr (kSSD) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {   // token 16 rt + j16, columns 16 ct + 4 g16 + e
          const int ra = 16 * rt + j16, ca = CW * wu + 16 * ct + 4 * g16;
          const uint2 tx = *reinterpret_cast<const uint2*>(&sV[pidx<DV>(ra, ca)]);
          const float xv[4] = {bf_lo(tx.x), bf_hi(tx.x), bf_lo(tx.y), bf_hi(tx.y)};
          float zz[4] = {1.f, 1.f, 1.f, 1.f};
          if (p.z) {
            const uint2 tz = *reinterpret_cast<const uint2*>(&sZ[pidx<DV>(ra, ca)]);
            const float zr[4] = {bf_lo(tz.x), bf_hi(tz.x), bf_lo(tz.y), bf_hi(tz.y)};
#pragma unroll
            for (int e = 0; e < 4; ++e) zz[e] = zr[e] * sigmoid_f(zr[e]);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) Y[ct][rt][e] = (Y[ct][rt][e] + f4get(Dc[ct], e) * xv[e]) * zz[e];
        }
    }
    {
      // row j16 + 16 rt, columns 16 ct + 4 g16 ..: a lane offset plus uniform row-tile
      // steps (the column tiles are instruction offsets).  Bounds-checked buffer stores
      // whose record range is the chunk's n rows: the hardware drops the rows past the
      // sequence end, so every step issues the same stores without a branch, which
      // keeps the count of memory operations in flight the same on every path (the
      // next landing then waits for the staged loads only, never for these stores).
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(out_base(t0), (short)0, (int)((uint32_t)n * ostride_b), kBufWord3);
      const uint32_t o0 = (uint32_t)j16 * ostride_b + (uint32_t)(4 * g16 * sizeof(OutT));
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const int off = (int)(o0 + (uint32_t)rt * (16u * ostride_b)) + 16 * ct * (int)sizeof(OutT);
          if constexpr (sizeof(OutT) == 2) {
            const u32x2 w = {cvt2(Y[ct][rt][0], Y[ct][rt][1]), cvt2(Y[ct][rt][2], Y[ct][rt][3])};
            __builtin_amdgcn_raw_buffer_store_b64(w, rs, off, 0, 0);
          } else {
            const u32x4 w = {__float_as_uint(Y[ct][rt][0]), __float_as_uint(Y[ct][rt][1]),
                             __float_as_uint(Y[ct][rt][2]), __float_as_uint(Y[ct][rt][3])};
            __builtin_amdgcn_raw_buffer_store_b128(w, rs, off, 0, 0);
          }
        }
    }

    // checkpoint inside the chunk, after its first m tokens: the state update with the
    // decays taken to token m - 1 and the later tokens left out,
    //   S_m^T = exp(G_{m-1}) S0^T + K^T diag(exp(G_{m-1} - G_i) r_k,i [i < m]) U
    // (r_k already in K^ on the fp16 path), written out tile by tile
    if (kCk && ck_b > C * c && ck_b < C * c + n) {
      __builtin_amdgcn_sched_barrier(0);   // (kept apart from the regular update: register pressure)
      const int m = ck_b - C * c;
      const float Gm = sGc[PAR][m - 1];
      const float gm = __expf(Gm);
      float cf[4][4];   // per token 16 rt + 4 g16 + e
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * rt + 4 * g16 + e;
          float rk = 1.f;
          if constexpr (!kF16) rk = sRk[PAR][i];
          cf[rt][e] = i < m ? __expf(Gm - sGc[PAR][i]) * rk : 0.f;
        }
      const int rb = 4 * g16 + (j16 >> 2);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {   // one column tile at a time (register pressure)
        f32x4 Uc[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int e = 0; e < 4; ++e) Uc[rt][e] = U[ct][rt][e] * cf[rt][e];
        if constexpr (kF16) {
          f16x8 Wc[2];
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) Wc[s2] = pair_to_op_h(Uc[2 * s2], Uc[2 * s2 + 1]);
#pragma unroll
          for (int tk = 0; tk < NTK; ++tk) {
            const int ca = 32 * (tk >> 1) + 8 * (j16 & 3) + 4 * (tk & 1);
            f32x4 acc = Sacc[ct][tk] * gm;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
              acc = mfma1632h(__builtin_bit_cast(f16x8, join(ldqtr<DK>(K, 32 * s2 + rb, ca), ldqtr<DK>(K, 32 * s2 + 16 + rb, ca))),
                              Wc[s2], acc);
            store_tile(ck_st, ct, tk, acc);
          }
        } else {
          bf16x8 Wh[2], Wl[2];
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) pair_split(Uc[2 * s2], Uc[2 * s2 + 1], Wh[s2], Wl[s2]);
#pragma unroll
          for (int tk = 0; tk < NTK; ++tk) {
            const int ca = 32 * (tk >> 1) + 8 * (j16 & 3) + 4 * (tk & 1);
            f32x4 acc = Sacc[ct][tk] * gm;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              const bf16x8 kt = join(ldqtr<DK>(K, 32 * s2 + rb, ca), ldqtr<DK>(K, 32 * s2 + 16 + rb, ca));
              acc = mfma1632(kt, Wh[s2], acc);
              acc = mfma1632(kt, Wl[s2], acc);
            }
            store_tile(ck_st, ct, tk, acc);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // state update: S^T = gamma_C S^T + K^T diag(CS) U  (fp16 K^ and CS U, or bf16 K with hi + lo splits)
    {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const float4 cs = ld_f4(&sCS[PAR][16 * rt + 4 * g16]);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) U[ct][rt][e] *= f4get(cs, e);
      }
      // A operand K^T: row j16 = d_k 32 (tk / 2) + 8 (j16 / 4) + 4 (tk % 2) + j16 % 4 (the
      // state's row order; a transpose read may take its four 4-column chunks from
      // anywhere); k slots: tokens 32 s2 + 4 g16 + e and 32 s2 + 16 + 4 g16 + e
      const int rb = 4 * g16 + (j16 >> 2);
      if constexpr (kF16) {   // K^^T (normalised rows) times the scaled U, fp16
        f16x8 Wf[CT][2];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) Wf[ct][s2] = pair_to_op_h(U[ct][2 * s2], U[ct][2 * s2 + 1]);
#pragma unroll
        for (int tk = 0; tk < NTK; ++tk) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) Sacc[ct][tk] *= gC;
          const int ca = 32 * (tk >> 1) + 8 * (j16 & 3) + 4 * (tk & 1);   // A row j16 = d_k ca + j16 % 4
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const f16x8 kt = __builtin_bit_cast(f16x8, join(ldqtr<DK>(K, 32 * s2 + rb, ca), ldqtr<DK>(K, 32 * s2 + 16 + rb, ca)));
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) Sacc[ct][tk] = mfma1632h(kt, Wf[ct][s2], Sacc[ct][tk]);
          }
        }
      } else {
        bf16x8 Wh[CT][2], Wl[CT][2];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) pair_split(U[ct][2 * s2], U[ct][2 * s2 + 1], Wh[ct][s2], Wl[ct][s2]);
#pragma unroll
        for (int tk = 0; tk < NTK; ++tk) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) Sacc[ct][tk] *= gC;
          const int ca = 32 * (tk >> 1) + 8 * (j16 & 3) + 4 * (tk & 1);   // A row j16 = d_k ca + j16 % 4
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const bf16x8 kt = join(ldqtr<DK>(K, 32 * s2 + rb, ca), ldqtr<DK>(K, 32 * s2 + 16 + rb, ca));
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              Sacc[ct][tk] = mfma1632(kt, Wh[ct][s2], Sacc[ct][tk]);
              Sacc[ct][tk] = mfma1632(kt, Wl[ct][s2], Sacc[ct][tk]);
            }
          }
        }
      }
    }
  };

  // ================================================================ producer waves

  // Tile (ti, tj) of K Q^T and K K^T (the transposes of Q K^T and K K^T: each lane
  // holds one query row i = 32 ti + l32 and keys m = 32 tj + 8 q4 + 4 hh + e).
  auto tile_mma = [&](const u16* Q, const u16* K, int ti, int tj, int l32, int hh, f32x16& qk, f32x16& kk) __attribute__((always_inline)) {
    qk = f32x16{};
    kk = f32x16{};
#pragma unroll
    for (int s = 0; s < DK / 16; ++s) {                        // 16-wide k-steps (32x32x16)
      const bf16x8 a = ldq8<DK>(K, 32 * tj + l32, 16 * s + 8 * hh);
      const bf16x8 bq = ldq8<DK>(Q, 32 * ti + l32, 16 * s + 8 * hh);
      if constexpr (kF16) {   // normalised fp16 rows
        const f16x8 ah = __builtin_bit_cast(f16x8, a);
        qk = mfma32h(ah, __builtin_bit_cast(f16x8, bq), qk);
        kk = mfma32h(ah, __builtin_bit_cast(f16x8, ldq8<DK>(K, 32 * ti + l32, 16 * s + 8 * hh)), kk);
      } else {
        qk = mfma32(a, bq, qk);
        if constexpr (!kSSD) kk = mfma32(a, ldq8<DK>(K, 32 * ti + l32, 16 * s + 8 * hh), kk);
      }
    }
  };
  uint32_t pgen = 0;                          // chunks prepared so far (uniform)
  constexpr float kLog2e = 1.4426950408889634f;

  // T = (I + A)^{-1} in place of A, in two parts.  The diagonal 16x16 blocks 2 t,
  // 2 t + 1 in fp32, by the wave that emitted diagonal tile t, right after it (lane
  // 16 b' + c of the lower half-wave solves column c of block 2 t + b'); the blocks of
  // A it reads were written by the same wave.
  auto solve_diag = [&](auto parq, int t) __attribute__((always_inline)) {
    constexpr int PQ = decltype(parq)::value;
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    lds_order();
    const int b = 2 * t + ((lane_o >> 4) & 1), c = lane_o & 15;   // (the upper half-wave repeats the lower)
    // The block's entries below the diagonal, row by row in 16-byte pieces, all read
    // up front (no wait for a read between the products), then forward substitution:
    // x_m = [m == c] - sum_{i < m} A_mi x_i.
    const float* Ab = sAd[PQ][b];
    float4 ar[36];
    {
      int k = 0;
#pragma unroll
      for (int mm = 1; mm < 16; ++mm)
#pragma unroll
        for (int q = 0; 4 * q < mm; ++q) ar[k++] = ld_f4(&Ab[20 * mm + 4 * q]);
    }
    float x[16];
    x[0] = c == 0 ? 1.f : 0.f;
    {
      int k = 0;
#pragma unroll
      for (int mm = 1; mm < 16; ++mm) {
        float acc = mm == c ? 1.f : 0.f;
#pragma unroll
        for (int q = 0; 4 * q < mm; ++q) {
          const float4 a4 = ar[k++];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * q + e < mm) acc -= f4get(a4, e) * x[4 * q + e];
        }
        x[mm] = acc;
      }
    }
    if (lane_o < 32) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sTb[PQ][16 * b + i][kperm(16 * b + c)] = f32_to_f16(x[i]);
    }
  };
  // Prepare chunk cp (buffers of parity PQ): its vectors, P (fp16, or bf16 hi + lo), and A stored in
  // T's buffer (fp16, kperm columns) plus A's fp32 diagonal 16x16 blocks.  Roles
  // (pr = wave - NSW):
  //   pr 3:    the chunk's vectors (lane = token): decay cumsum, the coefficient
  //            vectors (with the row norms from the landing) and the decay factors of
  //            the tiles; then the off-diagonal tile (rows 32..63, keys 0..31), whose
  //            decay factors into a row and a key factor split at token 31 (both <= 1);
  //   pr 0, 1: diagonal tile t = pr: its products, then P and A (one exp per
  //            element) and the two diagonal 16x16 blocks of T = (I + A)^{-1} inside it.
  // Entries of A on and above the diagonal are not needed; those inside the diagonal
  // 32x32 tiles come out as zeros or are overwritten by T's diagonal blocks.
  auto produce = [&](int cp, auto parq) __attribute__((always_inline)) {
    constexpr int PQ = decltype(parq)::value;
    const int t0 = tbeg + cp * C, n = min(C, tend - t0);
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int l32 = lane_o & 31, hh = lane_o >> 5;
    const int pr = wu - NSW;
    const u16* Q = sQ[PQ];
    const u16* K = sK[PQ];
    ++pgen;

    // P and A of tile (ti, tj) from its products
    auto emit = [&](auto kdiag, const f32x16& qk, const f32x16& kk) __attribute__((always_inline)) {
      constexpr bool kDiag = decltype(kdiag)::value;
      const int ti = kDiag ? pr : 1, tj = kDiag ? pr : 0;
      const int i = 32 * ti + l32;                                // this lane's row
      const float gi = kDiag ? sEG[i] : 0.f;
      const float rowP = kDiag ? sERp[i] : sEF[i];
      const float rowA = kDiag ? sERa[i] : sEFa[i];
      // every key factor is read before the first store (LDS accesses complete in
      // order: a read after the stores would wait for them)
      float4 kmv[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int mb = 32 * tj + 8 * q4 + 4 * hh;
        kmv[q4] = ld_f4(kDiag ? &sEB[mb] : &sEF[mb]);
      }
      // A's entries inside the diagonal 16x16 blocks: keys 16 (l32 / 16) + 4 hh + 0..3
      // (q4 = 2 (l32 / 16)) and + 8 (q4 + 1) of this lane's row
      f32x4 ad0 = {}, ad1 = {};   // (native vectors: selects of float4 structs go through scratch)
      const bool upper = l32 >= 16;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int mb = 32 * tj + 8 * q4 + 4 * hh;                 // keys mb .. mb + 3
        const float4 km = kmv[q4];
        float pv[4], av[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q4 + e;
          // decay and key norm of (i, m): diagonal tiles take one exp per element,
          // masked before the exp; the off-diagonal tile has them factored
          const float f = kDiag ? __builtin_amdgcn_exp2f(mb + e <= i ? gi - f4get(km, e) : -INFINITY) : f4get(km, e);
          pv[e] = (rowP * f) * qk[r];
          av[e] = (rowA * f) * kk[r];
        }
        if constexpr (kF16) {
          *reinterpret_cast<uint2*>(&sPh[PQ][i][kperm(mb)]) = make_uint2(cvt2h(pv[0], pv[1]), cvt2h(pv[2], pv[3]));
        } else {
          const uint32_t h0 = cvt2(pv[0], pv[1]), h1 = cvt2(pv[2], pv[3]);
          const uint32_t l0 = cvt2(sub_bf_lo(h0, pv[0]), sub_bf_hi(h0, pv[1]));
          const uint32_t l1 = cvt2(sub_bf_lo(h1, pv[2]), sub_bf_hi(h1, pv[3]));
          *reinterpret_cast<uint2*>(&sPh[PQ][i][kperm(mb)]) = make_uint2(h0, h1);
          *reinterpret_cast<uint2*>(&sPl[PQ][i][kperm(mb)]) = make_uint2(l0, l1);
        }
        if constexpr (!kSSD) {
          *reinterpret_cast<uint2*>(&sTb[PQ][i][kperm(mb)]) = make_uint2(cvt2h(av[0], av[1]), cvt2h(av[2], av[3]));
          if constexpr (kDiag) {
            const f32x4 a4 = {av[0], av[1], av[2], av[3]};
            if (q4 == 0) ad0 = a4;
            if (q4 == 1) ad1 = a4;
            if (q4 == 2) ad0 = upper ? a4 : ad0;
            if (q4 == 3) ad1 = upper ? a4 : ad1;
          }
        }
      }
      if constexpr (kDiag && !kSSD) {   // (branch-free: both stores from every lane)
        float* arow = &sAd[PQ][i >> 4][20 * (i & 15) + 4 * hh];
        *reinterpret_cast<f32x4*>(arow) = ad0;
        *reinterpret_cast<f32x4*>(arow + 8) = ad1;
      }
    };

    f32x16 qk, kk;
    if (pr == 3) {
      // cumulative decay within the chunk (padded tokens: log g = 0, beta = 0)
      const int i = lane_o;
      const float bt = i < n ? sBr[PQ][i] : 0.f;
      const float G = wave_inclusive_scan(i < n ? sGr[PQ][i] : 0.f);
      const float GC = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), C - 1));
      const float G31 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), 31));
      // 1 / |row| of q_i and k_i: from the landing (raw bf16 rows, zero past the end);
      // 1 with the fp16 operands, which land normalised (zero rows past the end); the
      // delta-off mode has no norms (zero past the end)
      float rq = 1.f, rk = 1.f;
      if constexpr (kSSD) {
        rq = rk = i < n ? 1.f : 0.f;
      } else if constexpr (!kF16) {
        rq = sRq[PQ][i];
        rk = sRk[PQ][i];
      }
      const float gam = __expf(G);
      sCR[PQ][i] = bt * gam * rk;                   // R = beta V - CR X
      sCO[PQ][i] = p.scale * gam * rq;              // O = CO (Q S0^T) + P U
      sCS[PQ][i] = __expf(GC - G) * rk;             // S1 = gamma_C S0 + K^T diag(CS) U
      if constexpr (kCk) sGc[PQ][i] = G;
      sBeta[PQ][i] = bt;
      if (i == 0) sGC[PQ][0] = __expf(GC);
      const float rowP = p.scale * rq, rowA = bt * rk;
      // diagonal tiles: P_im = rowP_i 2^(EG_i - EB_m) (Q K^T)_im, A likewise with rowA_i
      sEG[i] = G * kLog2e;
      sEB[i] = kF16 ? G * kLog2e : G * kLog2e - __builtin_amdgcn_logf(rk);   // (r_k = 0: +inf, the key drops out)
      sERp[i] = rowP;
      sERa[i] = rowA;
      // off-diagonal tile: exp(G_i - G_m) = exp(G_i - G_31) exp(G_31 - G_m)
      const float F = __expf(i < 32 ? G31 - G : G - G31);
      sEF[i] = (i < 32 ? rk : rowP) * F;
      sEFa[i] = rowA * F;
      arrive(&sSync[0]);
      tile_mma(Q, K, 1, 0, l32, hh, qk, kk);
      emit(std::false_type{}, qk, kk);
    } else {
      tile_mma(Q, K, pr, pr, l32, hh, qk, kk);
      wait_count(&sSync[0], pgen);
      emit(std::true_type{}, qk, kk);
      if constexpr (!kSSD) solve_diag(Par<PQ>{}, pr);
    }
  };

  // Then, early in the step that consumes the chunk, one wave merges them: the two
  // 16 -> 32 merges T10 = -T11 A10 T00 and the 32 -> 64 merge T[32..63][0..31] =
  // -T22 A21 T11.  Each merge reads its A block before it writes the T block in its
  // place.
  auto merge_T = [&](auto parc) __attribute__((always_inline)) {
    constexpr int PAR = decltype(parc)::value;
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int l32 = lane_o & 31, hh = lane_o >> 5;
    const int g16 = lane_o >> 4, j16 = lane_o & 15;
    auto T = sTb[PAR];
#pragma unroll
    for (int t = 0; t < 2; ++t) {   // 16 -> 32 inside diagonal tile t
      const int r0 = 32 * t;
      // B operand: column r0 + j16 of T00, rows r0 + 4 g16 + e (one transpose read)
      const f16x4 bD = __builtin_bit_cast(f16x4, tr_read(&T[r0 + 4 * g16 + (j16 >> 2)][kperm(r0 + 4 * (j16 & 3))]));
      f32x4 y = {};
      y = mfma16h(__builtin_bit_cast(f16x4, *reinterpret_cast<const uint2*>(&T[r0 + 16 + j16][kperm(r0 + 4 * g16)])), bD, y);
      f16x4 yb;
#pragma unroll
      for (int e = 0; e < 4; ++e) yb[e] = (_Float16)y[e];
      f32x4 zz = {};
      zz = mfma16h(__builtin_bit_cast(f16x4, *reinterpret_cast<const uint2*>(&T[r0 + 16 + j16][kperm(r0 + 16 + 4 * g16)])), yb, zz);
#pragma unroll
      for (int e = 0; e < 4; ++e) T[r0 + 16 + 4 * g16 + e][kperm(r0 + j16)] = f32_to_f16(-zz[e]);
    }
    lds_order();
    {   // 32 -> 64
      f32x16 y = {};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        // B operand: column l32 of T11, rows 16 s + 8 hh + 0..7 (two transpose reads; a
        // 16-lane group covers columns 16 (l32 / 16) .. + 15)
        const int cb = kperm((l32 & 16) + 4 * (j16 & 3));
        const f16x8 bT = __builtin_bit_cast(f16x8, join(tr_read(&T[16 * s + 8 * hh + (j16 >> 2)][cb]),
                                                        tr_read(&T[16 * s + 8 * hh + 4 + (j16 >> 2)][cb])));
        const f16x8 a = __builtin_bit_cast(f16x8, join(*reinterpret_cast<const uint2*>(&T[32 + l32][kperm(16 * s + 8 * hh)]),
                                                       *reinterpret_cast<const uint2*>(&T[32 + l32][kperm(16 * s + 8 * hh + 4)])));
        y = mfma32h(a, bT, y);
      }
      f32x16 zz = {};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u16* trow = &T[32 + l32][0];
        const int c0 = 32 + 16 * s + 4 * hh;      // k slots 0..3: columns c0.., 4..7: c0 + 8..
        zz = mfma32h(__builtin_bit_cast(f16x8, join(*reinterpret_cast<const uint2*>(trow + kperm(c0)),
                                                    *reinterpret_cast<const uint2*>(trow + kperm(c0 + 8)))),
                     acc_to_op_h(y, s), zz);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) T[32 + acc_row(r, hh)][kperm(l32)] = f32_to_f16(-zz[r]);
    }
    // the state waves apply L = T - I (U = R + L R): the unit diagonal, needed by
    // the merges above, is stored as zero once they are done
    lds_order();
    T[lane_o][kperm(lane_o)] = 0;
    arrive(&sSync[1]);
  };

  // ================================================================ step loop
  // Step c: the state waves consume chunk c while the producers prepare chunk c + 1.
  // Each role runs its own copy of the loop (kProd): the compiler's count of memory
  // operations in flight, and the waits it derives for the landing, then follow one
  // role's code only.
  auto step = [&](int c, auto parc, auto rolep, auto firstp) __attribute__((always_inline)) {
    constexpr int PAR = decltype(parc)::value;     // parity of chunk c
    constexpr int PQ = PAR ^ 1;                    // parity of chunk c + 1
    constexpr bool kProd = decltype(rolep)::value;
    constexpr bool hasS = !decltype(firstp)::value;   // step -1 has no chunk to consume
    const bool hasP = c + 1 < nch;
    lds_sync();                                    // previous step done (the step's one barrier)
    // Each role lands its staged rows and announces them.  Staging loads are issued
    // unconditionally (past the last chunk they re-read it, unused): a conditional
    // load would merge with the old values and force a wait for it.
    if constexpr (kProd) {
      // Q, K of chunk c + 1 (and, gate not folded in, its log g, beta)
      if (hasP) {
        if constexpr (kSSD) {
          rq_.template store<true>(sQ[PQ], siq);
          rk_.template store<true>(sK[PQ], siq);
        } else {
          land_qk(Par<PQ>{}, min(C, tend - (tbeg + (c + 1) * C)));
        }
      }
      if constexpr (!kGate) {
        if (hasP && wu - NSW == 2) {
          sGr[PQ][lane] = rg_;
          sBr[PQ][lane] = rb_;
        }
      }
      arrive(&sSync[3]);
      if (wu - NSW == 2) {   // T of chunk c (delta rule only); reads nothing landed here
        if constexpr (!kSSD) {
          if constexpr (hasS) merge_T(Par<PAR>{});
        }
        // (staged after the merge: issuing the loads first held T back by their issue
        // time, while the state waves wait for it)
        stage_qk(min(c + 2, nch - 1));
        gate_store(PAR);       // (gate folded in) chunk c + 2, staged just above
      } else {
        stage_qk(min(c + 2, nch - 1));
        if (hasP) {
          wait_count(&sSync[3], (uint32_t)kNP * (uint32_t)(c + 2));   // the producers' landing of this step done
          produce(c + 1, Par<PQ>{});
        }
      }
    } else {
      // V, z of chunk c
      if constexpr (hasS) {
        rv_.template store<false>(sV, siv);
        if constexpr (kSSD) {
          if (p.z) rz_.template store<false>(sZ, siv);
        }
      }
      arrive(&sSync[2]);
      if constexpr (hasS) {
        consume(c, Par<PAR>{});
      } else {   // step -1: no chunk to consume, stage chunk 0's rows here
        stage_v(min(c + 1, nch - 1));
      }
    }
  };

  if (nch > 0 && isP) stage_qk(0);
  if (tid < 8) sSync[tid] = 0u;   // visible to all after the first barrier
  // entry state and first staged loads retired on every path here, so no wait inside
  // the loop has to cover them
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  if (wu == NSW + 2) gate_store(0);    // (gate folded in) chunk 0
  // Step -1 (landing and the first chunk's preparation only) runs before the loop and
  // retires its loads, so that every step inside the loop has the same memory
  // operations in flight at its landing.
  auto run = [&](auto rolep) __attribute__((always_inline)) {
    if (nch == 0) return;   // (an empty sequence only stores its state)
    step(-1, Par<1>{}, rolep, std::true_type{});
    if constexpr (!decltype(rolep)::value) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    for (int c = 0; c < nch; c += 2) {
      step(c, Par<0>{}, rolep, std::false_type{});
      if (c + 1 < nch) step(c + 1, Par<1>{}, rolep, std::false_type{});
    }
  };
  // (each role ends in its own branch: no state-wave value stays live through the
  // producers' loop)
  if (isP) {
    run(std::true_type{});
    lds_sync();   // every wave's last wait is over
    return;
  }
  if (kCk) {   // checkpoint after ck_b tokens, ck_b in [0, len]
    const int tok = p.ck_token[nseq], cks = p.ck_slot[nseq];
    const int b = p.ck_relative ? tok : tok - tbeg;
    if (tok >= 0 && cks >= 0 && b >= 0 && b <= tend - tbeg) {
      ck_b = b;
      ck_st = p.ck_states + ((int64_t)cks * p.H_v + h) * (int64_t)(DV * DK);
    }
  }
  if (ck_b == 0) store_state(ck_st);
  run(std::false_type{});
  if (ck_b > 0 && ck_b == tend - tbeg) store_state(ck_st);
  lds_sync();   // every wave's last wait is over
  if (sSync[kFailFlag] != 0u) {   // a bounded wait ran out: poison this wave's results
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int tk = 0; tk < NTK; ++tk) Sacc[ct][tk] = f32x4{nan, nan, nan, nan};
    OutT* ob = reinterpret_cast<OutT*>(p.out);
    for (int t = tbeg + lane / CW; t < tend; t += kWave / CW)
      Elem<OutT>::store(ob, (int64_t)t * p.out_stride + (int64_t)h * DV + CW * wu + lane % CW, nan);
  }
  if (!p.keep_pool) store_state(state);
}

template <int DK, int DV, bool kSSD, typename OutT, bool kGate, bool kCk>
hipError_t launch_gated(const SeqLaunch& p, hipStream_t stream) {
  constexpr int CT = kSSD ? 1 : 2;   // d_v columns per state wave: 32 (GDN), 16 (delta-off)
  dim3 grid(p.H_v, p.N), block((DV / (16 * CT) + kNP) * kWave);
  hipLaunchKernelGGL((chunk_kernel<DK, DV, kSSD, OutT, CT, kGate, kCk>), grid, block, 0, stream, p);
  return hipGetLastError();
}
// (checkpoint capture is a separate instantiation: calls without it run no trace of it)
template <int DK, int DV, bool kSSD, typename OutT, bool kGate>
hipError_t launch_ck(const SeqLaunch& p, hipStream_t stream) {
  return p.ck_token ? launch_gated<DK, DV, kSSD, OutT, kGate, true>(p, stream)
                    : launch_gated<DK, DV, kSSD, OutT, kGate, false>(p, stream);
}
template <int DK, int DV, bool kSSD, typename OutT>
hipError_t launch_typed(const SeqLaunch& p, hipStream_t stream) {
  return p.gate_fused ? launch_ck<DK, DV, kSSD, OutT, true>(p, stream)
                      : launch_ck<DK, DV, kSSD, OutT, false>(p, stream);
}

}  // namespace

int chunked_obstacles(const SeqLaunch& p) {
  int why = 0;
  if (!p.in_bf16) why |= GDN_WHY_FP32;
  if (p.d_k != 128 || p.d_v != (p.ssd ? 64 : 128)) why |= GDN_WHY_HEAD_DIMS;
  if (p.N > 65535) why |= GDN_WHY_BATCH;
  // 16-byte row segments of q, k, v (z) are staged with single loads
  const uintptr_t ptrs = reinterpret_cast<uintptr_t>(p.q) | reinterpret_cast<uintptr_t>(p.k) |
                         reinterpret_cast<uintptr_t>(p.v) | reinterpret_cast<uintptr_t>(p.z);
  if (ptrs % 16 != 0 || (p.q_stride | p.k_stride | p.v_stride | (p.z ? p.z_stride : 0)) % 8 != 0)
    why |= GDN_WHY_ALIGN;
  // 32-bit row offsets within a chunk (outputs and staged input rows)
  const int64_t lim = (int64_t(1) << 31) / (C * 4);
  if (p.out_stride > lim || p.q_stride > lim || p.k_stride > lim || p.v_stride > lim ||
      (p.z && p.z_stride > lim))
    why |= GDN_WHY_STRIDE;
  // gate folded in: the raw bf16 gate inputs are read as aligned 32-bit words
  if (p.gate_fused) {
    if ((reinterpret_cast<uintptr_t>(p.ga) | reinterpret_cast<uintptr_t>(p.gb)) % 4 != 0 ||
        (p.ga_stride | (p.gb ? p.gb_stride : 0)) % 2 != 0)
      why |= GDN_WHY_GATE_ALIGN;
  }
  return why;
}

hipError_t launch_chunked(const SeqLaunch& p, hipStream_t stream) {
  if (p.N == 0) return hipSuccess;
  if (p.ssd) return p.out_bf16 ? launch_typed<128, 64, true, u16>(p, stream)
                               : launch_typed<128, 64, true, float>(p, stream);
  return p.out_bf16 ? launch_typed<128, 128, false, u16>(p, stream)
                    : launch_typed<128, 128, false, float>(p, stream);
}

}  // namespace gdn
