// Token-recurrent GDN kernel: the decode step, short extends and fp32 inputs.
//
// Per (sequence, v-head, row r of the [d_v, d_k] state), one token at a time:
//   x = S_r . khat,  y = S_r . qhat                       (one read of the row)
//   u = beta (v_r - g x)                                    (delta rule, GDN mode)
//   o_r = scale (g y + u (khat . qhat))                     (= scale * S_t qhat)
//   S_r <- g S_r + u khat^T
// which is S_t = g S_{t-1} (I - beta khat khat^T) + beta v khat^T, o_t = scale S_t qhat
// (gated delta rule, Gated DeltaNet, ICLR 2025) with both dot products taken from
// the same read of S_{t-1}.  Delta-off mode (flashinfer.mamba.ssd_combined_fwd
// semantics): u = beta v_r (beta = dt'), no L2 norm, then o += D v and o *= silu(z).
// A requested state checkpoint is the state after the sequence's first b tokens
// (the lane's rows, written when token b - 1 is done, or before the first token).
// Target verify records the state after every token; with a token tree each token
// starts from its parent's recorded state (a parent outside [0, index) or past the
// recorded steps: from the start state).
//
// Memory layout: the state row r of (slot, head) is 4*d_k contiguous bytes of the
// pool [slot][head][d_v][d_k].  A decode step (one token) gives a row to d_k/4 lanes,
// each a float4 of it, so a wave streams 64 * 16 B = 1 KiB per instruction, fully
// coalesced.  Short extends (a verify batch: a few tokens per sequence, where the
// token loop's arithmetic rather than the state's traffic sets the time) give a row
// to 16 lanes, each d_k/64 float4 of it (columns 4 (c + 16 f)): the per-row sums then
// take four lane steps instead of five (no cross-row permute), and the per-token work
// every wave repeats (the norms, q.k, the gate) is shared by twice the rows.  The
// state stays in registers across the tokens of a sequence and is written back once.
// Its loads are non-temporal (each byte of the pool is read once per launch); the
// stores keep the default policy (measured faster for an extend + decode step than
// streaming them past the caches).
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;
constexpr int kRowSteps = 4;  // rows per lane

// LR lanes own a row, each kVec float4 of it
template <int DK, int LR>
struct RecLayout {
  static constexpr int kLanesPerRow = LR;
  static constexpr int kVec = DK / (4 * LR);                        // float4 per lane and row
  static constexpr int kRowsPerStep = kWave / kLanesPerRow;         // rows per wave instr
  static constexpr int kRowsPerWave = kRowsPerStep * kRowSteps;
  static constexpr int kRowsPerBlock = kRowsPerWave * (kThreads / kWave);
  static_assert(kVec * 4 * LR == DK, "whole float4 per lane");
};

// Four consecutive inputs as loaded (bf16 kept packed until used: a staged token then
// holds half the registers) and as float4.
template <typename InT>
struct Raw4;
template <>
struct Raw4<float> {
  typedef float4 type;
  __device__ __forceinline__ static float4 load(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ static float4 cvt(float4 v) { return v; }
};
template <>
struct Raw4<u16> {
  typedef uint2 type;
  __device__ __forceinline__ static uint2 load(const u16* p) { return *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ static float4 cvt(uint2 w) {
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
  }
};

__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

// (Short extends without checkpoints or speculative states: at most 128 VGPRs, four
// waves per SIMD instead of three -- one more workgroup per CU in flight, ~2% faster
// on a 32 x 4 verify batch, same results; with them the bound would spill.)
template <int DK, int DV, typename InT, typename OutT, bool kSSD, bool kAux, int kPre, int LR>
__global__ void __launch_bounds__(kThreads, (kPre > 1 && !kAux ? 4 : 1)) recurrent_kernel(SeqLaunch p) {
  using L = RecLayout<DK, LR>;
  constexpr int V = L::kVec;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int c = lane % L::kLanesPerRow;       // column groups: columns 4 (c + LR f) .. + 3, f < V
  const int rsub = lane / L::kLanesPerRow;
  auto col = [&](int f) { return 4 * (c + LR * f); };
  const int h = blockIdx.y;
  const int n = blockIdx.z;
  const int row0 = blockIdx.x * L::kRowsPerBlock + wave * L::kRowsPerWave + rsub;

  const int sl = p.slot[n];
  if (sl < 0) return;                           // disabled sequence: nothing is touched
  int t0 = n, t1 = n + 1;
  if (p.cu_seqlens) { t0 = p.cu_seqlens[n]; t1 = p.cu_seqlens[n + 1]; }
  const bool init = p.has_init ? (p.has_init[n] != 0) : true;
  const int j = h / (p.H_v / p.H_qk);          // qk-head of this v-head

  float* state = p.pool + ((int64_t)sl * p.H_v + h) * (int64_t)(DV * DK);
  typedef float nf4 __attribute__((ext_vector_type(4)));   // (the nontemporal builtin takes native vectors)
  float4 st[kRowSteps][V];
#pragma unroll
  for (int s = 0; s < kRowSteps; ++s) {
    const int row = row0 + s * L::kRowsPerStep;
#pragma unroll
    for (int f = 0; f < V; ++f) {
      if (init) {
        const nf4 v = __builtin_nontemporal_load(reinterpret_cast<const nf4*>(state + (int64_t)row * DK + col(f)));
        st[s][f] = make_float4(v.x, v.y, v.z, v.w);
      } else {
        st[s][f] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }

  // state checkpoint: the state after ckb tokens of the sequence (ckb in [0, len])
  int ckb = -1;
  float* ckst = nullptr;
  if (kAux && p.ck_token) {
    const int tok = p.ck_token[n], cks = p.ck_slot[n];
    const int b = p.ck_relative ? tok : tok - t0;
    if (tok >= 0 && cks >= 0 && b >= 0 && b <= t1 - t0) {
      ckb = b;
      ckst = p.ck_states + ((int64_t)cks * p.H_v + h) * (int64_t)(DV * DK);
    }
  }
  auto write_ck = [&]() {
#pragma unroll
    for (int s = 0; s < kRowSteps; ++s)
#pragma unroll
      for (int f = 0; f < V; ++f)
        *reinterpret_cast<float4*>(ckst + (int64_t)(row0 + s * L::kRowsPerStep) * DK + col(f)) = st[s][f];
  };
  if (kAux && ckb == 0) write_ck();
  // target-verify states: the state after token i goes to row spr, step i; with a
  // token tree each token starts from its parent's recorded state (rows this thread
  // wrote itself) or from the start state
  float* spr = nullptr;
  if (kAux && p.sp_states) {
    const int r = p.sp_slot[n];
    if (r >= 0) spr = p.sp_states + (int64_t)r * p.sp_steps * p.H_v * (DV * DK) + (int64_t)h * (DV * DK);
  }
  const int64_t sp_step = (int64_t)p.H_v * (DV * DK);
  float4 st0[kRowSteps][V];
#pragma unroll
  for (int s = 0; s < kRowSteps; ++s)
#pragma unroll
    for (int f = 0; f < V; ++f) st0[s][f] = kAux ? st[s][f] : make_float4(0.f, 0.f, 0.f, 0.f);

  const InT* qb = reinterpret_cast<const InT*>(p.q);
  const InT* kb = reinterpret_cast<const InT*>(p.k);
  const InT* vb = reinterpret_cast<const InT*>(p.v);
  OutT* ob = reinterpret_cast<OutT*>(p.out);
  // delta-off D of this lane's rows (constant over the tokens)
  float Dr[kRowSteps];
#pragma unroll
  for (int s = 0; s < kRowSteps; ++s) {
    Dr[s] = 0.f;
    if (kSSD && p.D) {
      const int row = row0 + s * L::kRowsPerStep;
      Dr[s] = Elem<InT>::load(reinterpret_cast<const InT*>(p.D), p.D_per_dim ? (int64_t)h * DV + row : (int64_t)h);
    }
  }

  // A token's inputs: this lane's columns of k and q, its rows' v (and z), the gate's
  // inputs (raw a, b / dt with the gate folded in, else log g and beta).
  struct Tok {
    typename Raw4<InT>::type k[V], q[V];
    float v[kRowSteps], z[kRowSteps];
    float a, b;
  };
  auto load_tok = [&](int t, Tok& in) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < V; ++f) {
      in.k[f] = Raw4<InT>::load(kb + (int64_t)t * p.k_stride + (int64_t)j * DK + col(f));
      in.q[f] = Raw4<InT>::load(qb + (int64_t)t * p.q_stride + (int64_t)j * DK + col(f));
    }
    const int64_t vrow = (int64_t)t * p.v_stride + (int64_t)h * DV;
#pragma unroll
    for (int s = 0; s < kRowSteps; ++s) {
      const int row = row0 + s * L::kRowsPerStep;
      in.v[s] = Elem<InT>::load(vb, vrow + row);
      in.z[s] = 0.f;
      if (kSSD && p.z)
        in.z[s] = Elem<InT>::load(reinterpret_cast<const InT*>(p.z), (int64_t)t * p.z_stride + (int64_t)h * DV + row);
    }
    if (p.gate_fused) {   // (uniform branch)
      in.a = Elem<InT>::load(reinterpret_cast<const InT*>(p.ga), (int64_t)t * p.ga_stride + h);
      in.b = kSSD ? 0.f : Elem<InT>::load(reinterpret_cast<const InT*>(p.gb), (int64_t)t * p.gb_stride + h);
    } else {
      const int64_t gi = (int64_t)t * p.H_v + h;
      in.a = p.log_g[gi];
      in.b = p.beta[gi];
    }
  };

  // this lane's part of a row dot product (its V float4 of the row)
  auto dotv = [&](const float4* a, const float4* b) __attribute__((always_inline)) {
    float d = dot4(a[0], b[0]);
#pragma unroll
    for (int f = 1; f < V; ++f) d += dot4(a[f], b[f]);
    return d;
  };
  // A token's scalars, the same for every row: 1 / |k|, 1 / |q| (1 in delta-off mode),
  // khat . qhat, log g and beta.  Every lane group of a row computes them for the token
  // whose inputs its lanes hold (the staged tokens of a short extend, one per group).
  struct TokS {
    float rk, rq, kq, lg, bt;
  };
  auto scalars = [&](const typename Raw4<InT>::type* kr, const typename Raw4<InT>::type* qr, float a, float b)
      __attribute__((always_inline)) {
    TokS sc;
    float4 kv[V], qv[V];
#pragma unroll
    for (int f = 0; f < V; ++f) {
      kv[f] = Raw4<InT>::cvt(kr[f]);
      qv[f] = Raw4<InT>::cvt(qr[f]);
    }
    sc.rk = sc.rq = 1.f;
    if constexpr (!kSSD) {
      const float nk = group_sum<L::kLanesPerRow>(dotv(kv, kv));
      const float nq = group_sum<L::kLanesPerRow>(dotv(qv, qv));
      sc.rk = __builtin_amdgcn_rsqf(nk + 1e-6f);   // (1 ulp, as the chunked kernel's norms)
      sc.rq = __builtin_amdgcn_rsqf(nq + 1e-6f);
    }
    sc.kq = group_sum<L::kLanesPerRow>(dotv(kv, qv)) * sc.rk * sc.rq;
    if (p.gate_fused) {   // the gate's arithmetic on the raw inputs (uniform branch)
      const float bias = p.gdt_bias ? p.gdt_bias[h] : 0.f;
      if constexpr (kSSD)
        gate_ssd(a, p.gA[h], bias, p.g_softplus, p.g_lo, p.g_hi, sc.lg, sc.bt);
      else
        gate_gdn(a, b, expf(p.gA[h]), bias, sc.lg, sc.bt);
    } else {
      sc.lg = a;
      sc.bt = b;
    }
    return sc;
  };

  // step(t, in, hasp, sc): with hasp (std::true_type) the token's scalars come in sc,
  // else the step computes them itself (the decode step: its inputs' conversion and
  // normalisation then serve the scalars and the rows alike)
  auto step = [&](int t, const Tok& in, auto hasp, const TokS& sc) __attribute__((always_inline)) {
    constexpr bool kHasS = decltype(hasp)::value;
    if (kAux && p.sp_parent && spr) {   // token tree (uniform branch)
      // a parent outside [0, i) (i = the token's index in its sequence) or past the
      // recorded steps counts as -1: only rows this thread wrote earlier are read
      const int par = p.sp_parent[t];
      if (par < 0 || par >= t - t0 || par >= p.sp_steps) {
#pragma unroll
        for (int s = 0; s < kRowSteps; ++s)
#pragma unroll
          for (int f = 0; f < V; ++f) st[s][f] = st0[s][f];
      } else if (par != t - t0 - 1) {
#pragma unroll
        for (int s = 0; s < kRowSteps; ++s)
#pragma unroll
          for (int f = 0; f < V; ++f)
            st[s][f] = *reinterpret_cast<const float4*>(spr + par * sp_step + (int64_t)(row0 + s * L::kRowsPerStep) * DK + col(f));
      }
    }
    float4 kv[V], qv[V];
#pragma unroll
    for (int f = 0; f < V; ++f) {
      kv[f] = Raw4<InT>::cvt(in.k[f]);
      qv[f] = Raw4<InT>::cvt(in.q[f]);
    }
    float rk = 1.f, rq = 1.f;
    if constexpr (!kSSD) {
      if constexpr (kHasS) {
        rk = sc.rk;
        rq = sc.rq;
      } else {
        const float nk = group_sum<L::kLanesPerRow>(dotv(kv, kv));
        const float nq = group_sum<L::kLanesPerRow>(dotv(qv, qv));
        rk = __builtin_amdgcn_rsqf(nk + 1e-6f);   // (1 ulp, as the chunked kernel's norms)
        rq = __builtin_amdgcn_rsqf(nq + 1e-6f);
      }
#pragma unroll
      for (int f = 0; f < V; ++f) {
        kv[f].x *= rk; kv[f].y *= rk; kv[f].z *= rk; kv[f].w *= rk;
        qv[f].x *= rq; qv[f].y *= rq; qv[f].z *= rq; qv[f].w *= rq;
      }
    }
    float kq, lg, bt;
    if constexpr (kHasS) {
      kq = sc.kq;
      lg = sc.lg;
      bt = sc.bt;
    } else {
      kq = group_sum<L::kLanesPerRow>(dotv(kv, qv));
      if (p.gate_fused) {   // the gate's arithmetic on the raw inputs (uniform branch)
        const float bias = p.gdt_bias ? p.gdt_bias[h] : 0.f;
        if constexpr (kSSD)
          gate_ssd(in.a, p.gA[h], bias, p.g_softplus, p.g_lo, p.g_hi, lg, bt);
        else
          gate_gdn(in.a, in.b, expf(p.gA[h]), bias, lg, bt);
      } else {
        lg = in.a;
        bt = in.b;
      }
    }
    const float g = __expf(lg);
    const int64_t orow = (int64_t)t * p.out_stride + (int64_t)h * DV;
#pragma unroll
    for (int s = 0; s < kRowSteps; ++s) {
      const int row = row0 + s * L::kRowsPerStep;
      const float vr = in.v[s];
      const float y = group_sum<L::kLanesPerRow>(dotv(st[s], qv));
      float u, o;
      if constexpr (kSSD) {
        u = bt * vr;
        o = g * y + u * kq;
      } else {
        const float x = group_sum<L::kLanesPerRow>(dotv(st[s], kv));
        u = bt * (vr - g * x);
        o = p.scale * (g * y + u * kq);
      }
#pragma unroll
      for (int f = 0; f < V; ++f) {
        st[s][f].x = g * st[s][f].x + u * kv[f].x;
        st[s][f].y = g * st[s][f].y + u * kv[f].y;
        st[s][f].z = g * st[s][f].z + u * kv[f].z;
        st[s][f].w = g * st[s][f].w + u * kv[f].w;
      }
      if constexpr (kSSD) {
        o += Dr[s] * vr;
        if (p.z) o *= in.z[s] * sigmoid_f(in.z[s]);
      }
      if (c == 0) Elem<OutT>::store(ob, orow + row, o);
    }
    if (kAux && t - t0 + 1 == ckb) write_ck();
    if (kAux && spr && t - t0 < p.sp_steps) {
#pragma unroll
      for (int s = 0; s < kRowSteps; ++s)
#pragma unroll
        for (int f = 0; f < V; ++f)
          *reinterpret_cast<float4*>(spr + (t - t0) * sp_step + (int64_t)(row0 + s * L::kRowsPerStep) * DK + col(f)) = st[s][f];
    }
  };

  // The first kPre tokens' inputs are loaded together (issued right after the state's
  // loads), so that a short extend (a verify batch) waits for memory once rather than
  // once per token; later tokens load as they come.  (A decode step, one token per
  // sequence, takes kPre = 1: registers for more would cost occupancy.)
  Tok pre[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    if constexpr (kPre > 1) pre[i] = Tok{};   // (tokens past the end join the scalars' pass below)
    if (t0 + i < t1) load_tok(t0 + i, pre[i]);
  }
  if constexpr (kPre > 1) {
    // The staged tokens' scalars in one pass: the lane group of row r takes token r
    // (its lanes hold every token's columns), then each token's values go to all lanes.
    static_assert(L::kRowsPerStep == kPre, "one lane group per staged token");
    typename Raw4<InT>::type kr[V], qr[V];
    float a = pre[0].a, b = pre[0].b;
#pragma unroll
    for (int f = 0; f < V; ++f) {
      kr[f] = pre[0].k[f];
      qr[f] = pre[0].q[f];
    }
#pragma unroll
    for (int i = 1; i < kPre; ++i)
      if (rsub == i) {
#pragma unroll
        for (int f = 0; f < V; ++f) {
          kr[f] = pre[i].k[f];
          qr[f] = pre[i].q[f];
        }
        a = pre[i].a;
        b = pre[i].b;
      }
    const TokS mine = scalars(kr, qr, a, b);
    auto bcast = [&](float v, int i) {
      return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), L::kLanesPerRow * i));
    };
#pragma unroll
    for (int i = 0; i < kPre; ++i)
      if (t0 + i < t1) {
        const TokS sc = {bcast(mine.rk, i), bcast(mine.rq, i), bcast(mine.kq, i), bcast(mine.lg, i), bcast(mine.bt, i)};
        step(t0 + i, pre[i], std::true_type{}, sc);
      }
  } else {
    if (t0 < t1) step(t0, pre[0], std::false_type{}, TokS{});
  }
  for (int t = t0 + kPre; t < t1; ++t) {
    Tok in;
    load_tok(t, in);
    step(t, in, std::false_type{}, TokS{});
  }
  if (p.keep_pool) return;
#pragma unroll
  for (int s = 0; s < kRowSteps; ++s) {
    const int row = row0 + s * L::kRowsPerStep;
#pragma unroll
    for (int f = 0; f < V; ++f) *reinterpret_cast<float4*>(state + (int64_t)row * DK + col(f)) = st[s][f];
  }
}

template <int DK, int DV, typename InT, typename OutT, bool kSSD>
hipError_t launch_typed(const SeqLaunch& p, hipStream_t stream) {
  constexpr int LRd = DK / 4;                  // decode layout: a float4 per lane and row
  constexpr int LRs = DK / 4 < 16 ? DK / 4 : 16;   // short extends: 16 lanes per row
  static_assert(DV % RecLayout<DK, LRd>::kRowsPerBlock == 0 && DV % RecLayout<DK, LRs>::kRowsPerBlock == 0,
                "d_v must be a multiple of the rows per block");
  const dim3 gd(DV / RecLayout<DK, LRd>::kRowsPerBlock, p.H_v, p.N);
  const dim3 gs(DV / RecLayout<DK, LRs>::kRowsPerBlock, p.H_v, p.N), block(kThreads);
  // checkpoints and target-verify states are a separate instantiation: the decode
  // step runs none of their code; short extends (at most 8 tokens per sequence by the
  // host's hint) load their first 4 tokens' inputs up front
  const bool aux = p.ck_token || p.sp_states;
  const bool shrt = p.max_seqlen > 1 && p.max_seqlen <= 8;
  if (aux && shrt)
    hipLaunchKernelGGL((recurrent_kernel<DK, DV, InT, OutT, kSSD, true, 4, LRs>), gs, block, 0, stream, p);
  else if (aux)
    hipLaunchKernelGGL((recurrent_kernel<DK, DV, InT, OutT, kSSD, true, 1, LRd>), gd, block, 0, stream, p);
  else if (shrt)
    hipLaunchKernelGGL((recurrent_kernel<DK, DV, InT, OutT, kSSD, false, 4, LRs>), gs, block, 0, stream, p);
  else
    hipLaunchKernelGGL((recurrent_kernel<DK, DV, InT, OutT, kSSD, false, 1, LRd>), gd, block, 0, stream, p);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_dims(const SeqLaunch& p, hipStream_t stream) {
  if (p.in_bf16) {
    if (p.out_bf16) return p.ssd ? launch_typed<DK, DV, u16, u16, true>(p, stream)
                                 : launch_typed<DK, DV, u16, u16, false>(p, stream);
    return p.ssd ? launch_typed<DK, DV, u16, float, true>(p, stream)
                 : launch_typed<DK, DV, u16, float, false>(p, stream);
  }
  if (p.out_bf16) return p.ssd ? launch_typed<DK, DV, float, u16, true>(p, stream)
                               : launch_typed<DK, DV, float, u16, false>(p, stream);
  return p.ssd ? launch_typed<DK, DV, float, float, true>(p, stream)
               : launch_typed<DK, DV, float, float, false>(p, stream);
}

}  // namespace

hipError_t launch_recurrent(const SeqLaunch& p, hipStream_t stream) {
  if (p.N == 0) return hipSuccess;
  if (p.d_k == 128 && p.d_v == 128) return launch_dims<128, 128>(p, stream);
  if (p.d_k == 128 && p.d_v == 64) return launch_dims<128, 64>(p, stream);
  if (p.d_k == 64 && p.d_v == 64) return launch_dims<64, 64>(p, stream);
  if (p.d_k == 64 && p.d_v == 128) return launch_dims<64, 128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
