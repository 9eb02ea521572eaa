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
// starts from its parent's recorded state.
//
// Memory layout: the state row r of (slot, head) is 4*d_k contiguous bytes of the
// pool [slot][head][d_v][d_k]; d_k/4 lanes own one row, each a float4 of it, so a
// wave streams 64 * 16 B = 1 KiB per instruction, fully coalesced.  The state stays
// in registers across the tokens of a sequence and is written back once.  Its loads
// are non-temporal (each byte of the pool is read once per launch); the stores keep
// the default policy (measured faster for an extend + decode step than streaming
// them past the caches).
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;
constexpr int kRowSteps = 4;  // rows per lane

template <int DK>
struct RecLayout {
  static constexpr int kLanesPerRow = DK / 4;                       // float4 per lane
  static constexpr int kRowsPerStep = kWave / kLanesPerRow;         // rows per wave instr
  static constexpr int kRowsPerWave = kRowsPerStep * kRowSteps;
  static constexpr int kRowsPerBlock = kRowsPerWave * (kThreads / kWave);
};

template <typename InT>
__device__ __forceinline__ float4 load4(const InT* p);
template <>
__device__ __forceinline__ float4 load4<float>(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
template <>
__device__ __forceinline__ float4 load4<u16>(const u16* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
}

__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

template <int DK, int DV, typename InT, typename OutT, bool kSSD, bool kAux>
__global__ void __launch_bounds__(kThreads) recurrent_kernel(SeqLaunch p) {
  using L = RecLayout<DK>;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int c = lane % L::kLanesPerRow;       // column group: columns 4c .. 4c+3
  const int rsub = lane / L::kLanesPerRow;
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
  float4 st[kRowSteps];
#pragma unroll
  for (int s = 0; s < kRowSteps; ++s) {
    const int row = row0 + s * L::kRowsPerStep;
    if (init) {
      const nf4 v = __builtin_nontemporal_load(reinterpret_cast<const nf4*>(state + (int64_t)row * DK + 4 * c));
      st[s] = make_float4(v.x, v.y, v.z, v.w);
    } else {
      st[s] = make_float4(0.f, 0.f, 0.f, 0.f);
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
      *reinterpret_cast<float4*>(ckst + (int64_t)(row0 + s * L::kRowsPerStep) * DK + 4 * c) = st[s];
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
  float4 st0[kRowSteps];
#pragma unroll
  for (int s = 0; s < kRowSteps; ++s) st0[s] = kAux ? st[s] : make_float4(0.f, 0.f, 0.f, 0.f);

  const InT* qb = reinterpret_cast<const InT*>(p.q);
  const InT* kb = reinterpret_cast<const InT*>(p.k);
  const InT* vb = reinterpret_cast<const InT*>(p.v);
  OutT* ob = reinterpret_cast<OutT*>(p.out);

  for (int t = t0; t < t1; ++t) {
    if (kAux && p.sp_parent && spr) {   // token tree (uniform branch)
      const int par = p.sp_parent[t];
      if (par < 0) {
#pragma unroll
        for (int s = 0; s < kRowSteps; ++s) st[s] = st0[s];
      } else if (par != t - t0 - 1) {
#pragma unroll
        for (int s = 0; s < kRowSteps; ++s)
          st[s] = *reinterpret_cast<const float4*>(spr + par * sp_step + (int64_t)(row0 + s * L::kRowsPerStep) * DK + 4 * c);
      }
    }
    float4 kv = load4<InT>(kb + (int64_t)t * p.k_stride + (int64_t)j * DK + 4 * c);
    float4 qv = load4<InT>(qb + (int64_t)t * p.q_stride + (int64_t)j * DK + 4 * c);
    if constexpr (!kSSD) {
      const float nk = group_sum<L::kLanesPerRow>(dot4(kv, kv));
      const float nq = group_sum<L::kLanesPerRow>(dot4(qv, qv));
      const float rk = 1.0f / sqrtf(nk + 1e-6f);
      const float rq = 1.0f / sqrtf(nq + 1e-6f);
      kv.x *= rk; kv.y *= rk; kv.z *= rk; kv.w *= rk;
      qv.x *= rq; qv.y *= rq; qv.z *= rq; qv.w *= rq;
    }
    const float kq = group_sum<L::kLanesPerRow>(dot4(kv, qv));
    float lg, bt;
    if (p.gate_fused) {   // the gate's arithmetic on the raw inputs (uniform branch)
      const float x = Elem<InT>::load(reinterpret_cast<const InT*>(p.ga), (int64_t)t * p.ga_stride + h);
      const float bias = p.gdt_bias ? p.gdt_bias[h] : 0.f;
      if constexpr (kSSD)
        gate_ssd(x, p.gA[h], bias, p.g_softplus, p.g_lo, p.g_hi, lg, bt);
      else
        gate_gdn(x, Elem<InT>::load(reinterpret_cast<const InT*>(p.gb), (int64_t)t * p.gb_stride + h),
                 expf(p.gA[h]), bias, lg, bt);
    } else {
      const int64_t gi = (int64_t)t * p.H_v + h;
      lg = p.log_g[gi];
      bt = p.beta[gi];
    }
    const float g = __expf(lg);
    const int64_t vrow = (int64_t)t * p.v_stride + (int64_t)h * DV;
    const int64_t orow = (int64_t)t * p.out_stride + (int64_t)h * DV;
#pragma unroll
    for (int s = 0; s < kRowSteps; ++s) {
      const int row = row0 + s * L::kRowsPerStep;
      const float vr = Elem<InT>::load(vb, vrow + row);
      const float y = group_sum<L::kLanesPerRow>(dot4(st[s], qv));
      float u, o;
      if constexpr (kSSD) {
        u = bt * vr;
        o = g * y + u * kq;
      } else {
        const float x = group_sum<L::kLanesPerRow>(dot4(st[s], kv));
        u = bt * (vr - g * x);
        o = p.scale * (g * y + u * kq);
      }
      st[s].x = g * st[s].x + u * kv.x;
      st[s].y = g * st[s].y + u * kv.y;
      st[s].z = g * st[s].z + u * kv.z;
      st[s].w = g * st[s].w + u * kv.w;
      if constexpr (kSSD) {
        if (p.D) {
          const InT* Db = reinterpret_cast<const InT*>(p.D);
          o += Elem<InT>::load(Db, p.D_per_dim ? (int64_t)h * DV + row : (int64_t)h) * vr;
        }
        if (p.z) {
          const float zz = Elem<InT>::load(reinterpret_cast<const InT*>(p.z),
                                           (int64_t)t * p.z_stride + (int64_t)h * DV + row);
          o *= zz * sigmoid_f(zz);
        }
      }
      if (c == 0) Elem<OutT>::store(ob, orow + row, o);
    }
    if (kAux && t - t0 + 1 == ckb) write_ck();
    if (kAux && spr && t - t0 < p.sp_steps) {
#pragma unroll
      for (int s = 0; s < kRowSteps; ++s)
        *reinterpret_cast<float4*>(spr + (t - t0) * sp_step + (int64_t)(row0 + s * L::kRowsPerStep) * DK + 4 * c) = st[s];
    }
  }
  if (p.keep_pool) return;
#pragma unroll
  for (int s = 0; s < kRowSteps; ++s) {
    const int row = row0 + s * L::kRowsPerStep;
    *reinterpret_cast<float4*>(state + (int64_t)row * DK + 4 * c) = st[s];
  }
}

template <int DK, int DV, typename InT, typename OutT, bool kSSD>
hipError_t launch_typed(const SeqLaunch& p, hipStream_t stream) {
  using L = RecLayout<DK>;
  static_assert(DV % L::kRowsPerBlock == 0, "d_v must be a multiple of the rows per block");
  dim3 grid(DV / L::kRowsPerBlock, p.H_v, p.N), block(kThreads);
  // checkpoints and target-verify states are a separate instantiation: the decode
  // step runs none of their code
  if (p.ck_token || p.sp_states)
    hipLaunchKernelGGL((recurrent_kernel<DK, DV, InT, OutT, kSSD, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((recurrent_kernel<DK, DV, InT, OutT, kSSD, false>), grid, block, 0, stream, p);
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
