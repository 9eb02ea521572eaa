// C-ABI entry points of libgdn.so: host-side validation, then one launch per call.
// Declarations and the contract (ownership, layouts, errors) are in include/gdn.h.
#include "../../include/gdn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>

#include "gdn_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  g_last_hip_error = (int)e;
  return e == hipSuccess ? GDN_OK : GDN_E_HIP;
}

bool dtype_ok(int32_t d) { return d == GDN_F32 || d == GDN_BF16; }
bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }
// A row start aligned to 4 elements of its dtype (null pointers are checked elsewhere).
bool aligned4(const void* ptr, int32_t dtype) {
  const uintptr_t bytes = dtype == GDN_BF16 ? 8 : 16;
  return reinterpret_cast<uintptr_t>(ptr) % bytes == 0;
}

// Checks shared by gdn_extend and gdn_decode; fills everything but the
// per-call index fields.
int check_seq_common(int32_t in_dtype, int32_t out_dtype, int32_t H_qk, int32_t H_v, int32_t d_k,
                     int32_t d_v, int64_t q_stride, int64_t k_stride, int64_t v_stride,
                     int64_t out_stride, int64_t num_slots, float scale) {
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return GDN_E_DTYPE;
  if (H_qk <= 0 || H_v <= 0 || H_v % H_qk != 0) return GDN_E_SHAPE;
  if (!head_dim_ok(d_k) || !head_dim_ok(d_v)) return GDN_E_UNSUPPORTED;
  if (q_stride < (int64_t)H_qk * d_k || k_stride < (int64_t)H_qk * d_k) return GDN_E_SHAPE;
  if (v_stride < (int64_t)H_v * d_v || out_stride < (int64_t)H_v * d_v) return GDN_E_SHAPE;
  // rows are accessed 4 elements at a time
  if ((q_stride | k_stride | v_stride | out_stride) % 4 != 0) return GDN_E_SHAPE;
  if (num_slots <= 0) return GDN_E_SHAPE;
  if (!std::isfinite(scale)) return GDN_E_SHAPE;
  return GDN_OK;
}

// Checks of a gdn_gate_args description of the raw gate inputs (pointers only when
// T > 0); `outputs` asks for the log_g / beta outputs of gdn_gate as well.
int check_gate(const gdn_gate_args* a, bool outputs) {
  if (a->mode != GDN_MODE_GDN && a->mode != GDN_MODE_SSD) return GDN_E_UNSUPPORTED;
  if (!dtype_ok(a->in_dtype)) return GDN_E_DTYPE;
  if (a->T < 0 || a->H <= 0) return GDN_E_SHAPE;
  if (a->T == 0) return GDN_OK;
  if (!a->a || !a->A) return GDN_E_NULL;
  if (outputs && (!a->log_g || !a->beta)) return GDN_E_NULL;
  if (a->a_stride < a->H) return GDN_E_SHAPE;
  if (a->mode == GDN_MODE_GDN) {
    if (!a->b) return GDN_E_NULL;
    if (a->b_stride < a->H) return GDN_E_SHAPE;
  } else {
    if (a->b) return GDN_E_SHAPE;            // SSD mode has no b input
    if (std::isnan(a->dt_min) || std::isnan(a->dt_max) || a->dt_min > a->dt_max)
      return GDN_E_SHAPE;
  }
  return GDN_OK;
}

// The gate of a gated extend / decode call: same mode, dtype and [T, H_v] as the call.
int check_fused_gate(const gdn_gate_args* g, int32_t mode, int32_t in_dtype, int64_t T, int32_t H_v) {
  if (!g) return GDN_E_NULL;
  if (g->mode != mode) return GDN_E_UNSUPPORTED;
  if (g->in_dtype != in_dtype) return GDN_E_DTYPE;
  if (g->T != T || g->H != H_v) return GDN_E_SHAPE;
  return check_gate(g, false);
}

void fill_fused_gate(gdn::SeqLaunch& p, const gdn_gate_args* g) {
  p.gate_fused = 1;
  p.ga = g->a;
  p.ga_stride = g->a_stride;
  p.gb = g->b;
  p.gb_stride = g->b_stride;
  p.gA = g->A;
  p.gdt_bias = g->dt_bias;
  p.g_softplus = g->dt_softplus;
  p.g_lo = g->dt_min;
  p.g_hi = g->dt_max;
}

int plan_extend(const gdn_extend_args* a, const gdn_gate_args* gate, gdn::SeqLaunch& p, int& why);
int extend_impl(const gdn_extend_args* a, const gdn_gate_args* gate, void* stream);
int decode_impl(const gdn_decode_args* a, const gdn_gate_args* gate, void* stream);

// Workspace of gdn_extend_noalloc, for callers that cannot allocate: one copy per
// device, resolved on the first call on that device.  Host code never passes the
// array's name to a kernel or copy (on the host it is only a stand-in for the
// symbol): every use goes through the per-device address that scratch_address gives.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch`.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return GDN_E_UNSUPPORTED;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e);
      if (!ptr || reinterpret_cast<uintptr_t>(ptr) % 256 != 0) return GDN_E_HIP;
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

int gdn_last_hip_error(void) { return g_last_hip_error; }

const char* gdn_status_str(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_E_NULL: return "required pointer is NULL";
    case GDN_E_SHAPE: return "inconsistent sizes or strides";
    case GDN_E_DTYPE: return "unsupported dtype";
    case GDN_E_UNSUPPORTED: return "unsupported configuration";
    case GDN_E_INDEX: return "index argument out of range";
    case GDN_E_HIP: return "HIP runtime error";
    case GDN_E_SCRATCH: return "input needs more than the static scratch of gdn_extend_noalloc";
    default: return "unknown status";
  }
}

int gdn_gate(const gdn_gate_args* a, void* stream) {
  if (!a) return GDN_E_NULL;
  const int st = check_gate(a, true);
  if (st != GDN_OK || a->T == 0) return st;
  gdn::GateLaunch p{};
  p.T = a->T;
  p.H = a->H;
  p.bf16 = a->in_dtype == GDN_BF16;
  p.ssd = a->mode == GDN_MODE_SSD;
  p.a = a->a;
  p.a_stride = a->a_stride;
  p.b = a->b;
  p.b_stride = a->b_stride;
  p.A = a->A;
  p.dt_bias = a->dt_bias;
  p.dt_softplus = a->dt_softplus;
  p.dt_min = a->dt_min;
  p.dt_max = a->dt_max;
  p.log_g = a->log_g;
  p.beta = a->beta;
  return hip_status(gdn::launch_gate(p, (hipStream_t)stream));
}

int gdn_extend(const gdn_extend_args* a, void* stream) { return extend_impl(a, nullptr, stream); }
int gdn_extend_gated(const gdn_extend_args* a, const gdn_gate_args* gate, void* stream) {
  if (!gate) return GDN_E_NULL;
  return extend_impl(a, gate, stream);
}
int gdn_extend_kernel(const gdn_extend_args* a, const gdn_gate_args* gate, int32_t* why) {
  gdn::SeqLaunch p{};
  int w = 0;
  const int k = plan_extend(a, gate, p, w);
  if (why) *why = w;
  return k;
}
int64_t gdn_extend_workspace_size(const gdn_extend_args* a, const gdn_gate_args* gate) {
  if (!a || a->mode != GDN_MODE_SSD || a->chunk == 64 || a->N <= 0) return 0;
  gdn::SeqLaunch p{};
  int w = 0;
  gdn_extend_args probe = *a;                     // as if a large workspace were given
  probe.workspace = reinterpret_cast<void*>(uintptr_t(256));
  probe.workspace_bytes = INT64_MAX;
  if (plan_extend(&probe, gate, p, w) != GDN_KERNEL_SSD_CHUNKED) return 0;
  return gdn::ssd_workspace_bytes(p.T, p.N, p.H_qk, p.H_v, (p.ssd_segs - 1) * p.ssd_sub);
}
int gdn_extend_noalloc(const gdn_extend_args* a, const gdn_gate_args* gate, void* stream) {
  if (!a) return GDN_E_NULL;
  if (a->workspace || a->workspace_bytes != 0) return GDN_E_SHAPE;   // the library supplies it
  // the kernel the allocating entry point takes when given all the workspace it wants
  gdn_extend_args b = *a;
  b.workspace = reinterpret_cast<void*>(uintptr_t(256));
  b.workspace_bytes = INT64_MAX;
  gdn::SeqLaunch p{};
  int why = 0;
  const int k = plan_extend(&b, gate, p, why);
  if (k <= 0) return -k;
  if (k == GDN_KERNEL_SSD_CHUNKED &&
      gdn::ssd_workspace_bytes(p.T, p.N, p.H_qk, p.H_v, 0) > GDN_NOALLOC_SCRATCH_BYTES)
    return GDN_E_SCRATCH;
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != GDN_OK) return st;
  b.workspace = ws;
  b.workspace_bytes = GDN_NOALLOC_SCRATCH_BYTES;
  return extend_impl(&b, gate, stream);
}
int gdn_decode(const gdn_decode_args* a, void* stream) { return decode_impl(a, nullptr, stream); }
int gdn_decode_gated(const gdn_decode_args* a, const gdn_gate_args* gate, void* stream) {
  if (!gate) return GDN_E_NULL;
  return decode_impl(a, gate, stream);
}

}  // extern "C"

namespace {

// Compute units of the current device (cached per device; 256, an MI355X, when the
// runtime cannot tell): the segment plan of the chunk-128 delta-off kernel fills them.
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Segments per sequence for the chunk-128 delta-off kernel, and the pieces the
// state-only pass cuts each of the first segs - 1 into: the pair (s in 1..16, k in 1..4)
// that minimises the estimated makespan in chunk steps -- ceil(N U s / CUs) rounds (U
// the workgroups per sequence and segment, one per pair of heads) of ceil(chunks / s)
// chunk steps for the full pass, plus for s > 1 the state-only pass, ceil(N U (s - 1) k
// / CUs) rounds of ceil(chunks / (s k)) steps (about a third of a full step per chunk;
// smaller pieces fill more CUs) -- among those whose workspace fits in `budget` bytes.
// Unknown lengths (max_seqlen 0): one segment.
void ssd_plan(gdn::SeqLaunch& p, int max_seqlen, int64_t budget) {
  p.ssd_segs = 1;
  p.ssd_seg_chunks = 1 << 30;
  p.ssd_sub = 1;
  if (max_seqlen <= 0) return;
  const int nch = (max_seqlen + 127) / 128;
  const double units = (double)p.N * gdn::ssd_units_per_seq(p), cus = (double)device_cus();
  double best = 1e300;
  for (int s = 1; s <= 16 && s <= nch; ++s) {
    const int sc = (nch + s - 1) / s;
    const int se = (nch + sc - 1) / sc;           // segments that hold chunks
    if ((int64_t)p.N * se > 65535 || gdn::ssd_workspace_bytes(p.T, p.N, p.H_qk, p.H_v, se - 1) > budget) break;
    for (int k = 1; k <= (se > 1 ? 4 : 1) && k <= sc; ++k) {
      const int states = (se - 1) * k;
      if ((int64_t)p.N * states > 65535 || gdn::ssd_workspace_bytes(p.T, p.N, p.H_qk, p.H_v, states) > budget) break;
      // (a segment's workgroup also folds the states before it: about a quarter of a
      // chunk step per pair of them)
      double cost = std::ceil(units * se / cus) * (sc + 0.125 * states);
      if (se > 1) cost += std::ceil(units * states / cus) * ((sc + k - 1) / k) * 0.35;
      if (cost < best * 0.98) {                   // (ties go to fewer segments and pieces)
        best = cost;
        p.ssd_segs = se;
        p.ssd_seg_chunks = se > 1 ? sc : 1 << 30;
        p.ssd_sub = k;
      }
    }
  }
}

// Host-side plan of an extend call: every check, the launch descriptor and the kernel
// choice.  Returns the GDN_KERNEL_* to launch, 0 when the call launches nothing, or
// minus a gdn_status; `why` collects the GDN_WHY_* bits that keep it from the fastest
// kernel of its mode.
int plan_extend(const gdn_extend_args* a, const gdn_gate_args* gate, gdn::SeqLaunch& p, int& why) {
  why = 0;
  if (!a) return -GDN_E_NULL;
  if (a->mode != GDN_MODE_GDN && a->mode != GDN_MODE_SSD) return -GDN_E_UNSUPPORTED;
  int st = check_seq_common(a->in_dtype, a->out_dtype, a->H_qk, a->H_v, a->d_k, a->d_v,
                            a->q_stride, a->k_stride, a->v_stride, a->out_stride, a->num_slots,
                            a->scale);
  if (st != GDN_OK) return -st;
  if (a->N < 0 || a->T < 0 || a->max_seqlen < 0) return -GDN_E_SHAPE;
  const bool ssd = a->mode == GDN_MODE_SSD;
  if (a->chunk != 0 && a->chunk != 64 && !(ssd && a->chunk == 128)) return -GDN_E_UNSUPPORTED;
  if (!ssd && (a->D || a->z)) return -GDN_E_SHAPE;   // SSD-only inputs
  if (a->z && a->z_stride < (int64_t)a->H_v * a->d_v) return -GDN_E_SHAPE;
  if (gate) {
    st = check_fused_gate(gate, a->mode, a->in_dtype, a->T, a->H_v);
    if (st != GDN_OK) return -st;
  }
  // checkpoints: all three pointers or none
  const int nck = (a->ckpt_token != nullptr) + (a->ckpt_slot != nullptr) + (a->ckpt_states != nullptr);
  if (nck != 0 && nck != 3) return -GDN_E_NULL;
  if (a->num_ckpt < 0) return -GDN_E_SHAPE;
  if (nck == 3 && reinterpret_cast<uintptr_t>(a->ckpt_states) % 16 != 0) return -GDN_E_SHAPE;
  // target-verify states: spec_states and spec_slot together; spec_parent needs them
  const bool spec = a->spec_states != nullptr;
  if (spec != (a->spec_slot != nullptr) || (a->spec_parent && !spec)) return -GDN_E_NULL;
  if (spec && (a->num_spec < 0 || a->spec_steps < 1 ||
               reinterpret_cast<uintptr_t>(a->spec_states) % 16 != 0))
    return -GDN_E_SHAPE;
  if (a->workspace_bytes < 0 || reinterpret_cast<uintptr_t>(a->workspace) % 256 != 0) return -GDN_E_SHAPE;
  if (a->N == 0) return 0;
  if (!a->cu_seqlens || !a->slot || !a->pool) return -GDN_E_NULL;
  if (a->T > 0 && (!a->q || !a->k || !a->v || !a->out)) return -GDN_E_NULL;
  if (a->T > 0 && !gate && (!a->log_g || !a->beta)) return -GDN_E_NULL;
  if (a->T > INT32_MAX) return -GDN_E_SHAPE;      // cu_seqlens is int32
  if (!aligned4(a->q, a->in_dtype) || !aligned4(a->k, a->in_dtype) || !aligned4(a->v, a->in_dtype) ||
      !aligned4(a->z, a->in_dtype) || !aligned4(a->out, a->out_dtype) || a->z_stride % 4 != 0 ||
      reinterpret_cast<uintptr_t>(a->pool) % 16 != 0)
    return -GDN_E_SHAPE;

  p = gdn::SeqLaunch{};
  p.ssd = ssd;
  p.in_bf16 = a->in_dtype == GDN_BF16;
  p.out_bf16 = a->out_dtype == GDN_BF16;
  p.N = a->N;
  p.T = a->T;
  p.H_qk = a->H_qk;
  p.H_v = a->H_v;
  p.d_k = a->d_k;
  p.d_v = a->d_v;
  p.q = a->q;
  p.q_stride = a->q_stride;
  p.k = a->k;
  p.k_stride = a->k_stride;
  p.v = a->v;
  p.v_stride = a->v_stride;
  p.log_g = a->log_g;
  p.beta = a->beta;
  p.cu_seqlens = a->cu_seqlens;
  p.slot = a->slot;
  p.has_init = a->has_init;
  p.pool = a->pool;
  p.num_slots = a->num_slots;
  p.out = a->out;
  p.out_stride = a->out_stride;
  p.scale = ssd ? 1.0f : a->scale;
  p.D = a->D;
  p.D_per_dim = a->D_per_dim;
  p.z = a->z;
  p.z_stride = a->z_stride;
  p.max_seqlen = a->max_seqlen;
  if (gate) fill_fused_gate(p, gate);
  if (nck == 3 && a->num_ckpt > 0) {
    p.ck_token = a->ckpt_token;
    p.ck_slot = a->ckpt_slot;
    p.ck_states = a->ckpt_states;
    p.ck_relative = a->ckpt_relative != 0;
  }
  p.keep_pool = a->keep_pool != 0;
  if (spec && a->num_spec > 0) {
    p.sp_states = a->spec_states;
    p.sp_slot = a->spec_slot;
    p.sp_parent = a->spec_parent;
    p.sp_steps = a->spec_steps;
  }
  p.lpt = a->N >= 2 && a->N <= 128;

  const int common = (a->max_seqlen > 0 && a->max_seqlen <= 8 ? GDN_WHY_SHORT : 0) | (spec ? GDN_WHY_VERIFY : 0);
  if (ssd && a->chunk != 64) {                    // the chunk-128 delta-off kernel
    const int w = gdn::ssd_obstacles(p) | common;
    const bool ws = a->workspace && a->workspace_bytes >= gdn::ssd_workspace_bytes(p.T, p.N, p.H_qk, p.H_v, 0);
    if (a->chunk == 128) {
      if (w) return -GDN_E_UNSUPPORTED;
      if (!a->workspace) return -GDN_E_NULL;
      if (!ws) return -GDN_E_SHAPE;
    }
    if (!w && ws) {
      ssd_plan(p, a->max_seqlen, a->workspace_bytes);
      return GDN_KERNEL_SSD_CHUNKED;
    }
    why |= w | (ws ? 0 : GDN_WHY_WORKSPACE);
  } else if (ssd) {
    why |= GDN_WHY_CHUNK;
  }
  const int w = gdn::chunked_obstacles(p) | common;
  why |= w;
  return w ? GDN_KERNEL_RECURRENT : GDN_KERNEL_CHUNKED;
}

int extend_impl(const gdn_extend_args* a, const gdn_gate_args* gate, void* stream) {
  gdn::SeqLaunch p{};
  int why = 0;
  const int k = plan_extend(a, gate, p, why);
  if (k <= 0) return -k;
  switch (k) {
    case GDN_KERNEL_SSD_CHUNKED:
      gdn::ssd_bind_workspace(p, a->workspace);
      return hip_status(gdn::launch_ssd(p, (hipStream_t)stream));
    case GDN_KERNEL_CHUNKED:
      return hip_status(gdn::launch_chunked(p, (hipStream_t)stream));
    default:
      return hip_status(gdn::launch_recurrent(p, (hipStream_t)stream));
  }
}

int decode_impl(const gdn_decode_args* a, const gdn_gate_args* gate, void* stream) {
  if (!a) return GDN_E_NULL;
  int st = check_seq_common(a->in_dtype, a->out_dtype, a->H_qk, a->H_v, a->d_k, a->d_v,
                            a->q_stride, a->k_stride, a->v_stride, a->out_stride, a->num_slots,
                            a->scale);
  if (st != GDN_OK) return st;
  if (a->B < 0) return GDN_E_SHAPE;
  if (gate) {
    st = check_fused_gate(gate, GDN_MODE_GDN, a->in_dtype, a->B, a->H_v);
    if (st != GDN_OK) return st;
  }
  if (a->B == 0) return GDN_OK;
  if (!a->q || !a->k || !a->v || !a->slot || !a->pool || !a->out) return GDN_E_NULL;
  if (!gate && (!a->log_g || !a->beta)) return GDN_E_NULL;
  if (!aligned4(a->q, a->in_dtype) || !aligned4(a->k, a->in_dtype) || !aligned4(a->v, a->in_dtype) ||
      !aligned4(a->out, a->out_dtype) || reinterpret_cast<uintptr_t>(a->pool) % 16 != 0)
    return GDN_E_SHAPE;
  gdn::SeqLaunch p{};
  p.ssd = 0;
  p.in_bf16 = a->in_dtype == GDN_BF16;
  p.out_bf16 = a->out_dtype == GDN_BF16;
  p.N = a->B;
  p.T = a->B;
  p.H_qk = a->H_qk;
  p.H_v = a->H_v;
  p.d_k = a->d_k;
  p.d_v = a->d_v;
  p.q = a->q;
  p.q_stride = a->q_stride;
  p.k = a->k;
  p.k_stride = a->k_stride;
  p.v = a->v;
  p.v_stride = a->v_stride;
  p.log_g = a->log_g;
  p.beta = a->beta;
  p.cu_seqlens = nullptr;   // token b is sequence b
  p.slot = a->slot;
  p.has_init = nullptr;     // always resumes from the pool
  p.pool = a->pool;
  p.num_slots = a->num_slots;
  p.out = a->out;
  p.out_stride = a->out_stride;
  p.scale = a->scale;
  p.max_seqlen = 1;
  if (gate) fill_fused_gate(p, gate);
  return hip_status(gdn::launch_recurrent(p, (hipStream_t)stream));
}

// Short causal conv: host checks shared by gdn_conv1d and gdn_conv1d_update.
bool aligned16(const void* ptr) { return reinterpret_cast<uintptr_t>(ptr) % 16 == 0; }

// Byte ranges [lo, hi) of rows 0..rows-1 of a [rows, width] bf16 matrix with a row stride.
bool rows_overlap(const void* a, int64_t a_rows, int64_t a_stride, int64_t a_width, const void* b,
                  int64_t b_rows, int64_t b_stride, int64_t b_width) {
  if (a_rows <= 0 || b_rows <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  const uintptr_t a1 = a0 + (uintptr_t)((a_rows - 1) * a_stride + a_width) * 2;
  const uintptr_t b1 = b0 + (uintptr_t)((b_rows - 1) * b_stride + b_width) * 2;
  return a0 < b1 && b0 < a1;
}

int conv_impl(const gdn_conv_args* a, bool update, void* stream) {
  if (!a) return GDN_E_NULL;
  if (a->dtype != GDN_BF16) return GDN_E_DTYPE;
  if (a->K < 2 || a->K > 4) return GDN_E_UNSUPPORTED;
  if (a->N < 0 || a->T < 0 || a->T > INT32_MAX || a->D < 8 || a->D % 8 != 0 ||
      a->D > (int64_t)INT32_MAX / 8 || a->num_slots <= 0)
    return GDN_E_SHAPE;
  if (update ? a->T != a->N : (a->N == 0 && a->T != 0)) return GDN_E_SHAPE;
  if (a->x_stride < a->D || a->x_stride % 8 != 0 || a->out_stride < a->D || a->out_stride % 8 != 0 ||
      a->pool_stride < a->D * (a->K - 1) || a->pool_stride % 8 != 0)
    return GDN_E_SHAPE;
  if (!update && a->parent && !a->keep_pool) return GDN_E_SHAPE;   // a tree keeps the pool
  if (a->N == 0) return GDN_OK;
  if (!a->weight || !a->slot || !a->pool || (!update && !a->cu_seqlens)) return GDN_E_NULL;
  if (a->T > 0 && (!a->x || !a->out)) return GDN_E_NULL;
  if (!aligned16(a->x) || !aligned16(a->out) || !aligned16(a->weight) || !aligned16(a->bias) ||
      !aligned16(a->pool))
    return GDN_E_SHAPE;
  if (!update) {
    // out rows are written while later tiles still read x rows before them, and the
    // pool is read by the output pass: out may overlap neither
    if (rows_overlap(a->out, a->T, a->out_stride, a->D, a->x, a->T, a->x_stride, a->D) ||
        rows_overlap(a->out, a->T, a->out_stride, a->D, a->pool, a->num_slots, a->pool_stride,
                     a->D * (a->K - 1)))
      return GDN_E_SHAPE;
  }
  gdn::ConvLaunch p{};
  p.K = a->K;
  p.act = a->activation != 0;
  p.T = a->T;
  p.N = a->N;
  p.D = (int)a->D;
  p.x = static_cast<const uint16_t*>(a->x);
  p.x_stride = a->x_stride;
  p.weight = static_cast<const uint16_t*>(a->weight);
  p.bias = static_cast<const uint16_t*>(a->bias);
  p.cu = a->cu_seqlens;
  p.slot = a->slot;
  p.has_init = a->has_init;
  p.pool = static_cast<uint16_t*>(a->pool);
  p.pool_stride = a->pool_stride;
  p.out = static_cast<uint16_t*>(a->out);
  p.out_stride = a->out_stride;
  p.keep_pool = a->keep_pool != 0;
  p.parent = update ? nullptr : a->parent;
  return hip_status(update ? gdn::launch_conv_update(p, (hipStream_t)stream)
                           : gdn::launch_conv(p, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int gdn_conv1d(const gdn_conv_args* a, void* stream) { return conv_impl(a, false, stream); }
int gdn_conv1d_update(const gdn_conv_args* a, void* stream) { return conv_impl(a, true, stream); }

int gdn_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst) return GDN_E_NULL;
  const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
  if (bytes <= 0 || bytes % 16 != 0 || (s | d) % 16 != 0) return GDN_E_SHAPE;
  if (s != d && (s < d ? d - s : s - d) < (uint64_t)bytes) return GDN_E_SHAPE;   // partial overlap
  return hip_status(gdn::launch_copy_probe(src, dst, bytes, (hipStream_t)stream));
}
int gdn_probe_mfma(float* out, int32_t blocks, int32_t iters, void* stream) {
  if (!out) return GDN_E_NULL;
  if (blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 20)) return GDN_E_SHAPE;
  return hip_status(gdn::launch_mfma_probe(out, blocks, iters, (hipStream_t)stream));
}
int gdn_validate_slots(const int32_t* slot, int32_t n, int64_t num_slots, int32_t* flag,
                       void* stream) {
  if (!flag) return GDN_E_NULL;
  if (n < 0 || num_slots <= 0) return GDN_E_SHAPE;
  if (n > 0 && !slot) return GDN_E_NULL;
  return hip_status(gdn::launch_validate_slots(slot, n, num_slots, flag, (hipStream_t)stream));
}

}  // extern "C"
