// Internal launch descriptors between the C-ABI layer (gdn_abi.cpp) and the kernels.
// Validation happens before these are filled; the kernels trust them.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"
#include "gdn_common.h"

namespace gdn {

struct GateLaunch {
  int64_t T;
  int H;
  int bf16;                 // a/b stored as bf16 (else fp32)
  int ssd;                  // delta-off mode
  const void* a;
  int64_t a_stride;
  const void* b;
  int64_t b_stride;
  const float* A;           // GDN: A_log; SSD: A
  const float* dt_bias;     // may be null
  int dt_softplus;
  float dt_min, dt_max;
  float* log_g;
  float* beta;
};

// One packed-varlen call: sequence n owns tokens [cu[n], cu[n+1]) (or token n
// when cu is null), starts from pool[slot[n]] (zeros when has_init[n] == 0) and
// writes its final state back to pool[slot[n]]; slot[n] < 0 skips it.
struct SeqLaunch {
  int ssd;                  // delta-off mode: no delta rule, no L2 norm, D and z epilogue
  int in_bf16;              // q/k/v/z/D stored as bf16 (else fp32)
  int out_bf16;             // out stored as bf16 (else fp32)
  int N;
  int64_t T;
  int H_qk, H_v, d_k, d_v;
  const void* q;
  int64_t q_stride;         // elements between tokens; heads contiguous (stride d_k)
  const void* k;
  int64_t k_stride;
  const void* v;
  int64_t v_stride;         // heads contiguous (stride d_v)
  const float* log_g;       // [T, H_v]
  const float* beta;        // [T, H_v]
  const int32_t* cu_seqlens;  // [N+1] or null (unit lengths)
  const int32_t* slot;        // [N]
  const int32_t* has_init;    // [N] or null (all 1)
  float* pool;                // [num_slots, H_v, d_v, d_k]
  int64_t num_slots;
  void* out;                  // [T, H_v, d_v]
  int64_t out_stride;
  float scale;
  const void* D;              // delta-off: [H_v] or [H_v, d_v], or null
  int D_per_dim;
  const void* z;              // delta-off: like v, or null
  int64_t z_stride;
  int max_seqlen;             // host hint, 0 = unknown
  // Gate folded in (gate_fused != 0): log g and beta are computed from these raw
  // inputs (in_dtype, [T, H_v] with the given row strides) instead of read from
  // log_g / beta, with the gate kernel's arithmetic.
  int gate_fused;
  const void* ga;             // GDN: a; SSD: dt
  int64_t ga_stride;
  const void* gb;             // GDN: b; SSD: null
  int64_t gb_stride;
  const float* gA;            // [H_v]: GDN A_log, SSD A
  const float* gdt_bias;      // [H_v] or null
  int g_softplus;
  float g_lo, g_hi;
  // State checkpoints (ck_token null = none): sequence n with a boundary b in
  // [0, len] (absolute ck_token[n] - cu[n], or ck_token[n] when ck_relative) and
  // ck_slot[n] >= 0 writes its state after b tokens to ck_states[ck_slot[n]].
  const int32_t* ck_token;    // [N]
  const int32_t* ck_slot;     // [N]
  float* ck_states;           // [*, H_v, d_v, d_k]
  int ck_relative;
  // Target-verify states (token-recurrent kernel only): the state after token i of
  // sequence n goes to sp_states[sp_slot[n], i] (i < sp_steps); with sp_parent a
  // token starts from its parent's recorded state (-1: the start state).  keep_pool:
  // the pool is not written.
  float* sp_states;           // [*, sp_steps, H_v, d_v, d_k] or null
  const int32_t* sp_slot;     // [N]
  const int32_t* sp_parent;   // [T] or null
  int sp_steps;
  int keep_pool;
  int lpt;                    // chunked kernel: longest sequences first (small N)
  // Chunk-128 delta-off kernel: fp16 copies of B (k) and C (q), [T, H_qk, d_k], and the
  // chunks' raw C B^T tiles, in the caller's workspace; each sequence cut into ssd_segs
  // segments of ssd_seg_chunks chunks (the last takes the rest).  The state-only pass
  // cuts each of the first segs - 1 segments into ssd_sub pieces and writes their
  // states segR [N, (segs - 1) ssd_sub, H_v, d_v, d_k] and log decays
  // segL [N, (segs - 1) ssd_sub, H_v], in token order.
  const u16* ssd_Bh;
  const u16* ssd_Ch;
  const u16* ssd_CB;          // raw C B^T tiles per chunk slot and group (fp16)
  float* segR;
  float* segL;
  int ssd_segs;
  int ssd_seg_chunks;
  int ssd_sub;
};

// Short causal conv1d (bf16, width K) over packed sequences with a conv-state pool.
struct ConvLaunch {
  int K;
  int act;                     // silu after the sum
  int64_t T;
  int N;
  int D;
  const uint16_t* x;
  int64_t x_stride;
  const uint16_t* weight;      // [D, K]
  const uint16_t* bias;        // [D] or null
  const int32_t* cu;           // [N + 1] (extend)
  const int32_t* slot;         // [N]
  const int32_t* has_init;     // [N] or null (extend)
  uint16_t* pool;              // [*, D, K - 1], slot stride pool_stride
  int64_t pool_stride;
  uint16_t* out;
  int64_t out_stride;
  int keep_pool;
  const int32_t* parent;       // [T] token tree or null (extend)
};

hipError_t launch_gate(const GateLaunch& p, hipStream_t stream);
hipError_t launch_recurrent(const SeqLaunch& p, hipStream_t stream);
hipError_t launch_chunked(const SeqLaunch& p, hipStream_t stream);
hipError_t launch_validate_slots(const int32_t* slot, int n, int64_t num_slots, int32_t* flag,
                                 hipStream_t stream);
// Why the chunk-64 kernel cannot run this call (GDN_WHY_* bits of gdn.h), 0 if it can.
int chunked_obstacles(const SeqLaunch& p);
// Chunk-128 delta-off kernel: whether it has a tile plan for the head dims, what else
// keeps it from this call (GDN_WHY_* bits), its workspace bytes for `segs` segments per
// sequence, how a workspace is carved up, and the launch (prep, segment states, full pass).
bool ssd_chunked_shape(const SeqLaunch& p);
int ssd_units_per_seq(const SeqLaunch& p);
int ssd_obstacles(const SeqLaunch& p);
int64_t ssd_workspace_bytes(int64_t T, int N, int H_qk, int H_v, int states);
void ssd_bind_workspace(SeqLaunch& p, void* ws);
hipError_t launch_ssd(const SeqLaunch& p, hipStream_t stream);
hipError_t launch_conv(const ConvLaunch& p, hipStream_t stream);          // varlen: outputs, then states
hipError_t launch_conv_update(const ConvLaunch& p, hipStream_t stream);   // one token per row

// measurement helpers (probe.hip)
hipError_t launch_copy_probe(const void* src, void* dst, int64_t bytes, hipStream_t stream);
hipError_t launch_mfma_probe(float* out, int blocks, int iters, hipStream_t stream);

}  // namespace gdn
