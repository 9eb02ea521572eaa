/* gdn.h -- C ABI of libgdn.so, the MI355X (gfx950) GDN linear-attention layer.
 *
 * The layer is the Gated DeltaNet ("gated delta rule") linear attention that a
 * hybrid full-attention + GDN model reaches through
 * HybridAttnBackend.forward_gdn(layer, forward_batch, mixed_qkv, a, b)
 * (pymllm.layers.attention.hybrid_backend API page, HybridAttnBackend.forward_gdn:
 * "delegate GDN computation to the GDN backend").  The recurrence, per sequence and
 * v-head, with q and k L2-normalised per head, is
 *
 *     S_t = g_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = scale S_t q_t
 *     g_t = exp(-exp(A_log) softplus(a_t + dt_bias)),                beta_t = sigmoid(b_t)
 *
 * (Yang, Kautz & Hatamizadeh, Gated Delta Networks, ICLR 2025).  A delta-off mode
 * computes the Mamba2 SSD scan of flashinfer.mamba.ssd_combined_fwd (parameter
 * list of that page): S_t = exp(dt'_t A) S_{t-1} + dt'_t x_t B_t^T,
 * y_t = S_t C_t + D x_t, out_t = y_t silu(z_t).
 *
 * Conventions shared by every call
 *   - Every pointer in an args struct is DEVICE memory owned by the caller.  The
 *     library allocates nothing, keeps no state between calls (gdn_extend_noalloc's
 *     static scratch aside) and never synchronises: work is enqueued on `stream` (a
 *     hipStream_t; NULL = the legacy default stream) and the call returns at once.
 *   - Strides and sizes are in elements, not bytes.  Within a token, heads are
 *     contiguous: element (t, head, i) of q is q[t * q_stride + head * d_k + i].
 *   - Rows are accessed 4 elements at a time: q, k, v, z and out must be aligned
 *     to 4 elements of their dtype (8 bytes bf16, 16 bytes fp32), the pool to 16
 *     bytes, and every token stride must be a multiple of 4; otherwise GDN_E_SHAPE.
 *   - Host-side validation runs first; on any error the call returns a nonzero
 *     gdn_status, launches nothing and touches no buffer.  A failed launch returns
 *     GDN_E_HIP; gdn_last_hip_error() then gives the hipError_t (per thread).
 *   - Device-resident index data (cu_seqlens, slot, has_init) is trusted: checking
 *     it would need a host synchronisation.  Out-of-range or duplicate slots are
 *     undefined behaviour; gdn_validate_slots() is the opt-in device-side check.
 *   - A negative slot disables its sequence: no output row and no pool slot is
 *     touched (after the "negative entries disable" rule of the checkpoint
 *     arguments on the flashinfer.mamba.ssd_combined_fwd page).
 *   - Two calls that write the same pool slot must be ordered by the caller.
 */
#ifndef GDN_H
#define GDN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 8

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_E_NULL = 1,        /* a required pointer is NULL                        */
  GDN_E_SHAPE = 2,       /* inconsistent sizes / strides                      */
  GDN_E_DTYPE = 3,       /* unsupported dtype combination                     */
  GDN_E_UNSUPPORTED = 4, /* valid request this build has no kernel for        */
  GDN_E_INDEX = 5,       /* index argument out of range (host-checkable ones) */
  GDN_E_HIP = 6,         /* the HIP runtime reported an error at launch        */
  GDN_E_SCRATCH = 7      /* gdn_extend_noalloc: needs more than its static scratch */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

enum { GDN_MODE_GDN = 0, GDN_MODE_SSD = 1 };

/* ---------------------------------------------------------------- gdn_gate
 * a, b -> log g, beta for every (token, head).
 *   GDN mode: log_g = -exp(A[h]) * softplus(a[t,h] + dt_bias[h]); beta = sigmoid(b[t,h]).
 *             A holds A_log.  dt_softplus, dt_min, dt_max are ignored.
 *   SSD mode: dt' = a[t,h] + dt_bias[h], softplus'd when dt_softplus != 0, then
 *             clamped to [dt_min, dt_max] (inclusive, ssd_combined_fwd dt_limit);
 *             log_g = dt' * A[h] (A < 0); beta = dt'.  b must be NULL.
 * The decay is returned as log g (<= 0, fp32) because the chunked extend works with
 * in-chunk cumulative sums of it; g = exp(log_g).
 * Outputs log_g and beta are fp32 [T, H], row stride H (contiguous).  dt_bias may
 * be NULL (zero bias).  T = 0 is a no-op. */
typedef struct gdn_gate_args {
  int32_t mode;          /* GDN_MODE_GDN | GDN_MODE_SSD                 */
  int32_t in_dtype;      /* gdn_dtype of a and b                        */
  int64_t T;             /* tokens                                      */
  int32_t H;             /* heads (v-heads)                             */
  int32_t _pad0;
  const void* a;         /* [T, H], row stride a_stride (GDN: a; SSD: dt) */
  int64_t a_stride;
  const void* b;         /* [T, H], row stride b_stride (GDN only)      */
  int64_t b_stride;
  const float* A;        /* [H] fp32: GDN A_log, SSD A                  */
  const float* dt_bias;  /* [H] fp32 or NULL                            */
  int32_t dt_softplus;   /* SSD only                                    */
  float dt_min, dt_max;  /* SSD only; use 0 and +inf for "no limit"     */
  int32_t _pad1;
  float* log_g;          /* out [T, H] fp32                             */
  float* beta;           /* out [T, H] fp32                             */
} gdn_gate_args;

/* ---------------------------------------------------------------- gdn_extend
 * Packed-varlen prefill / extend.  Sequence n owns tokens [cu_seqlens[n],
 * cu_seqlens[n+1]) (cu_seqlens[0] = 0, non-decreasing, last <= T: tokens after the
 * last sequence are padding of a static buffer, e.g. under graph capture, and their
 * output rows are not written).  It starts from
 * pool[slot[n]] when has_init[n] != 0 (has_init NULL = all 1) and from zeros
 * otherwise, and writes its final state to pool[slot[n]] -- also for a
 * zero-length sequence, which writes its start state back.  slot[n] < 0 skips it.
 *
 *   q, k : [T, H_qk, d_k] (token stride q_stride / k_stride, heads contiguous)
 *   v    : [T, H_v, d_v]  (token stride v_stride)
 *   log_g, beta : [T, H_v] fp32 from gdn_gate
 *   pool : fp32 [num_slots, H_v, d_v, d_k] -- one [d_v, d_k] matrix S per
 *          (slot, v-head), d_k fastest; read and written in place
 *   out  : [T, H_v, d_v] in out_dtype (token stride out_stride), RNE rounding
 * v-head h reads qk-head h / (H_v / H_qk).  GDN mode L2-normalises q and k
 * (q / sqrt(|q|^2 + 1e-6)) and uses `scale`; SSD mode does not normalise, ignores
 * scale (1), and applies the D skip (D_per_dim ? D[h, i] : D[h]) and the silu(z)
 * gate when D / z are non-NULL (D and z in in_dtype, z laid out like v).
 * In SSD mode q = C, k = B (H_qk = ngroups, d_k = dstate), v = x (d_v = headdim),
 * log_g / beta from gdn_gate in SSD mode.
 *
 * Supported: d_k, d_v in {64, 128}; H_v % H_qk == 0; in_dtype bf16 or fp32 with
 * out_dtype bf16 or fp32.  bf16 inputs use the chunked MFMA kernels, fp32 inputs and
 * short batches (max_seqlen in 1..8) the token-recurrent kernel; gdn_extend_kernel()
 * tells which kernel a call takes and why.  max_seqlen is a host-side hint (an upper
 * bound of the longest sequence, 0 = unknown); a wrong hint changes speed, never
 * results.
 *   chunk, GDN mode : 0 (default) or 64 (the chunk-64 kernel; d_k = d_v = 128).
 *   chunk, SSD mode : 64, 128 or 0 (default: 128 when the call can take it, else 64).
 *     The chunk-128 delta-off kernel (d_k = dstate = 128, d_v = headdim = 64, the
 *     ssd_combined_fwd chunk size) needs a caller workspace: fp16 copies of B and C
 *     and the chunks' C B^T tiles (every head of a group reads them) and, to run the
 *     segments of a sequence in parallel, their states.  gdn_extend_workspace_size() gives the bytes it wants;
 *     a smaller workspace (at least the size for one segment) means fewer segments,
 *     i.e. speed only.  chunk = 128 without a usable workspace: GDN_E_NULL (none) or
 *     GDN_E_SHAPE (too small for one segment).  Its fp16 operands need |C.B|, |dt' x|
 *     and the state below 65504 (beyond that the outputs turn inf / NaN).  It reads z
 *     and writes out in 16-byte pieces: with z or out not 16-byte aligned, or a row
 *     stride of either that is not a multiple of 16 bytes, chunk 0 takes the chunk-64
 *     kernel and chunk 128 returns GDN_E_UNSUPPORTED.
 *
 * State checkpoints (optional; the checkpoint_token_indices / checkpoint_state_slots
 * / checkpoint_states arguments of the ssd_combined_fwd page, in both modes):
 *   ckpt_token  : int32 [N], one exclusive token boundary per sequence: absolute
 *                 packed-token index, or relative to the sequence's first token
 *                 when ckpt_relative != 0; negative disables the sequence's capture
 *   ckpt_slot   : int32 [N], row of ckpt_states; negative disables
 *   ckpt_states : fp32 [num_ckpt, H_v, d_v, d_k] (the pool's layout), caller-owned
 * Sequence n (slot[n] >= 0) with a boundary b inside [its first token, its end]
 * writes the state after its tokens before b to ckpt_states[ckpt_slot[n]]: its start
 * state for b at the first token, its final state for b at the end.  A boundary
 * outside the sequence captures nothing.  The three pointers are given together or
 * not at all (else GDN_E_NULL); num_ckpt >= 0.  As for the pool, ckpt_slot values
 * are device data and not range-checked: they must be < num_ckpt and distinct among
 * capturing sequences.
 *
 * Target-verify states (optional; the speculative state buffer of the target-verify
 * path in the SGLang GDN test article, chains and EAGLE trees):
 *   spec_states : fp32 [num_spec, spec_steps, H_v, d_v, d_k], caller-owned
 *   spec_slot   : int32 [N], row of spec_states; negative: the sequence records nothing
 *   spec_parent : int32 [T] or NULL; token tree: token i of a sequence (index within
 *                 it) starts from the state after its token spec_parent[t] (an earlier
 *                 index), or from the sequence's start state for -1; NULL = a chain.
 *                 A parent outside [0, i) or not below spec_steps counts as -1 (the
 *                 rule of gdn_conv1d's parent), so only recorded rows are ever read; a
 *                 sequence without a speculative row (spec_slot[n] < 0) runs as a chain
 *   keep_pool   : non-zero leaves the pool unwritten (read only)
 * Sequence n with spec_slot[n] >= 0 writes the state after its token i to
 * spec_states[spec_slot[n], i] for i < spec_steps.  With spec_parent every sequence
 * with tokens needs spec_slot[n] >= 0 and at most spec_steps tokens (device data, not
 * checked).  The pool receives the state after the sequence's last token (a chain's
 * final state) unless keep_pool.  spec_states and spec_slot go together, spec_parent
 * needs them (else GDN_E_NULL); spec_steps >= 1 with them.  Calls with target-verify
 * states run the token-recurrent kernel (verify batches are a few tokens per
 * sequence). */
typedef struct gdn_extend_args {
  int32_t mode;          /* GDN_MODE_GDN | GDN_MODE_SSD          */
  int32_t in_dtype;      /* q, k, v (and D, z)                   */
  int32_t out_dtype;
  int32_t N;             /* sequences                            */
  int64_t T;             /* packed tokens                        */
  int32_t H_qk, H_v, d_k, d_v;
  int32_t chunk;         /* 0 = default                          */
  int32_t max_seqlen;    /* hint, 0 = unknown                    */
  const void* q;
  int64_t q_stride;
  const void* k;
  int64_t k_stride;
  const void* v;
  int64_t v_stride;
  const float* log_g;
  const float* beta;
  const int32_t* cu_seqlens; /* [N+1]                            */
  const int32_t* slot;       /* [N]                              */
  const int32_t* has_init;   /* [N] or NULL                      */
  float* pool;
  int64_t num_slots;
  void* out;
  int64_t out_stride;
  float scale;
  int32_t D_per_dim;
  const void* D;         /* SSD only, or NULL                    */
  const void* z;         /* SSD only, or NULL                    */
  int64_t z_stride;
  const int32_t* ckpt_token; /* [N] or NULL (no checkpoints)     */
  const int32_t* ckpt_slot;  /* [N] or NULL                      */
  float* ckpt_states;        /* [num_ckpt, H_v, d_v, d_k] or NULL */
  int64_t num_ckpt;
  int32_t ckpt_relative;     /* boundaries relative to each sequence's first token */
  int32_t keep_pool;         /* non-zero: the pool is not written   */
  float* spec_states;        /* [num_spec, spec_steps, H_v, d_v, d_k] or NULL */
  const int32_t* spec_slot;  /* [N] or NULL                      */
  const int32_t* spec_parent;/* [T] or NULL (chain)              */
  int64_t num_spec;
  int32_t spec_steps;
  int32_t _pad_spec;
  void* workspace;           /* device scratch of the chunk-128 delta-off kernel, or NULL */
  int64_t workspace_bytes;
} gdn_extend_args;

/* Workspace bytes the chunk-128 delta-off kernel wants for a gdn_extend (gate NULL) or
 * gdn_extend_gated call with these arguments (fp16 B and C copies, the C B^T tiles of
 * every chunk, and the states of the pieces of the segments the library would run: it
 * grows with T and with N x H_v x pieces), or
 * 0 when the call would run another kernel or is invalid.  Host-side, launches nothing;
 * args->workspace / workspace_bytes are ignored.  The workspace must be 256-byte
 * aligned (else GDN_E_SHAPE) and is overwritten by the call (its contents need not be
 * initialised and mean nothing afterwards); calls in flight at once need their own. */
int64_t gdn_extend_workspace_size(const gdn_extend_args* args, const gdn_gate_args* gate);

/* Kernels of gdn_extend / gdn_extend_gated, and what keeps a call from a faster one. */
enum {
  GDN_KERNEL_RECURRENT = 1,   /* token-recurrent (decode kernel, a token at a time)   */
  GDN_KERNEL_CHUNKED = 2,     /* chunk-64 MFMA kernel                                 */
  GDN_KERNEL_SSD_CHUNKED = 3  /* chunk-128 delta-off MFMA kernel                      */
};
enum {
  GDN_WHY_FP32 = 1 << 0,        /* fp32 inputs                                          */
  GDN_WHY_SHORT = 1 << 1,       /* max_seqlen hint in 1..8 (short or verify batches)    */
  GDN_WHY_VERIFY = 1 << 2,      /* target-verify states requested                       */
  GDN_WHY_HEAD_DIMS = 1 << 3,   /* head sizes without a chunked tile plan               */
  GDN_WHY_ALIGN = 1 << 4,       /* rows not 16-byte aligned or strides not multiples of 8 */
  GDN_WHY_STRIDE = 1 << 5,      /* token strides beyond 32-bit in-chunk offsets         */
  GDN_WHY_BATCH = 1 << 6,       /* more than 65535 sequences                            */
  GDN_WHY_GATE_ALIGN = 1 << 7,  /* folded gate (GDN): a, b not 4-byte aligned, odd strides */
  GDN_WHY_WORKSPACE = 1 << 8,   /* delta-off: no workspace for the chunk-128 kernel     */
  GDN_WHY_CHUNK = 1 << 9        /* delta-off: chunk 64 requested                        */
};
/* The kernel a gdn_extend (gate NULL) or gdn_extend_gated call with these arguments
 * runs, decided on the host exactly as the call decides it; launches nothing.
 * Returns GDN_KERNEL_* (> 0), or minus the gdn_status the call would return.  *why
 * (may be NULL) receives the GDN_WHY_* bits of everything that keeps the call from
 * the fastest kernel of its mode (0 when it takes that kernel). */
int gdn_extend_kernel(const gdn_extend_args* args, const gdn_gate_args* gate, int32_t* why);

/* ---------------------------------------------------------------- gdn_decode
 * One token per sequence: token b belongs to sequence b, which always starts from
 * pool[slot[b]] and writes it back in place (state read-modify-write).  slot[b] < 0
 * marks a padding row: its output row and every pool slot stay untouched.
 * Layouts as gdn_extend with T = B; log_g / beta are [B, H_v].  GDN mode only. */
typedef struct gdn_decode_args {
  int32_t in_dtype;
  int32_t out_dtype;
  int32_t B;
  int32_t H_qk, H_v, d_k, d_v;
  int32_t _pad0;
  const void* q;
  int64_t q_stride;
  const void* k;
  int64_t k_stride;
  const void* v;
  int64_t v_stride;
  const float* log_g;
  const float* beta;
  const int32_t* slot;   /* [B] */
  float* pool;
  int64_t num_slots;
  void* out;
  int64_t out_stride;
  float scale;
  int32_t _pad1;
} gdn_decode_args;

/* `stream` is a hipStream_t passed as void* so this header needs no HIP include. */
int gdn_gate(const gdn_gate_args* args, void* stream);
int gdn_extend(const gdn_extend_args* args, void* stream);
int gdn_decode(const gdn_decode_args* args, void* stream);

/* ---------------------------------------------------------------- gated calls
 * gdn_extend / gdn_decode with the gate folded in: the kernels compute log g and
 * beta from the raw gate inputs that `gate` describes, with the arithmetic of
 * gdn_gate, instead of reading args->log_g / args->beta (ignored, may be NULL).
 * This is the same computation as gdn_gate followed by gdn_extend / gdn_decode,
 * bit for bit (one shared definition of the gate functions), with one launch and
 * the fp32 [T, H_v] round trip fewer: the shape of forward_gdn(layer,
 * forward_batch, mixed_qkv, a, b) on the hybrid_backend page, whose a, b are the
 * gate inputs.  The chunked kernel reads bf16 a, b as aligned 32-bit words: with a,
 * b not 4-byte aligned or an odd row stride the call runs the token-recurrent
 * kernel instead (speed only).
 *   gate->mode     : args->mode (extend) / GDN_MODE_GDN (decode), else
 *                    GDN_E_UNSUPPORTED
 *   gate->in_dtype : args->in_dtype, else GDN_E_DTYPE
 *   gate->T, H     : args->T (extend) or args->B (decode), and args->H_v, else
 *                    GDN_E_SHAPE
 *   gate->a, b, A, dt_bias, dt_softplus, dt_min, dt_max : as for gdn_gate
 *   gate->log_g, beta : not written, may be NULL
 * A NULL `gate` returns GDN_E_NULL; everything else is validated as for the
 * ungated call. */
int gdn_extend_gated(const gdn_extend_args* args, const gdn_gate_args* gate, void* stream);
int gdn_decode_gated(const gdn_decode_args* args, const gdn_gate_args* gate, void* stream);

/* ---------------------------------------------------------------- extend without allocation
 * For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  gdn_extend_gated (gate may be NULL:
 * then gdn_extend) with the chunk-128 delta-off kernel's workspace taken from a static
 * device array of the library, GDN_NOALLOC_SCRATCH_BYTES per device, instead of from
 * args->workspace, which must be NULL with workspace_bytes 0 (else GDN_E_SHAPE).  The
 * call allocates and frees nothing.
 *   - A call whose chunk-128 kernel needs more than the array holds at one segment per
 *     sequence (about T x H_qk > 99000 token-groups: 672 bytes per token and group)
 *     returns GDN_E_SCRATCH and launches nothing; gdn_extend_gated with a workspace of
 *     gdn_extend_workspace_size bytes runs it.  A need between one segment's and gdn_extend_workspace_size's means
 *     fewer segments per sequence (speed only).
 *   - The first call on a device, with that device current, resolves the device's copy
 *     of the array (a failure returns GDN_E_HIP); the copy stays allocated until the
 *     process ends.
 *   - Every call on one device shares its copy, which keeps the last call's contents:
 *     calls that overlap in time on one device (two streams, two threads) race and give
 *     undefined results, so the caller orders them.  No part of it needs to start at
 *     zero: a call writes every byte it reads before reading it, in stream order.
 * Every other argument, result and error as gdn_extend_gated. */
#define GDN_NOALLOC_SCRATCH_BYTES (64ll << 20)
int gdn_extend_noalloc(const gdn_extend_args* args, const gdn_gate_args* gate, void* stream);

/* ---------------------------------------------------------------- short causal conv
 * The depthwise causal conv1d of width K (and SiLU) that turns the input projection
 * into mixed_qkv in front of the layer, with each sequence's last K - 1 inputs kept
 * per slot in a conv-state pool: the per-layer conv state that sits next to the
 * temporal state in the hybrid model's memory pool (SGLang GDN test-matrix article,
 * framerc.cn, memory-pool section, its conv[0] buffer).  Channel c of sequence n
 * sees the window  w = (has_init[n] ? pool[slot[n]][c] : zeros) || its own inputs,
 * and its token i (= t - cu_seqlens[n]) gives
 *     out[t, c] = act(bias[c] + sum_{j < K} weight[c, j] * w[i + j])
 *     act(y) = y * sigmoid(y) when activation != 0, y otherwise
 * (the causal convolution: weight[c, K - 1] multiplies the current input).  The
 * slot's new state is the last K - 1 entries of w: partly the old state for a
 * sequence shorter than K - 1, the start state for an empty one.
 *   x      : bf16 [T, D], token stride x_stride (the projected mixed_qkv, before the conv)
 *   weight : bf16 [D, K], a channel's K taps contiguous, oldest input first
 *   bias   : bf16 [D], or NULL for none
 *   pool   : bf16 [num_slots, D, K - 1] with slot stride pool_stride (>= D (K - 1)),
 *            a channel's entries contiguous, oldest first; read, and written in place
 *            unless keep_pool != 0 (then only read: target-verify passes whose
 *            accepted prefix the caller commits later)
 *   out    : bf16 [T, D], token stride out_stride; the fp32 result rounded to nearest even
 *   parent : int32 [T] or NULL (gdn_conv1d only): a target-verify token tree, in the
 *            convention of gdn_extend's spec_parent (token i of a sequence continues
 *            its token parent[t], an earlier index, or the state for -1); the window of
 *            a token is then the state followed by the inputs along its root path.  A
 *            parent outside [0, i) counts as -1.  Requires keep_pool != 0 (which branch
 *            to keep is the caller's choice), else GDN_E_SHAPE.
 * cu_seqlens, slot, has_init (NULL = all 1) and num_slots follow gdn_extend, with
 * the same rules for negative slots, padding tokens after the last sequence and
 * device-resident indices.
 * Supported: dtype GDN_BF16 (else GDN_E_DTYPE); K in {2, 3, 4} (else
 * GDN_E_UNSUPPORTED).  D >= 8 and a multiple of 8; x, out, weight, bias and pool
 * 16-byte aligned; x_stride, out_stride >= D and pool_stride multiples of 8
 * (else GDN_E_SHAPE).  The fp32 arithmetic: the K products and the bias summed in
 * fp32, then the activation. */
typedef struct gdn_conv_args {
  int32_t dtype;
  int32_t K;
  int32_t activation;
  int32_t N;             /* sequences (gdn_conv1d) or rows (gdn_conv1d_update) */
  int64_t T;             /* tokens; gdn_conv1d_update: must equal N */
  int64_t D;             /* channels */
  const void* x;
  int64_t x_stride;
  const void* weight;
  const void* bias;
  const int32_t* cu_seqlens; /* [N + 1]; ignored by gdn_conv1d_update */
  const int32_t* slot;       /* [N] */
  const int32_t* has_init;   /* [N] or NULL; ignored by gdn_conv1d_update */
  void* pool;
  int64_t num_slots;
  int64_t pool_stride;
  void* out;
  int64_t out_stride;
  int32_t keep_pool;
  int32_t _pad0;
  const int32_t* parent;     /* [T] or NULL; ignored by gdn_conv1d_update */
} gdn_conv_args;

/* Packed varlen (prefill / extend): two launches on `stream`, the outputs (which
 * read the old states) and then the new states.  out must not overlap x or the pool
 * (else GDN_E_SHAPE).  T = 0 launches only the state pass (empty sequences keep or
 * clear their slot as above); N = 0 launches nothing. */
int gdn_conv1d(const gdn_conv_args* args, void* stream);
/* Decode: one token per row (T = N = rows), row b always starts from pool[slot[b]]
 * (cu_seqlens, has_init ignored); slot[b] < 0 marks a padding row whose output row
 * and slot stay untouched.  One launch; out may be x itself (same rows). */
int gdn_conv1d_update(const gdn_conv_args* args, void* stream);

/* Device-side check of slot[0..n): *flag (device int32) receives 0 when every
 * non-negative slot is < num_slots and no non-negative slot repeats, 1 when one
 * is out of range, 2 when one repeats (3 when both).  Negative slots are padding
 * and may repeat.  Asynchronous like the others; O(n^2) comparisons. */
int gdn_validate_slots(const int32_t* slot, int32_t n, int64_t num_slots, int32_t* flag,
                       void* stream);

/* Measurement helpers, not part of the layer: they give the achievable peaks of the
 * running GPU that the layer's kernels are reported against, beside the published ones.
 *
 * gdn_probe_copy: copies `bytes` bytes from src to dst (device pointers, 16-byte
 * aligned, bytes a positive multiple of 16; dst either equal to src -- in place, every
 * element read and rewritten -- or not overlapping it) with a streaming kernel; the
 * caller times it.  HBM traffic: 2 x bytes.
 * gdn_probe_mfma: `blocks` workgroups of four waves (1 <= blocks <= 65536), each wave
 * four chains of `iters` (1 <= iters <= 1 << 20) dependent 32x32x16 bf16 MFMAs with
 * fp32 accumulation: blocks x 4 x 4 x iters x 32768 flop.  out (device, blocks x 256
 * floats, caller-owned) receives one finite sum per thread.
 * Both are asynchronous on `stream`; GDN_E_NULL / GDN_E_SHAPE on bad arguments. */
int gdn_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);
int gdn_probe_mfma(float* out, int32_t blocks, int32_t iters, void* stream);

const char* gdn_status_str(int status);
int gdn_last_hip_error(void);
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
