"""MI355X-native GDN (Gated DeltaNet) linear-attention layer.

Thin Python binding over libgdn.so (include/gdn.h): every step of the layer runs
in the library's HIP kernels; this module only checks tensors, allocates outputs
the caller did not supply and passes pointers, strides and torch's current HIP
stream.  There is no fallback: without the built library every call raises.

Entry points (same names as the C ABI):
  gate / ssd_gate      a, b -> (log g, beta)               -> gdn_gate
  extend               packed varlen extend over a pool   -> gdn_extend
  extend_kernel        which kernel an extend call takes  -> gdn_extend_kernel
  extend_workspace_size  delta-off chunk-128 workspace    -> gdn_extend_workspace_size
  extend_noalloc       extend with the library's scratch  -> gdn_extend_noalloc
  decode               one token per sequence, in place   -> gdn_decode
  conv1d               short causal conv, varlen          -> gdn_conv1d
  conv1d_update        short causal conv, one token/row   -> gdn_conv1d_update
  validate_slots       opt-in device check of slots       -> gdn_validate_slots
and the two call shapes of the pages:
  forward_gdn(layer, forward_batch, mixed_qkv, a, b)  (pymllm HybridAttnBackend.forward_gdn)
  ssd_combined_fwd(x, dt, A, B, C, ...)               (flashinfer.mamba.ssd_combined_fwd subset)
"""
from __future__ import annotations

import ctypes as ct
import math

import torch

from . import _lib
from ._lib import GDN_BF16, GDN_F32, GDN_MODE_GDN, GDN_MODE_SSD, GDNError

__all__ = ["load", "gate", "ssd_gate", "extend", "extend_noalloc", "extend_kernel",
           "extend_workspace_size", "decode", "conv1d", "conv1d_update", "validate_slots", "forward_gdn",
           "ssd_combined_fwd", "GDNError", "split_mixed_qkv", "probe_copy", "probe_mfma"]


def load():
    """Load libgdn.so (raises RuntimeError when it is missing)."""
    return _lib.load()


# ------------------------------------------------------------------ helpers
def _dtype_code(t) -> int:
    """gdn_dtype of a tensor or a torch dtype."""
    dt = t if isinstance(t, torch.dtype) else t.dtype
    if dt == torch.bfloat16:
        return GDN_BF16
    if dt == torch.float32:
        return GDN_F32
    raise ValueError(f"unsupported dtype {dt} (bf16 or fp32)")


def _ptr(t):
    return None if t is None else ct.c_void_p(t.data_ptr())


def _stream(device) -> ct.c_void_p:
    return ct.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _on_gpu(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must live on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def _rows(t: torch.Tensor, name: str, heads: int, dim: int) -> int:
    """Token stride of a [T, heads, dim] view whose heads are contiguous."""
    if t.dim() != 3 or t.shape[1] != heads or t.shape[2] != dim:
        raise ValueError(f"{name} must be [T, {heads}, {dim}], got {tuple(t.shape)}")
    if t.stride(2) != 1 or (heads > 1 and t.stride(1) != dim):
        raise ValueError(f"{name} must have contiguous heads (strides {t.stride()})")
    return t.stride(0)


def _mat_rows(t: torch.Tensor, name: str, T: int, H: int) -> int:
    if t.dim() != 2 or t.shape[0] != T or t.shape[1] != H or (H > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be [{T}, {H}] with unit column stride, got "
                         f"{tuple(t.shape)} / {t.stride()}")
    return t.stride(0) if T > 1 else H


def _same_rows(n: int, what: str, **ts):
    """Every given tensor has n rows (tokens): the library sees plain pointers and
    cannot check how long a buffer is."""
    for name, t in ts.items():
        if t is not None and (t.dim() == 0 or t.shape[0] != n):
            raise ValueError(f"{name} must have {n} rows ({what}), got shape {tuple(t.shape)}")


def _i32(t: torch.Tensor, name: str, n: int) -> torch.Tensor:
    if t.dtype != torch.int32 or t.dim() != 1 or t.shape[0] != n or (n > 1 and t.stride(0) != 1):
        raise ValueError(f"{name} must be a contiguous int32 vector of length {n}")
    return t


def split_mixed_qkv(mixed_qkv: torch.Tensor, H_qk: int, H_v: int, d_k: int, d_v: int):
    """Views q [T,H_qk,d_k], k [T,H_qk,d_k], v [T,H_v,d_v] of a [T, 2 H_qk d_k + H_v d_v]
    projection laid out q | k | v with heads contiguous inside each block."""
    T, width = mixed_qkv.shape
    nq = H_qk * d_k
    if width != 2 * nq + H_v * d_v or mixed_qkv.stride(1) != 1:
        raise ValueError(f"mixed_qkv width {width} != 2*{H_qk}*{d_k} + {H_v}*{d_v}")
    q = mixed_qkv[:, :nq].unflatten(1, (H_qk, d_k))
    k = mixed_qkv[:, nq:2 * nq].unflatten(1, (H_qk, d_k))
    v = mixed_qkv[:, 2 * nq:].unflatten(1, (H_v, d_v))
    return q, k, v


# ------------------------------------------------------------------ gdn_gate
class GateInputs:
    """Raw gate inputs of one call (tensors kept alive with their ctypes description):
    GDN a, b [T, H] with A_log, dt_bias [H]; delta-off dt [T, H] with A, dt_bias [H] and
    the softplus / clamp settings.  Passed as `gate=` to extend / decode to fold the
    gate into those kernels, or used by gate() / ssd_gate() to materialise log g, beta."""

    def __init__(self, mode, a, b, A, dt_bias, dt_softplus, dt_limit):
        T, H = a.shape
        self.dev = _on_gpu(a, b, A, dt_bias)
        if b is not None and b.dtype != a.dtype:
            raise ValueError("a and b must share a dtype")
        for t, nm in ((A, "A_log" if mode == GDN_MODE_GDN else "A"), (dt_bias, "dt_bias")):
            if t is not None and (t.dtype != torch.float32 or t.shape != (H,) or not t.is_contiguous()):
                raise ValueError(f"{nm} must be contiguous fp32 [{H}]")
        self.T, self.H, self.mode, self.dtype = T, H, mode, a.dtype
        self._keep = (a, b, A, dt_bias)
        self.args = _lib.GateArgs(
            mode=mode, in_dtype=_dtype_code(a), T=T, H=H, a=_ptr(a),
            a_stride=_mat_rows(a, "a" if mode == GDN_MODE_GDN else "dt", T, H),
            b=_ptr(b), b_stride=_mat_rows(b, "b", T, H) if b is not None else 0, A=_ptr(A),
            dt_bias=_ptr(dt_bias), dt_softplus=int(bool(dt_softplus)),
            dt_min=float(dt_limit[0]), dt_max=float(dt_limit[1]), log_g=None, beta=None)


def gdn_gate_inputs(a, b, A_log, dt_bias=None) -> GateInputs:
    """GDN gate inputs: log_g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b)."""
    return GateInputs(GDN_MODE_GDN, a, b, A_log, dt_bias, 1, (0.0, math.inf))


def ssd_gate_inputs(dt, A, dt_bias=None, dt_softplus=False, dt_limit=(0.0, math.inf)) -> GateInputs:
    """Delta-off gate inputs: dt' = clamp(softplus?(dt + dt_bias), dt_limit); log_g = dt' A; beta = dt'."""
    return GateInputs(GDN_MODE_SSD, dt, None, A, dt_bias, dt_softplus, dt_limit)


def _run_gate(g: GateInputs, log_g, beta):
    lib = _lib.load()
    _on_gpu(log_g, beta)
    log_g = torch.empty((g.T, g.H), dtype=torch.float32, device=g.dev) if log_g is None else log_g
    beta = torch.empty((g.T, g.H), dtype=torch.float32, device=g.dev) if beta is None else beta
    for t, nm in ((log_g, "log_g"), (beta, "beta")):
        if t.dtype != torch.float32 or t.shape != (g.T, g.H) or not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous fp32 [{g.T}, {g.H}]")
    args = _lib.GateArgs.from_buffer_copy(g.args)
    args.log_g, args.beta = _ptr(log_g), _ptr(beta)
    _lib.check("gdn_gate", lib.gdn_gate(ct.byref(args), _stream(g.dev)))
    return log_g, beta


def gate(a: torch.Tensor, b: torch.Tensor, A_log: torch.Tensor, dt_bias: torch.Tensor | None = None,
         *, log_g: torch.Tensor | None = None, beta: torch.Tensor | None = None):
    """GDN gate: log_g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b); fp32 [T, H]."""
    return _run_gate(gdn_gate_inputs(a, b, A_log, dt_bias), log_g, beta)


def ssd_gate(dt: torch.Tensor, A: torch.Tensor, dt_bias: torch.Tensor | None = None,
             dt_softplus: bool = False, dt_limit=(0.0, math.inf), *,
             log_g: torch.Tensor | None = None, beta: torch.Tensor | None = None):
    """Delta-off gate: dt' = clamp(softplus?(dt + dt_bias), dt_limit); log_g = dt' A; beta = dt'."""
    return _run_gate(ssd_gate_inputs(dt, A, dt_bias, dt_softplus, dt_limit), log_g, beta)


# ------------------------------------------------------------------ gdn_extend
def _extend_args(q, k, v, log_g, beta, cu_seqlens, slot, pool, *, has_init=None, scale=None, out=None,
                 out_dtype=None, max_seqlen: int = 0, mode: str = "gdn", D=None, z=None, chunk: int = 0,
                 gate: GateInputs | None = None, ckpt_token=None, ckpt_slot=None, ckpt_states=None,
                 ckpt_relative: bool = False, spec_states=None, spec_slot=None, spec_parent=None,
                 keep_pool: bool = False, alloc_out: bool = True):
    """Checks and the ctypes argument struct of one gdn_extend call: (args, out, device)."""
    T, H_qk, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    N = cu_seqlens.shape[0] - 1
    _same_rows(T, "the tokens of q", k=k, v=v, out=out, z=z)
    dev = _on_gpu(q, k, v, log_g, beta, cu_seqlens, slot, pool, has_init, out, D, z)
    if gate is not None and gate.dev != dev:
        raise ValueError("gate inputs live on another device")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    ssd = mode == "ssd"
    if mode not in ("gdn", "ssd"):
        raise ValueError(f"mode must be 'gdn' or 'ssd', got {mode!r}")
    if pool.dtype != torch.float32 or pool.dim() != 4 or pool.shape[1:] != (H_v, d_v, d_k) \
            or not pool.is_contiguous():
        raise ValueError(f"pool must be contiguous fp32 [num_slots, {H_v}, {d_v}, {d_k}]")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None and alloc_out:
        out = torch.empty((T, H_v, d_v), dtype=out_dtype, device=dev)
    if scale is None:
        scale = 1.0 if ssd else d_k ** -0.5
    _i32(cu_seqlens, "cu_seqlens", N + 1)
    _i32(slot, "slot", N)
    if has_init is not None:
        _i32(has_init, "has_init", N)
    for t, nm in ((log_g, "log_g"), (beta, "beta")):
        if gate is not None and t is None:
            continue
        if t.dtype != torch.float32 or t.shape != (T, H_v) or not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous fp32 [{T}, {H_v}]")
    if D is not None and (D.dtype != q.dtype or not D.is_contiguous()
                          or D.shape not in ((H_v,), (H_v, d_v))):
        raise ValueError(f"D must be contiguous [{H_v}] or [{H_v}, {d_v}] in the input dtype")
    if z is not None and z.dtype != q.dtype:
        raise ValueError("z must share the input dtype")
    nck = sum(t is not None for t in (ckpt_token, ckpt_slot, ckpt_states))
    if nck not in (0, 3):
        raise ValueError("ckpt_token, ckpt_slot and ckpt_states go together")
    if nck:
        if _on_gpu(ckpt_token, ckpt_slot, ckpt_states) != dev:
            raise ValueError("checkpoint tensors live on another device")
        _i32(ckpt_token, "ckpt_token", N)
        _i32(ckpt_slot, "ckpt_slot", N)
        if ckpt_states.dtype != torch.float32 or ckpt_states.dim() != 4 \
                or ckpt_states.shape[1:] != (H_v, d_v, d_k) or not ckpt_states.is_contiguous():
            raise ValueError(f"ckpt_states must be contiguous fp32 [num_ckpt, {H_v}, {d_v}, {d_k}]")
    if (spec_states is None) != (spec_slot is None) or (spec_parent is not None and spec_states is None):
        raise ValueError("spec_states and spec_slot go together; spec_parent needs them")
    if spec_states is not None:
        if _on_gpu(spec_states, spec_slot, spec_parent) != dev:
            raise ValueError("target-verify tensors live on another device")
        _i32(spec_slot, "spec_slot", N)
        if spec_parent is not None:
            _i32(spec_parent, "spec_parent", T)
        if spec_states.dtype != torch.float32 or spec_states.dim() != 5 \
                or spec_states.shape[2:] != (H_v, d_v, d_k) or not spec_states.is_contiguous():
            raise ValueError(f"spec_states must be contiguous fp32 [num_spec, steps, {H_v}, {d_v}, {d_k}]")
    args = _lib.ExtendArgs(
        mode=GDN_MODE_SSD if ssd else GDN_MODE_GDN, in_dtype=_dtype_code(q),
        out_dtype=_dtype_code(out if out is not None else out_dtype),
        N=N, T=T, H_qk=H_qk, H_v=H_v, d_k=d_k, d_v=d_v, chunk=chunk,
        max_seqlen=int(max_seqlen), q=_ptr(q), q_stride=_rows(q, "q", H_qk, d_k), k=_ptr(k),
        k_stride=_rows(k, "k", H_qk, d_k), v=_ptr(v), v_stride=_rows(v, "v", H_v, d_v),
        log_g=_ptr(log_g), beta=_ptr(beta), cu_seqlens=_ptr(cu_seqlens), slot=_ptr(slot),
        has_init=_ptr(has_init), pool=_ptr(pool), num_slots=pool.shape[0], out=_ptr(out),
        out_stride=_rows(out, "out", H_v, d_v) if out is not None else H_v * d_v, scale=float(scale),
        D_per_dim=int(D is not None and D.dim() == 2), D=_ptr(D), z=_ptr(z),
        z_stride=_rows(z, "z", H_v, d_v) if z is not None else 0,
        ckpt_token=_ptr(ckpt_token), ckpt_slot=_ptr(ckpt_slot), ckpt_states=_ptr(ckpt_states),
        num_ckpt=ckpt_states.shape[0] if nck else 0, ckpt_relative=int(bool(ckpt_relative)),
        keep_pool=int(bool(keep_pool)), spec_states=_ptr(spec_states), spec_slot=_ptr(spec_slot),
        spec_parent=_ptr(spec_parent), num_spec=spec_states.shape[0] if spec_states is not None else 0,
        spec_steps=spec_states.shape[1] if spec_states is not None else 0)
    return args, out, dev


def _gate_ref(gate):
    return None if gate is None else ct.byref(gate.args)


def extend(q, k, v, log_g, beta, cu_seqlens, slot, pool, *, has_init=None, scale=None, out=None,
           out_dtype=None, max_seqlen: int = 0, mode: str = "gdn", D=None, z=None, chunk: int = 0,
           gate: GateInputs | None = None, ckpt_token=None, ckpt_slot=None, ckpt_states=None,
           ckpt_relative: bool = False, spec_states=None, spec_slot=None, spec_parent=None,
           keep_pool: bool = False, workspace: torch.Tensor | None = None):
    """Packed-varlen extend.  q, k [T, H_qk, d_k]; v [T, H_v, d_v]; log_g, beta [T, H_v] fp32;
    cu_seqlens [N+1], slot [N], has_init [N] int32; pool fp32 [num_slots, H_v, d_v, d_k]
    (updated in place).  With `gate` (GateInputs of the same mode, dtype and [T, H_v]) the
    gate is folded into the kernel and log_g / beta are not used (pass None).
    State checkpoints (all three or none): ckpt_token [N] int32 exclusive token boundaries
    (absolute, or per sequence with ckpt_relative), ckpt_slot [N] int32 rows of ckpt_states
    fp32 [num_ckpt, H_v, d_v, d_k]; negative entries disable.
    Target verify: spec_states fp32 [num_spec, steps, H_v, d_v, d_k] and spec_slot [N] int32
    record the state after every token; spec_parent [T] int32 (optional) makes the tokens
    of a sequence a tree; keep_pool leaves the pool unwritten.
    Delta-off mode (mode="ssd"): chunk 0 or 128 runs the chunk-128 kernel, which needs a
    workspace of gdn_extend_workspace_size bytes: pass a uint8 device tensor as `workspace`
    (e.g. a static buffer under graph capture), else one is allocated for the call.
    Returns out [T, H_v, d_v]."""
    lib = _lib.load()
    args, out, dev = _extend_args(q, k, v, log_g, beta, cu_seqlens, slot, pool, has_init=has_init,
                                  scale=scale, out=out, out_dtype=out_dtype, max_seqlen=max_seqlen,
                                  mode=mode, D=D, z=z, chunk=chunk, gate=gate, ckpt_token=ckpt_token,
                                  ckpt_slot=ckpt_slot, ckpt_states=ckpt_states,
                                  ckpt_relative=ckpt_relative, spec_states=spec_states,
                                  spec_slot=spec_slot, spec_parent=spec_parent, keep_pool=keep_pool)
    ws = _workspace(lib, args, gate, dev, workspace)
    if gate is None:
        _lib.check("gdn_extend", lib.gdn_extend(ct.byref(args), _stream(dev)))
    else:
        _lib.check("gdn_extend_gated", lib.gdn_extend_gated(ct.byref(args), ct.byref(gate.args), _stream(dev)))
    del ws
    return out


def extend_noalloc(q, k, v, log_g, beta, cu_seqlens, slot, pool, *, out, has_init=None, scale=None,
                   max_seqlen: int = 0, mode: str = "gdn", D=None, z=None, chunk: int = 0,
                   gate: GateInputs | None = None, ckpt_token=None, ckpt_slot=None, ckpt_states=None,
                   ckpt_relative: bool = False, spec_states=None, spec_slot=None, spec_parent=None,
                   keep_pool: bool = False):
    """extend() for callers that cannot allocate (gdn_extend_noalloc): the caller passes
    `out` ([T, H_v, d_v], bf16 or fp32), and the chunk-128 delta-off kernel's workspace
    comes from the library's static per-device scratch.  Calls that overlap in time on one
    device race on that scratch.  Returns out."""
    if out is None:
        raise ValueError("extend_noalloc writes into a caller-given out")
    lib = _lib.load()
    args, out, dev = _extend_args(q, k, v, log_g, beta, cu_seqlens, slot, pool, has_init=has_init,
                                  scale=scale, out=out, max_seqlen=max_seqlen, mode=mode, D=D, z=z,
                                  chunk=chunk, gate=gate, ckpt_token=ckpt_token, ckpt_slot=ckpt_slot,
                                  ckpt_states=ckpt_states, ckpt_relative=ckpt_relative,
                                  spec_states=spec_states, spec_slot=spec_slot,
                                  spec_parent=spec_parent, keep_pool=keep_pool)
    _lib.check("gdn_extend_noalloc", lib.gdn_extend_noalloc(ct.byref(args), _gate_ref(gate), _stream(dev)))
    return out


def _workspace(lib, args, gate, dev, workspace):
    """Attach the chunk-128 delta-off kernel's workspace to args: the caller's uint8 tensor,
    or (when the call wants one) a fresh allocation on the current stream."""
    if workspace is not None:
        if workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_contiguous() \
                or workspace.device != dev:
            raise ValueError("workspace must be a contiguous uint8 vector on the call's device")
        args.workspace, args.workspace_bytes = _ptr(workspace), workspace.numel()
        return workspace
    need = lib.gdn_extend_workspace_size(ct.byref(args), _gate_ref(gate)) if args.mode == GDN_MODE_SSD else 0
    if need <= 0:
        return None
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    args.workspace, args.workspace_bytes = _ptr(ws), need
    return ws


def extend_workspace_size(q, k, v, log_g, beta, cu_seqlens, slot, pool, **kw) -> int:
    """Bytes of workspace the delta-off chunk-128 kernel wants for extend(...) with these
    arguments (0 when the call runs another kernel): gdn_extend_workspace_size."""
    lib = _lib.load()
    kw.pop("workspace", None)
    args, _, _ = _extend_args(q, k, v, log_g, beta, cu_seqlens, slot, pool, alloc_out=False, **kw)
    _placeholder_out(args)
    return int(lib.gdn_extend_workspace_size(ct.byref(args), _gate_ref(kw.get("gate"))))


def _placeholder_out(args):
    """The host-side queries read no buffer; a call without `out` gets its output from
    extend(), so they are shown an aligned stand-in address."""
    if not args.out:
        args.out = ct.c_void_p(256)


def extend_kernel(q, k, v, log_g, beta, cu_seqlens, slot, pool, **kw):
    """(kernel, reasons): which kernel extend(...) with these arguments runs -- "chunked64",
    "ssd_chunked128" or "recurrent" -- and the names of the GDN_WHY_* reasons that keep it
    from the fastest kernel of its mode (empty when it takes that one).  Decided on the
    host exactly as the call decides it (gdn_extend_kernel); launches nothing."""
    lib = _lib.load()
    workspace = kw.pop("workspace", None)
    args, _, dev = _extend_args(q, k, v, log_g, beta, cu_seqlens, slot, pool, alloc_out=False, **kw)
    _placeholder_out(args)
    gate = kw.get("gate")
    if workspace is not None:
        args.workspace, args.workspace_bytes = _ptr(workspace), workspace.numel()
    elif args.mode == GDN_MODE_SSD:   # extend() would allocate what the call wants
        need = lib.gdn_extend_workspace_size(ct.byref(args), _gate_ref(gate))
        if need > 0:
            args.workspace, args.workspace_bytes = ct.c_void_p(256), need
    why = ct.c_int32(0)
    kern = lib.gdn_extend_kernel(ct.byref(args), _gate_ref(gate), ct.byref(why))
    if kern < 0:
        _lib.check("gdn_extend_kernel", -kern)
    return _lib.KERNEL_NAMES[kern], [n for i, n in enumerate(_lib.WHY_NAMES) if why.value >> i & 1]


# ------------------------------------------------------------------ gdn_decode
def decode(q, k, v, log_g, beta, slot, pool, *, scale=None, out=None, out_dtype=None,
           gate: GateInputs | None = None):
    """One token per sequence; pool slots are read and written in place.  With `gate`
    (GDN GateInputs of [B, H_v]) the gate is folded into the kernel (log_g, beta None)."""
    lib = _lib.load()
    B, H_qk, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    _same_rows(B, "one token per sequence of q", k=k, v=v, out=out)
    dev = _on_gpu(q, k, v, log_g, beta, slot, pool, out)
    if gate is not None and gate.dev != dev:
        raise ValueError("gate inputs live on another device")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    if pool.dtype != torch.float32 or pool.dim() != 4 or pool.shape[1:] != (H_v, d_v, d_k) \
            or not pool.is_contiguous():
        raise ValueError(f"pool must be contiguous fp32 [num_slots, {H_v}, {d_v}, {d_k}]")
    _i32(slot, "slot", B)
    for t, nm in ((log_g, "log_g"), (beta, "beta")):
        if gate is not None and t is None:
            continue
        if t.dtype != torch.float32 or t.shape != (B, H_v) or not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous fp32 [{B}, {H_v}]")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, H_v, d_v), dtype=out_dtype, device=dev)
    scale = d_k ** -0.5 if scale is None else scale
    args = _lib.DecodeArgs(
        in_dtype=_dtype_code(q), out_dtype=_dtype_code(out), B=B, H_qk=H_qk, H_v=H_v, d_k=d_k,
        d_v=d_v, q=_ptr(q), q_stride=_rows(q, "q", H_qk, d_k), k=_ptr(k),
        k_stride=_rows(k, "k", H_qk, d_k), v=_ptr(v), v_stride=_rows(v, "v", H_v, d_v),
        log_g=_ptr(log_g), beta=_ptr(beta), slot=_ptr(slot), pool=_ptr(pool),
        num_slots=pool.shape[0], out=_ptr(out), out_stride=_rows(out, "out", H_v, d_v),
        scale=float(scale))
    if gate is None:
        _lib.check("gdn_decode", lib.gdn_decode(ct.byref(args), _stream(dev)))
    else:
        _lib.check("gdn_decode_gated", lib.gdn_decode_gated(ct.byref(args), ct.byref(gate.args), _stream(dev)))
    return out


def validate_slots(slot: torch.Tensor, num_slots: int) -> int:
    """0 = ok, bit 1 = out of range, bit 2 = duplicate (synchronises to read the flag)."""
    lib = _lib.load()
    dev = _on_gpu(slot)
    _i32(slot, "slot", slot.shape[0])
    flag = torch.empty(1, dtype=torch.int32, device=dev)
    _lib.check("gdn_validate_slots", lib.gdn_validate_slots(_ptr(slot), slot.shape[0], num_slots,
                                                            _ptr(flag), _stream(dev)))
    return int(flag.item())


# ------------------------------------------------------------------ measurement helpers
def probe_copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    """gdn_probe_copy: stream src's bytes into dst (same size, contiguous device
    tensors; dst may be src itself: in place) on the current stream."""
    lib = _lib.load()
    dev = _on_gpu(src, dst)
    nbytes = src.numel() * src.element_size()
    if not (src.is_contiguous() and dst.is_contiguous()) or dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must be contiguous tensors of the same size in bytes")
    _lib.check("gdn_probe_copy", lib.gdn_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(dev)))


def probe_mfma(out: torch.Tensor, blocks: int, iters: int) -> int:
    """gdn_probe_mfma on the current stream: out is a float32 device tensor of blocks x 256
    elements.  Returns the flop the launch performs."""
    lib = _lib.load()
    dev = _on_gpu(out)
    if out.dtype != torch.float32 or not out.is_contiguous() or out.numel() < blocks * 256:
        raise ValueError(f"out must be a contiguous float32 tensor of at least {blocks * 256} elements")
    _lib.check("gdn_probe_mfma", lib.gdn_probe_mfma(_ptr(out), blocks, iters, _stream(dev)))
    return blocks * 4 * 4 * iters * 32 * 32 * 16 * 2


# ------------------------------------------------------------------ short causal conv
def _conv_args(x, weight, bias, slot, pool, activation, out, keep_pool, T, N):
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError(f"x must be [T, D] with unit channel stride, got {tuple(x.shape)} / {x.stride()}")
    D = x.shape[1]
    if weight.dim() != 2 or weight.shape[0] != D or not weight.is_contiguous():
        raise ValueError(f"weight must be a contiguous [{D}, K] tensor, got {tuple(weight.shape)}")
    K = weight.shape[1]
    if pool.dim() != 3 or pool.shape[1:] != (D, K - 1) or pool.stride(2) != 1 or pool.stride(1) != K - 1:
        raise ValueError(f"pool must be [num_slots, {D}, {K - 1}] with contiguous slots' rows, got "
                         f"{tuple(pool.shape)} / {pool.stride()}")
    for t, nm in ((weight, "weight"), (bias, "bias"), (pool, "pool")):
        if t is not None and t.dtype != torch.bfloat16:
            raise ValueError(f"{nm} must be bf16")
    if bias is not None and (bias.shape != (D,) or not bias.is_contiguous()):
        raise ValueError(f"bias must be a contiguous [{D}] vector")
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16")
    if out is None:
        out = torch.empty((T, D), dtype=torch.bfloat16, device=x.device)
    elif out.shape != (T, D) or out.dtype != torch.bfloat16 or out.stride(1) != 1:
        raise ValueError(f"out must be bf16 [{T}, {D}] with unit channel stride")
    _i32(slot, "slot", N)
    a = _lib.ConvArgs(dtype=GDN_BF16, K=K, activation=int(bool(activation)), N=N, T=T, D=D,
                      x=_ptr(x), x_stride=x.stride(0) if T > 1 else D, weight=_ptr(weight),
                      bias=_ptr(bias), slot=_ptr(slot), pool=_ptr(pool), num_slots=pool.shape[0],
                      pool_stride=pool.stride(0) if pool.shape[0] > 1 else D * (K - 1),
                      out=_ptr(out), out_stride=out.stride(0) if T > 1 else D,
                      keep_pool=int(bool(keep_pool)))
    return a, out


def conv1d(x, weight, bias, cu_seqlens, slot, pool, *, has_init=None, activation=True, out=None,
           keep_pool=False, parent=None):
    """Short causal depthwise conv1d over packed sequences with a conv-state pool
    (gdn_conv1d).  x [T, D] bf16; weight [D, K] bf16 (K in 2..4, the last tap on the
    current input); bias [D] bf16 or None; cu_seqlens int32 [N+1]; slot int32 [N]
    (negative skips the sequence); pool bf16 [num_slots, D, K-1], the last K-1 inputs
    per slot, updated in place unless keep_pool; has_init int32 [N] or None (= all 1).
    parent: optional int32 [T] token tree (target verify; needs keep_pool): token i of a
    sequence continues its token parent[t] (an earlier index, -1 = the state).
    Returns out [T, D] bf16 = silu(conv) (or the plain conv without activation)."""
    lib = _lib.load()
    dev = _on_gpu(x, weight, bias, cu_seqlens, slot, pool, has_init, out, parent)
    N = slot.shape[0]
    T = x.shape[0]
    _i32(cu_seqlens, "cu_seqlens", N + 1)
    if has_init is not None:
        _i32(has_init, "has_init", N)
    if parent is not None:
        _i32(parent, "parent", T)
    a, out = _conv_args(x, weight, bias, slot, pool, activation, out, keep_pool, T, N)
    a.cu_seqlens = _ptr(cu_seqlens)
    a.has_init = _ptr(has_init)
    a.parent = _ptr(parent)
    _lib.check("gdn_conv1d", lib.gdn_conv1d(ct.byref(a), _stream(dev)))
    return out


def conv1d_update(x, weight, bias, slot, pool, *, activation=True, out=None, keep_pool=False):
    """One token per row (gdn_conv1d_update): x [B, D] bf16, row b continues
    pool[slot[b]] (negative = padding row, left untouched); out may be x itself."""
    lib = _lib.load()
    dev = _on_gpu(x, weight, bias, slot, pool, out)
    B = x.shape[0]
    a, out = _conv_args(x, weight, bias, slot, pool, activation, out, keep_pool, B, B)
    _lib.check("gdn_conv1d_update", lib.gdn_conv1d_update(ct.byref(a), _stream(dev)))
    return out


# ------------------------------------------------------------------ forward_gdn adapter
_DECODE_MODES = {"decode", "idle"}
_EXTEND_MODES = {"extend", "mixed", "draft_extend", "draft_extend_v2", "target_verify",
                 "split_prefill", "dllm_extend"}


def _is_target_verify(forward_mode) -> bool:
    if hasattr(forward_mode, "is_target_verify"):
        return bool(forward_mode.is_target_verify())
    name = getattr(forward_mode, "name", forward_mode)
    return isinstance(name, str) and name.lower() == "target_verify"


def _mode_kind(forward_mode) -> str:
    """'decode' or 'extend' for the legal forward modes, else ValueError.

    The legal set follows the SGLang GDN test-matrix article (framerc.cn), section
    on unsupported production combinations: decode-or-idle, or the extend family
    (EXTEND, MIXED, DRAFT_EXTEND, DRAFT_EXTEND_V2, TARGET_VERIFY, SPLIT_PREFILL,
    DLLM_EXTEND).  Objects with is_decode_or_idle() / is_extend() predicates are
    accepted as well as plain names."""
    if hasattr(forward_mode, "is_decode_or_idle") and forward_mode.is_decode_or_idle():
        return "decode"
    if hasattr(forward_mode, "is_extend"):
        try:
            ext = forward_mode.is_extend(include_draft_extend_v2=True)
        except TypeError:
            ext = forward_mode.is_extend()
        if ext:
            return "extend"
    name = getattr(forward_mode, "name", forward_mode)
    if isinstance(name, str):
        key = name.lower()
        if key in _DECODE_MODES:
            return "decode"
        if key in _EXTEND_MODES:
            return "extend"
    raise ValueError(f"Invalid forward mode: {forward_mode=}")


def forward_gdn(layer, forward_batch, mixed_qkv: torch.Tensor, a: torch.Tensor, b: torch.Tensor):
    """GDN layer call of a hybrid model (pymllm HybridAttnBackend.forward_gdn).

    layer: num_k_heads, num_v_heads, head_k_dim, head_v_dim, A_log [H_v] fp32,
           dt_bias [H_v] fp32, optional scale (default head_k_dim ** -0.5), layer_id.
    forward_batch: forward_mode; state_slots int32 [N]; state_pool indexable by
           layer_id -> fp32 [num_slots, H_v, d_v, d_k]; for extend modes also
           cu_seqlens int32 [N+1], optional has_initial_state int32 [N] and max_seqlen;
           for target verify the speculative state buffer spec_states (indexable by
           layer_id -> fp32 [rows, steps, H_v, d_v, d_k]) with spec_state_slots int32
           [N] and optionally spec_parents int32 [T] (token trees): the state after
           every draft token is recorded there and the pool is left unwritten (without
           spec_states / spec_state_slots target verify raises ValueError).
    mixed_qkv: [T, 2 H_qk d_k + H_v d_v]; a, b: [T, H_v].  mixed_qkv is taken as
    already convolved unless the layer carries the short conv's taps: conv_weight
    bf16 [D, K] (or [D, 1, K]) with optional conv_bias [D]; then forward_batch.conv_pool
    (indexable by layer_id -> bf16 [num_slots, D, K-1]) holds the conv states of the
    same slots, and the conv (with silu) runs first -- gdn_conv1d / gdn_conv1d_update,
    leaving the conv pool unwritten in target verify (with spec_parents the conv
    windows follow the token tree).
    Returns out [T, H_v * d_v] in mixed_qkv's dtype."""
    kind = _mode_kind(forward_batch.forward_mode)
    H_qk, H_v = layer.num_k_heads, layer.num_v_heads
    d_k, d_v = layer.head_k_dim, layer.head_v_dim
    scale = getattr(layer, "scale", None)
    scale = d_k ** -0.5 if scale is None else scale
    pool = forward_batch.state_pool[layer.layer_id]
    T = mixed_qkv.shape[0]
    if T == 0:
        return mixed_qkv.new_empty((0, H_v * d_v))
    verify = kind == "extend" and _is_target_verify(forward_batch.forward_mode)
    spec = getattr(forward_batch, "spec_states", None)
    if verify and (spec is None or getattr(forward_batch, "spec_state_slots", None) is None):
        # without a speculative buffer the verify pass would write the state after the
        # rejected draft tokens into the pool (and read a token tree as a chain)
        raise ValueError("target verify needs forward_batch.spec_states and spec_state_slots")
    conv_w = getattr(layer, "conv_weight", None)
    if conv_w is not None:
        if conv_w.dim() == 3:
            conv_w = conv_w.reshape(conv_w.shape[0], conv_w.shape[2])
        cpool = forward_batch.conv_pool[layer.layer_id]
        cbias = getattr(layer, "conv_bias", None)
        if kind == "decode":
            mixed_qkv = conv1d_update(mixed_qkv, conv_w, cbias, forward_batch.state_slots, cpool)
        else:
            mixed_qkv = conv1d(mixed_qkv, conv_w, cbias, forward_batch.cu_seqlens,
                               forward_batch.state_slots, cpool,
                               has_init=getattr(forward_batch, "has_initial_state", None),
                               keep_pool=verify,
                               parent=getattr(forward_batch, "spec_parents", None) if verify else None)
    q, k, v = split_mixed_qkv(mixed_qkv, H_qk, H_v, d_k, d_v)
    g = gdn_gate_inputs(a, b, layer.A_log, layer.dt_bias)
    # the gate is folded into the layer kernel when a, b share q's dtype (else its own launch)
    log_g = beta = None
    if g.dtype != q.dtype:
        log_g, beta = _run_gate(g, None, None)
        g = None
    if kind == "decode":
        o = decode(q, k, v, log_g, beta, forward_batch.state_slots, pool, scale=scale, gate=g)
    else:
        o = extend(q, k, v, log_g, beta, forward_batch.cu_seqlens, forward_batch.state_slots, pool,
                   has_init=getattr(forward_batch, "has_initial_state", None), scale=scale,
                   max_seqlen=int(getattr(forward_batch, "max_seqlen", 0) or 0), gate=g,
                   spec_states=spec[layer.layer_id] if verify else None,
                   spec_slot=forward_batch.spec_state_slots if verify else None,
                   spec_parent=getattr(forward_batch, "spec_parents", None) if verify else None,
                   keep_pool=verify)
    return o.view(T, H_v * d_v)


# ------------------------------------------------------------------ ssd_combined_fwd subset
def ssd_combined_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=False,
                     dt_limit=(0.0, math.inf), initial_states=None, seq_idx=None,
                     chunk_indices=None, chunk_offsets=None, seq_chunk_cumsum=None,
                     update_seq_chunk_cumsum=False, checkpoint_token_indices=None,
                     checkpoint_state_slots=None, checkpoint_states=None, out=None,
                     return_final_states=True, out_dtype=None):
    """flashinfer.mamba.ssd_combined_fwd on the delta-off kernels, batched and packed.

    x [batch, L, H, P] bf16; dt [batch, L, H]; A [H] fp32; B, C [batch, L, G, N];
    D [H] or [H, P]; z like x.  States are fp32.
    Batched mode: initial_states [batch, H, P, N]; returns (out [batch, L, H, P],
    final_states [batch, H, P, N] or None); checkpoint boundaries are relative to each
    batch element.
    Packed-varlen mode (seq_idx [1, L] given): the sequences are the runs of equal ids,
    0, 1, ... in order (ids non-decreasing); initial_states [num_seqs, H, P, N];
    final_states [num_seqs, H, P, N]; checkpoint boundaries are absolute token indices.
    num_seqs is initial_states' first dimension, else the last id + 1 (read back to the
    host).  chunk_indices, chunk_offsets and seq_chunk_cumsum describe another kernel's
    physical chunk layout and are not needed here (accepted, unused).
    Checkpoints: checkpoint_token_indices, checkpoint_state_slots [sequences] int32,
    checkpoint_states fp32 [num_checkpoints, H, P, N], all three together.
    update_seq_chunk_cumsum and the caller-owned 5-D `out` storage raise
    NotImplementedError.  out_dtype (an extension) selects the output dtype; default
    x's dtype."""
    if out is not None or update_seq_chunk_cumsum:
        raise NotImplementedError("caller-owned out and update_seq_chunk_cumsum are not supported")
    batch, L, H, P = x.shape
    G, Nst = B.shape[2], B.shape[3]
    dev = _on_gpu(x, dt, A, B, C, D, z, dt_bias, initial_states)
    if H % G:
        raise ValueError("nheads must be a multiple of ngroups")
    T = batch * L
    for t, nm in ((x, "x"), (dt, "dt"), (B, "B"), (C, "C"), (z, "z")):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    g = ssd_gate_inputs(dt.view(T, H), A, dt_bias, dt_softplus, dt_limit)
    log_g = dtp = None
    if g.dtype != x.dtype:   # folded into the extend kernel only when dt shares x's dtype
        log_g, dtp = _run_gate(g, None, None)
        g = None
    if seq_idx is not None:                     # packed varlen: runs of equal ids
        if batch != 1 or seq_idx.shape != (1, L):
            raise ValueError("packed-varlen mode takes batch 1 and seq_idx [1, seqlen]")
        if seq_idx.device != dev:
            raise ValueError("seq_idx must be on x's device")
        ids = seq_idx[0].to(torch.int64).contiguous()
        nseq = (initial_states.shape[0] if initial_states is not None
                else (int(ids[-1].item()) + 1 if L > 0 else 0))
        cu = torch.searchsorted(ids, torch.arange(nseq + 1, device=dev)).to(torch.int32)
        relative = False
    else:
        nseq = batch
        cu = torch.arange(0, T + 1, L, dtype=torch.int32, device=dev)
        relative = True
    if initial_states is not None:
        pool = initial_states.to(torch.float32).contiguous().clone()
    else:
        pool = torch.empty((nseq, H, P, Nst), dtype=torch.float32, device=dev)
    slot = torch.arange(nseq, dtype=torch.int32, device=dev)
    has_init = torch.full((nseq,), int(initial_states is not None), dtype=torch.int32, device=dev)
    o = extend(C.view(T, G, Nst), B.view(T, G, Nst), x.view(T, H, P), log_g, dtp, cu, slot, pool,
               has_init=has_init, mode="ssd", D=D, z=None if z is None else z.view(T, H, P),
               max_seqlen=L if seq_idx is None else 0, out_dtype=out_dtype, gate=g,
               ckpt_token=checkpoint_token_indices, ckpt_slot=checkpoint_state_slots,
               ckpt_states=checkpoint_states, ckpt_relative=relative)
    return o.view(batch, L, H, P), (pool if return_final_states else None)
