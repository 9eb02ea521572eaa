"""ctypes view of libgdn.so (include/gdn.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK, GDN_E_NULL, GDN_E_SHAPE, GDN_E_DTYPE, GDN_E_UNSUPPORTED, GDN_E_INDEX, GDN_E_HIP, GDN_E_SCRATCH = range(8)
GDN_F32, GDN_BF16 = 0, 1
GDN_MODE_GDN, GDN_MODE_SSD = 0, 1
ABI_VERSION = 8

EXPORTED = ["gdn_gate", "gdn_extend", "gdn_decode", "gdn_extend_gated", "gdn_decode_gated",
            "gdn_conv1d", "gdn_conv1d_update", "gdn_validate_slots", "gdn_status_str",
            "gdn_last_hip_error", "gdn_abi_version", "gdn_extend_workspace_size", "gdn_extend_kernel",
            "gdn_extend_noalloc", "gdn_probe_copy", "gdn_probe_mfma"]

# gdn_extend_kernel results and reason bits (include/gdn.h)
GDN_KERNEL_RECURRENT, GDN_KERNEL_CHUNKED, GDN_KERNEL_SSD_CHUNKED = 1, 2, 3
KERNEL_NAMES = {0: "none", GDN_KERNEL_RECURRENT: "recurrent", GDN_KERNEL_CHUNKED: "chunked64",
                GDN_KERNEL_SSD_CHUNKED: "ssd_chunked128"}
WHY_NAMES = ["fp32_inputs", "short_batch", "target_verify", "head_dims", "alignment", "stride",
             "batch", "gate_alignment", "no_workspace", "chunk64_requested"]


class GateArgs(C.Structure):
    _fields_ = [("mode", C.c_int32), ("in_dtype", C.c_int32), ("T", C.c_int64), ("H", C.c_int32),
                ("_pad0", C.c_int32), ("a", C.c_void_p), ("a_stride", C.c_int64),
                ("b", C.c_void_p), ("b_stride", C.c_int64), ("A", C.c_void_p),
                ("dt_bias", C.c_void_p), ("dt_softplus", C.c_int32), ("dt_min", C.c_float),
                ("dt_max", C.c_float), ("_pad1", C.c_int32), ("log_g", C.c_void_p),
                ("beta", C.c_void_p)]


class ExtendArgs(C.Structure):
    _fields_ = [("mode", C.c_int32), ("in_dtype", C.c_int32), ("out_dtype", C.c_int32),
                ("N", C.c_int32), ("T", C.c_int64), ("H_qk", C.c_int32), ("H_v", C.c_int32),
                ("d_k", C.c_int32), ("d_v", C.c_int32), ("chunk", C.c_int32),
                ("max_seqlen", C.c_int32), ("q", C.c_void_p), ("q_stride", C.c_int64),
                ("k", C.c_void_p), ("k_stride", C.c_int64), ("v", C.c_void_p),
                ("v_stride", C.c_int64), ("log_g", C.c_void_p), ("beta", C.c_void_p),
                ("cu_seqlens", C.c_void_p), ("slot", C.c_void_p), ("has_init", C.c_void_p),
                ("pool", C.c_void_p), ("num_slots", C.c_int64), ("out", C.c_void_p),
                ("out_stride", C.c_int64), ("scale", C.c_float), ("D_per_dim", C.c_int32),
                ("D", C.c_void_p), ("z", C.c_void_p), ("z_stride", C.c_int64),
                ("ckpt_token", C.c_void_p), ("ckpt_slot", C.c_void_p), ("ckpt_states", C.c_void_p),
                ("num_ckpt", C.c_int64), ("ckpt_relative", C.c_int32), ("keep_pool", C.c_int32),
                ("spec_states", C.c_void_p), ("spec_slot", C.c_void_p), ("spec_parent", C.c_void_p),
                ("num_spec", C.c_int64), ("spec_steps", C.c_int32), ("_pad_spec", C.c_int32),
                ("workspace", C.c_void_p), ("workspace_bytes", C.c_int64)]


class DecodeArgs(C.Structure):
    _fields_ = [("in_dtype", C.c_int32), ("out_dtype", C.c_int32), ("B", C.c_int32),
                ("H_qk", C.c_int32), ("H_v", C.c_int32), ("d_k", C.c_int32), ("d_v", C.c_int32),
                ("_pad0", C.c_int32), ("q", C.c_void_p), ("q_stride", C.c_int64),
                ("k", C.c_void_p), ("k_stride", C.c_int64), ("v", C.c_void_p),
                ("v_stride", C.c_int64), ("log_g", C.c_void_p), ("beta", C.c_void_p),
                ("slot", C.c_void_p), ("pool", C.c_void_p), ("num_slots", C.c_int64),
                ("out", C.c_void_p), ("out_stride", C.c_int64), ("scale", C.c_float),
                ("_pad1", C.c_int32)]


class ConvArgs(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("K", C.c_int32), ("activation", C.c_int32), ("N", C.c_int32),
                ("T", C.c_int64), ("D", C.c_int64), ("x", C.c_void_p), ("x_stride", C.c_int64),
                ("weight", C.c_void_p), ("bias", C.c_void_p), ("cu_seqlens", C.c_void_p),
                ("slot", C.c_void_p), ("has_init", C.c_void_p), ("pool", C.c_void_p),
                ("num_slots", C.c_int64), ("pool_stride", C.c_int64), ("out", C.c_void_p),
                ("out_stride", C.c_int64), ("keep_pool", C.c_int32), ("_pad0", C.c_int32),
                ("parent", C.c_void_p)]


_lib = None


def load(path: str | None = None) -> C.CDLL:
    """Load libgdn.so once.  Raises RuntimeError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m hybrid_model_linear_amd.build`"
                           " (the GDN layer has no fallback implementation)")
    lib = C.CDLL(path)
    lib.gdn_gate.argtypes = [C.POINTER(GateArgs), C.c_void_p]
    lib.gdn_extend.argtypes = [C.POINTER(ExtendArgs), C.c_void_p]
    lib.gdn_decode.argtypes = [C.POINTER(DecodeArgs), C.c_void_p]
    lib.gdn_extend_gated.argtypes = [C.POINTER(ExtendArgs), C.POINTER(GateArgs), C.c_void_p]
    lib.gdn_decode_gated.argtypes = [C.POINTER(DecodeArgs), C.POINTER(GateArgs), C.c_void_p]
    lib.gdn_conv1d.argtypes = [C.POINTER(ConvArgs), C.c_void_p]
    lib.gdn_conv1d_update.argtypes = [C.POINTER(ConvArgs), C.c_void_p]
    lib.gdn_validate_slots.argtypes = [C.c_void_p, C.c_int32, C.c_int64, C.c_void_p, C.c_void_p]
    for fn in ("gdn_gate", "gdn_extend", "gdn_decode", "gdn_extend_gated", "gdn_decode_gated",
               "gdn_conv1d", "gdn_conv1d_update", "gdn_validate_slots", "gdn_last_hip_error",
               "gdn_abi_version"):
        getattr(lib, fn).restype = C.c_int
    lib.gdn_extend_workspace_size.argtypes = [C.POINTER(ExtendArgs), C.POINTER(GateArgs)]
    lib.gdn_extend_workspace_size.restype = C.c_int64
    lib.gdn_extend_kernel.argtypes = [C.POINTER(ExtendArgs), C.POINTER(GateArgs), C.POINTER(C.c_int32)]
    lib.gdn_extend_kernel.restype = C.c_int
    lib.gdn_extend_noalloc.argtypes = [C.POINTER(ExtendArgs), C.POINTER(GateArgs), C.c_void_p]
    lib.gdn_extend_noalloc.restype = C.c_int
    lib.gdn_probe_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]
    lib.gdn_probe_copy.restype = C.c_int
    lib.gdn_probe_mfma.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p]
    lib.gdn_probe_mfma.restype = C.c_int
    lib.gdn_status_str.argtypes = [C.c_int]
    lib.gdn_status_str.restype = C.c_char_p
    lib.gdn_last_hip_error.argtypes = []
    lib.gdn_abi_version.argtypes = []
    if lib.gdn_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libgdn.so ABI {lib.gdn_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = lib
    return lib


class GDNError(RuntimeError):
    def __init__(self, fn: str, status: int, hip: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {status}, hipError {hip})")
        self.status = status
        self.hip_error = hip


def check(fn: str, status: int) -> None:
    if status == GDN_OK:
        return
    lib = load()
    msg = lib.gdn_status_str(status).decode()
    hip = lib.gdn_last_hip_error()
    if status in (GDN_E_SHAPE, GDN_E_DTYPE, GDN_E_NULL, GDN_E_UNSUPPORTED, GDN_E_INDEX, GDN_E_SCRATCH):
        err = ValueError(f"{fn} rejected its arguments: {msg} (status {status})")
        err.status = status
        raise err
    raise GDNError(fn, status, hip, msg)
