"""Host-side tests of the C-ABI library and the Python binding (no GPU needed).

The library is loaded and its error conventions are exercised with arguments
that fail validation, so nothing is ever launched.  The forward_gdn adapter is
tested with mocked library calls (spy technique of the SGLang GDN test-matrix
article, section "Hybrid dispatch fan-out tests": sentinel identity, not exact
argument shapes)."""
import ctypes as ct
import os
import re
import subprocess
import tempfile
from types import SimpleNamespace
from unittest import mock

import pytest
import torch

import hybrid_model_linear_amd as gdn
from hybrid_model_linear_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int|int64_t)\s+(gdn_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = gdn.load()
    names = _declared_functions()
    assert set(names) == set(_lib.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.gdn_abi_version() == _lib.ABI_VERSION


def test_struct_layouts_match_header():
    """offsetof/sizeof from the C compiler == ctypes layout used by the binding."""
    structs = {"gdn_gate_args": _lib.GateArgs, "gdn_extend_args": _lib.ExtendArgs,
               "gdn_decode_args": _lib.DecodeArgs, "gdn_conv_args": _lib.ConvArgs}
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', 'int main(void){']
    for cname, cls in structs.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0;}")
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "l.c"), os.path.join(d, "l")
        open(src, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-std=c99", "-o", exe, src], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    got = {}
    for line in out.splitlines():
        s, f, v = line.split()
        got[(s, f)] = int(v)
    for cname, cls in structs.items():
        assert got[(cname, "size")] == ct.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert got[(cname, f)] == getattr(cls, f).offset, (cname, f)


def _ext(**kw):
    base = dict(mode=0, in_dtype=1, out_dtype=1, N=1, T=4, H_qk=2, H_v=4, d_k=128, d_v=128,
                chunk=0, max_seqlen=0, q_stride=2 * 2 * 128 + 4 * 128, k_stride=2 * 2 * 128 + 4 * 128,
                v_stride=2 * 2 * 128 + 4 * 128, num_slots=8, out_stride=4 * 128, scale=0.088)
    base.update(kw)
    return _lib.ExtendArgs(**base)


FAKE = ct.c_void_p(0x1000)   # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("kw,status", [
    (dict(), _lib.GDN_E_NULL),                                   # q/k/v/... are NULL
    (dict(H_v=3), _lib.GDN_E_SHAPE),                             # H_v % H_qk
    (dict(d_k=96), _lib.GDN_E_UNSUPPORTED),
    (dict(d_v=32), _lib.GDN_E_UNSUPPORTED),
    (dict(in_dtype=7), _lib.GDN_E_DTYPE),
    (dict(chunk=128), _lib.GDN_E_UNSUPPORTED),
    (dict(mode=5), _lib.GDN_E_UNSUPPORTED),
    (dict(q_stride=100), _lib.GDN_E_SHAPE),
    (dict(out_stride=100), _lib.GDN_E_SHAPE),
    (dict(num_slots=0), _lib.GDN_E_SHAPE),
    (dict(scale=float("nan")), _lib.GDN_E_SHAPE),
    (dict(D=FAKE), _lib.GDN_E_SHAPE),                            # SSD-only input in GDN mode
    (dict(N=-1), _lib.GDN_E_SHAPE),
    (dict(q_stride=2 * 2 * 128 + 4 * 128 + 2), _lib.GDN_E_SHAPE),  # stride not a multiple of 4
    (dict(cu_seqlens=FAKE, slot=FAKE, pool=FAKE, q=ct.c_void_p(0x1002), k=FAKE, v=FAKE, log_g=FAKE,
          beta=FAKE, out=FAKE), _lib.GDN_E_SHAPE),               # q not 8-byte aligned (bf16)
    (dict(ckpt_token=FAKE), _lib.GDN_E_NULL),                    # checkpoint arguments: all or none
    (dict(ckpt_token=FAKE, ckpt_slot=FAKE), _lib.GDN_E_NULL),
    (dict(ckpt_token=FAKE, ckpt_slot=FAKE, ckpt_states=FAKE, num_ckpt=-1), _lib.GDN_E_SHAPE),
    (dict(ckpt_token=FAKE, ckpt_slot=FAKE, ckpt_states=ct.c_void_p(0x1008), num_ckpt=2),
     _lib.GDN_E_SHAPE),                                          # checkpoint states not 16-byte aligned
    (dict(N=0, ckpt_states=FAKE), _lib.GDN_E_NULL),              # checked before the empty-call exit
    (dict(spec_states=FAKE, spec_steps=4), _lib.GDN_E_NULL),     # target-verify states need their rows
    (dict(spec_slot=FAKE), _lib.GDN_E_NULL),
    (dict(spec_parent=FAKE), _lib.GDN_E_NULL),                   # a token tree needs the state buffer
    (dict(spec_states=FAKE, spec_slot=FAKE, spec_steps=0, num_spec=2), _lib.GDN_E_SHAPE),
    (dict(spec_states=ct.c_void_p(0x1008), spec_slot=FAKE, spec_steps=4, num_spec=2), _lib.GDN_E_SHAPE),
])
def test_extend_validation(kw, status):
    lib = gdn.load()
    assert lib.gdn_extend(ct.byref(_ext(**kw)), None) == status


def test_extend_null_and_empty():
    lib = gdn.load()
    assert lib.gdn_extend(None, None) == _lib.GDN_E_NULL
    assert lib.gdn_extend(ct.byref(_ext(N=0)), None) == _lib.GDN_OK      # nothing to do
    a = _ext(cu_seqlens=FAKE, slot=FAKE, pool=FAKE)                      # q..out missing
    assert lib.gdn_extend(ct.byref(a), None) == _lib.GDN_E_NULL


# ------------------------------------------------------------------ kernel choice and workspace
# Host-side planning only: gdn_extend_kernel and gdn_extend_workspace_size decide exactly
# as gdn_extend does and launch nothing, so fake (aligned, never dereferenced) pointers do.
def _ptrs(**kw):
    d = dict(q=ct.c_void_p(0x10000), k=ct.c_void_p(0x20000), v=ct.c_void_p(0x30000),
             log_g=ct.c_void_p(0x40000), beta=ct.c_void_p(0x50000), cu_seqlens=FAKE, slot=FAKE,
             pool=ct.c_void_p(0x60000), out=ct.c_void_p(0x70000))
    d.update(kw)
    return d


def _ssd(**kw):
    """Delta-off arguments shaped like the Mamba2 workload (2 x 8192 tokens, 80 heads of
    headdim 64, one group of dstate 128)."""
    base = dict(mode=1, in_dtype=1, out_dtype=1, N=2, T=16384, H_qk=1, H_v=80, d_k=128, d_v=64,
                chunk=0, max_seqlen=8192, q_stride=128, k_stride=128, v_stride=80 * 64,
                num_slots=2, out_stride=80 * 64, scale=1.0, **_ptrs())
    base.update(kw)
    return _lib.ExtendArgs(**base)


def _kernel(args, gate=None):
    lib = gdn.load()
    why = ct.c_int32(-1)
    k = lib.gdn_extend_kernel(ct.byref(args), None if gate is None else ct.byref(gate), ct.byref(why))
    return k, why.value


W = {n: 1 << i for i, n in enumerate(_lib.WHY_NAMES)}


@pytest.mark.parametrize("kw,kernel,why", [
    (dict(), _lib.GDN_KERNEL_CHUNKED, 0),
    (dict(in_dtype=0, out_dtype=0), _lib.GDN_KERNEL_RECURRENT, W["fp32_inputs"]),
    (dict(max_seqlen=4), _lib.GDN_KERNEL_RECURRENT, W["short_batch"]),
    (dict(d_k=64, q_stride=2 * 2 * 64 + 4 * 128, k_stride=2 * 2 * 64 + 4 * 128, v_stride=2 * 2 * 64 + 4 * 128),
     _lib.GDN_KERNEL_RECURRENT, W["head_dims"]),
    (dict(q=ct.c_void_p(0x10008)), _lib.GDN_KERNEL_RECURRENT, W["alignment"]),
    (dict(q_stride=16 * 1024 * 1024), _lib.GDN_KERNEL_RECURRENT, W["stride"]),
    (dict(spec_states=ct.c_void_p(0x80000), spec_slot=FAKE, num_spec=1, spec_steps=4),
     _lib.GDN_KERNEL_RECURRENT, W["target_verify"]),
    (dict(N=0), 0, 0),                                            # launches nothing
    (dict(chunk=128), -_lib.GDN_E_UNSUPPORTED, 0),                # GDN mode has chunk 64 only
])
def test_extend_kernel_choice_gdn(kw, kernel, why):
    a = _ext(**_ptrs())
    for k, v in kw.items():
        setattr(a, k, v)
    assert _kernel(a) == (kernel, why)


def test_extend_kernel_choice_folded_gate_alignment():
    g = _lib.GateArgs(mode=0, in_dtype=1, T=4, H=4, a=ct.c_void_p(0x90002), a_stride=4,
                      b=ct.c_void_p(0xA0000), b_stride=4, A=FAKE)
    a = _ext(**_ptrs(log_g=None, beta=None))
    assert _kernel(a, g) == (_lib.GDN_KERNEL_RECURRENT, W["gate_alignment"])
    g.a = ct.c_void_p(0x90000)
    assert _kernel(a, g) == (_lib.GDN_KERNEL_CHUNKED, 0)


def test_ssd_kernel_choice_and_workspace():
    lib = gdn.load()
    a = _ssd()
    need = lib.gdn_extend_workspace_size(ct.byref(a), None)
    # fp16 B and C copies (16384 x 128 x 2 bytes each), the raw C B^T tiles of the
    # 16384 / 128 + 2 chunk slots (ten 32 x 32 fp16 tiles each), plus segment states
    bc = 16384 * 128 * 2
    cb = (16384 // 128 + 2) * 10 * 32 * 32 * 2
    one = 2 * bc + cb                                                          # one segment's workspace
    assert need > one and (need - one) % 256 == 0
    assert _kernel(a) == (_lib.GDN_KERNEL_CHUNKED, W["no_workspace"])          # chunk 64 without it
    a.workspace, a.workspace_bytes = ct.c_void_p(0x1000000), need
    assert _kernel(a) == (_lib.GDN_KERNEL_SSD_CHUNKED, 0)
    a.workspace_bytes = one                                                    # one segment still fits
    assert _kernel(a) == (_lib.GDN_KERNEL_SSD_CHUNKED, 0)
    a.workspace_bytes = one - 256                                              # too small: chunk 64
    assert _kernel(a) == (_lib.GDN_KERNEL_CHUNKED, W["no_workspace"])
    a.chunk = 128                                                              # ... unless 128 is asked for
    assert _kernel(a)[0] == -_lib.GDN_E_SHAPE
    a.workspace, a.workspace_bytes = None, 0
    assert _kernel(a)[0] == -_lib.GDN_E_NULL
    a.workspace, a.workspace_bytes, a.chunk = ct.c_void_p(0x1000000), need, 64
    assert _kernel(a) == (_lib.GDN_KERNEL_CHUNKED, W["chunk64_requested"])
    assert lib.gdn_extend_workspace_size(ct.byref(a), None) == 0              # chunk 64 needs none
    a.chunk = 0
    a.workspace = ct.c_void_p(0x1000010)                                      # not 256-byte aligned
    assert _kernel(a)[0] == -_lib.GDN_E_SHAPE
    a.workspace = ct.c_void_p(0x1000000)
    a.in_dtype = a.out_dtype = 0                                               # fp32 inputs: token-recurrent
    assert _kernel(a) == (_lib.GDN_KERNEL_RECURRENT, W["fp32_inputs"])
    assert lib.gdn_extend_workspace_size(ct.byref(a), None) == 0
    a.chunk = 128
    assert _kernel(a)[0] == -_lib.GDN_E_UNSUPPORTED
    assert lib.gdn_extend_workspace_size(ct.byref(_ext(**_ptrs())), None) == 0  # GDN mode: none


def test_ssd_chunk128_needs_16_byte_rows_of_z_and_out():
    """The chunk-128 delta-off kernel reads z and writes out as 16-byte pieces of whole
    rows: an out pointer or row stride off 16 bytes sends chunk 0 to the chunk-64 kernel
    (reason: alignment; a z off 16 bytes, which the chunk-64 kernel also stages in
    16-byte segments, to the token-recurrent one) and makes chunk 128 unsupported."""
    lib = gdn.load()
    a = _ssd(z=ct.c_void_p(0x80000), z_stride=80 * 64)
    a.workspace = ct.c_void_p(0x1000000)
    a.workspace_bytes = lib.gdn_extend_workspace_size(ct.byref(a), None)
    assert _kernel(a) == (_lib.GDN_KERNEL_SSD_CHUNKED, 0)
    for field, value, kernel in (("out_stride", 80 * 64 + 4, _lib.GDN_KERNEL_CHUNKED),
                                 ("out", ct.c_void_p(0x70008), _lib.GDN_KERNEL_CHUNKED),
                                 ("z_stride", 80 * 64 + 4, _lib.GDN_KERNEL_RECURRENT),
                                 ("z", ct.c_void_p(0x80008), _lib.GDN_KERNEL_RECURRENT)):
        b = _ssd(z=ct.c_void_p(0x80000), z_stride=80 * 64, workspace=a.workspace,
                 workspace_bytes=a.workspace_bytes)
        setattr(b, field, value)
        assert _kernel(b) == (kernel, W["alignment"]), field
        b.chunk = 128
        assert _kernel(b)[0] == -_lib.GDN_E_UNSUPPORTED, field
    f = _ssd(out_dtype=0, out_stride=80 * 64 + 4, workspace=a.workspace,   # fp32 out: 16-byte rows
             workspace_bytes=a.workspace_bytes)
    assert _kernel(f) == (_lib.GDN_KERNEL_SSD_CHUNKED, 0)


def test_ssd_workspace_grows_with_segments_and_unknown_length_needs_one():
    """Without a length hint the kernel runs one segment per sequence: the workspace holds
    only the B and C copies and the chunks' raw C B^T tiles.  With the hint, the segment
    states come on top."""
    lib = gdn.load()
    a = _ssd(max_seqlen=0)
    one = lib.gdn_extend_workspace_size(ct.byref(a), None)
    assert one == 2 * 16384 * 128 * 2 + (16384 // 128 + 2) * 10 * 32 * 32 * 2
    a.max_seqlen = 8192
    assert lib.gdn_extend_workspace_size(ct.byref(a), None) > one


def test_ssd_plan_cuts_the_state_pass_finer_than_the_segments():
    """The Mamba2-shaped call on 256 CUs (the count the host assumes without a device):
    three segments per sequence for the full pass (2 x 40 head pairs x 3 = 240
    workgroups), and the state-only pass cuts each of the first two into three pieces
    (480 workgroups of ~7 chunks instead of 160 of 22): six pieces' fp32 states
    [80, 64, 128] and log decays per sequence on top of the one-segment workspace."""
    lib = gdn.load()
    one = lib.gdn_extend_workspace_size(ct.byref(_ssd(max_seqlen=0)), None)
    up = lambda b: (b + 255) & ~255
    pieces = 2 * 6
    assert lib.gdn_extend_workspace_size(ct.byref(_ssd()), None) == \
        one + up(pieces * 80 * 64 * 128 * 4) + up(pieces * 80 * 4)


def test_extend_noalloc_host_checks_come_before_any_device_call():
    """gdn_extend_noalloc validates everything on the host before it touches a device:
    the workspace fields are its own (a caller's workspace is refused), invalid
    arguments fail as in gdn_extend, and a delta-off call whose chunk-128 kernel needs
    more than the static scratch at one segment per sequence is refused."""
    lib = gdn.load()
    assert _lib.GDN_E_SCRATCH == 7
    assert lib.gdn_extend_noalloc(None, None, None) == _lib.GDN_E_NULL
    a = _ssd(workspace=ct.c_void_p(0x1000000), workspace_bytes=1 << 20)
    assert lib.gdn_extend_noalloc(ct.byref(a), None, None) == _lib.GDN_E_SHAPE
    a = _ssd(workspace_bytes=256)
    assert lib.gdn_extend_noalloc(ct.byref(a), None, None) == _lib.GDN_E_SHAPE
    assert lib.gdn_extend_noalloc(ct.byref(_ext(H_v=3)), None, None) == _lib.GDN_E_SHAPE
    assert lib.gdn_extend_noalloc(ct.byref(_ext(N=0)), None, None) == _lib.GDN_OK   # nothing to do
    limit = 64 << 20
    # B and C copies alone: 2 x T x H_qk x 128 x 2 bytes at one segment
    T = limit // (2 * 128 * 2) + 256
    big = _ssd(T=T, max_seqlen=0, N=2)
    assert lib.gdn_extend_workspace_size(ct.byref(big), None) > limit
    assert lib.gdn_extend_noalloc(ct.byref(big), None, None) == _lib.GDN_E_SCRATCH
    with pytest.raises(ValueError, match="static scratch"):
        _lib.check("gdn_extend_noalloc", _lib.GDN_E_SCRATCH)
    big.chunk = 128
    assert lib.gdn_extend_noalloc(ct.byref(big), None, None) == _lib.GDN_E_SCRATCH
    big.chunk, big.in_dtype, big.out_dtype = 0, 0, 0            # fp32: another kernel, no scratch
    assert _kernel(big)[0] == _lib.GDN_KERNEL_RECURRENT
    big.chunk = 128                                             # fp32 has no chunk-128 kernel
    assert lib.gdn_extend_noalloc(ct.byref(big), None, None) == _lib.GDN_E_UNSUPPORTED


def _conv(**kw):
    base = dict(dtype=1, K=4, activation=1, N=2, T=10, D=64, x=ct.c_void_p(0x10000), x_stride=64,
                weight=ct.c_void_p(0x20000), cu_seqlens=FAKE, slot=FAKE, pool=ct.c_void_p(0x30000),
                num_slots=4, pool_stride=192, out=ct.c_void_p(0x40000), out_stride=64)
    base.update(kw)
    return _lib.ConvArgs(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=0), _lib.GDN_E_DTYPE),                           # bf16 only
    (dict(K=5), _lib.GDN_E_UNSUPPORTED),
    (dict(K=1), _lib.GDN_E_UNSUPPORTED),
    (dict(D=12), _lib.GDN_E_SHAPE),                              # channels in vectors of 8
    (dict(D=0), _lib.GDN_E_SHAPE),
    (dict(x_stride=60), _lib.GDN_E_SHAPE),                       # row stride < D
    (dict(out_stride=72 + 4), _lib.GDN_E_SHAPE),                 # not a multiple of 8
    (dict(pool_stride=184), _lib.GDN_E_SHAPE),                   # < D (K - 1)
    (dict(num_slots=0), _lib.GDN_E_SHAPE),
    (dict(N=0), _lib.GDN_E_SHAPE),                               # tokens without sequences
    (dict(N=0, T=0), _lib.GDN_OK),                               # nothing to do
    (dict(weight=None), _lib.GDN_E_NULL),
    (dict(cu_seqlens=None), _lib.GDN_E_NULL),
    (dict(x=None), _lib.GDN_E_NULL),
    (dict(x=ct.c_void_p(0x10008)), _lib.GDN_E_SHAPE),            # not 16-byte aligned
    (dict(bias=ct.c_void_p(0x50004)), _lib.GDN_E_SHAPE),
    (dict(out=ct.c_void_p(0x10000 + 2 * 64 * 9)), _lib.GDN_E_SHAPE),   # out overlaps x's last row
    (dict(out=ct.c_void_p(0x30000 + 16)), _lib.GDN_E_SHAPE),     # out overlaps the pool
    (dict(parent=FAKE), _lib.GDN_E_SHAPE),                       # a token tree must keep the pool
])
def test_conv_validation(kw, status):
    lib = gdn.load()
    assert lib.gdn_conv1d(ct.byref(_conv(**kw)), None) == status


def test_conv_update_validation():
    lib = gdn.load()
    assert lib.gdn_conv1d_update(None, None) == _lib.GDN_E_NULL
    assert lib.gdn_conv1d_update(ct.byref(_conv(N=3, T=4)), None) == _lib.GDN_E_SHAPE   # T != rows
    assert lib.gdn_conv1d_update(ct.byref(_conv(N=0, T=0)), None) == _lib.GDN_OK
    # cu_seqlens is not needed; out may be x itself (checked only for the varlen call)
    a = _conv(N=3, T=3, cu_seqlens=None, out=ct.c_void_p(0x10000), slot=None)
    assert lib.gdn_conv1d_update(ct.byref(a), None) == _lib.GDN_E_NULL                # slot missing


def test_gate_and_decode_validation():
    lib = gdn.load()
    g = _lib.GateArgs(mode=0, in_dtype=1, T=0, H=4)
    assert lib.gdn_gate(ct.byref(g), None) == _lib.GDN_OK              # T = 0 is a no-op
    g = _lib.GateArgs(mode=0, in_dtype=1, T=3, H=4)
    assert lib.gdn_gate(ct.byref(g), None) == _lib.GDN_E_NULL
    g = _lib.GateArgs(mode=1, in_dtype=1, T=3, H=4, a=FAKE, a_stride=4, A=FAKE, log_g=FAKE,
                      beta=FAKE, b=FAKE, b_stride=4)
    assert lib.gdn_gate(ct.byref(g), None) == _lib.GDN_E_SHAPE         # b given in SSD mode
    g = _lib.GateArgs(mode=1, in_dtype=1, T=3, H=4, a=FAKE, a_stride=4, A=FAKE, log_g=FAKE,
                      beta=FAKE, dt_min=2.0, dt_max=1.0)
    assert lib.gdn_gate(ct.byref(g), None) == _lib.GDN_E_SHAPE         # empty clamp range
    g = _lib.GateArgs(mode=0, in_dtype=1, T=3, H=4, a=FAKE, a_stride=2, A=FAKE, log_g=FAKE,
                      beta=FAKE, b=FAKE, b_stride=4)
    assert lib.gdn_gate(ct.byref(g), None) == _lib.GDN_E_SHAPE         # row stride < H
    d = _lib.DecodeArgs(in_dtype=1, out_dtype=1, B=2, H_qk=2, H_v=4, d_k=128, d_v=128,
                        q_stride=1024, k_stride=1024, v_stride=1024, num_slots=4, out_stride=512,
                        scale=0.1)
    assert lib.gdn_decode(ct.byref(d), None) == _lib.GDN_E_NULL
    d.B = 0
    assert lib.gdn_decode(ct.byref(d), None) == _lib.GDN_OK
    d.B, d.H_v = 2, 5
    assert lib.gdn_decode(ct.byref(d), None) == _lib.GDN_E_SHAPE
    assert lib.gdn_validate_slots(None, 3, 4, None, None) == _lib.GDN_E_NULL
    assert lib.gdn_validate_slots(None, 3, 4, FAKE, None) == _lib.GDN_E_NULL
    assert lib.gdn_validate_slots(None, -1, 4, FAKE, None) == _lib.GDN_E_SHAPE
    assert lib.gdn_status_str(_lib.GDN_E_HIP) == b"HIP runtime error"


def test_gated_calls_validation():
    lib = gdn.load()
    e = _ext(cu_seqlens=FAKE, slot=FAKE, pool=FAKE, q=FAKE, k=FAKE, v=FAKE, out=FAKE)   # no log_g/beta
    g = _lib.GateArgs(mode=0, in_dtype=1, T=4, H=4, a=FAKE, a_stride=4, b=FAKE, b_stride=4, A=FAKE)
    assert lib.gdn_extend_gated(ct.byref(e), None, None) == _lib.GDN_E_NULL
    assert lib.gdn_extend(ct.byref(e), None) == _lib.GDN_E_NULL                 # ungated needs log_g
    for kw, status in ((dict(mode=1, b=None), _lib.GDN_E_UNSUPPORTED),        # mode differs
                       (dict(in_dtype=0), _lib.GDN_E_DTYPE),                   # dtype differs
                       (dict(T=5), _lib.GDN_E_SHAPE),                          # token count differs
                       (dict(H=2, a_stride=2, b_stride=2), _lib.GDN_E_SHAPE),  # head count differs
                       (dict(a=None), _lib.GDN_E_NULL),
                       (dict(b=None), _lib.GDN_E_NULL),
                       (dict(a_stride=3), _lib.GDN_E_SHAPE)):
        bad = _lib.GateArgs.from_buffer_copy(g)
        for f, val in kw.items():
            setattr(bad, f, val)
        assert lib.gdn_extend_gated(ct.byref(e), ct.byref(bad), None) == status, kw
    d = _lib.DecodeArgs(in_dtype=1, out_dtype=1, B=4, H_qk=2, H_v=4, d_k=128, d_v=128,
                        q_stride=1024, k_stride=1024, v_stride=1024, num_slots=4, out_stride=512,
                        scale=0.1)
    assert lib.gdn_decode_gated(ct.byref(d), None, None) == _lib.GDN_E_NULL
    assert lib.gdn_decode_gated(ct.byref(d), ct.byref(g), None) == _lib.GDN_E_NULL   # q .. missing
    gs = _lib.GateArgs.from_buffer_copy(g)
    gs.mode, gs.b = 1, None
    assert lib.gdn_decode_gated(ct.byref(d), ct.byref(gs), None) == _lib.GDN_E_UNSUPPORTED   # decode is GDN only


def test_binding_checks_token_counts():
    """k, v, out and z must have q's token count (the library cannot see buffer
    lengths): a shorter one is refused before anything runs."""
    T, N = 6, 2
    q = torch.zeros(T, 2, 128, dtype=torch.bfloat16)
    v = torch.zeros(T, 4, 128, dtype=torch.bfloat16)
    cu = torch.tensor([0, 3, 6], dtype=torch.int32)
    slot = torch.arange(N, dtype=torch.int32)
    pool = torch.zeros(N, 4, 128, 128)
    lg = torch.zeros(T, 4)
    for kw, name in ((dict(k=q[:5]), "k"), (dict(v=v[:4]), "v"), (dict(out=torch.zeros(T - 1, 4, 128)), "out")):
        a = dict(k=q, v=v, out=None)
        a.update(kw)
        with pytest.raises(ValueError, match=f"{name} must have {T} rows"):
            gdn.extend(q, a["k"], a["v"], lg, lg, cu, slot, pool, out=a["out"])
    with pytest.raises(ValueError, match=f"z must have {T} rows"):
        gdn.extend(q, q, v, lg, lg, cu, slot, pool, mode="ssd", z=v[:2])
    with pytest.raises(ValueError, match="v must have 6 rows"):
        gdn.decode(q, q, v[:3], lg, lg, torch.arange(T, dtype=torch.int32), pool)


def test_binding_rejects_cpu_tensors():
    q = torch.zeros(4, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gdn.gate(q[:, :, 0], q[:, :, 1], torch.zeros(2), torch.zeros(2))


# ------------------------------------------------------------------ forward_gdn dispatch
class _Mode:
    def __init__(self, name):
        self.name = name

    def is_decode_or_idle(self):
        return self.name in ("DECODE", "IDLE")

    def is_extend(self, include_draft_extend_v2=False):
        fam = {"EXTEND", "MIXED", "DRAFT_EXTEND", "TARGET_VERIFY", "SPLIT_PREFILL", "DLLM_EXTEND"}
        return self.name in fam or (include_draft_extend_v2 and self.name == "DRAFT_EXTEND_V2")

    def __repr__(self):
        return f"ForwardMode.{self.name}"


@pytest.mark.parametrize("mode,kind", [("DECODE", "decode"), ("IDLE", "decode"),
                                       ("EXTEND", "extend"), ("MIXED", "extend"),
                                       ("DRAFT_EXTEND", "extend"), ("DRAFT_EXTEND_V2", "extend"),
                                       ("TARGET_VERIFY", "extend"), ("SPLIT_PREFILL", "extend"),
                                       ("DLLM_EXTEND", "extend"), ("decode", "decode"),
                                       ("target_verify", "extend")])
def test_mode_kind(mode, kind):
    m = _Mode(mode) if mode.isupper() else mode
    assert gdn._mode_kind(m) == kind


@pytest.mark.parametrize("mode", [_Mode("DUMMY_FIRST"), "prefill_only", 3])
def test_mode_kind_rejects(mode):
    with pytest.raises(ValueError, match="Invalid forward mode"):
        gdn._mode_kind(mode)


def _layer():
    return SimpleNamespace(num_k_heads=2, num_v_heads=4, head_k_dim=128, head_v_dim=128,
                           A_log=object(), dt_bias=object(), scale=None, layer_id=3)


@pytest.mark.parametrize("mode,expect", [("DECODE", "decode"), ("TARGET_VERIFY", "extend"),
                                         ("EXTEND", "extend")])
@pytest.mark.parametrize("gate_dtype_matches", [True, False])
def test_forward_gdn_routes_by_mode(mode, expect, gate_dtype_matches):
    T = 5
    mixed = torch.zeros(T, 2 * 2 * 128 + 4 * 128)
    a, b = torch.zeros(T, 4), torch.zeros(T, 4)
    pool, slots, cu, hi = object(), object(), object(), object()
    fb = SimpleNamespace(forward_mode=_Mode(mode), state_pool={3: pool}, state_slots=slots,
                         cu_seqlens=cu, has_initial_state=hi, max_seqlen=7)
    spec_buf, spec_rows = object(), object()
    if mode == "TARGET_VERIFY":
        fb.spec_states, fb.spec_state_slots = {3: spec_buf}, spec_rows
    layer = _layer()
    gsent = SimpleNamespace(dtype=mixed.dtype if gate_dtype_matches else torch.bfloat16)
    lg, bt = object(), object()
    out = torch.zeros(T, 4, 128)
    with mock.patch.object(gdn, "gdn_gate_inputs", return_value=gsent) as mg, \
            mock.patch.object(gdn, "_run_gate", return_value=(lg, bt)) as mr, \
            mock.patch.object(gdn, "decode", return_value=out) as md, \
            mock.patch.object(gdn, "extend", return_value=out) as me:
        res = gdn.forward_gdn(layer, fb, mixed, a, b)
    assert res.shape == (T, 512)
    mg.assert_called_once()
    assert mg.call_args.args[0] is a and mg.call_args.args[1] is b
    assert mg.call_args.args[2] is layer.A_log and mg.call_args.args[3] is layer.dt_bias
    called, other = (md, me) if expect == "decode" else (me, md)
    called.assert_called_once()
    other.assert_not_called()
    sent = list(called.call_args.args) + list(called.call_args.kwargs.values())
    assert any(x is pool for x in sent) and any(x is slots for x in sent)
    if gate_dtype_matches:   # gate folded into the layer kernel
        mr.assert_not_called()
        assert called.call_args.kwargs["gate"] is gsent
        assert called.call_args.args[3] is None and called.call_args.args[4] is None
    else:                    # gate launched on its own, its outputs passed on
        mr.assert_called_once()
        assert called.call_args.kwargs["gate"] is None
        assert called.call_args.args[3] is lg and called.call_args.args[4] is bt
    if expect == "extend":
        assert any(x is cu for x in sent) and any(x is hi for x in sent)
        assert called.call_args.kwargs["max_seqlen"] == 7
        kw = called.call_args.kwargs
        verify = mode == "TARGET_VERIFY"
        assert kw["keep_pool"] == verify
        assert kw["spec_states"] is (spec_buf if verify else None)
        assert kw["spec_slot"] is (spec_rows if verify else None)
        assert kw["spec_parent"] is None
    # q, k, v are views of mixed_qkv, not copies
    q, k, v = called.call_args.args[:3]
    assert q.data_ptr() == mixed.data_ptr()
    assert k.data_ptr() == mixed.data_ptr() + 2 * 128 * mixed.element_size()
    assert v.data_ptr() == mixed.data_ptr() + 4 * 128 * mixed.element_size()


@pytest.mark.parametrize("mode,tree", [("DECODE", False), ("EXTEND", False), ("TARGET_VERIFY", False),
                                       ("TARGET_VERIFY", True)])
def test_forward_gdn_runs_the_conv_first(mode, tree):
    """With conv taps on the layer, forward_gdn convolves mixed_qkv first (decode ->
    conv1d_update, extend family -> conv1d with the same slots; target verify leaves the
    conv pool unwritten and passes the token tree) and splits q, k, v from the result."""
    T = 5
    mixed = torch.zeros(T, 2 * 2 * 128 + 4 * 128)
    conv_out = torch.ones_like(mixed)
    a, b = torch.zeros(T, 4), torch.zeros(T, 4)
    cpool, slots, cu, hi, par = object(), object(), object(), object(), object()
    fb = SimpleNamespace(forward_mode=_Mode(mode), state_pool={3: object()}, conv_pool={3: cpool},
                         state_slots=slots, cu_seqlens=cu, has_initial_state=hi, max_seqlen=7)
    if mode == "TARGET_VERIFY":
        fb.spec_states, fb.spec_state_slots = {3: object()}, object()
    if tree:
        fb.spec_parents = par
    layer = _layer()
    layer.conv_weight = torch.zeros(1024, 1, 4)
    layer.conv_bias = object()
    out = torch.zeros(T, 4, 128)
    with mock.patch.object(gdn, "gdn_gate_inputs", return_value=SimpleNamespace(dtype=mixed.dtype)), \
            mock.patch.object(gdn, "conv1d", return_value=conv_out) as mc, \
            mock.patch.object(gdn, "conv1d_update", return_value=conv_out) as mu, \
            mock.patch.object(gdn, "decode", return_value=out) as md, \
            mock.patch.object(gdn, "extend", return_value=out) as me:
        gdn.forward_gdn(layer, fb, mixed, a, b)
    if mode == "DECODE":
        mu.assert_called_once()
        mc.assert_not_called()
        args = mu.call_args.args
        assert args[0] is mixed and args[1].shape == (1024, 4) and args[2] is layer.conv_bias
        assert args[3] is slots and args[4] is cpool
        layer_call = md
    else:
        mc.assert_called_once()
        mu.assert_not_called()
        args, kw = mc.call_args.args, mc.call_args.kwargs
        assert args[0] is mixed and args[1].shape == (1024, 4) and args[3] is cu and args[4] is slots
        assert args[5] is cpool and kw["has_init"] is hi
        assert kw["keep_pool"] == (mode == "TARGET_VERIFY")
        assert kw["parent"] is (par if tree else None)
        layer_call = me
        ekw = me.call_args.kwargs
        assert ekw["keep_pool"] == (mode == "TARGET_VERIFY")
        assert ekw["spec_parent"] is (par if tree else None)
    q = layer_call.call_args.args[0]
    assert q.data_ptr() == conv_out.data_ptr()      # q, k, v come from the conv output


@pytest.mark.parametrize("missing", ["spec_states", "spec_state_slots", "both"])
def test_forward_gdn_target_verify_without_buffer_raises_before_any_call(missing):
    """Target verify without a speculative state buffer would commit the rejected draft
    tokens' state to the pool: it raises before the conv or the layer runs."""
    fb = SimpleNamespace(forward_mode=_Mode("TARGET_VERIFY"), state_pool={3: object()},
                         conv_pool={3: object()}, state_slots=object(), cu_seqlens=object(),
                         max_seqlen=4, spec_states={3: object()}, spec_state_slots=object())
    if missing in ("spec_states", "both"):
        del fb.spec_states
    if missing in ("spec_state_slots", "both"):
        del fb.spec_state_slots
    layer = _layer()
    layer.conv_weight = torch.zeros(1024, 4)
    with mock.patch.object(gdn, "conv1d") as mc, mock.patch.object(gdn, "extend") as me, \
            mock.patch.object(gdn, "gdn_gate_inputs") as mg:
        with pytest.raises(ValueError, match="target verify needs"):
            gdn.forward_gdn(layer, fb, torch.zeros(3, 1024), torch.zeros(3, 4), torch.zeros(3, 4))
    mc.assert_not_called()
    me.assert_not_called()
    mg.assert_not_called()


def test_forward_gdn_invalid_mode_raises_before_any_call():
    fb = SimpleNamespace(forward_mode=_Mode("DUMMY_FIRST"))
    with mock.patch.object(gdn, "gdn_gate_inputs") as mg:
        with pytest.raises(ValueError, match="Invalid forward mode"):
            gdn.forward_gdn(_layer(), fb, torch.zeros(1, 1024), torch.zeros(1, 4), torch.zeros(1, 4))
    mg.assert_not_called()


def test_ssd_combined_rejects_unsupported_arguments():
    x = torch.zeros(1, 4, 2, 64)
    with pytest.raises(NotImplementedError):
        gdn.ssd_combined_fwd(x, x[..., 0], None, x, x, out=x)
    with pytest.raises(NotImplementedError):
        gdn.ssd_combined_fwd(x, x[..., 0], None, x, x, update_seq_chunk_cumsum=True)


def test_probe_argument_checks():
    """The measurement probes refuse bad arguments before any launch."""
    lib = gdn.load()
    p = ct.c_void_p(0x100000)
    assert lib.gdn_probe_copy(None, p, 1024, None) == _lib.GDN_E_NULL
    assert lib.gdn_probe_copy(p, p, 1000, None) == _lib.GDN_E_SHAPE          # not a multiple of 16
    assert lib.gdn_probe_copy(p, ct.c_void_p(0x100008), 1024, None) == _lib.GDN_E_SHAPE   # misaligned
    assert lib.gdn_probe_copy(p, p, 0, None) == _lib.GDN_E_SHAPE
    assert lib.gdn_probe_copy(p, ct.c_void_p(0x100000 + 512), 1024, None) == _lib.GDN_E_SHAPE   # overlap
    assert lib.gdn_probe_mfma(None, 1, 1, None) == _lib.GDN_E_NULL
    assert lib.gdn_probe_mfma(p, 0, 1, None) == _lib.GDN_E_SHAPE
    assert lib.gdn_probe_mfma(p, 1, 0, None) == _lib.GDN_E_SHAPE
    assert lib.gdn_probe_mfma(p, 65537, 1, None) == _lib.GDN_E_SHAPE
    assert lib.gdn_probe_mfma(p, 1, (1 << 20) + 1, None) == _lib.GDN_E_SHAPE
