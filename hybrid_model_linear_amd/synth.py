"""Seeded synthetic inputs for the GDN layer, shared by the tests, the bench and
the oracle's callers.

This module holds no arithmetic of the method itself: it draws random numbers,
rounds them to the storage dtype, lays them out the way the layer receives them
and builds the varlen/slot metadata.  Everything here is plain numpy so that it
can run on a CPU-only host.

Shapes follow the Qwen3-Next-shaped layer (H_qk=16, H_v=32, d_k=d_v=128) and the
small cases of the SGLang GDN test matrix article (framerc.cn), sections
"torch_native" (prefix_lens (0,8,16), extend_lens (15,8,1)) and "Input & config
coverage" (page-boundary and batch-1 patterns).  The Mamba2-shaped delta-off
case follows the parameter list of the flashinfer.mamba.ssd_combined_fwd page.

Distributions (sigma is a standard deviation):
  q, k, v, a, b ~ N(0, 1); A_log = log U(1, 16); dt_bias ~ N(0, 0.5);
  prefix states ~ N(0, 0.1) (decode pool: N(0, 0.05)).
bf16 tensors are drawn in fp32 and rounded to bf16 with round-to-nearest-even,
so the values handed to the GPU and to the oracle are bit-identical.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "bf16_round", "bf16_bits", "GDNCase", "SSDCase", "make_gdn_case",
    "config0_tiny", "config1_decode", "config2_prefill", "config3_ragged",
    "config3_verify", "config4_ssd", "ragged_lengths", "edge_case",
]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even (finite inputs)."""
    return (bf16_round(x).view(np.uint32) >> 16).astype(np.uint16)


def bf16_round(x: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value (RNE, ties to even); fp32 result.
    Works in 32-bit integer arithmetic in place so that it scales to ~1e9 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    res = np.array(x, copy=True) if out is None else out
    if res is not x:
        np.copyto(res, x)
    u = res.view(np.uint32)
    lsb = (u >> 16) & 1
    lsb += 0x7FFF
    u += lsb
    u &= 0xFFFF0000
    return res


def _normal(rng, shape, sigma=1.0):
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma))


@dataclass
class GDNCase:
    """One gdn_extend / gdn_decode call's inputs (host copies, fp32 values).

    mixed_qkv is [T, 2*H_qk*d_k + H_v*d_v] with the q | k | v blocks in that
    order and heads contiguous inside each block; q, k, v are strided views of
    it.  pool is [num_slots, H_v, d_v, d_k] (or None when the caller fills the
    pool on the device; then pool_seed/pool_sigma describe it).
    """
    name: str
    dtype: str                      # "bf16" or "f32": storage type of q/k/v/a/b/out
    H_qk: int
    H_v: int
    d_k: int
    d_v: int
    scale: float
    mixed_qkv: np.ndarray
    a: np.ndarray                   # [T, H_v]
    b: np.ndarray                   # [T, H_v]
    A_log: np.ndarray               # [H_v] fp32
    dt_bias: np.ndarray             # [H_v] fp32
    cu_seqlens: np.ndarray          # [N+1] int32
    slot: np.ndarray                # [N] int32, <0 = skipped
    has_init: np.ndarray            # [N] int32
    num_slots: int
    pool: Optional[np.ndarray]      # [num_slots, H_v, d_v, d_k] fp32
    pool_sigma: float = 0.1
    pool_seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.mixed_qkv.shape[0])

    @property
    def N(self) -> int:
        return int(self.slot.shape[0])

    @property
    def q(self) -> np.ndarray:
        n = self.H_qk * self.d_k
        return self.mixed_qkv[:, :n].reshape(self.T, self.H_qk, self.d_k)

    @property
    def k(self) -> np.ndarray:
        n = self.H_qk * self.d_k
        return self.mixed_qkv[:, n:2 * n].reshape(self.T, self.H_qk, self.d_k)

    @property
    def v(self) -> np.ndarray:
        n = self.H_qk * self.d_k
        return self.mixed_qkv[:, 2 * n:].reshape(self.T, self.H_v, self.d_v)


@dataclass
class SSDCase:
    """Inputs of the Mamba2-shaped delta-off call (ssd_combined_fwd layout)."""
    name: str
    x: np.ndarray        # [batch, L, H, P] (bf16 values)
    dt: np.ndarray       # [batch, L, H]
    A: np.ndarray        # [H] fp32, negative
    B: np.ndarray        # [batch, L, G, N]
    C: np.ndarray        # [batch, L, G, N]
    D: Optional[np.ndarray]   # [H] or [H, P]
    z: Optional[np.ndarray]   # like x
    dt_bias: Optional[np.ndarray]  # [H] fp32
    dt_softplus: bool
    dt_limit: tuple
    initial_states: Optional[np.ndarray]  # [batch, H, P, N] fp32


def _round_if(x, dtype):
    return bf16_round(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def make_gdn_case(name, *, seed, lens, has_init, H_qk, H_v, d_k, d_v, dtype="bf16",
                  num_slots=None, slot=None, pool_sigma=0.1, scale=None,
                  host_pool=True, a_sigma=1.0, b_sigma=1.0, qk_sigma=1.0,
                  v_sigma=1.0, A_log=None, dt_bias=None, meta=None) -> GDNCase:
    """Build a packed-varlen case.  lens: token counts per sequence."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    N = len(lens)
    T = int(lens.sum())
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    width = 2 * H_qk * d_k + H_v * d_v
    mixed = rng.standard_normal(size=(T, width), dtype=np.float32)   # q | k | v
    if qk_sigma != 1.0:
        mixed[:, :2 * H_qk * d_k] *= np.float32(qk_sigma)
    if v_sigma != 1.0:
        mixed[:, 2 * H_qk * d_k:] *= np.float32(v_sigma)
    if dtype == "bf16":
        bf16_round(mixed, out=mixed)
    a = _round_if(_normal(rng, (T, H_v), a_sigma), dtype)
    b = _round_if(_normal(rng, (T, H_v), b_sigma), dtype)
    if A_log is None:
        A_log = np.log(rng.uniform(1.0, 16.0, size=H_v)).astype(np.float32)
    if dt_bias is None:
        dt_bias = _normal(rng, (H_v,), 0.5)
    if num_slots is None:
        num_slots = max(16, 2 * N)
    if slot is None:
        slot = rng.permutation(num_slots)[:N].astype(np.int32)
    slot = np.asarray(slot, dtype=np.int32)
    has_init = np.broadcast_to(np.asarray(has_init, dtype=np.int32), (N,)).copy()
    pool = None
    pool_seed = int(rng.integers(0, 2**31 - 1))
    if host_pool:
        prng = np.random.default_rng(pool_seed)
        pool = _normal(prng, (num_slots, H_v, d_v, d_k), pool_sigma)
    if scale is None:
        scale = float(d_k) ** -0.5
    return GDNCase(name=name, dtype=dtype, H_qk=H_qk, H_v=H_v, d_k=d_k, d_v=d_v,
                   scale=float(scale), mixed_qkv=mixed, a=a, b=b,
                   A_log=np.asarray(A_log, np.float32), dt_bias=np.asarray(dt_bias, np.float32),
                   cu_seqlens=cu, slot=slot, has_init=has_init, num_slots=int(num_slots),
                   pool=pool, pool_sigma=pool_sigma, pool_seed=pool_seed, meta=dict(meta or {}))


@dataclass
class ConvCase:
    """Inputs of one short causal conv call (gdn_conv1d), bf16 values held as fp32.

    x is the projected mixed_qkv before the conv (standard normal); weight [D, K] and
    bias [D] are uniform in +-1/sqrt(K), the default init of a depthwise Conv1d with
    K taps; pool [num_slots, D, K-1] holds earlier inputs (standard normal)."""
    x: np.ndarray
    weight: np.ndarray
    bias: np.ndarray
    cu_seqlens: np.ndarray
    slot: np.ndarray
    has_init: np.ndarray
    pool: np.ndarray

    @property
    def T(self) -> int:
        return int(self.x.shape[0])


def make_conv_case(*, seed, lens, D, K=4, has_init=1, num_slots=None, slot=None) -> ConvCase:
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    N = len(lens)
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    x = bf16_round(rng.standard_normal((int(lens.sum()), D), dtype=np.float32))
    lim = np.float32(1.0 / np.sqrt(K))
    weight = bf16_round(rng.uniform(-lim, lim, (D, K)).astype(np.float32))
    bias = bf16_round(rng.uniform(-lim, lim, D).astype(np.float32))
    if num_slots is None:
        num_slots = max(8, 2 * N)
    if slot is None:
        slot = rng.permutation(num_slots)[:N].astype(np.int32)
    pool = bf16_round(rng.standard_normal((num_slots, D, K - 1), dtype=np.float32))
    return ConvCase(x=x, weight=weight, bias=bias, cu_seqlens=cu,
                    slot=np.asarray(slot, np.int32),
                    has_init=np.broadcast_to(np.asarray(has_init, np.int32), (N,)).copy(), pool=pool)


def config0_tiny(seed: int = 1000):
    """Tiny fp32 extend followed by one decode token per sequence.

    3 sequences, prefix_lens (0, 8, 16) -> has_init (0, 1, 1), extend_lens
    (15, 8, 1); H_qk = H_v = 2, d = 64, scale 1/8; 16-slot pool, slots drawn
    from a permutation.  Returns (extend_case, decode_case); the decode case
    reuses the same slots and must start from the extend's final states.
    """
    ext = make_gdn_case("tiny-extend", seed=seed, lens=(15, 8, 1), has_init=(0, 1, 1),
                        H_qk=2, H_v=2, d_k=64, d_v=64, dtype="f32", num_slots=16,
                        pool_sigma=0.1, scale=0.125)
    dec = make_gdn_case("tiny-decode", seed=seed + 1, lens=(1, 1, 1), has_init=1,
                        H_qk=2, H_v=2, d_k=64, d_v=64, dtype="f32", num_slots=16,
                        slot=ext.slot, pool_sigma=0.1, scale=0.125,
                        A_log=ext.A_log, dt_bias=ext.dt_bias, host_pool=False)
    return ext, dec


def config1_decode(seed: int = 1001, batch: int = 256, num_slots: int = 1024, host_pool=False):
    """Qwen3-Next-shaped decode: 256 sequences x 1 token, pool [1024,32,128,128]."""
    rng = np.random.default_rng(seed + 7)
    slot = rng.choice(num_slots, size=batch, replace=False).astype(np.int32)
    return make_gdn_case("decode-256", seed=seed, lens=np.ones(batch, np.int64), has_init=1,
                         H_qk=16, H_v=32, d_k=128, d_v=128, dtype="bf16",
                         num_slots=num_slots, slot=slot, pool_sigma=0.05,
                         host_pool=host_pool)


def config2_prefill(seed: int = 1002, nseq: int = 8, seqlen: int = 4096):
    """Prefill: 8 x 4096 packed tokens, zero initial states, 16-slot pool."""
    return make_gdn_case("prefill-8x4096", seed=seed, lens=[seqlen] * nseq, has_init=0,
                         H_qk=16, H_v=32, d_k=128, d_v=128, dtype="bf16", num_slots=16,
                         host_pool=False, pool_sigma=0.1)


def ragged_lengths(seed: int, n: int = 64, lo: int = 1, hi: int = 8192,
                   total: int = 131072, tol: int = 64) -> np.ndarray:
    """n log-uniform lengths in [lo, hi], rescaled by one common factor so that
    the clamped, rounded lengths sum to total +- tol (bisection on the factor)."""
    rng = np.random.default_rng(seed)
    base = np.exp(rng.uniform(np.log(lo), np.log(hi), size=n))

    def realise(s):
        return np.clip(np.rint(s * base), lo, hi).astype(np.int64)

    s_lo, s_hi = 1e-3, 1e4
    for _ in range(200):
        mid = 0.5 * (s_lo + s_hi)
        if realise(mid).sum() < total:
            s_lo = mid
        else:
            s_hi = mid
        if abs(int(realise(mid).sum()) - total) <= tol:
            return realise(mid)
    return realise(s_hi)


def config3_ragged(seed: int = 1003, num_slots: int = 512):
    """Ragged extend from cached states: 64 sequences, log-uniform lengths scaled
    to ~131072 tokens, has_init = 1, slots = permutation(512)[:64]."""
    lens = ragged_lengths(seed)
    rng = np.random.default_rng(seed + 11)
    perm = rng.permutation(num_slots).astype(np.int32)
    case = make_gdn_case("ragged-64", seed=seed, lens=lens, has_init=1, H_qk=16, H_v=32,
                         d_k=128, d_v=128, dtype="bf16", num_slots=num_slots,
                         slot=perm[:64], host_pool=False, pool_sigma=0.1,
                         meta={"perm": perm})
    return case


def config3_verify(seed: int = 1003, num_slots: int = 512):
    """Verify-style batch: 32 sequences x 4 tokens from pooled states, on slots
    permutation(512)[64:96] (disjoint from the ragged call's slots)."""
    rng = np.random.default_rng(seed + 11)
    perm = rng.permutation(num_slots).astype(np.int32)
    return make_gdn_case("verify-32x4", seed=seed + 100, lens=[4] * 32, has_init=1,
                         H_qk=16, H_v=32, d_k=128, d_v=128, dtype="bf16",
                         num_slots=num_slots, slot=perm[64:96], host_pool=False,
                         pool_sigma=0.1)


def config4_ssd(seed: int = 1004, batch: int = 2, L: int = 8192, H: int = 80, P: int = 64,
                G: int = 1, Nst: int = 128, with_D=True, with_z=True, initial=False) -> SSDCase:
    """Mamba2-shaped delta-off call: x [2,8192,80,64], B/C [2,8192,1,128]."""
    rng = np.random.default_rng(seed)
    x = bf16_round(_normal(rng, (batch, L, H, P)))
    dt = bf16_round(_normal(rng, (batch, L, H)))
    A = (-rng.uniform(1.0, 16.0, size=H)).astype(np.float32)
    B = bf16_round(_normal(rng, (batch, L, G, Nst)))
    C = bf16_round(_normal(rng, (batch, L, G, Nst)))
    D = bf16_round(_normal(rng, (H,))) if with_D else None
    z = bf16_round(_normal(rng, (batch, L, H, P))) if with_z else None
    dt_bias = _normal(rng, (H,), 0.5)
    init = _normal(rng, (batch, H, P, Nst), 0.1) if initial else None
    return SSDCase(name=f"ssd-{batch}x{L}x{H}x{P}", x=x, dt=dt, A=A, B=B, C=C, D=D, z=z,
                   dt_bias=dt_bias, dt_softplus=True, dt_limit=(0.0, float("inf")),
                   initial_states=init)


def edge_case(name, lens, has_init=1, seed=7, H_qk=2, H_v=4, d_k=128, d_v=128,
              dtype="bf16", num_slots=None, slot=None):
    """Small bf16 case with the Qwen head dims, for boundary patterns such as
    lengths 1/63/64/65/127/128/129 or the page-boundary tuples."""
    return make_gdn_case(name, seed=seed, lens=lens, has_init=has_init, H_qk=H_qk, H_v=H_v,
                         d_k=d_k, d_v=d_v, dtype=dtype, num_slots=num_slots, slot=slot)


# ------------------------------------------------------------------ device-side generation
# The full-size layer shapes are generated on the GPU with torch's seeded Philox
# generator (same distributions, bf16 by round-to-nearest-even conversion): host
# generation of ~1e9 values is too slow to sit in a test.  The oracle then reads
# back only the rows it samples.
def device_case(name, *, seed, lens, has_init, H_qk, H_v, d_k, d_v, num_slots, slot=None,
                pool_sigma=0.1, scale=None, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    N = len(lens)
    T = int(lens.sum())
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    width = 2 * H_qk * d_k + H_v * d_v
    mixed = torch.empty((T, width), dtype=torch.bfloat16, device=device)
    step = 4096
    for r0 in range(0, T, step):                       # bounded fp32 temporaries
        r1 = min(T, r0 + step)
        mixed[r0:r1] = torch.randn((r1 - r0, width), generator=g, device=device).to(torch.bfloat16)
    a = torch.randn((T, H_v), generator=g, device=device).to(torch.bfloat16)
    b = torch.randn((T, H_v), generator=g, device=device).to(torch.bfloat16)
    A_log = np.log(rng.uniform(1.0, 16.0, size=H_v)).astype(np.float32)
    dt_bias = _normal(rng, (H_v,), 0.5)
    if slot is None:
        slot = rng.permutation(num_slots)[:N].astype(np.int32)
    has_init = np.broadcast_to(np.asarray(has_init, dtype=np.int32), (N,)).copy()
    return GDNCase(name=name, dtype="bf16", H_qk=H_qk, H_v=H_v, d_k=d_k, d_v=d_v,
                   scale=float(d_k) ** -0.5 if scale is None else float(scale), mixed_qkv=mixed,
                   a=a, b=b, A_log=A_log, dt_bias=dt_bias, cu_seqlens=cu,
                   slot=np.asarray(slot, np.int32), has_init=has_init, num_slots=int(num_slots),
                   pool=None, pool_sigma=pool_sigma, pool_seed=int(rng.integers(0, 2**31 - 1)))


def device_pool(case: GDNCase, device="cuda"):
    """fp32 pool [num_slots, H_v, d_v, d_k] ~ N(0, pool_sigma), filled on the device."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(case.pool_seed)
    shape = (case.num_slots, case.H_v, case.d_v, case.d_k)
    pool = torch.empty(shape, dtype=torch.float32, device=device)
    for s0 in range(0, case.num_slots, 64):
        s1 = min(case.num_slots, s0 + 64)
        pool[s0:s1] = torch.randn((s1 - s0,) + shape[1:], generator=g, device=device) * case.pool_sigma
    return pool


def device_config1_decode(seed: int = 1001, device="cuda"):
    rng = np.random.default_rng(seed + 7)
    slot = rng.choice(1024, size=256, replace=False).astype(np.int32)
    return device_case("decode-256", seed=seed, lens=np.ones(256, np.int64), has_init=1,
                       H_qk=16, H_v=32, d_k=128, d_v=128, num_slots=1024, slot=slot,
                       pool_sigma=0.05, device=device)


def device_config2_prefill(seed: int = 1002, device="cuda"):
    return device_case("prefill-8x4096", seed=seed, lens=[4096] * 8, has_init=0, H_qk=16,
                       H_v=32, d_k=128, d_v=128, num_slots=16, device=device)


def device_config3_ragged(seed: int = 1003, device="cuda"):
    lens = ragged_lengths(seed)
    rng = np.random.default_rng(seed + 11)
    perm = rng.permutation(512).astype(np.int32)
    return device_case("ragged-64", seed=seed, lens=lens, has_init=1, H_qk=16, H_v=32, d_k=128,
                       d_v=128, num_slots=512, slot=perm[:64], device=device)


def device_config3_verify(seed: int = 1003, device="cuda"):
    rng = np.random.default_rng(seed + 11)
    perm = rng.permutation(512).astype(np.int32)
    return device_case("verify-32x4", seed=seed + 100, lens=[4] * 32, has_init=1, H_qk=16,
                       H_v=32, d_k=128, d_v=128, num_slots=512, slot=perm[64:96], device=device)


def device_config4_ssd(seed: int = 1004, batch=2, L=8192, H=80, P=64, G=1, Nst=128, device="cuda"):
    """Mamba2-shaped delta-off inputs as torch tensors on the device."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    rng = np.random.default_rng(seed)

    def bf(shape):
        return torch.randn(shape, generator=g, device=device).to(torch.bfloat16)

    x = bf((batch, L, H, P))
    dt = bf((batch, L, H))
    B = bf((batch, L, G, Nst))
    C = bf((batch, L, G, Nst))
    D = bf((H,))
    z = bf((batch, L, H, P))
    A = torch.from_numpy((-rng.uniform(1.0, 16.0, size=H)).astype(np.float32)).to(device)
    dt_bias = torch.from_numpy(_normal(rng, (H,), 0.5)).to(device)
    return SSDCase(name=f"ssd-{batch}x{L}x{H}x{P}", x=x, dt=dt, A=A, B=B, C=C, D=D, z=z,
                   dt_bias=dt_bias, dt_softplus=True, dt_limit=(0.0, float("inf")),
                   initial_states=None)
