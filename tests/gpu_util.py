"""Helpers of the GPU parity tests: upload seeded cases, run the HIP path through
the binding, run the oracle on (sampled) sequences and heads, compare."""
import numpy as np
import torch

import oracle

REL_L2 = 2e-3      # relative L2 bound on outputs and final states (bf16 in, fp32 state)
MAX_ABS = 1e-2     # max-abs bound on the same


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def assert_close(got, ref, what, rel=REL_L2, mx=MAX_ABS, peak_rel=False):
    """rel-L2 <= rel and max-abs <= mx.  The max-abs bound is absolute, except with
    peak_rel (delta-off outputs and states only), where it is mx times the peak
    magnitude when that exceeds one: delta-off outputs reach |y| ~ 1e2, where a single
    bf16 ulp of the output alone exceeds 1e-2."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    r = rel_l2(got, ref)
    m = float(np.max(np.abs(got - ref))) if got.size else 0.0
    peak = float(np.max(np.abs(ref))) if ref.size else 0.0
    mx_eff = mx * max(1.0, peak) if peak_rel else mx
    print(f"  {what}: rel-L2 {r:.3e}  max-abs {m:.3e} (bound {mx_eff:.3e}, peak {peak:.3e})", flush=True)
    assert r <= rel and m <= mx_eff, f"{what}: rel-L2 {r:.3e} (<= {rel}) max-abs {m:.3e} (<= {mx_eff:.3e})"
    return r, m


def tdtype(case):
    return torch.bfloat16 if case.dtype == "bf16" else torch.float32


def upload(case, device="cuda", pool=None):
    """Torch tensors of a synth.GDNCase (numpy or already on the device)."""
    def dev(x, dt):
        if isinstance(x, torch.Tensor):
            return x.to(device)
        return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=dt)
    dt = tdtype(case)
    d = dict(mixed=dev(case.mixed_qkv, dt), a=dev(case.a, dt), b=dev(case.b, dt),
             A_log=dev(case.A_log, torch.float32), dt_bias=dev(case.dt_bias, torch.float32),
             cu=dev(case.cu_seqlens, torch.int32), slot=dev(case.slot, torch.int32),
             has_init=dev(case.has_init, torch.int32))
    if pool is not None:
        d["pool"] = pool
    elif case.pool is not None:
        d["pool"] = dev(case.pool, torch.float32)
    return d


def run_extend(gdn, case, d, out_dtype=None, max_seqlen=0, out=None):
    q, k, v = gdn.split_mixed_qkv(d["mixed"], case.H_qk, case.H_v, case.d_k, case.d_v)
    log_g, beta = gdn.gate(d["a"], d["b"], d["A_log"], d["dt_bias"])
    return gdn.extend(q, k, v, log_g, beta, d["cu"], d["slot"], d["pool"], has_init=d["has_init"],
                      scale=case.scale, out_dtype=out_dtype, max_seqlen=max_seqlen, out=out)


def host_rows(x, t0, t1):
    if isinstance(x, torch.Tensor):
        return x[t0:t1].float().cpu().numpy()
    return np.asarray(x[t0:t1], np.float32)


def oracle_seq(case, n, heads, init_state):
    """Oracle outputs [L, len(heads), d_v] and final state [len(heads), d_v, d_k] of
    sequence n, starting from init_state [H_v, d_v, d_k] (ignored if has_init == 0)."""
    t0, t1 = int(case.cu_seqlens[n]), int(case.cu_seqlens[n + 1])
    mixed = host_rows(case.mixed_qkv, t0, t1)
    L = t1 - t0
    nq = case.H_qk * case.d_k
    q = mixed[:, :nq].reshape(L, case.H_qk, case.d_k)
    k = mixed[:, nq:2 * nq].reshape(L, case.H_qk, case.d_k)
    v = mixed[:, 2 * nq:].reshape(L, case.H_v, case.d_v)
    a = host_rows(case.a, t0, t1)
    b = host_rows(case.b, t0, t1)
    pool = {0: init_state}
    out, _, fin = oracle.gdn_extend(q, k, v, a, b, case.A_log, case.dt_bias, np.array([0, L]),
                                    np.array([0]), np.array([int(case.has_init[n])]), pool,
                                    case.scale, heads=heads)
    return out, fin[0]
