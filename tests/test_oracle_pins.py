"""Pins of the CPU oracle to things other than itself.

Each check is a function of an implementation with the signature of
oracle.gdn_extend, so the same checks can be run against planted mistakes
(test_pins_reject_mutants) to show they are sensitive to them.

What pins what:
  * gate            : closed forms and library special cases (numpy logaddexp,
                      scipy expit)
  * recurrence      : dense transition-matrix brute force; exact rational
                      arithmetic on a hand-checkable 2-d example
  * beta = 0        : closed-form pure decay
  * g = 1, beta = 1 : exact key -> value recall with orthonormal keys, and the
                      delta-rule overwrite of a repeated key
  * split / resume  : extend(A||B) == extend(A) -> extend(B) == extend(A) -> decode*
  * grouped heads   : shared-head run == duplicated-head run
  * pool / indices  : untouched slots, skipped sequences, has_init = 0,
                      zero-length sequences, per-slot ownership
  * delta-off (SSD) : quadratic (masked matmul) dual form, A = 0 prefix sums,
                      D / silu(z) epilogue, dt clamp, initial-state term
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle
from hybrid_model_linear_amd import synth

RTOL = 1e-12


def _close(a, b, tol=RTOL):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"max abs err {err:.3e} > {tol * scale:.3e}"


def _run(impl, case, pool=None, **kw):
    pool = case.pool if pool is None else pool
    return impl(case.q, case.k, case.v, case.a, case.b, case.A_log, case.dt_bias,
                case.cu_seqlens, case.slot, case.has_init, pool, case.scale, **kw)


# ------------------------------------------------------------------ gate
def test_gate_closed_forms():
    # b = 0 => beta = 1/2 exactly; A_log = 0 and a + dt_bias = 0 => log g = -ln 2.
    lg, beta = oracle.gdn_gate(np.zeros((1, 1)), np.zeros((1, 1)), np.zeros(1), np.zeros(1))
    assert beta[0, 0] == 0.5
    assert abs(lg[0, 0] + np.log(2.0)) < 1e-16
    # a + dt_bias -> -inf => g -> 1 (log g ~ -exp(A_log) * exp(a)).
    lg, _ = oracle.gdn_gate(np.array([[-40.0]]), np.zeros((1, 1)), np.array([np.log(3.0)]), np.zeros(1))
    assert abs(lg[0, 0] + 3.0 * np.exp(-40.0)) < 1e-30
    # large positive argument => softplus(x) ~ x.
    lg, _ = oracle.gdn_gate(np.array([[50.0]]), np.zeros((1, 1)), np.array([np.log(2.0)]), np.array([1.0]))
    assert abs(lg[0, 0] + 2.0 * 51.0) < 1e-12
    # the dt_bias is added before the softplus, the exp(A_log) multiplies after.
    lg1, _ = oracle.gdn_gate(np.array([[0.3]]), np.zeros((1, 1)), np.array([0.7]), np.array([-0.1]))
    assert abs(lg1[0, 0] + np.exp(0.7) * np.log1p(np.exp(0.2))) < 1e-15


def test_gate_matches_library_special_functions():
    x = np.linspace(-60, 60, 2401)
    assert np.max(np.abs(oracle.softplus(x) - np.logaddexp(0.0, x))) < 1e-13
    assert np.max(np.abs(oracle.sigmoid(x) - scipy.special.expit(x))) < 1e-15
    rng = np.random.default_rng(0)
    a = rng.standard_normal((7, 5))
    b = rng.standard_normal((7, 5))
    A_log = np.log(rng.uniform(1, 16, 5))
    bias = rng.standard_normal(5) * 0.5
    lg, beta = oracle.gdn_gate(a, b, A_log, bias)
    _close(lg, -np.exp(A_log) * np.logaddexp(0.0, a + bias))
    _close(beta, scipy.special.expit(b))
    assert np.all(lg < 0) and np.all((beta > 0) & (beta < 1))


def test_ssd_gate_order_and_clamp():
    dt = np.array([[-3.0, 0.0, 2.0]])
    A = np.array([-1.0, -2.0, -4.0])
    bias = np.array([1.0, 0.5, -0.5])
    lg, dtp = oracle.ssd_gate(dt, A, bias, True, (0.2, 1.0))
    expect = np.clip(np.logaddexp(0.0, dt + bias), 0.2, 1.0)
    _close(dtp, expect)
    _close(lg, expect * A)
    lg, dtp = oracle.ssd_gate(dt, A, None, False, (0.0, np.inf))
    _close(dtp, np.clip(dt, 0.0, np.inf))
    assert dtp[0, 0] == 0.0                     # inclusive lower limit reached


# ------------------------------------------------------------------ checks (impl-generic)
def tiny_case(seed=3, lens=(5, 3, 4), H_qk=2, H_v=4, d_k=6, d_v=5, has_init=(1, 0, 1), scale=0.7):
    return synth.make_gdn_case("pin", seed=seed, lens=lens, has_init=has_init, H_qk=H_qk,
                               H_v=H_v, d_k=d_k, d_v=d_v, dtype="f32", num_slots=9,
                               pool_sigma=0.3, scale=scale)


def check_dense_bruteforce(impl):
    """S_t = S_{t-1} M_t + beta_t v_t khat_t^T with M_t = g_t (I - beta_t khat khat^T)
    formed densely; d_k != d_v and H_v = 2 H_qk so transposes and head maps show."""
    c = tiny_case()
    out, written, finals = _run(impl, c)
    r = c.H_v // c.H_qk
    for n in range(c.N):
        t0, t1 = c.cu_seqlens[n], c.cu_seqlens[n + 1]
        for h in range(c.H_v):
            j = h // r
            S = c.pool[c.slot[n], h].astype(np.float64) if c.has_init[n] else np.zeros((c.d_v, c.d_k))
            for t in range(t0, t1):
                sp = np.logaddexp(0.0, float(c.a[t, h]) + float(c.dt_bias[h]))
                g = np.exp(-np.exp(float(c.A_log[h])) * sp)
                beta = scipy.special.expit(float(c.b[t, h]))
                kk = c.k[t, j].astype(np.float64)
                kk = kk / np.sqrt(kk @ kk + 1e-6)
                qq = c.q[t, j].astype(np.float64)
                qq = qq / np.sqrt(qq @ qq + 1e-6)
                M = g * (np.eye(c.d_k) - beta * np.outer(kk, kk))
                S = S @ M + beta * np.outer(c.v[t, h].astype(np.float64), kk)
                _close(out[t, h], c.scale * S @ qq)
            _close(finals[c.slot[n]][h], S)
    assert written.all()


def check_exact_rational(impl):
    """Hand-checkable 2-d example in exact rational arithmetic.

    A_log = 0 and a = -dt_bias give g = exp(-softplus(0)) = 1/2; b = 0 gives
    beta = 1/2; keys (3,4) and (4,-3) normalise to (3/5,4/5) and (4/5,-3/5)
    (eps = 0); queries (1,0), (0,2), (5,12).
    """
    keys = [(3, 4), (4, -3), (3, 4)]
    qs = [(1, 0), (0, 2), (5, 12)]
    vs = [(2, -1), (1, 3), (-4, 1)]
    S = [[Fraction(1, 2), Fraction(-1, 3)], [Fraction(0), Fraction(1, 4)]]   # [d_v][d_k]
    g = beta = Fraction(1, 2)
    expect_out = []
    for kv, qv, vv in zip(keys, qs, vs):
        nk = Fraction(int(round(np.hypot(*kv))))
        kh = [Fraction(x) / nk for x in kv]
        nq = Fraction(int(round(np.hypot(*qv))))
        qh = [Fraction(x) / nq for x in qv]
        # S <- g S (I - beta kh kh^T) + beta v kh^T, element by element
        M = [[g * ((1 if i == j else 0) - beta * kh[i] * kh[j]) for j in range(2)] for i in range(2)]
        S = [[sum(S[r][m] * M[m][c] for m in range(2)) + beta * vv[r] * kh[c] for c in range(2)]
             for r in range(2)]
        expect_out.append([sum(S[r][c] * qh[c] for c in range(2)) for r in range(2)])
    T = 3
    q = np.array(qs, dtype=np.float64).reshape(T, 1, 2)
    k = np.array(keys, dtype=np.float64).reshape(T, 1, 2)
    v = np.array(vs, dtype=np.float64).reshape(T, 1, 2)
    a = np.full((T, 1), 0.25)
    bias = np.array([-0.25])
    pool = np.array([[[[0.5, -1 / 3], [0.0, 0.25]]]])
    out, _, finals = impl(q, k, v, a, np.zeros((T, 1)), np.zeros(1), bias, np.array([0, T]),
                          np.array([0]), np.array([1]), pool, 1.0, eps=0.0)
    _close(out[:, 0, :], np.array([[float(x) for x in row] for row in expect_out]), 1e-14)
    _close(finals[0][0], np.array([[float(x) for x in row] for row in S]), 1e-14)


def check_beta_zero_pure_decay(impl):
    """beta = 0 (b = -1000 underflows sigmoid to 0): S_t = gamma_t S_0 and
    o_t = scale * gamma_t S_0 qhat_t with gamma_t the running product of g."""
    c = tiny_case(lens=(7,), has_init=(1,))
    c.b[:] = -1000.0
    out, _, finals = _run(impl, c)
    r = c.H_v // c.H_qk
    lg, _ = oracle.gdn_gate(c.a, np.zeros_like(c.a), c.A_log, c.dt_bias)  # decay only
    gamma = np.exp(np.cumsum(lg, axis=0))                                 # [T, H_v]
    S0 = c.pool[c.slot[0]].astype(np.float64)
    for t in range(c.T):
        for h in range(c.H_v):
            qq = c.q[t, h // r].astype(np.float64)
            qq = qq / np.sqrt(qq @ qq + 1e-6)
            _close(out[t, h], c.scale * gamma[t, h] * S0[h] @ qq)
    _close(finals[c.slot[0]], gamma[-1][:, None, None] * S0)


def check_exact_recall(impl):
    """g = 1 (a = -1000), beta = 1 (b = +1000), S_0 = 0, orthonormal keys: after
    writing (k_j, v_j), a read token (beta = 0, q = k_j) returns scale * v_j; a key
    written twice keeps only its second value (delta-rule overwrite)."""
    rng = np.random.default_rng(5)
    d_k, d_v, m = 8, 3, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((d_k, d_k)))
    keys = Qm[:m] * rng.uniform(0.5, 3.0, size=(m, 1))          # any length: normalised
    vals = rng.standard_normal((m, d_v))
    newv = rng.standard_normal(d_v)
    # write m pairs, overwrite key 0 with newv, then read all m keys
    K = np.concatenate([keys, keys[:1], keys])
    V = np.concatenate([vals, newv[None], np.zeros((m, d_v))])
    Q = np.concatenate([keys, keys[:1], keys * 2.0])
    T = len(K)
    a = np.full((T, 1), -1000.0)
    b = np.concatenate([np.full(m + 1, 1000.0), np.full(m, -1000.0)])[:, None]
    out, _, _ = impl(Q[:, None], K[:, None], V[:, None], a, b, np.zeros(1), np.zeros(1),
                     np.array([0, T]), np.array([0]), np.array([0]),
                     np.zeros((1, 1, d_v, d_k)), 0.5, eps=0.0)
    expect = vals.copy()
    expect[0] = newv
    _close(out[m + 1:, 0], 0.5 * expect, 1e-12)
    _close(out[0, 0], 0.5 * vals[0], 1e-12)          # read-after-write within a token


def check_split_invariance(impl):
    """extend over [A;B] == extend(A) then extend(B) from the saved state, at every
    cut, and == extend(A) followed by single-token steps."""
    c = tiny_case(lens=(9,), has_init=(1,))
    full, _, ffin = _run(impl, c)
    for cut in range(0, 10):
        pool = c.pool.copy()
        parts = [(0, cut), (cut, 9)] if cut not in (0, 9) else [(0, 9)]
        outs = np.full_like(full, np.nan)
        for (t0, t1) in parts:
            sl = slice(t0, t1)
            o, _, fin = impl(c.q[sl], c.k[sl], c.v[sl], c.a[sl], c.b[sl], c.A_log, c.dt_bias,
                             np.array([0, t1 - t0]), c.slot, np.array([1]), pool, c.scale)
            outs[sl] = o
            pool = oracle.apply_final_states(pool, fin)
        _close(outs, full)
        _close(pool[c.slot[0]], ffin[c.slot[0]])
    # extend(A) then one token at a time
    pool = c.pool.copy()
    o, _, fin = impl(c.q[:4], c.k[:4], c.v[:4], c.a[:4], c.b[:4], c.A_log, c.dt_bias,
                     np.array([0, 4]), c.slot, np.array([1]), pool, c.scale)
    pool = oracle.apply_final_states(pool, fin)
    for t in range(4, 9):
        sl = slice(t, t + 1)
        o, _, fin = impl(c.q[sl], c.k[sl], c.v[sl], c.a[sl], c.b[sl], c.A_log, c.dt_bias,
                         np.array([0, 1]), c.slot, np.array([1]), pool, c.scale)
        _close(o[0], full[t])
        pool = oracle.apply_final_states(pool, fin)
    _close(pool[c.slot[0]], ffin[c.slot[0]])


def check_grouped_heads(impl):
    """H_v = 2 H_qk with shared qk-heads == H_qk = H_v with each qk-head duplicated
    for its two v-heads."""
    c = tiny_case(H_qk=2, H_v=4)
    out, _, fin = _run(impl, c)
    q2 = np.repeat(c.q, 2, axis=1)
    k2 = np.repeat(c.k, 2, axis=1)
    out2, _, fin2 = impl(q2, k2, c.v, c.a, c.b, c.A_log, c.dt_bias, c.cu_seqlens, c.slot,
                         c.has_init, c.pool, c.scale)
    _close(out, out2)
    for s in fin:
        _close(fin[s], fin2[s])


def check_pool_and_indices(impl):
    """slot < 0 skips (no row, no state); has_init = 0 ignores the pool; a
    zero-length sequence writes its start state back; each slot gets its own
    sequence's state (distinct per-slot initial states)."""
    c = tiny_case(lens=(4, 0, 3, 0, 2), has_init=(1, 1, 0, 0, 1))
    c.slot[:] = [6, 2, 8, 0, -1]
    out, written, fin = _run(impl, c)
    assert sorted(fin) == [0, 2, 6, 8]
    assert not written[7:].any() and written[:7].all()
    assert np.isnan(out[7:]).all()
    _close(fin[2], c.pool[2])                        # zero-length, has_init = 1
    _close(fin[0], np.zeros_like(c.pool[0]))         # zero-length, has_init = 0
    # has_init = 0: poisoning the pool slot must not change anything
    pool2 = c.pool.copy()
    pool2[8] = 1e6
    out2, _, fin2 = _run(impl, c, pool=pool2)
    _close(out2[:7], out[:7])
    _close(fin2[8], fin[8])
    # ownership: sequence 0 (slot 6) must not see slot 8's or slot 2's contents
    pool3 = c.pool.copy()
    pool3[[0, 1, 3, 4, 5, 7]] = -7.0
    out3, _, fin3 = _run(impl, c, pool=pool3)
    _close(out3[:4], out[:4])
    _close(fin3[6], fin[6])


def check_norm_scale_invariance(impl):
    """q and k are L2-normalised: scaling them by positive constants changes nothing
    (up to eps, set to 0 here)."""
    c = tiny_case()
    o1, _, f1 = _run(impl, c, eps=0.0)
    mixed = c.mixed_qkv.copy()
    n = c.H_qk * c.d_k
    mixed[:, :n] *= 4.0            # powers of two keep the fp32 inputs exact
    mixed[:, n:2 * n] *= 0.25
    c2 = synth.GDNCase(**{**c.__dict__, "mixed_qkv": mixed})
    o2, _, f2 = _run(impl, c2, eps=0.0)
    _close(o1, o2, 1e-11)
    for s in f1:
        _close(f1[s], f2[s], 1e-11)


def check_state_orientation(impl):
    """One token from zero with g = 1, beta = 1: S = v khat^T, so the stored
    matrix is [d_v][d_k] with S[r, c] = v_r khat_c."""
    d_k, d_v = 4, 3
    k = np.array([[[0.0, 3.0, 0.0, 4.0]]])
    v = np.array([[[1.0, -2.0, 5.0]]])
    q = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    _, _, fin = impl(q, k, v, np.array([[-1000.0]]), np.array([[1000.0]]), np.zeros(1),
                     np.zeros(1), np.array([0, 1]), np.array([0]), np.array([0]),
                     np.zeros((1, 1, d_v, d_k)), 1.0, eps=0.0)
    _close(fin[0][0], np.outer(v[0, 0], [0.0, 0.6, 0.0, 0.8]))


CHECKS = [check_dense_bruteforce, check_exact_rational, check_beta_zero_pure_decay,
          check_exact_recall, check_split_invariance, check_grouped_heads,
          check_pool_and_indices, check_norm_scale_invariance, check_state_orientation]


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle.gdn_extend)


def test_decode_is_unit_length_extend():
    c = tiny_case(lens=(1, 1, 1, 1), has_init=1)
    o1, _, f1 = oracle.gdn_decode(c.q, c.k, c.v, c.a, c.b, c.A_log, c.dt_bias, c.slot,
                                  c.pool, c.scale)
    o2, _, f2 = _run(oracle.gdn_extend, c)
    _close(o1, o2)
    # and each decode step equals the dense one-step update
    check_dense_bruteforce(oracle.gdn_extend)


def test_heads_subset_matches_full():
    c = tiny_case()
    out, _, fin = _run(oracle.gdn_extend, c)
    sub, _, fsub = _run(oracle.gdn_extend, c, heads=[3, 0])
    _close(sub, out[:, [3, 0]])
    for s in fin:
        _close(fsub[s], fin[s][[3, 0]])


# ------------------------------------------------------------------ planted mistakes
def _mutant(kind):
    """A re-typed recurrence with one planted mistake (kind), used only to show
    that the checks above reject it.  kind=None must equal the oracle."""
    def impl(q, k, v, a, b, A_log, dt_bias, cu, slot, has_init, pool, scale, eps=1e-6,
             heads=None, seqs=None):
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
        A_log, dt_bias = np.asarray(A_log, np.float64), np.asarray(dt_bias, np.float64)
        T, H_qk, d_k = q.shape
        H_v, d_v = v.shape[1:]
        r = H_v // H_qk
        out = np.full((T, H_v, d_v), np.nan)
        written = np.zeros(T, bool)
        fin = {}
        for n in range(len(cu) - 1):
            if slot[n] < 0:
                continue
            S = (np.array(pool[slot[n]], np.float64) if has_init[n]
                 else np.zeros((H_v, d_v, d_k)))
            for t in range(cu[n], cu[n + 1]):
                for h in range(H_v):
                    j = (h % H_qk) if kind == "head_mod" else h // r
                    sp = np.logaddexp(0.0, a[t, h] + dt_bias[h])
                    g = np.exp(-np.exp(A_log[h]) * sp)
                    if kind == "gate_sign":
                        g = np.exp(-np.exp(A_log[h]) * np.logaddexp(0.0, a[t, h] - dt_bias[h]))
                    beta = scipy.special.expit(b[t, h])
                    kk = k[t, j] / np.sqrt(k[t, j] @ k[t, j] + eps)
                    qq = q[t, j] / np.sqrt(q[t, j] @ q[t, j] + eps)
                    if kind == "no_qnorm":
                        qq = q[t, j]
                    Sp = S[h].copy()
                    if kind == "decay_after":
                        S[h] = g * (S[h] + beta * np.outer(v[t, h] - S[h] @ kk, kk))
                    elif kind == "undecayed_read":
                        S[h] = g * S[h] + beta * np.outer(v[t, h] - Sp @ kk, kk)
                    elif kind == "sign":
                        S[h] = g * S[h] + beta * np.outer(v[t, h] + g * Sp @ kk, kk)
                    else:
                        S[h] = g * S[h]
                        S[h] = S[h] + beta * np.outer(v[t, h] - S[h] @ kk, kk)
                    Sread = Sp if kind == "read_prev_state" else S[h]
                    out[t, h] = scale * Sread @ qq
                    written[t] = True
            fin[slot[n]] = S.swapaxes(1, 2).copy() if kind == "transpose_state" else S.copy()
        return out, written, fin
    return impl


MUTANTS = ["head_mod", "gate_sign", "no_qnorm", "decay_after", "undecayed_read", "sign",
           "read_prev_state", "transpose_state"]


def test_mutant_baseline_equals_oracle():
    c = tiny_case()
    o1, _, f1 = _run(oracle.gdn_extend, c)
    o2, _, f2 = _run(_mutant(None), c)
    _close(o1, o2)
    for s in f1:
        _close(f1[s], f2[s])


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_reject_mutants(kind):
    impl = _mutant(kind)
    failed = 0
    for check in CHECKS:
        try:
            check(impl)
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed > 0, f"no pin rejects the planted mistake {kind!r}"


# ------------------------------------------------------------------ delta-off (SSD)
def _ssd_small(seed=2, batch=2, L=11, H=6, P=3, G=2, Nst=5, initial=False, with_D=True, with_z=True):
    c = synth.config4_ssd(seed=seed, batch=batch, L=L, H=H, P=P, G=G, Nst=Nst,
                          with_D=with_D, with_z=with_z, initial=initial)
    return c


def test_ssd_quadratic_dual_form():
    """Zero initial state: y = (C B^T o L) diag(dt') X with L_ij = exp(G_i - G_j)
    (i >= j) -- the SSD dual (masked matmul) form -- plus D x, times silu(z)."""
    c = _ssd_small()
    out, fin = oracle.ssd_combined(c.x, c.dt, c.A, c.B, c.C, c.D, c.z, c.dt_bias, True,
                                   (0.0, np.inf), None, True)
    H = c.x.shape[2]
    G = c.B.shape[2]
    for bi in range(c.x.shape[0]):
        for h in range(H):
            gi = h // (H // G)
            dtp = np.logaddexp(0.0, c.dt[bi, :, h].astype(np.float64) + c.dt_bias[h])
            Gc = np.cumsum(dtp * c.A[h])
            L = np.tril(np.exp(Gc[:, None] - Gc[None, :]))
            Bm = c.B[bi, :, gi].astype(np.float64)
            Cm = c.C[bi, :, gi].astype(np.float64)
            X = c.x[bi, :, h].astype(np.float64)
            y = ((Cm @ Bm.T) * L) @ (dtp[:, None] * X) + float(c.D[h]) * X
            zz = c.z[bi, :, h].astype(np.float64)
            y = y * zz * scipy.special.expit(zz)
            _close(out[bi, :, h], y, 1e-11)
            # final state: sum_j exp(G_L - G_j) dt'_j x_j B_j^T
            w = np.exp(Gc[-1] - Gc) * dtp
            _close(fin[bi, h], (w[:, None] * X).T @ Bm, 1e-11)


def test_ssd_initial_state_term():
    """Linearity in the initial state: out(S0) - out(0) = diag(gamma) C S0^T (times the
    gate), final(S0) - final(0) = gamma_L S0."""
    c = _ssd_small(initial=True, with_D=False, with_z=False)
    o1, f1 = oracle.ssd_combined(c.x, c.dt, c.A, c.B, c.C, None, None, c.dt_bias, True,
                                 (0.0, np.inf), c.initial_states, True)
    o0, f0 = oracle.ssd_combined(c.x, c.dt, c.A, c.B, c.C, None, None, c.dt_bias, True,
                                 (0.0, np.inf), None, True)
    H = c.x.shape[2]
    G = c.B.shape[2]
    for bi in range(c.x.shape[0]):
        for h in range(H):
            dtp = np.logaddexp(0.0, c.dt[bi, :, h].astype(np.float64) + c.dt_bias[h])
            gam = np.exp(np.cumsum(dtp * c.A[h]))
            S0 = c.initial_states[bi, h].astype(np.float64)
            Cm = c.C[bi, :, h // (H // G)].astype(np.float64)
            _close(o1[bi, :, h] - o0[bi, :, h], gam[:, None] * (Cm @ S0.T), 1e-11)
            _close(f1[bi, h] - f0[bi, h], gam[-1] * S0, 1e-11)


def test_ssd_no_decay_prefix_sum_and_clamp():
    """A = 0 => g = 1 and y_t = sum_{m<=t} dt'_m (C_t . B_m) x_m; with dt_softplus off
    and dt_limit (0.1, 0.4) the step is the clamped raw dt + dt_bias."""
    c = _ssd_small(with_D=False, with_z=False, G=1)
    A = np.zeros_like(c.A)
    out, _ = oracle.ssd_combined(c.x, c.dt, A, c.B, c.C, None, None, c.dt_bias, False,
                                 (0.1, 0.4), None, True)
    for bi in range(c.x.shape[0]):
        for h in range(c.x.shape[2]):
            dtp = np.clip(c.dt[bi, :, h].astype(np.float64) + c.dt_bias[h], 0.1, 0.4)
            Bm = c.B[bi, :, 0].astype(np.float64)
            Cm = c.C[bi, :, 0].astype(np.float64)
            X = c.x[bi, :, h].astype(np.float64)
            for t in range(c.x.shape[1]):
                y = sum(dtp[m] * (Cm[t] @ Bm[m]) * X[m] for m in range(t + 1))
                _close(out[bi, t, h], y, 1e-11)


def test_ssd_D_per_dim_and_heads_subset():
    c = _ssd_small(with_z=False)
    Dfull = np.tile(np.asarray(c.D, np.float64)[:, None], (1, c.x.shape[3]))
    o1, _ = oracle.ssd_combined(c.x, c.dt, c.A, c.B, c.C, c.D, None, c.dt_bias, True)
    o2, _ = oracle.ssd_combined(c.x, c.dt, c.A, c.B, c.C, Dfull, None, c.dt_bias, True)
    _close(o1, o2)
    o3, _ = oracle.ssd_combined(c.x, c.dt, c.A, c.B, c.C, c.D, None, c.dt_bias, True, heads=[5, 1])
    _close(o3, o1[:, :, [5, 1]])


# ------------------------------------------------------------------ generators
def test_generators_shapes_and_rounding():
    ext, dec = synth.config0_tiny()
    assert ext.T == 24 and list(ext.cu_seqlens) == [0, 15, 23, 24]
    assert list(ext.has_init) == [0, 1, 1] and ext.pool.shape == (16, 2, 64, 64)
    assert len(set(ext.slot.tolist())) == 3 and list(dec.slot) == list(ext.slot)
    lens = synth.ragged_lengths(1003)
    assert len(lens) == 64 and abs(int(lens.sum()) - 131072) <= 64
    assert lens.min() >= 1 and lens.max() <= 8192
    x = np.array([1.0, 1.00390625, 1.0048828125, -3.3e-5, np.inf], np.float32)
    r = synth.bf16_round(x)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.0078125 and np.isinf(r[4])
    c = synth.edge_case("e", (3, 2))
    assert np.array_equal(synth.bf16_round(c.mixed_qkv), c.mixed_qkv)


# ------------------------------------------------------------------ state checkpoints
def _dense_prefix_state(c, n, h, b):
    """State of sequence n, head h after its tokens before absolute index b, by the
    dense transition-matrix recurrence (independent of the oracle's loop)."""
    r = c.H_v // c.H_qk
    j = h // r
    S = c.pool[c.slot[n], h].astype(np.float64) if c.has_init[n] else np.zeros((c.d_v, c.d_k))
    for t in range(int(c.cu_seqlens[n]), b):
        sp = np.logaddexp(0.0, float(c.a[t, h]) + float(c.dt_bias[h]))
        g = np.exp(-np.exp(float(c.A_log[h])) * sp)
        beta = scipy.special.expit(float(c.b[t, h]))
        kk = c.k[t, j].astype(np.float64)
        kk = kk / np.sqrt(kk @ kk + 1e-6)
        S = S @ (g * (np.eye(c.d_k) - beta * np.outer(kk, kk))) + beta * np.outer(c.v[t, h].astype(np.float64), kk)
    return S


def test_checkpoint_states_every_boundary():
    """A checkpoint at exclusive boundary b holds the state after the sequence's tokens
    before b, for every b from the first token (the initial state, or zeros) to the end
    (the final state); the outputs and final states are unchanged by capturing."""
    c = tiny_case(lens=(5, 3, 4), has_init=(1, 0, 1))
    ref_out, _, ref_fin = _run(oracle.gdn_extend, c)
    for n in range(c.N):
        t0, t1 = int(c.cu_seqlens[n]), int(c.cu_seqlens[n + 1])
        for b in range(t0, t1 + 1):
            tok = np.full(c.N, -1, np.int64)
            tok[n] = b
            ck_slot = np.full(c.N, -1, np.int64)
            ck_slot[n] = 7
            ck = {}
            out, _, fin = _run(oracle.gdn_extend, c, ckpt_token=tok, ckpt_slot=ck_slot, ckpts=ck)
            assert list(ck) == [7]
            for h in range(c.H_v):
                _close(ck[7][h], _dense_prefix_state(c, n, h, b))
            _close(out, ref_out)
            for s in fin:
                _close(fin[s], ref_fin[s])
        _close(ck[7], ref_fin[c.slot[n]])            # b = end: the final state


def test_checkpoint_disabled_entries():
    """Negative boundary or slot, a skipped sequence, or a boundary outside the
    sequence records nothing; several sequences record into their own rows."""
    c = tiny_case(lens=(5, 3, 4), has_init=(1, 0, 1))
    cu = c.cu_seqlens
    ck = {}
    _run(oracle.gdn_extend, c, ckpt_token=np.array([-1, cu[1] + 1, cu[2] + 2]),
         ckpt_slot=np.array([0, -1, 4]), ckpts=ck)
    assert list(ck) == [4]
    c.slot[2] = -1
    ck = {}
    _run(oracle.gdn_extend, c, ckpt_token=np.array([cu[0] + 2, cu[1] + 4, cu[2] + 2]),
         ckpt_slot=np.array([1, 2, 3]), ckpts=ck)
    assert list(ck) == [1]                           # seq 1: 4 > its 3 tokens; seq 2 skipped


def test_ssd_checkpoint_relative_boundary():
    """Delta-off checkpoints (batched, boundary relative to the batch element): the
    state after the first b tokens is gamma_b S0 + sum_{j<b} exp(G_{b-1} - G_j) dt'_j x_j B_j^T."""
    c = _ssd_small(initial=True, with_D=False, with_z=False)
    H = c.x.shape[2]
    G = c.B.shape[2]
    L = c.x.shape[1]
    for b in (0, 1, 4, L):
        ck = {}
        oracle.ssd_combined(c.x, c.dt, c.A, c.B, c.C, None, None, c.dt_bias, True, (0.0, np.inf),
                            c.initial_states, True, ckpt_token=np.array([b, -1]),
                            ckpt_slot=np.array([5, 6]), ckpts=ck)
        assert list(ck) == [5]
        for h in range(H):
            dtp = np.logaddexp(0.0, c.dt[0, :b, h].astype(np.float64) + c.dt_bias[h])
            Gc = np.cumsum(dtp * c.A[h])
            Gb = Gc[-1] if b else 0.0
            S = np.exp(Gb) * c.initial_states[0, h].astype(np.float64)
            if b:
                X = c.x[0, :b, h].astype(np.float64)
                Bm = c.B[0, :b, h // (H // G)].astype(np.float64)
                S = S + ((np.exp(Gb - Gc) * dtp)[:, None] * X).T @ Bm
            _close(ck[5][h], S, 1e-11)


# ------------------------------------------------------------------ target-verify states
def _dense_path_state(c, n, h, path):
    """State of sequence n, head h after applying its tokens `path` (absolute indices,
    in order) to its start state, by the dense transition-matrix recurrence."""
    r = c.H_v // c.H_qk
    j = h // r
    S = c.pool[c.slot[n], h].astype(np.float64) if c.has_init[n] else np.zeros((c.d_v, c.d_k))
    for t in path:
        sp = np.logaddexp(0.0, float(c.a[t, h]) + float(c.dt_bias[h]))
        g = np.exp(-np.exp(float(c.A_log[h])) * sp)
        beta = scipy.special.expit(float(c.b[t, h]))
        kk = c.k[t, j].astype(np.float64)
        kk = kk / np.sqrt(kk @ kk + 1e-6)
        S = S @ (g * (np.eye(c.d_k) - beta * np.outer(kk, kk))) + beta * np.outer(c.v[t, h].astype(np.float64), kk)
    return S


def test_verify_chain_states():
    """Chain verify: the state after token i of each sequence is the dense recurrence over
    its first i + 1 tokens; outputs and final states equal the plain extend's."""
    c = tiny_case(lens=(4, 3, 5), has_init=(1, 1, 0))
    ref_out, _, ref_fin = _run(oracle.gdn_extend, c)
    spec = {}
    out, _, fin = _run(oracle.gdn_extend, c, spec_slot=np.array([2, -1, 0]), spec=spec)
    _close(out, ref_out)
    assert sorted(spec) == [(0, i) for i in range(5)] + [(2, i) for i in range(4)]
    for n, row in ((0, 2), (2, 0)):
        t0 = int(c.cu_seqlens[n])
        for i in range(int(c.cu_seqlens[n + 1]) - t0):
            for h in range(c.H_v):
                _close(spec[(row, i)][h], _dense_path_state(c, n, h, range(t0, t0 + i + 1)))


def test_verify_tree_states_and_outputs():
    """Tree verify: each token continues its parent's state; its state and output equal
    the dense recurrence over the path root -> token alone (siblings do not see each
    other)."""
    c = tiny_case(lens=(5, 4), has_init=(1, 0))
    parents = np.array([-1, 0, 0, 1, 2, -1, 0, 1, 1])        # per token, within its sequence
    spec = {}
    out, _, _ = _run(oracle.gdn_extend, c, spec_slot=np.array([1, 0]), spec_parent=parents, spec=spec)
    for n, row in ((0, 1), (1, 0)):
        t0, t1 = int(c.cu_seqlens[n]), int(c.cu_seqlens[n + 1])
        for i in range(t1 - t0):
            path, x = [], i
            while x >= 0:
                path.append(t0 + x)
                x = int(parents[t0 + x])
            path = path[::-1]
            r = c.H_v // c.H_qk
            for h in range(c.H_v):
                S = _dense_path_state(c, n, h, path)
                _close(spec[(row, i)][h], S)
                qq = c.q[t0 + i, h // r].astype(np.float64)
                _close(out[t0 + i, h], c.scale * S @ (qq / np.sqrt(qq @ qq + 1e-6)))


def test_verify_tree_parent_outside_the_past_is_the_start():
    """A parent outside [0, i) (forward, self or far past the end) or not below the
    recorded steps counts as -1: the token's state is the dense recurrence from the
    sequence's start state over the token alone, or over its root path where the chain of
    parents stays inside the past."""
    c = tiny_case(lens=(6, 4), has_init=(1, 1))
    # seq 0: token 1 -> 3 (forward), 2 -> 2 (itself), 3 -> 1, 4 -> 99 (past the end),
    # 5 -> 4 (whose own parent was forward); seq 1: token 2 -> 3 (forward), 3 -> 2
    parents = np.array([-1, 3, 2, 1, 99, 4, -1, 0, 3, 2])
    spec = {}
    out, _, _ = _run(oracle.gdn_extend, c, spec_slot=np.array([0, 1]), spec_parent=parents, spec=spec)

    def path_of(t0, i, steps=None):
        path, x = [], i
        while x >= 0:
            path.append(t0 + x)
            p_ = int(parents[t0 + x])
            x = p_ if (0 <= p_ < x and (steps is None or p_ < steps)) else -1
        return path[::-1]
    r = c.H_v // c.H_qk
    for n, row in ((0, 0), (1, 1)):
        t0, t1 = int(c.cu_seqlens[n]), int(c.cu_seqlens[n + 1])
        for i in range(t1 - t0):
            for h in range(c.H_v):
                S = _dense_path_state(c, n, h, path_of(t0, i))
                _close(spec[(row, i)][h], S)
                qq = c.q[t0 + i, h // r].astype(np.float64)
                _close(out[t0 + i, h], c.scale * S @ (qq / np.sqrt(qq @ qq + 1e-6)))
    # with 3 recorded steps, token 5's parent 4 is not recorded: it starts from the start
    spec3 = {}
    _run(oracle.gdn_extend, c, spec_slot=np.array([0, 1]), spec_parent=parents, spec=spec3, spec_steps=3)
    for h in range(c.H_v):
        _close(spec3[(0, 5)][h], _dense_path_state(c, 0, h, path_of(0, 5, steps=3)))
        _close(spec3[(0, 3)][h], _dense_path_state(c, 0, h, path_of(0, 3, steps=3)))
    # the root paths the rule gives (token indices)
    assert path_of(0, 1) == [1] and path_of(0, 2) == [2] and path_of(0, 3) == [1, 3]
    assert path_of(0, 4) == [4] and path_of(0, 5) == [4, 5] and path_of(6, 3) == [8, 9]
    assert path_of(0, 5, steps=3) == [5] and path_of(0, 3, steps=3) == [1, 3]


# ------------------------------------------------------------------ short causal conv1d
# The checks take the implementation as an argument so that the same checks can be
# run against re-typed versions with planted mistakes (below).
def _conv_case(seed=4, lens=(6, 2, 5, 0), C=7, K=4, has_init=(1, 1, 0, 1)):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return dict(x=rng.standard_normal((T, C)), w=rng.standard_normal((C, K)), b=rng.standard_normal(C),
                cu=cu, slot=np.array([3, 0, 2, 1]), has_init=np.array(has_init),
                pool=rng.standard_normal((5, C, K - 1)))


def _check_conv_convolve(impl):
    """Each channel of each sequence equals numpy's full convolution of [state; x] with the
    reversed kernel (valid part), plus bias, through silu (scipy expit); the new state is
    the last K-1 window rows."""
    c = _conv_case()
    out, st = impl(c["x"], c["w"], c["b"], c["cu"], c["slot"], c["has_init"], c["pool"])
    K = c["w"].shape[1]
    for n in range(4):
        t0, t1 = c["cu"][n], c["cu"][n + 1]
        s = c["slot"][n]
        prev = c["pool"][s].T if c["has_init"][n] else np.zeros((K - 1, c["x"].shape[1]))
        win = np.concatenate([prev, c["x"][t0:t1]])
        for ch in range(c["x"].shape[1] if t1 > t0 else 0):
            y = np.convolve(win[:, ch], c["w"][ch, ::-1], mode="valid") + c["b"][ch]
            _close(out[t0:t1, ch], y * scipy.special.expit(y))
        _close(st[s], win[-(K - 1):].T)
    assert list(st) == [3, 0, 2, 1]                  # the empty sequence keeps its state
    _close(st[1], c["pool"][1])


def _check_conv_split_resume(impl):
    """conv(A || B) == conv(A) then conv(B) from the state == conv(A) then one token at a
    time; without activation the map is linear in x (bias 0)."""
    c = _conv_case(lens=(9,), has_init=(1,))
    c["slot"] = np.array([2])
    full, fst = impl(c["x"], c["w"], c["b"], np.array([0, 9]), c["slot"], None, c["pool"])
    for cut in range(10):
        pool = c["pool"].copy()
        outs = []
        for (a0, a1) in ((0, cut), (cut, 9)):
            o, st = impl(c["x"][a0:a1], c["w"], c["b"], np.array([0, a1 - a0]), c["slot"], None, pool)
            outs.append(o)
            pool[2] = st[2]
        _close(np.concatenate(outs), full)
        _close(pool[2], fst[2])
    pool = c["pool"].copy()
    for t in range(9):
        o, st = impl(c["x"][t:t + 1], c["w"], c["b"], np.array([0, 1]), c["slot"], None, pool)
        _close(o[0], full[t])
        pool[2] = st[2]
    o1, _ = impl(c["x"], c["w"], None, np.array([0, 9]), c["slot"], np.array([0]), c["pool"], False)
    o2, _ = impl(2 * c["x"], c["w"], None, np.array([0, 9]), c["slot"], np.array([0]), c["pool"], False)
    _close(o2, 2 * o1)


def _check_conv_token_tree(impl):
    """A chain given as a tree (parent = i - 1) is the plain conv; every token of a tree
    gives the last output of the plain conv over its explicit root path; no states."""
    c = _conv_case(lens=(7, 5), has_init=(1, 0))
    c["slot"] = np.array([2, 4])
    cu = np.array([0, 7, 12])
    chain = np.array([-1, 0, 1, 2, 3, 4, 5, -1, 0, 1, 2, 3])
    ref, _ = impl(c["x"][:12], c["w"], c["b"], cu, c["slot"], c["has_init"][:2], c["pool"])
    got, st = impl(c["x"][:12], c["w"], c["b"], cu, c["slot"], c["has_init"][:2], c["pool"], parent=chain)
    _close(got, ref)
    assert st == {}
    tree = np.array([-1, 0, 0, 1, 2, 2, -1, -1, 0, 0, 1, 3])     # two branches, a second root
    got, _ = impl(c["x"][:12], c["w"], c["b"], cu, c["slot"], c["has_init"][:2], c["pool"], parent=tree)
    for n in range(2):
        t0 = cu[n]
        for i in range(cu[n + 1] - t0):
            path = [i]
            while tree[t0 + path[-1]] >= 0:
                path.append(tree[t0 + path[-1]])
            xs = c["x"][[t0 + j for j in reversed(path)]]
            o, _ = impl(xs, c["w"], c["b"], np.array([0, len(xs)]), c["slot"][n:n + 1],
                        c["has_init"][n:n + 1], c["pool"])
            _close(got[t0 + i], o[-1])


CONV_CHECKS = [_check_conv_convolve, _check_conv_split_resume, _check_conv_token_tree]


def test_conv_matches_numpy_convolve():
    _check_conv_convolve(oracle.causal_conv1d)


def test_conv_split_resume_and_decode():
    _check_conv_split_resume(oracle.causal_conv1d)


def test_conv_token_tree():
    _check_conv_token_tree(oracle.causal_conv1d)


def _conv_mutant(kind):
    """A re-typed conv with one planted mistake (kind); kind=None must equal the oracle."""
    def impl(x, weight, bias, cu_seqlens, slot, has_init, conv_pool, activation=True, parent=None):
        x = np.asarray(x, np.float64)
        w = np.asarray(weight, np.float64)
        if kind == "reversed_taps":
            w = w[:, ::-1]
        T, C = x.shape
        K = w.shape[1]
        b = np.zeros(C) if (bias is None or kind == "no_bias") else np.asarray(bias, np.float64)
        N = len(cu_seqlens) - 1
        hi = np.ones(N, np.int64) if has_init is None else np.asarray(has_init)
        out = np.full((T, C), np.nan)
        states = {}
        for n in range(N):
            s = int(slot[n])
            if s < 0:
                continue
            t0, t1 = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
            prev = np.asarray(conv_pool[s], np.float64).T if hi[n] else np.zeros((K - 1, C))
            if kind == "state_newest_first":
                prev = prev[::-1]
            for t in range(t0, t1):
                rows = list(range(t0, t + 1))
                if parent is not None and kind != "tree_as_chain":
                    rows = [t]
                    while int(parent[rows[0]]) >= 0:
                        rows.insert(0, t0 + int(parent[rows[0]]))
                win = np.concatenate([prev, x[rows]])[-K:]
                y = b + np.einsum("ck,kc->c", w, win)
                if activation:
                    y = scipy.special.expit(y) if kind == "sigmoid_not_silu" else y * scipy.special.expit(y)
                out[t] = y
            if parent is None:
                allrows = np.concatenate([prev, x[t0:t1]])
                states[s] = (prev.T.copy() if kind == "stale_state" else allrows[-(K - 1):].T.copy())
        return out, states
    return impl


CONV_MUTANTS = ["reversed_taps", "no_bias", "state_newest_first", "tree_as_chain",
                "sigmoid_not_silu", "stale_state"]


def test_conv_mutant_baseline_passes():
    for check in CONV_CHECKS:
        check(_conv_mutant(None))


@pytest.mark.parametrize("kind", CONV_MUTANTS)
def test_conv_pins_reject_mutants(kind):
    impl = _conv_mutant(kind)
    failed = 0
    for check in CONV_CHECKS:
        try:
            check(impl)
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed > 0, f"no pin rejects the planted mistake {kind!r}"


# ------------------------------------------------------------------ committed fixture
def test_oracle_reproduces_committed_config0_fixture():
    """tests/golden/config0_oracle.npz (written by tests/golden/make_golden.py through the
    oracle alone) is a regression fixture: any later change to the oracle's arithmetic
    that moves the tiny fp32 extend + decode case shows up here as a difference from the
    committed values (the oracle is float64 throughout; 1e-12 allows for BLAS order)."""
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "config0_oracle.npz")
    ref = np.load(path)
    ext, dec = synth.config0_tiny()
    out_e, _, fin_e = oracle.gdn_extend(ext.q, ext.k, ext.v, ext.a, ext.b, ext.A_log, ext.dt_bias,
                                        ext.cu_seqlens, ext.slot, ext.has_init, ext.pool, ext.scale)
    pool1 = oracle.apply_final_states(ext.pool, fin_e)
    out_d, _, fin_d = oracle.gdn_decode(dec.q, dec.k, dec.v, dec.a, dec.b, dec.A_log, dec.dt_bias,
                                        dec.slot, pool1, dec.scale)
    pool2 = oracle.apply_final_states(pool1, fin_d)
    assert np.array_equal(ref["slots"], ext.slot)
    for name, got in (("extend_out", out_e), ("decode_out", out_d),
                      ("state_after_extend", pool1[ext.slot]), ("state_after_decode", pool2[ext.slot])):
        np.testing.assert_allclose(got, ref[name], rtol=1e-12, atol=1e-14, err_msg=name)

