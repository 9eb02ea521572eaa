"""Token-by-token float64 oracle for the GDN layer and the delta-off SSD mode.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.  Parity pins live in tests/test_oracle_pins.py.

Conventions (the pages leave these open; the readings are the plainest the
rest supports):
  * state layout: one [d_v, d_k] matrix per (slot, v-head), i.e. S as written
    in v k^T; the pool is [num_slots, H_v, d_v, d_k].  The flashinfer
    ssd_combined_fwd page orders initial states as [.., nheads, headdim, dstate],
    which is the same (value dim, key dim) order.
  * grouped heads: v-head h reads qk-head h // (H_v // H_qk) (contiguous groups).
  * L2 normalisation: x / sqrt(sum(x^2) + eps), eps = 1e-6.
  * the output uses the post-update state S_t.
  * has_init[n] == 0 starts sequence n from zeros and ignores the pool;
    slot[n] < 0 skips sequence n entirely (no output row, no pool write), after
    the "negative entries disable" rule of the ssd_combined_fwd page;
    a zero-length sequence writes its initial state (or zeros) back unchanged.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------- scalar maps
def softplus(x):
    """softplus(x) = log(1 + exp(x)), written as max(x, 0) + log1p(exp(-|x|))
    so that it neither overflows nor loses the small-x tail."""
    x = np.asarray(x, dtype=F64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    """sigmoid(x) = 1 / (1 + exp(-x)), evaluated on the side that cannot overflow."""
    x = np.asarray(x, dtype=F64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def gdn_gate(a, b, A_log, dt_bias):
    """GDN gate (gated delta rule parameterisation):
        log g = -exp(A_log[h]) * softplus(a[t, h] + dt_bias[h]),  beta = sigmoid(b[t, h]).
    Returns (log_g, beta), both float64 [T, H].  g itself is exp(log_g)."""
    a = np.asarray(a, dtype=F64)
    b = np.asarray(b, dtype=F64)
    A_log = np.asarray(A_log, dtype=F64)
    bias = np.zeros_like(A_log) if dt_bias is None else np.asarray(dt_bias, dtype=F64)
    log_g = -np.exp(A_log)[None, :] * softplus(a + bias[None, :])
    beta = sigmoid(b)
    return log_g, beta


def ssd_gate(dt, A, dt_bias=None, dt_softplus=False, dt_limit=(0.0, float("inf"))):
    """Delta-off (Mamba2 SSD) gate after the ssd_combined_fwd parameter list:
    dt' = clamp(softplus(dt + dt_bias) if dt_softplus else dt + dt_bias, lo, hi)
    (inclusive limits), log g = dt' * A[h].  Returns (log_g, dt') float64 [.., H]."""
    dt = np.asarray(dt, dtype=F64)
    A = np.asarray(A, dtype=F64)
    x = dt if dt_bias is None else dt + np.asarray(dt_bias, dtype=F64)
    if dt_softplus:
        x = softplus(x)
    lo, hi = dt_limit
    x = np.clip(x, lo, hi)
    return x * A, x


def l2_normalize(x, eps=1e-6):
    """x / sqrt(sum(x^2, last axis) + eps), float64."""
    x = np.asarray(x, dtype=F64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


# ---------------------------------------------------------------- GDN layer
def gdn_extend(q, k, v, a, b, A_log, dt_bias, cu_seqlens, slot, has_init, pool,
               scale, eps=1e-6, heads=None, seqs=None, ckpt_token=None, ckpt_slot=None,
               ckpts=None, spec_slot=None, spec_parent=None, spec=None, spec_steps=None):
    """Packed-varlen GDN extend, token by token.

    q, k : [T, H_qk, d_k]; v : [T, H_v, d_v]; a, b : [T, H_v]
    A_log, dt_bias : [H_v]; cu_seqlens : [N+1]; slot, has_init : [N]
    pool : anything indexable as pool[slot] -> [H_v, d_v, d_k] (initial states).
    heads : optional list of v-heads to compute (heads are independent);
    seqs  : optional list of sequence indices to compute.
    ckpt_token, ckpt_slot : optional [N] state checkpoints after the
      checkpoint_token_indices / checkpoint_state_slots arguments of the
      ssd_combined_fwd page: sequence n records the state after its tokens before
      the absolute token index ckpt_token[n] (an exclusive boundary in
      [cu[n], cu[n+1]]) under the key ckpt_slot[n] of the dict `ckpts`; a negative
      entry (either one), a skipped sequence or a boundary outside the sequence
      records nothing.
    spec_slot : optional [N] rows for the target-verify states: sequence n with
      spec_slot[n] >= 0 records the state after each of its tokens (index i within the
      sequence) under spec[(spec_slot[n], i)].
    spec_parent : optional [T] token tree: token i of a sequence starts from the state
      after token spec_parent[t] of the same sequence (an earlier index), or from the
      sequence's start state for -1, instead of from the state after token i - 1 (a
      chain).  A parent outside [0, i), or not below spec_steps when that is given
      (the number of recorded steps per row), counts as -1; a sequence without a row
      (spec_slot[n] < 0) runs as a chain.

    Returns (out, written, finals):
      out     float64 [T, len(heads), d_v]   (NaN where not written)
      written bool [T]                       (rows this call writes)
      finals  dict slot -> float64 [len(heads), d_v, d_k]  (final states)
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    T, H_qk, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    assert H_v % H_qk == 0, "H_v must be a multiple of H_qk"
    r = H_v // H_qk
    heads = list(range(H_v)) if heads is None else [int(h) for h in heads]
    hsel = np.asarray(heads, dtype=np.int64)
    jsel = hsel // r                                    # qk-head of each v-head
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    slot = np.asarray(slot, dtype=np.int64)
    has_init = np.ones(N, np.int64) if has_init is None else np.asarray(has_init, np.int64)
    seqs = range(N) if seqs is None else seqs

    out = np.full((T, len(heads), d_v), np.nan, dtype=F64)
    written = np.zeros(T, dtype=bool)
    finals = {}
    for n in seqs:
        s = int(slot[n])
        if s < 0:
            continue
        t0, t1 = int(cu[n]), int(cu[n + 1])
        ck = -1
        if ckpt_token is not None and int(ckpt_token[n]) >= 0 and int(ckpt_slot[n]) >= 0:
            ck = int(ckpt_token[n])
        if has_init[n]:
            S = np.array(pool[s], dtype=F64)[hsel].copy()          # [Hs, d_v, d_k]
        else:
            S = np.zeros((len(heads), d_v, d_k), dtype=F64)
        S_start = S.copy()
        row = -1 if spec_slot is None else int(spec_slot[n])
        for t in range(t0, t1):
            if t == ck:                                            # state before token t
                ckpts[int(ckpt_slot[n])] = S.copy()
            if spec_parent is not None and row >= 0:               # token tree: start from the parent
                par = int(spec_parent[t])
                i = t - t0
                if par < 0 or par >= i or (spec_steps is not None and par >= spec_steps):
                    par = -1                                       # outside the recorded past
                S = (S_start if par < 0 else spec[(row, par)]).copy()
            log_g, beta = gdn_gate(np.asarray(a[t:t + 1])[:, hsel], np.asarray(b[t:t + 1])[:, hsel],
                                   np.asarray(A_log)[hsel], np.asarray(dt_bias)[hsel])
            g = np.exp(log_g[0])[:, None, None]                    # [Hs,1,1]
            bt = beta[0][:, None]                                  # [Hs,1]
            kh = l2_normalize(np.asarray(k[t], dtype=F64)[jsel], eps)   # [Hs, d_k]
            qh = l2_normalize(np.asarray(q[t], dtype=F64)[jsel], eps)
            vt = np.asarray(v[t], dtype=F64)[hsel]                 # [Hs, d_v]
            S = g * S                                              # decay
            u = np.einsum("hvk,hk->hv", S, kh)                     # S k
            S = S + np.einsum("hv,hk->hvk", bt * (vt - u), kh)     # delta-rule write
            out[t] = scale * np.einsum("hvk,hk->hv", S, qh)        # read with S_t
            written[t] = True
            if row >= 0:
                spec[(row, t - t0)] = S.copy()
        if ck == t1:                                               # boundary at the end
            ckpts[int(ckpt_slot[n])] = S.copy()
        finals[s] = S
    return out, written, finals


def gdn_decode(q, k, v, a, b, A_log, dt_bias, slot, pool, scale, eps=1e-6, heads=None):
    """One token per sequence: token n belongs to sequence n, which always starts
    from its pool state (the decode step is the extend with unit lengths)."""
    B = np.asarray(q).shape[0]
    cu = np.arange(B + 1, dtype=np.int64)
    return gdn_extend(q, k, v, a, b, A_log, dt_bias, cu, slot, np.ones(B, np.int64), pool,
                      scale, eps=eps, heads=heads)


def apply_final_states(pool, finals, heads=None):
    """Return a float64 copy of pool with the final states written to their slots."""
    new = np.array(pool, dtype=F64, copy=True)
    for s, S in finals.items():
        if heads is None:
            new[s] = S
        else:
            new[s][np.asarray(heads)] = S
    return new


# ---------------------------------------------------------------- delta-off (SSD) mode
def ssd_combined(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=False,
                 dt_limit=(0.0, float("inf")), initial_states=None, return_final_states=True,
                 heads=None, ckpt_token=None, ckpt_slot=None, ckpts=None):
    """Mamba2 SSD scan, token by token, batched mode of ssd_combined_fwd.

    x [batch, L, H, P], dt [batch, L, H], A [H], B/C [batch, L, G, N],
    D [H] or [H, P] (optional), z like x (optional), initial_states
    [batch, H, P, N] (optional, zeros otherwise).  Head h uses group
    h // (H // G).  Per token:
        dt' = clamp(softplus(dt + dt_bias) | dt + dt_bias, dt_limit)
        S   = exp(dt' A) S + dt' x_t B_t^T            ([P, N] per head)
        y_t = S C_t + D x_t ;  out_t = y_t * silu(z_t)
    Returns (out float64 [batch, L, Hs, P], final float64 [batch, Hs, P, N] | None).
    ckpt_token, ckpt_slot : optional [batch] checkpoints as in gdn_extend, with the
    boundary relative to the batch element's first token (batched mode of the
    ssd_combined_fwd page); the states go to the dict `ckpts`.
    """
    x = np.asarray(x)
    batch, L, H, P = x.shape
    G, Nst = np.asarray(B).shape[2], np.asarray(B).shape[3]
    heads = list(range(H)) if heads is None else [int(h) for h in heads]
    hsel = np.asarray(heads, dtype=np.int64)
    gsel = hsel // (H // G)
    out = np.zeros((batch, L, len(heads), P), dtype=F64)
    finals = np.zeros((batch, len(heads), P, Nst), dtype=F64)
    Dv = None
    if D is not None:
        Dv = np.asarray(D, dtype=F64)[hsel]
        Dv = Dv[:, None] if Dv.ndim == 1 else Dv                  # [Hs, 1 | P]
    bias = None if dt_bias is None else np.asarray(dt_bias, dtype=F64)[hsel]
    for bi in range(batch):
        if initial_states is None:
            S = np.zeros((len(heads), P, Nst), dtype=F64)
        else:
            S = np.array(initial_states[bi], dtype=F64)[hsel].copy()
        ck = -1
        if ckpt_token is not None and int(ckpt_token[bi]) >= 0 and int(ckpt_slot[bi]) >= 0:
            ck = int(ckpt_token[bi])
        for t in range(L):
            if t == ck:
                ckpts[int(ckpt_slot[bi])] = S.copy()
            log_g, dtp = ssd_gate(np.asarray(dt[bi, t], dtype=F64)[hsel],
                                  np.asarray(A, dtype=F64)[hsel], bias, dt_softplus, dt_limit)
            xt = np.asarray(x[bi, t], dtype=F64)[hsel]             # [Hs, P]
            Bt = np.asarray(B[bi, t], dtype=F64)[gsel]             # [Hs, N]
            Ct = np.asarray(C[bi, t], dtype=F64)[gsel]
            S = np.exp(log_g)[:, None, None] * S + np.einsum("hp,hn->hpn", dtp[:, None] * xt, Bt)
            y = np.einsum("hpn,hn->hp", S, Ct)
            if Dv is not None:
                y = y + Dv * xt
            if z is not None:
                zt = np.asarray(z[bi, t], dtype=F64)[hsel]
                y = y * zt * sigmoid(zt)
            out[bi, t] = y
        if ck == L:
            ckpts[int(ckpt_slot[bi])] = S.copy()
        finals[bi] = S
    return out, (finals if return_final_states else None)


# ---------------------------------------------------------------- short causal conv1d
def causal_conv1d(x, weight, bias, cu_seqlens, slot, has_init, conv_pool, activation=True,
                  seqs=None, parent=None):
    """Depthwise causal conv1d over packed sequences with a per-slot conv state (the
    short convolution in front of the GDN layer; the plain reading of the conv[0]
    state buffer of the SGLang GDN test article).

    x [T, C]; weight [C, K]; bias [C] or None; conv_pool[slot] -> [C, K - 1] holds the
    last K - 1 inputs of the slot's sequence so far, oldest first.  Sequence n with
    slot[n] >= 0 sees the window w = (conv_pool[slot[n]] if has_init[n] else zeros)
    followed by its own inputs:
        y_t = sum_j weight[:, j] * w[t - t0 + j] + bias     (j = 0 .. K-1)
        out_t = silu(y_t) if activation else y_t
    and its new state is the last K - 1 rows of w (for a short sequence partly the
    old state).  slot[n] < 0 skips the sequence.
    parent: optional [T] token tree of target verify (the reading of the SGLang GDN test
    article's tree verify): token i of a sequence continues token parent[t] (an earlier
    index within the sequence, -1 = the state), so its window is the state followed by
    the inputs along its root path; no state is returned (the caller commits the
    accepted branch).
    Returns (out float64 [T, C] (NaN where not written), states dict slot -> [C, K-1]).
    """
    x = np.asarray(x, dtype=F64)
    w = np.asarray(weight, dtype=F64)
    T, Cn = x.shape
    K = w.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    b = np.zeros(Cn) if bias is None else np.asarray(bias, dtype=F64)
    has_init = np.ones(N, np.int64) if has_init is None else np.asarray(has_init, np.int64)
    out = np.full((T, Cn), np.nan, dtype=F64)
    states = {}
    for n in (range(N) if seqs is None else seqs):
        s = int(slot[n])
        if s < 0:
            continue
        t0, t1 = int(cu[n]), int(cu[n + 1])
        prev = np.asarray(conv_pool[s], dtype=F64).T if has_init[n] else np.zeros((K - 1, Cn))
        if parent is not None:
            for t in range(t0, t1):
                path = [t - t0]                                      # root path, newest first
                while int(parent[t0 + path[-1]]) >= 0:
                    path.append(int(parent[t0 + path[-1]]))
                win = np.concatenate([prev, x[[t0 + i for i in reversed(path)]]], axis=0)
                y = b + np.sum(win[len(win) - K:] * w.T, axis=0)
                out[t] = y / (1.0 + np.exp(-y)) if activation else y
            continue
        win = np.concatenate([prev, x[t0:t1]], axis=0)              # [K-1 + len, C]
        for t in range(t0, t1):
            i = t - t0
            y = b + np.sum(win[i:i + K] * w.T, axis=0)
            out[t] = y / (1.0 + np.exp(-y)) if activation else y
        states[s] = win[len(win) - (K - 1):].T.copy()               # [C, K-1]
    return out, states
