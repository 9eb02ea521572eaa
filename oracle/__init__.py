"""CPU oracle for the GDN (Gated DeltaNet) layer and its delta-off (Mamba2 SSD) mode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link or
execute this package: only the tests, the graft entry's smoke check and the
bench's CPU-baseline leg use it.  It shares no code with the HIP library or its
Python binding and imports neither.

It is the plain definition, token by token, in float64 (inputs stored as bf16 or
fp32 are widened exactly).  The chunked GPU algorithm is an exact re-association
of the same recurrence, so the oracle is the definition, not the algorithm.

Sources.  The pages call the expected output a "pure-PyTorch gated-delta
recurrence reference" (SGLang GDN test-matrix article, framerc.cn, section
"GDN hybrid linear attention & test positioning") without writing it out; the
recurrence, gate and normalisation are those of the published gated delta rule
(Yang, Kautz & Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with Delta
Rule", ICLR 2025, the gated delta rule and its gate parameterisation):

    S_t = g_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
    o_t = scale * S_t q_t        (q, k L2-normalised per head)
    g_t = exp(-exp(A_log) * softplus(a_t + dt_bias)),  beta_t = sigmoid(b_t)

The delta-off mode follows the parameter list of the flashinfer page
"flashinfer.mamba.ssd_combined_fwd" (x, dt, A, B, C, D, z, dt_bias, dt_softplus,
dt_limit, initial_states, return_final_states).

Parity pins: every function here is pinned by tests in tests/test_oracle_pins.py
(closed forms, brute force, exact rational arithmetic, invariants).  No function
is "parity unpinned".
"""
from .gdn import (softplus, sigmoid, gdn_gate, ssd_gate, l2_normalize, gdn_extend,
                  gdn_decode, apply_final_states, ssd_combined, causal_conv1d)

__all__ = ["softplus", "sigmoid", "gdn_gate", "ssd_gate", "l2_normalize", "gdn_extend",
           "gdn_decode", "apply_final_states", "ssd_combined", "causal_conv1d"]
