"""CPU oracle of the Kimi Delta Attention (KDA) core -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import, call, link or run anything in this package. The GPU library
(linear_attention_05_amd) never does; the two share no code.

Contents:
  recurrence  fp64 token-by-token recurrence in plain C (kda_oracle.c) via ctypes:
              the definition S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1}
              + beta_t k_t v_t^T, o_t = S_t^T q_t, with optional initial state,
              final state and periodic state checkpoints; plus the decode step.
  chunked     fp64 NumPy chunked formulation (UT-transform form) of the same map.
  brute       exact-rational brute force with explicit transition matrices.

Pins (tests/test_oracle.py): state unchanged for alpha = 1, beta = 0; closed
form of pure decay; exact retrieval S_t^T k_t = v_t for beta = 1 and unit
keys; closed form for one-hot keys; exact rationals; joint linearity in
(V, S_0); chunked == recurrence; packing, column-block, thread-count,
decode-step, checkpoint and resume invariances.
"""
