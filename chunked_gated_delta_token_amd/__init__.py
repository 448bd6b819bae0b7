"""Fused chunk-local KKT + triangular solve of the chunked Gated DeltaNet
forward pass, for AMD Instinct MI355X (gfx950).

    from chunked_gated_delta_token_amd import kkt_solve
    X = kkt_solve(k, g, beta)          # [B, T, H, 64] rows of (I + A)^{-1}
    A = kkt_scaled_dot(k, g, beta)     # the unfused chain: A alone (fp32) ...
    X = kkt_solve_tril(A)              # ... then its solve
    X, g = kkt_solve_gate_cumsum(k, a, beta, return_gate=True)  # a: per-token log-decay

The computation is the HIP library ``libkkt_solve.so`` (C ABI in
``include/kkt_solve.h``); this package only marshals arguments.
"""
from .kkt import (KKTError, KKTInvalidArgument, KKTUnsupported,  # noqa: F401
                  chunk_gated_delta_rule_fwd_kkt_solve, chunk_scaled_dot_kkt_fwd,
                  kkt_scaled_dot, kkt_solve, kkt_solve_gate_cumsum, kkt_solve_tril, last_error, load_library,
                  solve_tril, version)
