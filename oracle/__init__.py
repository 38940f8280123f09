"""fp64 CPU oracle of the Gated DeltaNet layer (TEST INFRASTRUCTURE ONLY).

Only tests/, the smoke entry point and the benchmark's CPU-baseline leg may
import this package. The HIP product path never imports or calls it.

`gdn_oracle.c` holds the arithmetic (plain fp64 loops); `oracle.py` wraps it
with numpy arrays; `build.py` compiles it with gcc.
"""
from .oracle import (  # noqa: F401
    OracleParams, build_oracle, conv1d_silu, front_end, delta_rule, gdn_forward,
    verify_commit, set_mutation, mutation, MUTATIONS, default_threads, gate_beta, gated_rmsnorm,
)
