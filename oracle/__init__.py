"""float64 CPU oracle for the KDA forward -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the cpu_baseline leg of bench.py may
import this package.  It wraps ``kda_oracle.c`` (plain C, compiled with gcc) and
shares nothing with the HIP library in ``gated_delta_rule_log2_amd``.
"""
from .kda_oracle import (  # noqa: F401
    GATE_LOWER_BOUND,
    GATE_PRE,
    GATE_SOFTPLUS,
    BETA_AS_GIVEN,
    BETA_SIGMOID,
    BETA_TWO_SIGMOID,
    build_oracle,
    load_oracle,
    oracle_fwd,
    oracle_gate_cumsum,
    oracle_num_threads,
)
