"""fp64 CPU oracle for causal attention forward/backward.

TEST INFRASTRUCTURE ONLY: tests/, the smoke check and the benchmark's CPU
baseline may import this package; the product path (``bwd_head_rms_amd``)
never does.
"""
from .oracle import Oracle, OracleError, default  # noqa: F401
