"""fp64 CPU oracles: causal attention forward/backward, the per-head RMS
QK-norm + RoPE step with its backward, and decode attention.

TEST INFRASTRUCTURE ONLY: tests/, the smoke check and the benchmark's CPU
baseline may import this package; the product path (``bwd_head_rms_amd``)
never does.
"""
from .decode_oracle import DecodeOracle, default_decode  # noqa: F401
from .norm_oracle import NormOracle, default_norm  # noqa: F401
from .oracle import Oracle, OracleError, default  # noqa: F401
