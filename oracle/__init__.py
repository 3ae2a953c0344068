"""fp64 CPU oracle for the fused attention forward (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It wraps ``mfa_oracle.c`` (plain C, double precision) through
ctypes and shares no code with the HIP library.
"""
from .oracle import Oracle, build_oracle, default_oracle, ORACLE_DIR  # noqa: F401
