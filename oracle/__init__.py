"""CPU oracle of the VAR-Q packed KV-cache path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package; the GPU library never does.
"""
from . import varq_oracle  # noqa: F401
