"""fp64 CPU oracle for KSA attention and its KV cache (test infrastructure only).

Only ``tests/``, the package's ``smoke()`` check and the benchmark's CPU-baseline
leg may import this package; the HIP library never does.
"""
from .ksa_oracle import *  # noqa: F401,F403
