"""CPU oracle for the MSA hot path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python
binding) never imports, links or calls anything here.
"""
from .msa_oracle import *  # noqa: F401,F403
