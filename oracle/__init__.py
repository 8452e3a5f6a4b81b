"""CPU oracle for MLA latent-KV attention (test infrastructure only).

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the HIP library or its Python binding.
"""
from .mla_oracle import *  # noqa: F401,F403
