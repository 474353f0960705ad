"""CPU oracle for the Prox sparse SwiGLU decode step (test infrastructure only).

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the product library or its binding.
"""
from .prox_oracle import *  # noqa: F401,F403
