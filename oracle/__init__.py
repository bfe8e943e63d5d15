"""CPU oracle for the Transformer-XL relative-attention hot path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its Python binding.
"""
from .oracle import *  # noqa: F401,F403
from . import brute  # noqa: F401
from . import backward  # noqa: F401
