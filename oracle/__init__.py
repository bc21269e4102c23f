"""CPU oracle for the KV-block codec and relative RoPE shift.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.  It shares no
code with the HIP library.
"""
from .hkv_oracle import *  # noqa: F401,F403
from . import hkv_oracle  # noqa: F401
