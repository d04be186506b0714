"""CPU oracle for the QAD hot path (NVFP4 simulated quantization + KL loss).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product library
never loads it and shares no code with it.  The arithmetic lives in
``oracle.c`` (plain C, binary32 for the quantizer, binary64 for the KL loss);
this module compiles it with gcc and marshals numpy arrays through ctypes.
"""
from .oracle import *  # noqa: F401,F403
