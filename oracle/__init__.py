"""CPU oracle for the GPT-2 training step.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may use this package; the product path never does.

`build()` compiles oracle/gpt2_oracle.c twice with gcc: in double precision
(the parity reference, `liboracle_f64.so`) and in single precision
(`liboracle_f32.so`, the fp32 step as a plain C program would run it).
`Oracle` wraps one model instance through ctypes.
"""
from .wrapper import Oracle, build, load, lib_path  # noqa: F401
