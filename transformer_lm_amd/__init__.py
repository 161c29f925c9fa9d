"""GPT-2 training step (forward, hand-derived backward, AdamW) on MI355X.

The step runs in hand-written HIP kernels for gfx950 behind the C ABI declared
in include/gpt2.h (library: libgpt2.so, built from csrc/). The Python layer,
transformer_lm_amd.gpt2, only marshals arguments; PyTorch supplies device
memory and streams.

Importing this package does not load the native library; importing
transformer_lm_amd.gpt2 does, and fails loudly when it is missing.
"""
from .workloads import WORKLOADS, Workload, param_shapes, param_offsets  # noqa: F401
