"""Infini-attention layer forward for MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``libinfini_attn.so``, built by ``build.py``); ``binding`` wraps it for torch tensors.
``workloads`` generates the seeded synthetic inputs.
"""

__all__ = ["binding", "workloads", "build"]
