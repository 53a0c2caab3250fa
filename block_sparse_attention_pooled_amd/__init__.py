"""MI355X-native pooled block-sparse attention for diffusion-LLM denoising.

The computation lives in the HIP library ``libstepdllm.so`` (C ABI in
``include/stepdllm.h``); ``binding`` is its thin ctypes layer and ``inputs``
the seeded synthetic workloads.
"""
from . import binding  # noqa: F401
