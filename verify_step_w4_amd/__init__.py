"""verify_step_w4_amd — batched verify step of MTP self-speculative decoding on MI355X.

The compute path is the HIP library libvw4.so (C ABI in include/vw4.h):
W4 skinny GEMM, verify_logits (LM head + temperature/top-p statistics) and
spec_accept (Leviathan–Chen acceptance with residual resampling and a bonus
token).  ``binding`` is the thin ctypes layer over it; ``synth`` draws the
seeded synthetic workloads.
"""
from . import binding  # noqa: F401

__all__ = ["binding"]
