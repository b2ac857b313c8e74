"""Device-resident workloads of the verify step, built on the C ABI.

torch provides device memory, streams and the synthetic random draws; every
step of the verify path is a libvw4 call.
"""
from __future__ import annotations

import numpy as np

from . import binding as B

BYTES_PER_WEIGHT = 0.5 + 2.0 / 64.0  # int4 code + fp16 scale per 64


class W4Linear:
    """Packed W4 weights of an [N][K] linear layer, resident in HBM."""

    def __init__(self, packed, pscales, N: int, K: int):
        self.packed, self.pscales, self.N, self.K = packed, pscales, N, K

    @classmethod
    def from_fp32(cls, w, stream=None):
        N, K = w.shape
        packed, pscales = B.w4_quantize_packed(w, stream=stream)
        return cls(packed, pscales, N, K)

    @classmethod
    def random(cls, N: int, K: int, std: float, gen, device="cuda", chunk_rows: int = 8192):
        """~N(0, std) fp32 weights drawn on the device (seeded torch generator),
        quantised straight into the packed layout chunk by chunk."""
        import torch
        cb, sb = B.packed_sizes(N, K)
        packed = torch.empty(cb, dtype=torch.uint8, device=device)
        pscales = torch.empty(sb // 2, dtype=torch.int16, device=device)
        # quantise whole 64-row tiles per chunk so the packed offsets line up
        chunk_rows = max(64, chunk_rows // 64 * 64)
        for r0 in range(0, N, chunk_rows):
            rows = min(chunk_rows, N - r0)
            w = torch.randn((rows, K), generator=gen, device=device, dtype=torch.float32) * std
            t0 = r0 // 64
            ntile = (rows + 63) // 64
            sub_p = packed[t0 * K * 32: (t0 + ntile) * K * 32]
            sub_s = pscales[t0 * (K // 64) * 64: (t0 + ntile) * (K // 64) * 64]
            B.w4_quantize_packed(w, out=(sub_p, sub_s))
            del w
        return cls(packed, pscales, N, K)

    def nbytes(self) -> int:
        return int(self.N * self.K * BYTES_PER_WEIGHT)


class LMHeadVerify:
    """One verify step on an LM head: W4 GEMM of the M rows, temperature/top-p
    statistics, Leviathan–Chen acceptance.  All buffers are allocated once."""

    def __init__(self, V: int, d: int, M: int, device="cuda"):
        import torch
        self.V, self.d, self.M, self.D = V, d, M, M - 1
        self.logits = torch.empty((M, V), dtype=torch.float32, device=device)
        self.stats = torch.zeros(M * B.ROWSTAT_BYTES, dtype=torch.uint8, device=device)
        self.gemm_ws = B.workspace(B.gemm_workspace_bytes(M, V, d), device)
        self.stat_ws = B.workspace(B.verify_workspace_bytes(M, V), device)
        self.acc_ws = B.workspace(B.accept_workspace_bytes(1, V), device)
        self.tokens = torch.empty((1, M), dtype=torch.int32, device=device)
        self.n_acc = torch.empty(1, dtype=torch.int32, device=device)
        self.flags = torch.empty(1, dtype=torch.int32, device=device)

    def gemm(self, x, head: W4Linear, stream=None):
        B.w4_skinny_gemm(x, head.packed, head.pscales, self.logits, self.M, self.V, self.d, ws=self.gemm_ws,
                         stream=stream)

    def stats_and_accept(self, q, drafts, T: float, top_p: float, seed: int, step: int, stream=None,
                         tokens=None, n_acc=None, flags=None):
        B.verify_logits(None, None, None, self.M, self.V, self.d, T, top_p, self.logits, self.stats, self.stat_ws,
                        stream=stream)
        B.spec_accept(self.logits, 0, self.stats, 0, q, 0, drafts, 1, self.D, self.V, T, seed, step,
                      self.tokens if tokens is None else tokens, self.n_acc if n_acc is None else n_acc,
                      self.flags if flags is None else flags, self.acc_ws, stream=stream)

    def step(self, x, head: W4Linear, q, drafts, T, top_p, seed, step, stream=None, **out):
        self.gemm(x, head, stream)
        self.stats_and_accept(q, drafts, T, top_p, seed, step, stream, **out)
