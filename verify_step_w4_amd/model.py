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

    # the interface every weight format's matrix offers the decoder
    def partials(self, x, part, M: int, stream=None):
        B.w4_skinny_gemm_partials(x, self.packed, self.pscales, part, M, self.N, self.K, stream)

    def partials_layout(self, M: int):
        return B.gemm_partials_layout(M, self.N, self.K)

    def gemm(self, x, y, M: int, ws=None, stream=None):
        B.w4_skinny_gemm(x, self.packed, self.pscales, y, M, self.N, self.K, ws=ws, stream=stream)

    def workspace_bytes(self, M: int) -> int:
        return B.gemm_workspace_bytes(M, self.N, self.K)

    def swiglu(self, x, a, M: int, stream=None):
        """a[:M][:N/2] = bf16(silu(gate) * up): this matrix holds gate/up-interleaved rows (B.interleave_gate_up)."""
        B.w4_skinny_gemm_swiglu(x, self.packed, self.pscales, a, a.stride(0), M, self.N // 2, self.K, stream)

    def nbytes(self) -> int:
        return int(self.N * self.K * BYTES_PER_WEIGHT)


class _TwoPlaneOps:
    """The decoder interface of the two-plane formats (hi, lo planes and packed
    scales), through the binding's calls named after _FMT."""
    _FMT = ""

    def partials(self, x, part, M: int, stream=None):
        getattr(B, f"{self._FMT}_skinny_gemm_partials")(x, self.hi, self.lo, self.pscales, part, M, self.N, self.K,
                                                         stream)

    def partials_layout(self, M: int):
        return getattr(B, f"{self._FMT}_partials_layout")(M, self.N, self.K)

    def gemm(self, x, y, M: int, ws=None, stream=None):
        getattr(B, f"{self._FMT}_skinny_gemm")(x, self.hi, self.lo, self.pscales, y, M, self.N, self.K, ws=ws,
                                               stream=stream)

    def workspace_bytes(self, M: int) -> int:
        return getattr(B, f"{self._FMT}_workspace_bytes")(M, self.N, self.K)

    def swiglu(self, x, a, M: int, stream=None):
        B.two_plane_gemm_swiglu(self._FMT, x, self.hi, self.lo, self.pscales, a, a.stride(0), M, self.N // 2, self.K,
                                stream)


class W8Linear(_TwoPlaneOps):
    """A [N][K] matrix in the W8 format (int8 codes, fp16 scale per 64 K), kept
    as its two packed nibble planes and the packed scales."""
    _FMT = "w8"

    def __init__(self, hi, lo, pscales, N: int, K: int):
        self.hi, self.lo, self.pscales, self.N, self.K = hi, lo, pscales, N, K

    @classmethod
    def from_codes(cls, codes, scales, stream=None):
        """codes: uint8 device [N][K] (c + 128); scales: int16 device [N][K/64] (fp16 bits)."""
        import torch
        N, K = codes.shape
        cb, sb = B.packed_sizes(N, K)
        hi = torch.empty(cb, dtype=torch.uint8, device=codes.device)
        lo = torch.empty(cb, dtype=torch.uint8, device=codes.device)
        ps = torch.empty(sb // 2, dtype=torch.int16, device=codes.device)
        B.w8_pack(codes, scales, N, K, hi, lo, ps, stream)
        return cls(hi, lo, ps, N, K)

    @classmethod
    def from_fp32(cls, w, device="cuda"):
        """w: fp32 [N][K] (numpy or torch); quantised by the library's host quantiser."""
        import torch
        wn = w.detach().cpu().numpy() if hasattr(w, "detach") else w
        codes, scales = B.w8_quantize_host(wn)
        return cls.from_codes(torch.from_numpy(codes).to(device), torch.from_numpy(scales.view("int16")).to(device))

    @classmethod
    def random(cls, N: int, K: int, gen, device="cuda"):
        """Uniform codes in [-127, 127] and fp16 scales in [1e-4, 3e-4] (timing inputs)."""
        import torch
        codes = torch.randint(1, 256, (N, K), generator=gen, device=device, dtype=torch.int32).to(torch.uint8)
        scales = (1e-4 + 2e-4 * torch.rand((N, K // 64), generator=gen, device=device)).to(torch.float16)
        return cls.from_codes(codes, scales.view(torch.int16))

    def nbytes(self) -> int:
        return self.N * self.K + self.N * (self.K // 64) * 2


class W16Linear:
    """A [N][K] matrix of unquantised 16-bit float weights (kind "f16": fp16,
    "bf16": bf16) in the operand-tiled layout; no scales."""

    def __init__(self, packed, N: int, K: int, kind: str):
        self.packed, self.N, self.K, self.kind = packed, N, K, kind

    @classmethod
    def from_bits(cls, w, kind: str, stream=None):
        """w: int16/uint16-bit device tensor [N][K] of fp16 or bf16 bit patterns."""
        import torch
        N, K = w.shape
        packed = torch.empty(int(B.lib().vw4_w16_packed_bytes(N, K)), dtype=torch.uint8, device=w.device)
        B.w16_pack(w, N, K, packed, stream)
        return cls(packed, N, K, kind)

    @classmethod
    def random(cls, N: int, K: int, gen, kind: str, device="cuda"):
        """N(0, 0.02) weights rounded to the kind's type (timing inputs)."""
        import torch
        dt = torch.float16 if kind == "f16" else torch.bfloat16
        w = (0.02 * torch.randn((N, K), generator=gen, device=device)).to(dt).view(torch.int16)
        return cls.from_bits(w, kind)

    @classmethod
    def from_fp32(cls, w, kind: str, device="cuda"):
        """fp32 weights rounded to the kind's type (round to nearest even) and packed."""
        import torch
        wt = w.detach() if hasattr(w, "detach") else torch.from_numpy(w)
        dt = torch.float16 if kind == "f16" else torch.bfloat16
        return cls.from_bits(wt.to(device).to(dt).view(torch.int16), kind)

    def partials(self, x, part, M: int, stream=None):
        B.w16_skinny_gemm_partials(x, self.packed, part, M, self.N, self.K, kind=self.kind, stream=stream)

    def partials_layout(self, M: int):
        return B.w16_partials_layout(M, self.N, self.K, self.kind)

    def gemm(self, x, y, M: int, ws=None, stream=None):
        B.w16_skinny_gemm(x, self.packed, y, M, self.N, self.K, kind=self.kind, ws=ws, stream=stream)

    def workspace_bytes(self, M: int) -> int:
        return B.w16_workspace_bytes(M, self.N, self.K, self.kind)

    def swiglu(self, x, a, M: int, stream=None):
        B.w16_skinny_gemm_swiglu(x, self.packed, a, a.stride(0), M, self.N // 2, self.K, kind=self.kind, stream=stream)

    def nbytes(self) -> int:
        return self.N * self.K * 2


class W3Linear(_TwoPlaneOps):
    """A [N][K] matrix in the W3 format (3-bit codes, fp16 scale per 64 K): the
    1-bit high plane, the 2-bit low plane and the packed scales."""
    _FMT = "w3"

    def __init__(self, hi, lo, pscales, N: int, K: int):
        self.hi, self.lo, self.pscales, self.N, self.K = hi, lo, pscales, N, K

    @classmethod
    def from_codes(cls, codes, scales, stream=None):
        """codes: uint8 device [N][K] (c + 4); scales: int16 device [N][K/64] (fp16 bits)."""
        import torch
        N, K = codes.shape
        _, sb = B.packed_sizes(N, K)
        cb = int(B.lib().vw4_w3_lo_plane_bytes(N, K))
        hb = int(B.lib().vw4_w3_hi_plane_bytes(N, K))
        hi = torch.empty(hb, dtype=torch.uint8, device=codes.device)
        lo = torch.empty(cb, dtype=torch.uint8, device=codes.device)
        ps = torch.empty(sb // 2, dtype=torch.int16, device=codes.device)
        B.w3_pack(codes, scales, N, K, hi, lo, ps, stream)
        return cls(hi, lo, ps, N, K)

    @classmethod
    def from_fp32(cls, w, device="cuda"):
        import torch
        wn = w.detach().cpu().numpy() if hasattr(w, "detach") else w
        codes, scales = B.w3_quantize_host(wn)
        return cls.from_codes(torch.from_numpy(codes).to(device), torch.from_numpy(scales.view("int16")).to(device))

    @classmethod
    def random(cls, N: int, K: int, gen, device="cuda"):
        """Uniform codes in [-3, 3] and fp16 scales in [4e-4, 1.2e-3] (timing inputs)."""
        import torch
        codes = torch.randint(1, 8, (N, K), generator=gen, device=device, dtype=torch.int32).to(torch.uint8)
        scales = (4e-4 + 8e-4 * torch.rand((N, K // 64), generator=gen, device=device)).to(torch.float16)
        return cls.from_codes(codes, scales.view(torch.int16))

    def nbytes(self) -> int:
        return self.N * self.K * 3 // 8 + self.N * (self.K // 64) * 2


class W2Linear:
    """A [N][K] matrix in the W2 format (2-bit codes, fp16 scale per 64 K): one
    2-bit plane and the packed scales."""

    def __init__(self, packed, pscales, N: int, K: int):
        self.packed, self.pscales, self.N, self.K = packed, pscales, N, K

    @classmethod
    def from_codes(cls, codes, scales, stream=None):
        """codes: uint8 device [N][K] (c + 1); scales: int16 device [N][K/64] (fp16 bits)."""
        import torch
        N, K = codes.shape
        _, sb = B.packed_sizes(N, K)
        pb = int(B.lib().vw4_w2_packed_bytes(N, K))
        packed = torch.empty(pb, dtype=torch.uint8, device=codes.device)
        ps = torch.empty(sb // 2, dtype=torch.int16, device=codes.device)
        B.w2_pack(codes, scales, N, K, packed, ps, stream)
        return cls(packed, ps, N, K)

    @classmethod
    def from_fp32(cls, w, device="cuda"):
        import torch
        wn = w.detach().cpu().numpy() if hasattr(w, "detach") else w
        codes, scales = B.w2_quantize_host(wn)
        return cls.from_codes(torch.from_numpy(codes).to(device), torch.from_numpy(scales.view("int16")).to(device))

    @classmethod
    def random(cls, N: int, K: int, gen, device="cuda"):
        """Uniform codes in [-1, 1] and fp16 scales in [4e-4, 1.2e-3] (timing inputs)."""
        import torch
        codes = torch.randint(0, 3, (N, K), generator=gen, device=device, dtype=torch.int32).to(torch.uint8)
        scales = (4e-4 + 8e-4 * torch.rand((N, K // 64), generator=gen, device=device)).to(torch.float16)
        return cls.from_codes(codes, scales.view(torch.int16))

    def partials(self, x, part, M: int, stream=None):
        B.w2_skinny_gemm_partials(x, self.packed, self.pscales, part, M, self.N, self.K, stream)

    def partials_layout(self, M: int):
        return B.w2_partials_layout(M, self.N, self.K)

    def gemm(self, x, y, M: int, ws=None, stream=None):
        B.w2_skinny_gemm(x, self.packed, self.pscales, y, M, self.N, self.K, ws=ws, stream=stream)

    def workspace_bytes(self, M: int) -> int:
        return B.w2_workspace_bytes(M, self.N, self.K)

    def swiglu(self, x, a, M: int, stream=None):
        B.w2_skinny_gemm_swiglu(x, self.packed, self.pscales, a, a.stride(0), M, self.N // 2, self.K, stream)

    def nbytes(self) -> int:
        return self.N * self.K // 4 + self.N * (self.K // 64) * 2


class W5Linear(_TwoPlaneOps):
    """A [N][K] matrix in the W5 format (5-bit codes, fp16 scale per 64 K): the
    1-bit high plane, the 4-bit low plane (W4 layout) and the packed scales."""
    _FMT = "w5"

    def __init__(self, hi, lo, pscales, N: int, K: int):
        self.hi, self.lo, self.pscales, self.N, self.K = hi, lo, pscales, N, K

    @classmethod
    def from_codes(cls, codes, scales, stream=None):
        """codes: uint8 device [N][K] (c + 16); scales: int16 device [N][K/64] (fp16 bits)."""
        import torch
        N, K = codes.shape
        cb, sb = B.packed_sizes(N, K)
        hb = int(B.lib().vw4_w5_hi_plane_bytes(N, K))
        hi = torch.empty(hb, dtype=torch.uint8, device=codes.device)
        lo = torch.empty(cb, dtype=torch.uint8, device=codes.device)
        ps = torch.empty(sb // 2, dtype=torch.int16, device=codes.device)
        B.w5_pack(codes, scales, N, K, hi, lo, ps, stream)
        return cls(hi, lo, ps, N, K)

    @classmethod
    def from_fp32(cls, w, device="cuda"):
        import torch
        wn = w.detach().cpu().numpy() if hasattr(w, "detach") else w
        codes, scales = B.w5_quantize_host(wn)
        return cls.from_codes(torch.from_numpy(codes).to(device), torch.from_numpy(scales.view("int16")).to(device))

    @classmethod
    def random(cls, N: int, K: int, gen, device="cuda"):
        """Uniform codes in [-15, 15] and fp16 scales in [4e-4, 1.2e-3] (timing inputs)."""
        import torch
        codes = torch.randint(1, 32, (N, K), generator=gen, device=device, dtype=torch.int32).to(torch.uint8)
        scales = (4e-4 + 8e-4 * torch.rand((N, K // 64), generator=gen, device=device)).to(torch.float16)
        return cls.from_codes(codes, scales.view(torch.int16))

    def nbytes(self) -> int:
        return self.N * self.K * 5 // 8 + self.N * (self.K // 64) * 2


class W6Linear(_TwoPlaneOps):
    """A [N][K] matrix in the W6 format (6-bit codes, fp16 scale per 64 K): the
    2-bit high plane, the 4-bit low plane (W4 layout) and the packed scales."""
    _FMT = "w6"

    def __init__(self, hi, lo, pscales, N: int, K: int):
        self.hi, self.lo, self.pscales, self.N, self.K = hi, lo, pscales, N, K

    @classmethod
    def from_codes(cls, codes, scales, stream=None):
        """codes: uint8 device [N][K] (c + 32); scales: int16 device [N][K/64] (fp16 bits)."""
        import torch
        N, K = codes.shape
        cb, sb = B.packed_sizes(N, K)
        hb = int(B.lib().vw4_w6_hi_plane_bytes(N, K))
        hi = torch.empty(hb, dtype=torch.uint8, device=codes.device)
        lo = torch.empty(cb, dtype=torch.uint8, device=codes.device)
        ps = torch.empty(sb // 2, dtype=torch.int16, device=codes.device)
        B.w6_pack(codes, scales, N, K, hi, lo, ps, stream)
        return cls(hi, lo, ps, N, K)

    @classmethod
    def from_fp32(cls, w, device="cuda"):
        import torch
        wn = w.detach().cpu().numpy() if hasattr(w, "detach") else w
        codes, scales = B.w6_quantize_host(wn)
        return cls.from_codes(torch.from_numpy(codes).to(device), torch.from_numpy(scales.view("int16")).to(device))

    @classmethod
    def random(cls, N: int, K: int, gen, device="cuda"):
        """Uniform codes in [-31, 31] and fp16 scales in [4e-4, 1.2e-3] (timing inputs)."""
        import torch
        codes = torch.randint(1, 64, (N, K), generator=gen, device=device, dtype=torch.int32).to(torch.uint8)
        scales = (4e-4 + 8e-4 * torch.rand((N, K // 64), generator=gen, device=device)).to(torch.float16)
        return cls.from_codes(codes, scales.view(torch.int16))

    def nbytes(self) -> int:
        return self.N * self.K * 3 // 4 + self.N * (self.K // 64) * 2


# the quantised formats whose matrices come from (N, K, gen, device) random draws
LINEAR_FORMATS = {"w8": W8Linear, "w6": W6Linear, "w5": W5Linear, "w3": W3Linear, "w2": W2Linear}
WEIGHT_FORMATS = ("w4", "w8", "w6", "w5", "w3", "w2", "f16", "bf16")


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


# ---------------------------------------------------------------------------
# Full verify forward of a dense decoder (synthetic weights)
# ---------------------------------------------------------------------------
DENSE_27B = dict(d=5120, nq=40, nkv=8, hd=128, F=17408, layers=64, V=151936, eps=1e-6, theta=10000.0)


class Decoder:
    """Pre-norm dense decoder with GQA attention and a SwiGLU FFN, every linear
    a skinny GEMM in one weight format (fmt, one of WEIGHT_FORMATS).  In every
    format the gate|up matrix is in the gate/up-interleaved row order of
    B.interleave_gate_up, with the SwiGLU in that GEMM's epilogue.  One call of ``forward`` scores M rows at positions
    L .. L+M-1 (the verify pass); M = 1 is an autoregressive step.  Weights,
    KV caches and activation buffers are allocated once (device-resident)."""

    def __init__(self, cfg: dict, M_max: int, Lmax: int, gen=None, device="cuda", weights=None,
                 kv_fill: bool = True, fmt: str = "w4"):
        import torch
        self.cfg = dict(cfg)
        c = self.cfg
        Lmax = (Lmax + 31) // 32 * 32                  # the value cache is stored in 32-position blocks
        self.M_max, self.Lmax, self.device = M_max, Lmax, device
        d, nq, nkv, hd, F, nl, V = c["d"], c["nq"], c["nkv"], c["hd"], c["F"], c["layers"], c["V"]
        self.nqkv = (nq + 2 * nkv) * hd
        self.shapes = {"qkv": (self.nqkv, d), "o": (d, nq * hd), "gate_up": (2 * F, d), "down": (d, F)}
        if weights is None:
            weights = self.random_weights(cfg, gen, device, fmt)
        self.layers = weights["layers"]
        self.final_gamma = weights["final_gamma"]
        self.lm_head = weights["lm_head"]
        # KV caches bf16: keys [layer][nkv][Lmax][hd], values in 32-position
        # blocks [layer][nkv][Lmax / 32][hd][32]; synthetic N(0,1) context
        self.Kc, self.Vc = [], []
        for _ in range(nl):
            if kv_fill:
                k = torch.randn((nkv, Lmax, hd), generator=gen, device=device).to(torch.bfloat16).view(torch.int16)
                v = torch.randn((nkv, Lmax // 32, hd, 32), generator=gen,
                                device=device).to(torch.bfloat16).view(torch.int16)
            else:
                k = torch.zeros((nkv, Lmax, hd), dtype=torch.int16, device=device)
                v = torch.zeros((nkv, Lmax // 32, hd, 32), dtype=torch.int16, device=device)
            self.Kc.append(k)
            self.Vc.append(v)
        # activation buffers
        i16 = torch.int16
        # two residual buffers: the one-launch add + RMSNorm writes the new
        # residual out of place
        self.resid = torch.empty((M_max, d), dtype=i16, device=device)
        self.resid2 = torch.empty((M_max, d), dtype=i16, device=device)
        self.h = torch.empty((M_max, d), dtype=i16, device=device)
        self.q = torch.empty((M_max, nq, hd), dtype=i16, device=device)
        self.attn = torch.empty((M_max, nq * hd), dtype=i16, device=device)
        self.a = torch.empty((M_max, F), dtype=i16, device=device)
        self.parts = {}
        for name in self.shapes:
            S, ldp = self.layers[0][name].partials_layout(M_max)
            self.parts[name] = torch.empty(S * ldp * M_max, dtype=torch.float32, device=device)
        self.attn_ws = B.workspace(B.attn_workspace_bytes(M_max, nq, nkv, hd, Lmax), device)
        self.norm_ws = B.workspace(B.norm_workspace_bytes(M_max, d), device)
        self.logits = torch.empty((M_max, V), dtype=torch.float32, device=device)
        self.lm_ws = B.workspace(self.lm_head.workspace_bytes(M_max), device)

    @staticmethod
    def random_weights(cfg: dict, gen, device="cuda", fmt: str = "w4"):
        """W4: ~N(0, 0.02) fp32 weights drawn on the device and quantised; W8:
        uniform int8 codes with fp16 scales in [1e-4, 3e-4] (the same spread);
        W6, W5, W3, W2: uniform codes with fp16 scales in [4e-4, 1.2e-3]; f16,
        bf16: N(0, 0.02) rounded to the type.  RMSNorm gains ~N(1, 0.02) in
        bf16.  The gate|up matrices are random draws, so their row order is
        immaterial; weights from a checkpoint would be interleaved with
        B.interleave_gate_up before packing."""
        import torch
        d, nq, nkv, hd, F, nl, V = (cfg[k] for k in ("d", "nq", "nkv", "hd", "F", "layers", "V"))
        nqkv = (nq + 2 * nkv) * hd

        def gamma():
            return (1.0 + 0.02 * torch.randn(d, generator=gen, device=device)).to(torch.bfloat16).view(torch.int16)

        def lin(N, K):
            if fmt == "w4":
                return W4Linear.random(N, K, 0.02, gen, device)
            if fmt in ("f16", "bf16"):
                return W16Linear.random(N, K, gen, fmt, device)
            return LINEAR_FORMATS[fmt].random(N, K, gen, device)

        layers = []
        for _ in range(nl):
            layers.append(dict(qkv=lin(nqkv, d), o=lin(d, nq * hd), gate_up=lin(2 * F, d), down=lin(d, F),
                               g1=gamma(), g2=gamma()))
        return dict(layers=layers, final_gamma=gamma(), lm_head=lin(V, d))

    def weight_bytes(self) -> int:
        n = sum(l[k].nbytes() for l in self.layers for k in ("qkv", "o", "gate_up", "down"))
        return n + self.lm_head.nbytes()

    def kv_bytes(self, L: int, M: int) -> int:
        c = self.cfg
        return c["layers"] * 2 * c["nkv"] * (L + M) * c["hd"] * 2

    def forward(self, x, L: int, M: int, stream=None, gemm_hook=None):
        """x: int16 (bf16 bits) [M][d] hidden rows; fills self.logits[:M].
        gemm_hook(when, name), if given, is called right before ("pre") and
        after ("post") each W4 GEMM launch (used to time the GEMMs in place)."""
        hook = gemm_hook or (lambda when, name: None)
        c = self.cfg
        d, nq, nkv, hd, F, eps = c["d"], c["nq"], c["nkv"], c["hd"], c["F"], c["eps"]
        assert 1 <= M <= self.M_max and L + M <= self.Lmax
        h = self.h[:M]
        bufs = (self.resid[:M], self.resid2[:M])
        cur = [x[:M], 0]                 # current residual rows, next output buffer

        def add_norm(part, S, ldp, gamma):
            """resid <- resid + sum of the partials; h <- rmsnorm(resid) * gamma."""
            out = bufs[cur[1]]
            if d % 4 == 0 and d <= 8192 and (part is None or (S <= 8 and ldp % 4 == 0)):
                B.add_rmsnorm_out(cur[0], part, S, ldp, gamma, eps, M, d, out, h, stream)
            else:
                out.copy_(cur[0])
                B.add_rmsnorm(out, part, S, ldp, gamma, eps, M, d, h, self.norm_ws, stream)
            cur[0], cur[1] = out, 1 - cur[1]

        lay = self.layers
        add_norm(None, 1, d, lay[0]["g1"])
        for li, W in enumerate(lay):
            # attention block
            N, K = self.shapes["qkv"]
            hook("pre", "qkv")
            S, ldp = self._partials(W, "qkv", h, M, stream)
            hook("post", "qkv")
            B.rope_kv_append(self.parts["qkv"], S, ldp, M, nq, nkv, hd, L, c["theta"], self.q, self.Kc[li],
                             self.Vc[li], self.Lmax, stream)
            B.decode_attn(self.q, self.Kc[li], self.Vc[li], self.Lmax, L, M, nq, nkv, hd, self.attn, self.attn_ws,
                          stream)
            hook("pre", "o")
            S, ldp = self._partials(W, "o", self.attn[:M], M, stream)
            hook("post", "o")
            add_norm(self.parts["o"], S, ldp, W["g2"])
            # FFN block: gate|up with the SwiGLU in the GEMM epilogue
            N, K = self.shapes["gate_up"]
            hook("pre", "gate_up")
            W["gate_up"].swiglu(h, self.a, M, stream)
            hook("post", "gate_up")
            hook("pre", "down")
            S, ldp = self._partials(W, "down", self.a[:M], M, stream)
            hook("post", "down")
            g_next = lay[li + 1]["g1"] if li + 1 < len(lay) else self.final_gamma
            add_norm(self.parts["down"], S, ldp, g_next)
        self.last_resid = cur[0]         # residual rows after the last layer (before the final norm)
        hook("pre", "lm_head")
        self._lm_head(h, M, stream)
        hook("post", "lm_head")
        return self.logits[:M]

    def _partials(self, W, name, x, M, stream):
        """Split-K partial sums of linear `name` into self.parts[name]; returns (S, ldp)."""
        lin = W[name]
        lin.partials(x, self.parts[name], M, stream)
        return lin.partials_layout(M)

    def _lm_head(self, h, M, stream):
        self.lm_head.gemm(h, self.logits[:M], M, ws=self.lm_ws, stream=stream)

    def gemm_pass(self, M: int, stream=None, names=("qkv", "o", "gate_up", "down", "lm_head")):
        """Only the W4 GEMM launches of one forward (same shapes, weights and
        buffers, in the same order; optionally only the named linears), for
        timing the GEMM kernel by itself.  Returns the launch count."""
        c = self.cfg
        eps, F = c["eps"], c["F"]
        n = 0
        for W in self.layers:
            for name in ("qkv", "o", "gate_up", "down"):
                if name not in names:
                    continue
                N, K = self.shapes[name]
                if name == "gate_up":
                    W[name].swiglu(self.h[:M], self.a, M, stream)
                else:
                    x = {"qkv": self.h, "o": self.attn, "gate_up": self.h, "down": self.a}[name]
                    self._partials(W, name, x[:M], M, stream)
                n += 1
        if "lm_head" in names:
            self._lm_head(self.h[:M], M, stream)
            n += 1
        return n

    def gemm_alg_bytes(self, M: int) -> int:
        """Algorithmic bytes of one forward's GEMMs: each weight (code + scale,
        or 16-bit weight) once, activations in, fp32 outputs out (gate|up: the
        bf16 SwiGLU of its epilogue)."""
        c = self.cfg
        tot = 0.0
        for name, (N, K) in self.shapes.items():
            # SwiGLU epilogue output (bf16) of gate|up, fp32 partial sums otherwise
            out = M * (N // 2) * 2 if name == "gate_up" else M * N * 4
            tot += sum(l[name].nbytes() for l in self.layers) + c["layers"] * (M * K * 2 + out)
        tot += self.lm_head.nbytes() + M * c["d"] * 2 + M * c["V"] * 4
        return int(tot)


class VerifyStep:
    """Decoder forward over the M = D + 1 verify rows, then the temperature /
    top-p statistics and Leviathan–Chen acceptance (D = 0: one plain
    autoregressive sampling step)."""

    def __init__(self, dec: Decoder, M: int):
        import torch
        self.dec, self.M, self.D = dec, M, M - 1
        V = dec.cfg["V"]
        dev = dec.device
        self.stats = torch.zeros(M * B.ROWSTAT_BYTES, dtype=torch.uint8, device=dev)
        self.stat_ws = B.workspace(B.verify_workspace_bytes(M, V), dev)
        self.acc_ws = B.workspace(B.accept_workspace_bytes(1, V), dev)
        # tokens [1][M], n_acc and flags in one int32 block: one copy reads a
        # step's outputs
        self.outputs = torch.empty(M + 2, dtype=torch.int32, device=dev)
        self.tokens = self.outputs[:M].view(1, M)
        self.n_acc = self.outputs[M:M + 1]
        self.flags = self.outputs[M + 1:M + 2]

    def run_graphable(self, x, L: int, q, drafts, T: float, top_p: float, seed: int, step_dev, stream=None):
        """The same step with the Philox step read from device memory and
        advanced by one at the end, so the sequence can be captured once and
        replayed (each replay is a new verify step)."""
        dec, M, V = self.dec, self.M, self.dec.cfg["V"]
        logits = dec.forward(x, L, M, stream)
        B.verify_logits(None, None, None, M, V, dec.cfg["d"], T, top_p, logits, self.stats, self.stat_ws,
                        stream=stream)
        B.spec_accept_ex(logits, 0, self.stats, 0, q, 0, drafts, 1, self.D, V, T, seed, step_dev, self.tokens,
                         self.n_acc, self.flags, self.acc_ws, stream=stream)
        B.step_advance(step_dev, 1, stream)

    def capture(self, x, L: int, q, drafts, T: float, top_p: float, seed: int, step_dev):
        """Record the verify step into a HIP graph (torch.cuda.CUDAGraph) on a
        side stream; replay() then re-issues every kernel with one launch."""
        import torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.run_graphable(x, L, q, drafts, T, top_p, seed, step_dev)  # warm (plans, code objects)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run_graphable(x, L, q, drafts, T, top_p, seed, step_dev)
        torch.cuda.synchronize()
        return g

    def run(self, x, L: int, q, drafts, T: float, top_p: float, seed: int, step: int, stream=None, gemm_hook=None,
            **out):
        dec, M, V = self.dec, self.M, self.dec.cfg["V"]
        logits = dec.forward(x, L, M, stream, gemm_hook=gemm_hook)
        B.verify_logits(None, None, None, M, V, dec.cfg["d"], T, top_p, logits, self.stats, self.stat_ws,
                        stream=stream)
        B.spec_accept(logits, 0, self.stats, 0, q, 0, drafts, 1, self.D, V, T, seed, step,
                      out.get("tokens", self.tokens), out.get("n_acc", self.n_acc), out.get("flags", self.flags),
                      self.acc_ws, stream=stream)
        return self.tokens, self.n_acc, self.flags


# ---------------------------------------------------------------------------
# The draft side and the closed cycle: MTP head -> verify -> accept
# ---------------------------------------------------------------------------
class MTPHead:
    """The drafter: the MTP head of the same checkpoint (hazakura.dev mtplx page,
    section "4層のアーキテクチャ", Layers 0-2).  The pages do not describe its
    inside; this is the common MTP head: the hidden row h of the last processed
    position and the embedding of the next token, each RMS-normalised with its
    own gain and concatenated, a W4 projection from 2d back to d, one decoder
    layer (own KV cache), the final norm and the target's LM head -- or, with
    ``lm_head`` given, a draft-only head (the pages' draft-only 4-bit LM head
    beside a higher-precision target head).  One ``draft`` call is one depth:
    its output row and drawn token feed the next."""

    def __init__(self, target: "Decoder", embed, gen=None, weights=None, kv_fill: bool = True, lm_head=None):
        import torch
        cfg = dict(target.cfg, layers=1)
        d, V = cfg["d"], cfg["V"]
        dev = target.device
        if weights is None:
            weights = self.random_weights(cfg, gen, dev)
        self.cfg, self.embed = cfg, embed
        self.gamma_h, self.gamma_e, self.proj = weights["gamma_h"], weights["gamma_e"], weights["proj"]
        self.block = Decoder(cfg, 1, target.Lmax, gen=gen, device=dev, kv_fill=kv_fill,
                             weights=dict(layers=[weights["layer"]], final_gamma=weights["final_gamma"],
                                          lm_head=target.lm_head if lm_head is None else lm_head))
        self.inp = torch.empty((1, 2 * d), dtype=torch.int16, device=dev)
        self.x = torch.empty((1, d), dtype=torch.int16, device=dev)
        self.proj_ws = B.workspace(B.gemm_workspace_bytes(1, d, 2 * d), dev)
        self.stats = torch.zeros(B.ROWSTAT_BYTES, dtype=torch.uint8, device=dev)
        self.stat_ws = B.workspace(B.verify_workspace_bytes(1, V), dev)
        self.ws = B.workspace(B.draft_workspace_bytes(V), dev)
        self.flags = torch.zeros(1, dtype=torch.int32, device=dev)

    @staticmethod
    def random_weights(cfg: dict, gen, device="cuda"):
        import torch
        d = cfg["d"]

        def gamma():
            return (1.0 + 0.02 * torch.randn(d, generator=gen, device=device)).to(torch.bfloat16).view(torch.int16)

        lay = Decoder.random_weights(dict(cfg, layers=1, V=1), gen, device)["layers"][0]
        return dict(gamma_h=gamma(), gamma_e=gamma(), final_gamma=gamma(), layer=lay,
                    proj=W4Linear.random(d, 2 * d, 0.02, gen, device))

    def draft(self, h, h_rows: int, h_row, token, pos: int, T: float, top_p: float, seed: int, step, depth: int,
              q_out, token_out, stream=None, gemm_hook=None):
        """One depth at position pos: h [h_rows][d] (row *h_row, or 0 if h_row is
        None), token (int32 on the device) -> q_out [V] (fp32 draft distribution)
        and token_out (the drawn draft).  step: an int, or an int64 device
        tensor read when the kernels run.  gemm_hook: passed to the block's
        forward (see Decoder.forward)."""
        c = self.cfg
        d, V = c["d"], c["V"]
        B.mtp_input(h, h_rows, h_row, self.embed, token, self.gamma_h, self.gamma_e, c["eps"], self.inp, stream)
        B.w4_skinny_gemm(self.inp, self.proj.packed, self.proj.pscales, self.x, 1, d, 2 * d, ws=self.proj_ws,
                         stream=stream)
        logits = self.block.forward(self.x, pos, 1, stream, gemm_hook=gemm_hook)
        B.verify_logits(None, None, None, 1, V, d, T, top_p, logits, self.stats, self.stat_ws, stream=stream)
        dev_step = step if hasattr(step, "data_ptr") else None
        B.draft_sample(logits, self.stats, V, T, seed, 0 if dev_step is not None else step, depth, q_out,
                       token_out, self.flags, self.ws, step_dev=dev_step, stream=stream)
        return logits


class SpecLoop:
    """The closed cycle (hazakura.dev mtplx page, "4層のアーキテクチャ" Layer 2):
    D drafts from the MTP head, one verify pass of the target over M = D + 1
    rows, Leviathan–Chen acceptance with residual / bonus sampling.  State
    between cycles: L positions processed (0 .. L-1 in the KV caches), the
    target's residual row h of position L-1 and the next token y (position L,
    not processed yet).  A cycle emits the accepted drafts and the corrected or
    bonus token; rejected positions need no rollback beyond L, whose rows the
    next cycle overwrites.  The verify rows are the embedding rows of
    [y, x_0 .. x_{D-1}] at positions L .. L+D."""

    def __init__(self, target: "Decoder", head: MTPHead, D: int):
        import torch
        assert 1 <= D <= 7 and D + 1 <= target.M_max
        dev = target.device
        V, d = target.cfg["V"], target.cfg["d"]
        self.target, self.head, self.D = target, head, D
        self.vs = VerifyStep(target, D + 1)
        self.tokens_in = torch.zeros(D + 1, dtype=torch.int32, device=dev)     # y, x_0 .. x_{D-1}
        self.q = torch.zeros((D, V), dtype=torch.float32, device=dev)
        self.x = torch.empty((D + 1, d), dtype=torch.int16, device=dev)
        self.h_row = torch.zeros(1, dtype=torch.int32, device=dev)
        self.h_src, self.h_rows = None, 1
        self.ar_vs = VerifyStep(target, 1)
        self.L = 0

    def start(self, L0: int, t0: int, T: float, top_p: float, seed: int, step: int):
        """Process token t0 at position L0 (an autoregressive step) and draw y."""
        self.tokens_in[:1].fill_(int(t0))
        B.embed_rows(self.head.embed, self.tokens_in, 1, self.x)
        tok, n_acc, flags = self.ar_vs.run(self.x, L0, None, None, T, top_p, seed, step)
        self.tokens_in[:1].copy_(tok.view(-1)[:1])
        self.h_src, self.h_rows = self.target.last_resid, 1
        self.h_row.zero_()
        self.L = L0 + 1
        return int(tok.view(-1)[0].item())

    def draft(self, T: float, top_p: float, seed: int, step):
        """D head steps from (h, y) at positions L-1 .. L+D-2; fills q and x_0 ..."""
        head, D = self.head, self.D
        h, rows, row = self.h_src, self.h_rows, self.h_row
        for i in range(D):
            head.draft(h, rows, row, self.tokens_in[i:i + 1], self.L - 1 + i, T, top_p, seed, step, i, self.q[i],
                       self.tokens_in[i + 1:i + 2])
            h, rows, row = head.block.last_resid, 1, None

    def verify(self, T: float, top_p: float, seed: int, step: int):
        D, M = self.D, self.D + 1
        B.embed_rows(self.head.embed, self.tokens_in, M, self.x)
        return self.vs.run(self.x, self.L, self.q, self.tokens_in[1:], T, top_p, seed, step)

    def ar_graphable(self, T: float, top_p: float, seed: int, step_dev):
        """One autoregressive step of the pending token at the current L (no
        drafts: D = 0 sampling), Philox step from device memory."""
        B.embed_rows(self.head.embed, self.tokens_in, 1, self.x)
        self.ar_vs.run_graphable(self.x, self.L, None, None, T, top_p, seed, step_dev)

    def ar_step(self, T: float, top_p: float, seed: int, step: int):
        """The same eagerly: processes the pending token at L, returns the next
        one (host int) and makes it the pending token."""
        B.embed_rows(self.head.embed, self.tokens_in, 1, self.x)
        tok, _, _ = self.ar_vs.run(self.x, self.L, None, None, T, top_p, seed, step)
        self.tokens_in[:1].copy_(tok.view(-1)[:1])
        self.h_src, self.h_rows = self.target.last_resid, 1
        self.h_row.zero_()
        self.L += 1
        t = int(tok.view(-1)[0].item())
        if t < 0:
            raise RuntimeError("the autoregressive row was not finite")
        return t

    def run_graphable(self, T: float, top_p: float, seed: int, step_dev):
        """A cycle at the current L with the Philox step read from device memory
        (drafts and verify draw with the same step; the verify advances it)."""
        self.draft(T, top_p, seed, step_dev)
        B.embed_rows(self.head.embed, self.tokens_in, self.D + 1, self.x)
        self.vs.run_graphable(self.x, self.L, self.q, self.tokens_in[1:], T, top_p, seed, step_dev)

    def capture(self, fn):
        """Record fn() (launches only) into a HIP graph on a side stream."""
        import torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()                                    # warm (plans, code objects)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def cycle(self, T: float, top_p: float, seed: int, step: int, drafts=None):
        """One cycle; returns the emitted tokens (host list).  drafts (int32
        device [D]) replaces the head's drafts (with one-hot q): any other
        drafter can drive the same verify."""
        if drafts is None:
            self.draft(T, top_p, seed, step)
        else:
            self.tokens_in[1:].copy_(drafts)
            self.q.zero_()
            self.q.scatter_(1, drafts.view(-1, 1).long(), 1.0)
        tok, n_acc, flags = self.verify(T, top_p, seed, step)
        k = int(n_acc.item())
        out = tok.view(-1)[:k + 1].tolist()
        if k < 0:
            raise RuntimeError("verify rows were not finite")
        self.tokens_in[:1].copy_(tok.view(-1)[k:k + 1])
        self.h_src, self.h_rows = self.target.last_resid, self.D + 1
        self.h_row.fill_(k)
        self.L += k + 1
        return out


def _graph_ms(g, reps: int, warm: int = 2) -> float:
    """Mean time of one replay of a captured graph, from HIP events on the
    current stream (where replay() launches)."""
    import torch
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


class DepthTuner:
    """Draft-depth autotune with the autoregressive fallback (devtrends.cc,
    "Apple Silicon上でローカルLLMを最大2倍高速化するMTPLX", section "主な機能":
    the tool tries draft depths 1 to 3 on the machine itself, keeps the
    fastest, and leaves drafting off where plain decoding is faster).

    Each candidate is measured on the device, from the same start state:
    * cost: one cycle of depth D (D head steps, the verify of D + 1 rows and
      the acceptance) captured as a HIP graph at the current context and
      replayed; D = 0 is the one-row autoregressive step, timed the same way;
    * yield: the tokens that real cycles of depth D emit (accepted drafts plus
      the corrected or bonus token), averaged over `cycles` cycles; D = 0
      emits one token per step.
    The depth with the most tokens per second is locked (a tie goes to the
    smaller depth, so AR wins ties).  ``decode`` then generates with it."""

    def __init__(self, target: "Decoder", head: MTPHead, depths=(1, 2, 3)):
        assert all(1 <= D <= 7 and D + 1 <= target.M_max for D in depths)
        self.target, self.head, self.depths = target, head, tuple(sorted(depths))
        self.depth = None
        self.report = None

    @staticmethod
    def choose(tokens_per_s: dict) -> int:
        """The depth with the most tokens per second; depth 0 (AR) is the
        default, and a tie keeps the smaller depth."""
        best = 0
        for D in sorted(tokens_per_s):
            if tokens_per_s[D] > tokens_per_s.get(best, float("-inf")):
                best = D
        return best

    def tune(self, L0: int, t0: int, T: float, top_p: float, seed: int, cycles: int = 8, reps: int = 10,
             drafts_fn=None):
        """Measure every candidate and lock the best.  drafts_fn(loop, emitted),
        if given, returns the int32 device drafts of the next cycle (None: the
        head drafts); emitted is the token list so far, starting with the token
        that follows t0."""
        import torch
        dev = self.target.device
        step_dev = torch.zeros(1, dtype=torch.int64, device=dev)
        ms, per_cycle = {}, {}
        ar = SpecLoop(self.target, self.head, self.depths[0])
        ar.start(L0, t0, T, top_p, seed, 0)
        ms[0] = _graph_ms(ar.capture(lambda: ar.ar_graphable(T, top_p, seed, step_dev)), reps)
        per_cycle[0] = 1.0
        for D in self.depths:
            loop = SpecLoop(self.target, self.head, D)
            loop.start(L0, t0, T, top_p, seed, 0)
            ms[D] = _graph_ms(loop.capture(lambda: loop.run_graphable(T, top_p, seed, step_dev)), reps)
            # real cycles from the same start state (rows past L are overwritten)
            emitted = [loop.start(L0, t0, T, top_p, seed, 0)]
            n = 0
            for c in range(cycles):
                drafts = drafts_fn(loop, emitted) if drafts_fn is not None else None
                out = loop.cycle(T, top_p, seed, c + 1, drafts=drafts)
                n += len(out)
                emitted += out
            per_cycle[D] = n / cycles
        tps = {D: per_cycle[D] * 1e3 / ms[D] for D in ms}
        best = self.choose(tps)
        self.depth = best
        self.report = {"pick": "ar" if best == 0 else f"D{best}", "depth": best,
                       "ms": {("ar" if D == 0 else f"D{D}"): v for D, v in ms.items()},
                       "tokens_per_cycle": {f"D{D}": per_cycle[D] for D in self.depths},
                       "tokens_per_s": {("ar" if D == 0 else f"D{D}"): v for D, v in tps.items()},
                       "alpha": {f"D{D}": round((per_cycle[D] - 1.0) / D, 4) for D in self.depths}}
        return self.report

    def decode(self, L0: int, t0: int, n: int, T: float, top_p: float, seed: int):
        """At least n tokens after t0 (processed at L0) with the locked depth:
        autoregressive steps for depth 0, else draft -> verify -> accept cycles.
        Returns (tokens, the loop)."""
        assert self.depth is not None, "tune() first"
        D = self.depth
        loop = SpecLoop(self.target, self.head, D if D else self.depths[0])
        seq = [loop.start(L0, t0, T, top_p, seed, 0)]
        k = 1
        while len(seq) < n:
            if D == 0:
                seq.append(loop.ar_step(T, top_p, seed, k))
            else:
                seq += loop.cycle(T, top_p, seed, k)
            k += 1
        return seq, loop


# ---------------------------------------------------------------------------
# MoE-shaped verify step (synthetic weights)
# ---------------------------------------------------------------------------
MOE_30B = dict(n_exp=128, topk=8, d=2048, F=768, V=151936, eps=1e-6)


class ExpertBank:
    """W4 weights of E SwiGLU experts, each stored as a contiguous slice of two
    stacked matrices: gate|up [E * 2F][d] (each expert's 2F rows in the
    gate/up-interleaved order of B.interleave_gate_up) and down [E * d][F]."""

    def __init__(self, gate_up: W4Linear, down: W4Linear, E: int, d: int, F: int):
        assert (2 * F) % 64 == 0 and d % 64 == 0 and F % 64 == 0
        self.gate_up, self.down, self.E, self.d, self.F = gate_up, down, E, d, F
        self.gu_estride = (2 * F * d // 2, 2 * F * d // 64)   # (bytes, fp16 scales) per expert
        self.dn_estride = (d * F // 2, d * F // 64)

    @classmethod
    def random(cls, E: int, d: int, F: int, std: float, gen, device="cuda"):
        return cls(W4Linear.random(E * 2 * F, d, std, gen, device), W4Linear.random(E * d, F, std, gen, device),
                   E, d, F)

    @classmethod
    def from_fp32(cls, gate_up, down):
        """gate_up: [E][2F][d], down: [E][d][F] fp32 device tensors."""
        E, F2, d = gate_up.shape
        gu = B.interleave_gate_up(gate_up.reshape(E, F2, d).permute(1, 0, 2).reshape(F2, E * d))
        gu = gu.reshape(F2, E, d).permute(1, 0, 2).contiguous()     # per expert, gate/up-interleaved rows
        return cls(W4Linear.from_fp32(gu.reshape(E * F2, d)), W4Linear.from_fp32(down.reshape(E * d, F2 // 2)),
                   E, d, F2 // 2)

    def expert_bytes(self) -> int:
        return int(3 * self.d * self.F * BYTES_PER_WEIGHT)


class MoEVerify:
    """Verify step of an MoE-shaped model: the M hidden rows go through one
    routed SwiGLU expert layer (router top-k, grouped W4 GEMMs over the
    distinct chosen experts, weighted combine), the residual add and the final
    RMSNorm, then the LM head, the temperature / top-p statistics and
    Leviathan–Chen acceptance.  Routing stays on the device (slot list), so the
    step can be captured as a graph."""

    def __init__(self, cfg: dict, M: int, lm_head: W4Linear, final_gamma, device="cuda"):
        import torch
        self.cfg = dict(cfg)
        E, topk, d, F, V = (cfg[k] for k in ("n_exp", "topk", "d", "F", "V"))
        self.M, self.D, self.E, self.topk, self.d, self.F, self.V = M, M - 1, E, topk, d, F, V
        self.lm_head, self.final_gamma, self.device = lm_head, final_gamma, device
        self.max_slots = min(E, M * topk)
        i32 = torch.int32
        self.experts = torch.empty((M, topk), dtype=i32, device=device)
        self.weights = torch.empty((M, topk), dtype=torch.float32, device=device)
        self.slot_expert = torch.zeros(self.max_slots, dtype=i32, device=device)
        # tokens [1][M], n_acc, flags and the routed slot count in one int32
        # block: one copy reads a step's outputs
        self.outputs = torch.zeros(M + 3, dtype=i32, device=device)
        self.n_slots = self.outputs[M + 2:M + 3]
        self.row_slot = torch.empty((M, topk), dtype=i32, device=device)
        self.dn_S, self.dn_ldp = B.grouped_gemm_layout(M, d, F, self.max_slots)
        self.dn_sstride = self.dn_S * M * self.dn_ldp
        self.part_dn = torch.empty(self.max_slots * self.dn_sstride, dtype=torch.float32, device=device)
        self.a = torch.empty((self.max_slots, M, F), dtype=torch.int16, device=device)
        self.y = torch.empty((M, d), dtype=torch.float32, device=device)
        self.resid = torch.empty((M, d), dtype=torch.int16, device=device)
        self.h = torch.empty((M, d), dtype=torch.int16, device=device)
        # the expert combine inside the final add + RMSNorm launch; False runs
        # vw4_moe_combine and vw4_add_rmsnorm_out
        self.fuse_combine = True
        self.norm_ws = B.workspace(B.norm_workspace_bytes(M, d), device)
        self.logits = torch.empty((M, V), dtype=torch.float32, device=device)
        self.lm_ws = B.workspace(B.gemm_workspace_bytes(M, V, d), device)
        self.stats = torch.zeros(M * B.ROWSTAT_BYTES, dtype=torch.uint8, device=device)
        self.stat_ws = B.workspace(B.verify_workspace_bytes(M, V), device)
        self.acc_ws = B.workspace(B.accept_workspace_bytes(1, V), device)
        self.tokens = self.outputs[:M].view(1, M)
        self.n_acc = self.outputs[M:M + 1]
        self.flags = self.outputs[M + 1:M + 2]

    def moe(self, x, router_logits, bank: ExpertBank, stream=None, gemm_hook=None, combine: bool = True):
        """y[M][d] (fp32) = routed SwiGLU experts of the bf16 rows x (combine=False
        stops at the down-projection partials, for a consumer that combines them)."""
        hook = gemm_hook or (lambda when, name: None)
        M, d, F, ms = self.M, self.d, self.F, self.max_slots
        B.moe_route(router_logits, M, self.E, self.topk, self.experts, self.weights, self.slot_expert, self.n_slots,
                    self.row_slot, stream)
        hook("pre", "gate_up")
        B.w4_grouped_gemm_swiglu(x, x.stride(0), 0, bank.gate_up.packed, bank.gu_estride[0], bank.gate_up.pscales,
                                 bank.gu_estride[1], self.slot_expert, self.n_slots, ms, self.a, M * F, M, F, d,
                                 stream)
        hook("post", "gate_up")
        hook("pre", "down")
        B.w4_grouped_gemm(self.a, F, M * F, bank.down.packed, bank.dn_estride[0], bank.down.pscales,
                          bank.dn_estride[1], self.slot_expert, self.n_slots, ms, self.part_dn, self.dn_sstride,
                          M, d, F, stream)
        hook("post", "down")
        if combine:
            B.moe_combine(self.part_dn, self.dn_S, self.dn_ldp, self.dn_sstride, self.row_slot, self.weights, M,
                          self.topk, d, self.y, d, stream)
        return self.y

    def gemm_pass(self, bank: ExpertBank, stream=None):
        """Only the W4 GEMM launches of one step (grouped gate|up, grouped
        down, LM head) on the current routing and buffers."""
        M, d, F, ms = self.M, self.d, self.F, self.max_slots
        B.w4_grouped_gemm_swiglu(self.h, d, 0, bank.gate_up.packed, bank.gu_estride[0], bank.gate_up.pscales,
                                 bank.gu_estride[1], self.slot_expert, self.n_slots, ms, self.a, M * F, M, F, d,
                                 stream)
        B.w4_grouped_gemm(self.a, F, M * F, bank.down.packed, bank.dn_estride[0], bank.down.pscales,
                          bank.dn_estride[1], self.slot_expert, self.n_slots, ms, self.part_dn, self.dn_sstride,
                          M, d, F, stream)
        B.w4_skinny_gemm(self.h, self.lm_head.packed, self.lm_head.pscales, self.logits, M, self.V, d, ws=self.lm_ws,
                         stream=stream)
        return 3

    def forward(self, x, router_logits, bank: ExpertBank, stream=None, gemm_hook=None):
        """Logits [M][V] of the M rows: LM head of bf16(rmsnorm(x + moe(x)) * gamma)."""
        hook = gemm_hook or (lambda when, name: None)
        M, d = self.M, self.d
        nch = (d + 255) // 256
        cpw = 1 if nch <= 8 else (2 if nch <= 16 else 3)
        if self.fuse_combine and self.topk <= 8 and self.dn_S * 8 * cpw <= 32 and d % 4 == 0:
            # the expert combine inside the add + RMSNorm launch (bitwise the two calls)
            self.moe(x, router_logits, bank, stream, gemm_hook, combine=False)
            B.moe_add_rmsnorm(x[:M], self.part_dn, self.dn_S, self.dn_ldp, self.dn_sstride, self.row_slot,
                              self.weights, self.topk, self.final_gamma, self.cfg["eps"], M, d, self.resid, self.h,
                              stream)
        else:
            self.moe(x, router_logits, bank, stream, gemm_hook)
            B.add_rmsnorm_out(x[:M], self.y, 1, d, self.final_gamma, self.cfg["eps"], M, d, self.resid, self.h,
                              stream)
        hook("pre", "lm_head")
        B.w4_skinny_gemm(self.h, self.lm_head.packed, self.lm_head.pscales, self.logits, M, self.V, d, ws=self.lm_ws,
                         stream=stream)
        hook("post", "lm_head")
        return self.logits

    def _accept(self, q, drafts, T, top_p, seed, step=None, step_dev=None, stream=None):
        B.verify_logits(None, None, None, self.M, self.V, self.d, T, top_p, self.logits, self.stats, self.stat_ws,
                        stream=stream)
        if step_dev is None:
            B.spec_accept(self.logits, 0, self.stats, 0, q, 0, drafts, 1, self.D, self.V, T, seed, step, self.tokens,
                          self.n_acc, self.flags, self.acc_ws, stream=stream)
        else:
            B.spec_accept_ex(self.logits, 0, self.stats, 0, q, 0, drafts, 1, self.D, self.V, T, seed, step_dev,
                             self.tokens, self.n_acc, self.flags, self.acc_ws, stream=stream)
            B.step_advance(step_dev, 1, stream)

    def run(self, x, router_logits, bank, q, drafts, T, top_p, seed, step, stream=None, gemm_hook=None):
        self.forward(x, router_logits, bank, stream, gemm_hook)
        self._accept(q, drafts, T, top_p, seed, step=step, stream=stream)
        return self.tokens, self.n_acc, self.flags

    def run_graphable(self, x, router_logits, bank, q, drafts, T, top_p, seed, step_dev, stream=None):
        self.forward(x, router_logits, bank, stream)
        self._accept(q, drafts, T, top_p, seed, step_dev=step_dev, stream=stream)

    def capture(self, x, router_logits, bank, q, drafts, T, top_p, seed, step_dev):
        import torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.run_graphable(x, router_logits, bank, q, drafts, T, top_p, seed, step_dev)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run_graphable(x, router_logits, bank, q, drafts, T, top_p, seed, step_dev)
        torch.cuda.synchronize()
        return g

    def step_bytes(self, n_distinct: int) -> int:
        """Algorithmic HBM bytes of one step with n_distinct experts chosen:
        each chosen expert's weights and the LM head once (activations and
        logits are < 0.5 % and left out)."""
        return int(n_distinct * 3 * self.d * self.F * BYTES_PER_WEIGHT + self.V * self.d * BYTES_PER_WEIGHT)
