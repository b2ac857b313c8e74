"""ctypes binding of libvw4.so (the C ABI declared in include/vw4.h).

Argument marshalling only: every step of the verify path runs in the HIP
kernels of libvw4.so.  torch is used for device memory and streams: tensors
are passed as raw device pointers and the current torch stream is passed as
the hipStream_t.  Loading fails loudly when the library has not been built;
there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
# VW4_LIB selects another build of the same sources (the host-sanitizer build
# that tests/test_host_sanitizers.py runs the host-side ABI checks against)
LIB_PATH = os.environ.get("VW4_LIB") or os.path.join(PKG, "libvw4.so")

VW4_OK = 0
VW4_EINVAL = -1
VW4_EUNSUPPORTED = -2
VW4_EHIP = -3
VW4_EWORKSPACE = -4
VW4_F32 = 0
VW4_BF16 = 1
FLAG_NONFINITE = 1
FLAG_TOPP_TIE = 2
FLAG_ACCEPT_TIE = 4
FLAG_CDF_TIE = 8
FLAG_R_ZERO = 16

# numpy view of struct vw4_rowstat (32 bytes)
ROWSTAT_DTYPE = np.dtype([("max_logit", "<f4"), ("tau", "<f4"), ("log_z", "<f8"), ("argmax", "<i4"),
                          ("n_kept", "<i4"), ("flags", "<u4"), ("pad", "<u4")])
ROWSTAT_BYTES = 32
assert ROWSTAT_DTYPE.itemsize == ROWSTAT_BYTES

# name -> (restype, argtypes), mirroring include/vw4.h
_P, _I32, _I64, _U64, _F32, _SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                   ctypes.c_float, ctypes.c_size_t)
SIGNATURES = {
    "vw4_version": (ctypes.c_char_p, []),
    "vw4_last_error": (ctypes.c_char_p, []),
    "vw4_w4_quantize_host": (ctypes.c_int, [_P, _I64, _I64, _P, _P]),
    "vw4_w4_quantize": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "vw4_w4_packed_bytes": (_SZ, [_I64, _I64, ctypes.POINTER(ctypes.c_size_t)]),
    "vw4_w4_pack": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _P]),
    "vw4_w4_unpack": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _P]),
    "vw4_w4_quantize_packed": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "vw4_gemm_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "w4_skinny_gemm": (ctypes.c_int, [_P, _I64, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _SZ, _P]),
    "w4_skinny_gemm_noalloc": (ctypes.c_int, [_P, _I64, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P]),
    "vw4_noalloc_scratch_bytes": (_SZ, []),
    "vw4_stream_read": (ctypes.c_int, [_P, _SZ, _P, _I32, _P]),
    "vw4_workspace_bytes": (_SZ, [_I32, _I32]),
    "verify_logits": (ctypes.c_int, [_P, _I64, _P, _P, _I32, _I32, _I32, _F32, _F32, _P, _P, _P, _SZ, _P]),
    "vw4_accept_workspace_bytes": (_SZ, [_I32, _I32]),
    "spec_accept": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _I64, _P, _I32, _I32, _I32, _F32, _U64, _U64, _P, _P,
                                   _P, _P, _SZ, _P]),
    "spec_accept_ex": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _I64, _P, _I32, _I32, _I32, _F32, _U64, _P, _P, _P,
                                      _P, _P, _SZ, _P]),
    "vw4_step_advance": (ctypes.c_int, [_P, _U64, _P]),
    "vw4_embed_rows": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _I32, _P, _I64, _P]),
    "vw4_mtp_input": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _I64, _I32, _P, _P, _P, ctypes.c_float, _I32, _P, _P]),
    "vw4_draft_workspace_bytes": (_SZ, [_I32]),
    "vw4_w8_quantize_host": (ctypes.c_int, [_P, _I64, _I64, _P, _P]),
    "vw4_w8_pack": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _P, _P]),
    "vw4_w8_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "w8_skinny_gemm": (ctypes.c_int, [_P, _I64, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _SZ, _P]),
    "vw4_w8_partials_layout": (ctypes.c_int, [_I32, _I32, _I32, ctypes.POINTER(ctypes.c_int32),
                                              ctypes.POINTER(ctypes.c_int64)]),
    "w8_skinny_gemm_partials": (ctypes.c_int, [_P, _I64, _P, _P, _P, _P, _I32, _I32, _I32, _P]),
    "vw4_w16_packed_bytes": (_SZ, [_I64, _I64]),
    "vw4_w16_pack": (ctypes.c_int, [_P, _I64, _I64, _P, _P]),
    "vw4_f16_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "vw4_bf16_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "f16_skinny_gemm": (ctypes.c_int, [_P, _I64, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _SZ, _P]),
    "bf16_skinny_gemm": (ctypes.c_int, [_P, _I64, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _SZ, _P]),
    "vw4_f16_partials_layout": (ctypes.c_int, [_I32, _I32, _I32, ctypes.POINTER(ctypes.c_int32),
                                               ctypes.POINTER(ctypes.c_int64)]),
    "vw4_bf16_partials_layout": (ctypes.c_int, [_I32, _I32, _I32, ctypes.POINTER(ctypes.c_int32),
                                                ctypes.POINTER(ctypes.c_int64)]),
    "f16_skinny_gemm_partials": (ctypes.c_int, [_P, _I64, _P, _P, _I32, _I32, _I32, _P]),
    "bf16_skinny_gemm_partials": (ctypes.c_int, [_P, _I64, _P, _P, _I32, _I32, _I32, _P]),
    "vw4_w3_quantize_host": (ctypes.c_int, [_P, _I64, _I64, _P, _P]),
    "vw4_w3_hi_plane_bytes": (_SZ, [_I64, _I64]),
    "vw4_w3_lo_plane_bytes": (_SZ, [_I64, _I64]),
    "vw4_w3_pack": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _P, _P]),
    "vw4_w3_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "w3_skinny_gemm": (ctypes.c_int, [_P, _I64, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _SZ, _P]),
    "vw4_w3_partials_layout": (ctypes.c_int, [_I32, _I32, _I32, ctypes.POINTER(ctypes.c_int32),
                                              ctypes.POINTER(ctypes.c_int64)]),
    "w3_skinny_gemm_partials": (ctypes.c_int, [_P, _I64, _P, _P, _P, _P, _I32, _I32, _I32, _P]),
    "vw4_w2_quantize_host": (ctypes.c_int, [_P, _I64, _I64, _P, _P]),
    "vw4_w2_packed_bytes": (_SZ, [_I64, _I64]),
    "vw4_w2_pack": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _P]),
    "vw4_w2_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "w2_skinny_gemm": (ctypes.c_int, [_P, _I64, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _SZ, _P]),
    "vw4_w2_partials_layout": (ctypes.c_int, [_I32, _I32, _I32, ctypes.POINTER(ctypes.c_int32),
                                              ctypes.POINTER(ctypes.c_int64)]),
    "w2_skinny_gemm_partials": (ctypes.c_int, [_P, _I64, _P, _P, _P, _I32, _I32, _I32, _P]),
    "vw4_w5_quantize_host": (ctypes.c_int, [_P, _I64, _I64, _P, _P]),
    "vw4_w5_hi_plane_bytes": (_SZ, [_I64, _I64]),
    "vw4_w5_pack": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _P, _P]),
    "vw4_w5_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "w5_skinny_gemm": (ctypes.c_int, [_P, _I64, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _SZ, _P]),
    "vw4_w5_partials_layout": (ctypes.c_int, [_I32, _I32, _I32, ctypes.POINTER(ctypes.c_int32),
                                              ctypes.POINTER(ctypes.c_int64)]),
    "w5_skinny_gemm_partials": (ctypes.c_int, [_P, _I64, _P, _P, _P, _P, _I32, _I32, _I32, _P]),
    "vw4_w6_quantize_host": (ctypes.c_int, [_P, _I64, _I64, _P, _P]),
    "vw4_w6_hi_plane_bytes": (_SZ, [_I64, _I64]),
    "vw4_w6_pack": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _P, _P]),
    "vw4_w6_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "w6_skinny_gemm": (ctypes.c_int, [_P, _I64, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _SZ, _P]),
    "vw4_w6_partials_layout": (ctypes.c_int, [_I32, _I32, _I32, ctypes.POINTER(ctypes.c_int32),
                                              ctypes.POINTER(ctypes.c_int64)]),
    "w6_skinny_gemm_partials": (ctypes.c_int, [_P, _I64, _P, _P, _P, _P, _I32, _I32, _I32, _P]),
    "draft_sample": (ctypes.c_int, [_P, _P, _I32, ctypes.c_float, _U64, _P, _U64, _I32, _P, _P, _P, _P, _SZ, _P]),
    "vw4_gemm_partials_layout": (ctypes.c_int, [_I32, _I32, _I32, ctypes.POINTER(ctypes.c_int32),
                                                ctypes.POINTER(ctypes.c_int64)]),
    "w4_skinny_gemm_partials": (ctypes.c_int, [_P, _I64, _P, _P, _P, _I32, _I32, _I32, _P]),
    "vw4_norm_workspace_bytes": (_SZ, [_I32, _I32]),
    "vw4_add_rmsnorm": (ctypes.c_int, [_P, _P, _I32, _I64, _P, _F32, _I32, _I32, _P, _P, _SZ, _P]),
    "vw4_rope_kv_append": (ctypes.c_int, [_P, _I32, _I64, _I32, _I32, _I32, _I32, _I32, _F32, _P, _P, _P, _I64, _P]),
    "vw4_swiglu": (ctypes.c_int, [_P, _I32, _I64, _I32, _I32, _P, _P]),
    "vw4_attn_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I64]),
    "vw4_decode_attn": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "vw4_moe_add_rmsnorm": (ctypes.c_int, [_P, _P, _I32, _I64, _I64, _P, _P, _I32, _P, _F32, _I32, _I32, _P, _P, _P]),
    "vw4_add_sumsq": (ctypes.c_int, [_P, _P, _I32, _I64, _I32, _I32, _P, _SZ, _P]),
    "vw4_add_rmsnorm_out": (ctypes.c_int, [_P, _P, _I32, _I64, _P, _F32, _I32, _I32, _P, _P, _P]),
    "w4_skinny_gemm_rmsnorm_partials": (ctypes.c_int, [_P, _P, _P, _F32, _P, _P, _P, _I32, _I32, _I32, _P]),
    "w4_skinny_gemm_rmsnorm_swiglu": (ctypes.c_int, [_P, _P, _P, _F32, _P, _P, _P, _I64, _I32, _I32, _I32, _P]),
    "w4_skinny_gemm_swiglu": (ctypes.c_int, [_P, _I64, _P, _P, _P, _I64, _I32, _I32, _I32, _P]),
    "w8_skinny_gemm_swiglu": (ctypes.c_int, [_P, _I64, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _P]),
    "w6_skinny_gemm_swiglu": (ctypes.c_int, [_P, _I64, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _P]),
    "w5_skinny_gemm_swiglu": (ctypes.c_int, [_P, _I64, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _P]),
    "w3_skinny_gemm_swiglu": (ctypes.c_int, [_P, _I64, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _P]),
    "w2_skinny_gemm_swiglu": (ctypes.c_int, [_P, _I64, _P, _P, _P, _I64, _I32, _I32, _I32, _P]),
    "f16_skinny_gemm_swiglu": (ctypes.c_int, [_P, _I64, _P, _P, _I64, _I32, _I32, _I32, _P]),
    "bf16_skinny_gemm_swiglu": (ctypes.c_int, [_P, _I64, _P, _P, _I64, _I32, _I32, _I32, _P]),
    "w4_grouped_gemm_swiglu": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _I64, _P, _P, _I32, _P, _I64, _I32,
                                              _I32, _I32, _P]),
    "vw4_moe_route": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P]),
    "vw4_grouped_gemm_layout": (ctypes.c_int, [_I32, _I32, _I32, _I32, ctypes.POINTER(ctypes.c_int32),
                                               ctypes.POINTER(ctypes.c_int64)]),
    "w4_grouped_gemm": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _I64, _P, _P, _I32, _P, _I64, _I32, _I32, _I32,
                                       _P]),
    "vw4_grouped_swiglu": (ctypes.c_int, [_P, _I32, _I64, _I64, _I32, _I32, _P, _I64, _P, _I32, _P]),
    "vw4_moe_combine": (ctypes.c_int, [_P, _I32, _I64, _I64, _P, _P, _I32, _I32, _I32, _P, _I64, _P]),
}


class VW4Error(RuntimeError):
    def __init__(self, name: str, rc: int, msg: str):
        super().__init__(f"{name} failed with {rc}: {msg}")
        self.rc = rc


_lib = None


def lib() -> ctypes.CDLL:
    """Load libvw4.so; raises if it is missing (build it with build.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(python -m verify_step_w4_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().vw4_last_error().decode()


def version() -> str:
    return lib().vw4_version().decode()


def _check(name: str, rc: int):
    if rc != VW4_OK:
        raise VW4Error(name, rc, last_error())


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev_tensor(t, name):
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous device tensor")


# ---------------------------------------------------------------------------
# W4 weight format
# ---------------------------------------------------------------------------
def w4_quantize_host(w: np.ndarray):
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    codes = np.zeros((N, K // 2), dtype=np.uint8)
    scales = np.zeros((N, K // 64), dtype=np.uint16)
    _check("vw4_w4_quantize_host", lib().vw4_w4_quantize_host(
        w.ctypes.data_as(_P), N, K, codes.ctypes.data_as(_P), scales.ctypes.data_as(_P)))
    return codes, scales


def packed_sizes(N: int, K: int):
    sb = ctypes.c_size_t(0)
    cb = lib().vw4_w4_packed_bytes(N, K, ctypes.byref(sb))
    if cb == 0:
        raise VW4Error("vw4_w4_packed_bytes", VW4_EINVAL, f"invalid shape N={N} K={K}")
    return int(cb), int(sb.value)


def w4_quantize(w, stream=None):
    """Device fp32 [N][K] -> device canonical (codes u8 [N][K/2], scales i16-bits [N][K/64])."""
    import torch
    _dev_tensor(w, "w")
    N, K = w.shape
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((N, K // 64), dtype=torch.int16, device=w.device)
    _check("vw4_w4_quantize", lib().vw4_w4_quantize(_ptr(w), N, K, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def w4_pack(codes, scales, N: int, K: int, stream=None):
    import torch
    cb, sb = packed_sizes(N, K)
    packed = torch.empty(cb, dtype=torch.uint8, device=codes.device)
    pscales = torch.empty(sb // 2, dtype=torch.int16, device=codes.device)
    _check("vw4_w4_pack", lib().vw4_w4_pack(_ptr(codes), _ptr(scales), N, K, _ptr(packed), _ptr(pscales),
                                            _stream(stream)))
    return packed, pscales


def w4_unpack(packed, pscales, N: int, K: int, stream=None):
    import torch
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=packed.device)
    scales = torch.empty((N, K // 64), dtype=torch.int16, device=packed.device)
    _check("vw4_w4_unpack", lib().vw4_w4_unpack(_ptr(packed), _ptr(pscales), N, K, _ptr(codes), _ptr(scales),
                                                _stream(stream)))
    return codes, scales


def w4_quantize_packed(w, stream=None, out=None):
    import torch
    _dev_tensor(w, "w")
    N, K = w.shape
    cb, sb = packed_sizes(N, K)
    if out is None:
        packed = torch.empty(cb, dtype=torch.uint8, device=w.device)
        pscales = torch.empty(sb // 2, dtype=torch.int16, device=w.device)
    else:
        packed, pscales = out
    _check("vw4_w4_quantize_packed", lib().vw4_w4_quantize_packed(_ptr(w), N, K, _ptr(packed), _ptr(pscales),
                                                                  _stream(stream)))
    return packed, pscales


# ---------------------------------------------------------------------------
# workspaces (caller-owned scratch; contents need no initialisation)
# ---------------------------------------------------------------------------
def workspace(nbytes: int, device="cuda"):
    import torch
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().vw4_gemm_workspace_bytes(M, N, K))


def verify_workspace_bytes(rows: int, V: int, d: int | None = None) -> int:
    n = int(lib().vw4_workspace_bytes(rows, V))
    if d is not None:
        n += gemm_workspace_bytes(rows, V, d)
    return n


def accept_workspace_bytes(B: int, V: int) -> int:
    return int(lib().vw4_accept_workspace_bytes(B, V))


# ---------------------------------------------------------------------------
# the three calls of the verify step
# ---------------------------------------------------------------------------
def w4_skinny_gemm(x, w_packed, scales_packed, y, M: int, N: int, K: int, ws=None, stream=None,
                   ldx: int | None = None, ldy: int | None = None):
    """y[M][N] (fp32 or bf16 tensor) = x[M][K] (bf16 bits as int16/bfloat16) @ W4^T."""
    import torch
    ydt = VW4_F32 if y.dtype == torch.float32 else VW4_BF16
    ldx = x.stride(0) if ldx is None else ldx
    ldy = y.stride(0) if ldy is None else ldy
    nbytes = ws.numel() if ws is not None else 0
    _check("w4_skinny_gemm", lib().w4_skinny_gemm(_ptr(x), ldx, _ptr(w_packed), _ptr(scales_packed), _ptr(y), ldy,
                                                  ydt, M, N, K, _ptr(ws), nbytes, _stream(stream)))
    return y


def w4_skinny_gemm_noalloc(x, w_packed, scales_packed, y, M: int, N: int, K: int, stream=None,
                           ldx: int | None = None, ldy: int | None = None):
    """w4_skinny_gemm with its partial sums in the library's static scratch
    array (no workspace, nothing allocated); calls on one GPU must not overlap."""
    import torch
    ydt = VW4_F32 if y.dtype == torch.float32 else VW4_BF16
    ldx = x.stride(0) if ldx is None else ldx
    ldy = y.stride(0) if ldy is None else ldy
    _check("w4_skinny_gemm_noalloc", lib().w4_skinny_gemm_noalloc(_ptr(x), ldx, _ptr(w_packed), _ptr(scales_packed),
                                                                  _ptr(y), ldy, ydt, M, N, K, _stream(stream)))
    return y


def stream_read(src, sink, blocks: int, nbytes: int | None = None, stream=None):
    """Read nbytes (default: all) of device tensor src; sink: int32/uint32
    device tensor of >= blocks words (per-workgroup XOR of what was read)."""
    n = src.numel() * src.element_size() if nbytes is None else nbytes
    _check("vw4_stream_read", lib().vw4_stream_read(_ptr(src), n, _ptr(sink), blocks, _stream(stream)))


def verify_logits(hidden, lm_packed, lm_scales, rows: int, V: int, d: int, temperature: float, top_p: float,
                  logits, stats, ws, stream=None, ldh: int | None = None):
    """stats: uint8 device tensor of rows * 32 bytes (struct vw4_rowstat)."""
    if hidden is not None:
        ldh = hidden.stride(0) if ldh is None else ldh
    _check("verify_logits", lib().verify_logits(_ptr(hidden), ldh or 0, _ptr(lm_packed), _ptr(lm_scales), rows, V,
                                                d, float(temperature), float(top_p), _ptr(logits), _ptr(stats),
                                                _ptr(ws), ws.numel(), _stream(stream)))
    return logits, stats


def spec_accept(logits, logits_bstride: int, stats, stats_bstride: int, q, q_bstride: int, draft, B: int, D: int,
                V: int, temperature: float, seed: int, step0: int, out_tokens, out_n_acc, out_flags, ws,
                stream=None):
    _check("spec_accept", lib().spec_accept(_ptr(logits), logits_bstride, _ptr(stats), stats_bstride, _ptr(q),
                                            q_bstride, _ptr(draft), B, D, V, float(temperature), int(seed),
                                            int(step0), _ptr(out_tokens), _ptr(out_n_acc), _ptr(out_flags),
                                            _ptr(ws), ws.numel(), _stream(stream)))
    return out_tokens, out_n_acc, out_flags


def spec_accept_ex(logits, logits_bstride: int, stats, stats_bstride: int, q, q_bstride: int, draft, B: int, D: int,
                   V: int, temperature: float, seed: int, step_dev, out_tokens, out_n_acc, out_flags, ws,
                   stream=None):
    _check("spec_accept_ex", lib().spec_accept_ex(_ptr(logits), logits_bstride, _ptr(stats), stats_bstride, _ptr(q),
                                                  q_bstride, _ptr(draft), B, D, V, float(temperature), int(seed),
                                                  _ptr(step_dev), _ptr(out_tokens), _ptr(out_n_acc),
                                                  _ptr(out_flags), _ptr(ws), ws.numel(), _stream(stream)))
    return out_tokens, out_n_acc, out_flags


def step_advance(step_dev, inc: int = 1, stream=None):
    _check("vw4_step_advance", lib().vw4_step_advance(_ptr(step_dev), int(inc), _stream(stream)))


def embed_rows(E, tokens, n: int, out, stream=None):
    """out[i] = E[tokens[i]] for i < n (bf16 bit tensors; tokens int32 on the device)."""
    V, d = E.shape
    _check("vw4_embed_rows", lib().vw4_embed_rows(_ptr(E), E.stride(0), V, d, _ptr(tokens), n, _ptr(out),
                                                  out.stride(0), _stream(stream)))


def mtp_input(h, h_rows: int, h_row, E, token, gamma_h, gamma_e, eps: float, out, stream=None):
    """out[0:2d] = [rmsnorm(h[*h_row]) * gamma_h ; rmsnorm(E[*token]) * gamma_e] (bf16)."""
    V, d = E.shape
    _check("vw4_mtp_input", lib().vw4_mtp_input(_ptr(h), h.stride(0), h_rows, _ptr(h_row), _ptr(E), E.stride(0), V,
                                                _ptr(token), _ptr(gamma_h), _ptr(gamma_e), float(eps), d, _ptr(out),
                                                _stream(stream)))


def draft_workspace_bytes(V: int) -> int:
    return int(lib().vw4_draft_workspace_bytes(V))


def draft_sample(logits, stats, V: int, temperature: float, seed: int, step: int, depth: int, q_out, token_out,
                 flags_out, ws, step_dev=None, stream=None):
    _check("draft_sample", lib().draft_sample(_ptr(logits), _ptr(stats), V, float(temperature), int(seed),
                                              _ptr(step_dev), int(step), int(depth), _ptr(q_out), _ptr(token_out),
                                              _ptr(flags_out), _ptr(ws), ws.numel(), _stream(stream)))


def w8_quantize_host(w: np.ndarray):
    """fp32 [N][K] host array -> (codes u8 [N][K] holding c + 128, scales u16 [N][K/64])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    codes = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N, K // 64), dtype=np.uint16)
    _check("vw4_w8_quantize_host", lib().vw4_w8_quantize_host(w.ctypes.data_as(ctypes.c_void_p), N, K,
                                                              codes.ctypes.data_as(ctypes.c_void_p),
                                                              scales.ctypes.data_as(ctypes.c_void_p)))
    return codes, scales


def w8_pack(codes, scales, N: int, K: int, hi, lo, pscales, stream=None):
    _check("vw4_w8_pack", lib().vw4_w8_pack(_ptr(codes), _ptr(scales), N, K, _ptr(hi), _ptr(lo), _ptr(pscales),
                                            _stream(stream)))


def w8_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().vw4_w8_workspace_bytes(M, N, K))


def w8_skinny_gemm(x, w_hi, w_lo, scales_packed, y, M: int, N: int, K: int, ws=None, stream=None,
                   ldx: int | None = None, ldy: int | None = None):
    """y[M][N] (fp32 or bf16 tensor) = x[M][K] (bf16 bits) @ W8^T."""
    import torch
    ydt = VW4_F32 if y.dtype == torch.float32 else VW4_BF16
    ldx = x.stride(0) if ldx is None else ldx
    ldy = y.stride(0) if ldy is None else ldy
    nbytes = ws.numel() if ws is not None else 0
    _check("w8_skinny_gemm", lib().w8_skinny_gemm(_ptr(x), ldx, _ptr(w_hi), _ptr(w_lo), _ptr(scales_packed), _ptr(y),
                                                  ldy, ydt, M, N, K, _ptr(ws), nbytes, _stream(stream)))
    return y


def w8_partials_layout(M: int, N: int, K: int):
    S, ldp = ctypes.c_int32(0), ctypes.c_int64(0)
    _check("vw4_w8_partials_layout", lib().vw4_w8_partials_layout(M, N, K, ctypes.byref(S), ctypes.byref(ldp)))
    return int(S.value), int(ldp.value)


def w8_skinny_gemm_partials(x, w_hi, w_lo, scales_packed, part, M: int, N: int, K: int, stream=None,
                            ldx: int | None = None):
    ldx = x.stride(0) if ldx is None else ldx
    _check("w8_skinny_gemm_partials", lib().w8_skinny_gemm_partials(_ptr(x), ldx, _ptr(w_hi), _ptr(w_lo),
                                                                    _ptr(scales_packed), _ptr(part), M, N, K,
                                                                    _stream(stream)))


def w16_pack(w, N: int, K: int, packed, stream=None):
    """16-bit weights (fp16 or bf16 bit patterns, device [N][K]) -> the operand-tiled layout."""
    _check("vw4_w16_pack", lib().vw4_w16_pack(_ptr(w), N, K, _ptr(packed), _stream(stream)))


def w16_workspace_bytes(M: int, N: int, K: int, kind: str = "f16") -> int:
    return int(getattr(lib(), f"vw4_{kind}_workspace_bytes")(M, N, K))


def w16_partials_layout(M: int, N: int, K: int, kind: str = "f16"):
    S, ldp = ctypes.c_int32(0), ctypes.c_int64(0)
    name = f"vw4_{kind}_partials_layout"
    _check(name, getattr(lib(), name)(M, N, K, ctypes.byref(S), ctypes.byref(ldp)))
    return int(S.value), int(ldp.value)


def w16_skinny_gemm(x, w_packed, y, M: int, N: int, K: int, kind: str = "f16", ws=None, stream=None,
                    ldx: int | None = None, ldy: int | None = None):
    """y[M][N] (fp32 or bf16 tensor) = x[M][K] (bf16 bits) @ W^T, W fp16 (kind "f16") or bf16 ("bf16")."""
    import torch
    assert kind in ("f16", "bf16")
    ydt = VW4_F32 if y.dtype == torch.float32 else VW4_BF16
    ldx = x.stride(0) if ldx is None else ldx
    ldy = y.stride(0) if ldy is None else ldy
    nbytes = ws.numel() if ws is not None else 0
    name = f"{kind}_skinny_gemm"
    _check(name, getattr(lib(), name)(_ptr(x), ldx, _ptr(w_packed), _ptr(y), ldy, ydt, M, N, K, _ptr(ws), nbytes,
                                      _stream(stream)))
    return y


def w16_skinny_gemm_partials(x, w_packed, part, M: int, N: int, K: int, kind: str = "f16", stream=None,
                             ldx: int | None = None):
    assert kind in ("f16", "bf16")
    ldx = x.stride(0) if ldx is None else ldx
    name = f"{kind}_skinny_gemm_partials"
    _check(name, getattr(lib(), name)(_ptr(x), ldx, _ptr(w_packed), _ptr(part), M, N, K, _stream(stream)))
    return part


def w3_quantize_host(w: np.ndarray):
    """fp32 [N][K] host array -> (codes u8 [N][K] holding c + 4, scales u16 [N][K/64])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    codes = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N, K // 64), dtype=np.uint16)
    _check("vw4_w3_quantize_host", lib().vw4_w3_quantize_host(w.ctypes.data_as(ctypes.c_void_p), N, K,
                                                              codes.ctypes.data_as(ctypes.c_void_p),
                                                              scales.ctypes.data_as(ctypes.c_void_p)))
    return codes, scales


def w3_pack(codes, scales, N: int, K: int, hi, lo, pscales, stream=None):
    _check("vw4_w3_pack", lib().vw4_w3_pack(_ptr(codes), _ptr(scales), N, K, _ptr(hi), _ptr(lo), _ptr(pscales),
                                            _stream(stream)))


def w3_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().vw4_w3_workspace_bytes(M, N, K))


def w3_partials_layout(M: int, N: int, K: int):
    S, ldp = ctypes.c_int32(0), ctypes.c_int64(0)
    _check("vw4_w3_partials_layout", lib().vw4_w3_partials_layout(M, N, K, ctypes.byref(S), ctypes.byref(ldp)))
    return int(S.value), int(ldp.value)


def w3_skinny_gemm_partials(x, w_hi, w_lo, scales_packed, part, M: int, N: int, K: int, stream=None,
                            ldx: int | None = None):
    ldx = x.stride(0) if ldx is None else ldx
    _check("w3_skinny_gemm_partials", lib().w3_skinny_gemm_partials(_ptr(x), ldx, _ptr(w_hi), _ptr(w_lo),
                                                                    _ptr(scales_packed), _ptr(part), M, N, K,
                                                                    _stream(stream)))


def w3_skinny_gemm(x, w_hi, w_lo, scales_packed, y, M: int, N: int, K: int, ws=None, stream=None,
                   ldx: int | None = None, ldy: int | None = None):
    """y[M][N] (fp32 or bf16 tensor) = x[M][K] (bf16 bits) @ W3^T."""
    import torch
    ydt = VW4_F32 if y.dtype == torch.float32 else VW4_BF16
    ldx = x.stride(0) if ldx is None else ldx
    ldy = y.stride(0) if ldy is None else ldy
    nbytes = ws.numel() if ws is not None else 0
    _check("w3_skinny_gemm", lib().w3_skinny_gemm(_ptr(x), ldx, _ptr(w_hi), _ptr(w_lo), _ptr(scales_packed), _ptr(y),
                                                  ldy, ydt, M, N, K, _ptr(ws), nbytes, _stream(stream)))
    return y


def w2_quantize_host(w: np.ndarray):
    """fp32 [N][K] host array -> (codes u8 [N][K] holding c + 1, scales u16 [N][K/64])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    codes = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N, K // 64), dtype=np.uint16)
    _check("vw4_w2_quantize_host", lib().vw4_w2_quantize_host(w.ctypes.data_as(ctypes.c_void_p), N, K,
                                                              codes.ctypes.data_as(ctypes.c_void_p),
                                                              scales.ctypes.data_as(ctypes.c_void_p)))
    return codes, scales


def w2_pack(codes, scales, N: int, K: int, packed, pscales, stream=None):
    _check("vw4_w2_pack", lib().vw4_w2_pack(_ptr(codes), _ptr(scales), N, K, _ptr(packed), _ptr(pscales),
                                            _stream(stream)))


def w2_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().vw4_w2_workspace_bytes(M, N, K))


def w2_partials_layout(M: int, N: int, K: int):
    S, ldp = ctypes.c_int32(0), ctypes.c_int64(0)
    _check("vw4_w2_partials_layout", lib().vw4_w2_partials_layout(M, N, K, ctypes.byref(S), ctypes.byref(ldp)))
    return int(S.value), int(ldp.value)


def w2_skinny_gemm_partials(x, w_packed, scales_packed, part, M: int, N: int, K: int, stream=None,
                            ldx: int | None = None):
    ldx = x.stride(0) if ldx is None else ldx
    _check("w2_skinny_gemm_partials", lib().w2_skinny_gemm_partials(_ptr(x), ldx, _ptr(w_packed),
                                                                    _ptr(scales_packed), _ptr(part), M, N, K,
                                                                    _stream(stream)))


def w2_skinny_gemm(x, w_packed, scales_packed, y, M: int, N: int, K: int, ws=None, stream=None,
                   ldx: int | None = None, ldy: int | None = None):
    """y[M][N] (fp32 or bf16 tensor) = x[M][K] (bf16 bits) @ W2^T."""
    import torch
    ydt = VW4_F32 if y.dtype == torch.float32 else VW4_BF16
    ldx = x.stride(0) if ldx is None else ldx
    ldy = y.stride(0) if ldy is None else ldy
    nbytes = ws.numel() if ws is not None else 0
    _check("w2_skinny_gemm", lib().w2_skinny_gemm(_ptr(x), ldx, _ptr(w_packed), _ptr(scales_packed), _ptr(y),
                                                  ldy, ydt, M, N, K, _ptr(ws), nbytes, _stream(stream)))
    return y


def w5_quantize_host(w: np.ndarray):
    """fp32 [N][K] host array -> (codes u8 [N][K] holding c + 16, scales u16 [N][K/64])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    codes = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N, K // 64), dtype=np.uint16)
    _check("vw4_w5_quantize_host", lib().vw4_w5_quantize_host(w.ctypes.data_as(ctypes.c_void_p), N, K,
                                                              codes.ctypes.data_as(ctypes.c_void_p),
                                                              scales.ctypes.data_as(ctypes.c_void_p)))
    return codes, scales


def w5_pack(codes, scales, N: int, K: int, hi, lo, pscales, stream=None):
    _check("vw4_w5_pack", lib().vw4_w5_pack(_ptr(codes), _ptr(scales), N, K, _ptr(hi), _ptr(lo), _ptr(pscales),
                                            _stream(stream)))


def w5_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().vw4_w5_workspace_bytes(M, N, K))


def w5_partials_layout(M: int, N: int, K: int):
    S, ldp = ctypes.c_int32(0), ctypes.c_int64(0)
    _check("vw4_w5_partials_layout", lib().vw4_w5_partials_layout(M, N, K, ctypes.byref(S), ctypes.byref(ldp)))
    return int(S.value), int(ldp.value)


def w5_skinny_gemm_partials(x, w_hi, w_lo, scales_packed, part, M: int, N: int, K: int, stream=None,
                            ldx: int | None = None):
    ldx = x.stride(0) if ldx is None else ldx
    _check("w5_skinny_gemm_partials", lib().w5_skinny_gemm_partials(_ptr(x), ldx, _ptr(w_hi), _ptr(w_lo),
                                                                    _ptr(scales_packed), _ptr(part), M, N, K,
                                                                    _stream(stream)))


def w5_skinny_gemm(x, w_hi, w_lo, scales_packed, y, M: int, N: int, K: int, ws=None, stream=None,
                   ldx: int | None = None, ldy: int | None = None):
    """y[M][N] (fp32 or bf16 tensor) = x[M][K] (bf16 bits) @ W5^T."""
    import torch
    ydt = VW4_F32 if y.dtype == torch.float32 else VW4_BF16
    ldx = x.stride(0) if ldx is None else ldx
    ldy = y.stride(0) if ldy is None else ldy
    nbytes = ws.numel() if ws is not None else 0
    _check("w5_skinny_gemm", lib().w5_skinny_gemm(_ptr(x), ldx, _ptr(w_hi), _ptr(w_lo), _ptr(scales_packed), _ptr(y),
                                                  ldy, ydt, M, N, K, _ptr(ws), nbytes, _stream(stream)))
    return y


def w6_quantize_host(w: np.ndarray):
    """fp32 [N][K] host array -> (codes u8 [N][K] holding c + 32, scales u16 [N][K/64])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    codes = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N, K // 64), dtype=np.uint16)
    _check("vw4_w6_quantize_host", lib().vw4_w6_quantize_host(w.ctypes.data_as(ctypes.c_void_p), N, K,
                                                              codes.ctypes.data_as(ctypes.c_void_p),
                                                              scales.ctypes.data_as(ctypes.c_void_p)))
    return codes, scales


def w6_pack(codes, scales, N: int, K: int, hi, lo, pscales, stream=None):
    _check("vw4_w6_pack", lib().vw4_w6_pack(_ptr(codes), _ptr(scales), N, K, _ptr(hi), _ptr(lo), _ptr(pscales),
                                            _stream(stream)))


def w6_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().vw4_w6_workspace_bytes(M, N, K))


def w6_partials_layout(M: int, N: int, K: int):
    S, ldp = ctypes.c_int32(0), ctypes.c_int64(0)
    _check("vw4_w6_partials_layout", lib().vw4_w6_partials_layout(M, N, K, ctypes.byref(S), ctypes.byref(ldp)))
    return int(S.value), int(ldp.value)


def w6_skinny_gemm_partials(x, w_hi, w_lo, scales_packed, part, M: int, N: int, K: int, stream=None,
                            ldx: int | None = None):
    ldx = x.stride(0) if ldx is None else ldx
    _check("w6_skinny_gemm_partials", lib().w6_skinny_gemm_partials(_ptr(x), ldx, _ptr(w_hi), _ptr(w_lo),
                                                                    _ptr(scales_packed), _ptr(part), M, N, K,
                                                                    _stream(stream)))


def w6_skinny_gemm(x, w_hi, w_lo, scales_packed, y, M: int, N: int, K: int, ws=None, stream=None,
                   ldx: int | None = None, ldy: int | None = None):
    """y[M][N] (fp32 or bf16 tensor) = x[M][K] (bf16 bits) @ W6^T."""
    import torch
    ydt = VW4_F32 if y.dtype == torch.float32 else VW4_BF16
    ldx = x.stride(0) if ldx is None else ldx
    ldy = y.stride(0) if ldy is None else ldy
    nbytes = ws.numel() if ws is not None else 0
    _check("w6_skinny_gemm", lib().w6_skinny_gemm(_ptr(x), ldx, _ptr(w_hi), _ptr(w_lo), _ptr(scales_packed), _ptr(y),
                                                  ldy, ydt, M, N, K, _ptr(ws), nbytes, _stream(stream)))
    return y


def rowstats_to_numpy(stats_tensor) -> np.ndarray:
    return stats_tensor.detach().cpu().numpy().view(ROWSTAT_DTYPE)


# ---------------------------------------------------------------------------
# decoder-layer calls
# ---------------------------------------------------------------------------
def gemm_partials_layout(M: int, N: int, K: int):
    S = ctypes.c_int32(0)
    ldp = ctypes.c_int64(0)
    _check("vw4_gemm_partials_layout", lib().vw4_gemm_partials_layout(M, N, K, ctypes.byref(S), ctypes.byref(ldp)))
    return int(S.value), int(ldp.value)


def w4_skinny_gemm_partials(x, w_packed, scales_packed, part, M: int, N: int, K: int, stream=None,
                            ldx: int | None = None):
    ldx = x.stride(0) if ldx is None else ldx
    _check("w4_skinny_gemm_partials", lib().w4_skinny_gemm_partials(_ptr(x), ldx, _ptr(w_packed), _ptr(scales_packed),
                                                                    _ptr(part), M, N, K, _stream(stream)))
    return part


def norm_workspace_bytes(M: int, D: int) -> int:
    return int(lib().vw4_norm_workspace_bytes(M, D))


def add_rmsnorm(resid, part, S: int, ldp: int, gamma, eps: float, M: int, D: int, h, ws, stream=None):
    _check("vw4_add_rmsnorm", lib().vw4_add_rmsnorm(_ptr(resid), _ptr(part), S, ldp, _ptr(gamma), float(eps), M, D,
                                                    _ptr(h), _ptr(ws), ws.numel(), _stream(stream)))
    return resid, h


def rope_kv_append(part, S: int, ldp: int, M: int, nq: int, nkv: int, hd: int, L: int, theta: float, q_out, Kc, Vc,
                   Lmax: int, stream=None):
    _check("vw4_rope_kv_append", lib().vw4_rope_kv_append(_ptr(part), S, ldp, M, nq, nkv, hd, L, float(theta),
                                                          _ptr(q_out), _ptr(Kc), _ptr(Vc), Lmax, _stream(stream)))
    return q_out


def swiglu(part, S: int, ldp: int, M: int, F: int, a, stream=None):
    _check("vw4_swiglu", lib().vw4_swiglu(_ptr(part), S, ldp, M, F, _ptr(a), _stream(stream)))
    return a


def attn_workspace_bytes(M: int, nq: int, nkv: int, hd: int, ctx: int) -> int:
    return int(lib().vw4_attn_workspace_bytes(M, nq, nkv, hd, ctx))


def moe_add_rmsnorm(resid_in, part, S: int, ldp: int, p_sstride: int, row_slot, weights, topk: int, gamma,
                    eps: float, M: int, D: int, resid_out, h, stream=None):
    _check("vw4_moe_add_rmsnorm",
           lib().vw4_moe_add_rmsnorm(_ptr(resid_in), _ptr(part), S, ldp, p_sstride, _ptr(row_slot), _ptr(weights),
                                     topk, _ptr(gamma), float(eps), M, D, _ptr(resid_out), _ptr(h), _stream(stream)))
    return resid_out, h


def decode_attn(q, Kc, Vc, Lmax: int, L: int, M: int, nq: int, nkv: int, hd: int, out, ws, stream=None):
    _check("vw4_decode_attn", lib().vw4_decode_attn(_ptr(q), _ptr(Kc), _ptr(Vc), Lmax, L, M, nq, nkv, hd, _ptr(out),
                                                    _ptr(ws), ws.numel(), _stream(stream)))
    return out


def moe_route(logits, M: int, E: int, topk: int, experts, weights, slot_expert, n_slots, row_slot, stream=None):
    _check("vw4_moe_route", lib().vw4_moe_route(_ptr(logits), M, E, topk, _ptr(experts), _ptr(weights),
                                                _ptr(slot_expert), _ptr(n_slots), _ptr(row_slot), _stream(stream)))


def grouped_gemm_layout(M: int, N: int, K: int, max_slots: int):
    S = ctypes.c_int32(0)
    ldp = ctypes.c_int64(0)
    _check("vw4_grouped_gemm_layout",
           lib().vw4_grouped_gemm_layout(M, N, K, max_slots, ctypes.byref(S), ctypes.byref(ldp)))
    return int(S.value), int(ldp.value)


def w4_grouped_gemm(x, ldx: int, x_sstride: int, w_bank, w_estride: int, s_bank, s_estride: int, slot_expert,
                    n_slots, max_slots: int, part, p_sstride: int, M: int, N: int, K: int, stream=None):
    _check("w4_grouped_gemm", lib().w4_grouped_gemm(_ptr(x), ldx, x_sstride, _ptr(w_bank), w_estride, _ptr(s_bank),
                                                    s_estride, _ptr(slot_expert), _ptr(n_slots), max_slots,
                                                    _ptr(part), p_sstride, M, N, K, _stream(stream)))
    return part


def grouped_swiglu(part, S: int, ldp: int, p_sstride: int, M: int, F: int, a, a_sstride: int, n_slots,
                   max_slots: int, stream=None):
    _check("vw4_grouped_swiglu", lib().vw4_grouped_swiglu(_ptr(part), S, ldp, p_sstride, M, F, _ptr(a), a_sstride,
                                                          _ptr(n_slots), max_slots, _stream(stream)))
    return a


def moe_combine(part, S: int, ldp: int, p_sstride: int, row_slot, weights, M: int, topk: int, D: int, y, ldy: int,
                stream=None):
    _check("vw4_moe_combine", lib().vw4_moe_combine(_ptr(part), S, ldp, p_sstride, _ptr(row_slot), _ptr(weights), M,
                                                    topk, D, _ptr(y), ldy, _stream(stream)))
    return y


def add_rmsnorm_out(resid_in, part, S: int, ldp: int, gamma, eps: float, M: int, D: int, resid_out, h,
                    stream=None):
    _check("vw4_add_rmsnorm_out", lib().vw4_add_rmsnorm_out(_ptr(resid_in), _ptr(part), S, ldp, _ptr(gamma),
                                                            float(eps), M, D, _ptr(resid_out), _ptr(h),
                                                            _stream(stream)))
    return resid_out, h


def add_sumsq(resid, part, S: int, ldp: int, M: int, D: int, ws, stream=None):
    _check("vw4_add_sumsq", lib().vw4_add_sumsq(_ptr(resid), _ptr(part), S, ldp, M, D, _ptr(ws), ws.numel(),
                                                _stream(stream)))


def w4_skinny_gemm_rmsnorm_partials(resid, gamma, norm_ws, eps: float, w_packed, scales_packed, part, M: int, N: int,
                                    K: int, stream=None):
    _check("w4_skinny_gemm_rmsnorm_partials",
           lib().w4_skinny_gemm_rmsnorm_partials(_ptr(resid), _ptr(gamma), _ptr(norm_ws), eps, _ptr(w_packed),
                                                 _ptr(scales_packed), _ptr(part), M, N, K, _stream(stream)))
    return part


def w4_skinny_gemm_rmsnorm_swiglu(resid, gamma, norm_ws, eps: float, w_packed, scales_packed, a, lda: int, M: int,
                                  F: int, K: int, stream=None):
    _check("w4_skinny_gemm_rmsnorm_swiglu",
           lib().w4_skinny_gemm_rmsnorm_swiglu(_ptr(resid), _ptr(gamma), _ptr(norm_ws), eps, _ptr(w_packed),
                                               _ptr(scales_packed), _ptr(a), lda, M, F, K, _stream(stream)))
    return a


def w4_grouped_gemm_swiglu(x, ldx: int, x_sstride: int, w_bank, w_estride: int, s_bank, s_estride: int, slot_expert,
                           n_slots, max_slots: int, a, a_sstride: int, M: int, F: int, K: int, stream=None):
    _check("w4_grouped_gemm_swiglu",
           lib().w4_grouped_gemm_swiglu(_ptr(x), ldx, x_sstride, _ptr(w_bank), w_estride, _ptr(s_bank), s_estride,
                                        _ptr(slot_expert), _ptr(n_slots), max_slots, _ptr(a), a_sstride, M, F, K,
                                        _stream(stream)))
    return a


def interleave_gate_up(w):
    """[2F][K] gate|up rows (gate rows 0..F-1, up rows F..2F-1; numpy or torch)
    -> the gate/up-interleaved row order of the fused SwiGLU GEMM: rows
    64 t .. +32 = gate rows 32 t .. +32, rows 64 t + 32 .. +32 = up rows
    32 t .. +32."""
    F = w.shape[0] // 2
    assert w.shape[0] == 2 * F and F % 32 == 0
    import numpy as _np
    order = _np.empty(2 * F, dtype=_np.int64)
    for t in range(F // 32):
        order[64 * t:64 * t + 32] = _np.arange(32 * t, 32 * t + 32)
        order[64 * t + 32:64 * t + 64] = F + _np.arange(32 * t, 32 * t + 32)
    if isinstance(w, _np.ndarray):
        return _np.ascontiguousarray(w[order])
    import torch
    return w[torch.as_tensor(order, device=w.device)].contiguous()


def two_plane_gemm_swiglu(fmt: str, x, w_hi, w_lo, scales_packed, a, lda: int, M: int, F: int, K: int,
                          stream=None, ldx: int | None = None):
    """Gate|up with the SwiGLU epilogue in a two-plane format (fmt w8, w6, w5, w3; gate/up-interleaved rows)."""
    assert fmt in ("w8", "w6", "w5", "w3")
    ldx = x.stride(0) if ldx is None else ldx
    name = f"{fmt}_skinny_gemm_swiglu"
    _check(name, getattr(lib(), name)(_ptr(x), ldx, _ptr(w_hi), _ptr(w_lo), _ptr(scales_packed), _ptr(a), lda, M, F,
                                      K, _stream(stream)))
    return a


def w2_skinny_gemm_swiglu(x, w_packed, scales_packed, a, lda: int, M: int, F: int, K: int, stream=None,
                          ldx: int | None = None):
    ldx = x.stride(0) if ldx is None else ldx
    _check("w2_skinny_gemm_swiglu", lib().w2_skinny_gemm_swiglu(_ptr(x), ldx, _ptr(w_packed), _ptr(scales_packed),
                                                                _ptr(a), lda, M, F, K, _stream(stream)))
    return a


def w16_skinny_gemm_swiglu(x, w_packed, a, lda: int, M: int, F: int, K: int, kind: str = "f16", stream=None,
                           ldx: int | None = None):
    assert kind in ("f16", "bf16")
    ldx = x.stride(0) if ldx is None else ldx
    name = f"{kind}_skinny_gemm_swiglu"
    _check(name, getattr(lib(), name)(_ptr(x), ldx, _ptr(w_packed), _ptr(a), lda, M, F, K, _stream(stream)))
    return a


def w4_skinny_gemm_swiglu(x, w_packed, scales_packed, a, lda: int, M: int, F: int, K: int, stream=None,
                          ldx: int | None = None):
    ldx = x.stride(0) if ldx is None else ldx
    _check("w4_skinny_gemm_swiglu", lib().w4_skinny_gemm_swiglu(_ptr(x), ldx, _ptr(w_packed), _ptr(scales_packed),
                                                                _ptr(a), lda, M, F, K, _stream(stream)))
    return a
