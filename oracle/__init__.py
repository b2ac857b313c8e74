"""CPU oracle for the batched verify step (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library under
``verify_step_w4_amd/`` never imports, links or calls it, and it imports
nothing from the product: the two share only the seeded input generators in
``verify_step_w4_amd/synth.py`` (which hold none of the method's arithmetic).

The arithmetic lives in ``oracle/oracle.c`` (plain C, IEEE binary64,
sequential sums in the order of each definition) and ``oracle/exact_law.py``
(rational arithmetic).  This module is argument marshalling over ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# VW4_ORACLE_LIB selects another build of the same source (the sanitizer build
# that tests/test_host_sanitizers.py runs the oracle pins against)
_LIB_PATH = os.environ.get("VW4_ORACLE_LIB") or os.path.join(_HERE, "_build", "liboracle.so")

_FLAGS = ["-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-fno-fast-math", "-ffp-contract=off"]
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into oracle/_build/liboracle.so."""
    path = os.path.join(_HERE, "_build", "liboracle.so")
    if not force and os.path.exists(path):
        return path
    os.makedirs(os.path.dirname(path), exist_ok=True)
    tmp = path + ".tmp"
    subprocess.run(["gcc", "-O2", *_FLAGS, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, path)
    return path


def build_sanitized(path: str) -> str:
    """The same source with AddressSanitizer and UndefinedBehaviorSanitizer
    (gcc; any report aborts).  Load it only in a process that preloads gcc's
    libasan first."""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    subprocess.run(["gcc", *SANITIZE_FLAGS, *_FLAGS, "-o", path, _SRC, "-lm"], check=True)
    return path


class WarpStat(ctypes.Structure):
    _fields_ = [("m", ctypes.c_double), ("tau", ctypes.c_double), ("E", ctypes.c_double),
                ("Z", ctypes.c_double), ("log_z", ctypes.c_double), ("P", ctypes.c_double),
                ("S_at", ctypes.c_double), ("S_before", ctypes.c_double),
                ("argmax", ctypes.c_int64), ("n_kept", ctypes.c_int64), ("k_star", ctypes.c_int64),
                ("flags", ctypes.c_uint32), ("pad", ctypes.c_uint32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_ if f != "pad"}


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_U64 = ctypes.c_uint64
_F32 = ctypes.c_float
_F64 = ctypes.c_double


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) and not os.environ.get("VW4_ORACLE_LIB"):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_f32_to_f16.argtypes = [_F32]
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_f16_value.argtypes = [ctypes.c_uint16]
        L.oracle_f16_value.restype = _F64
        L.oracle_bf16_round.argtypes = [_F64]
        L.oracle_bf16_round.restype = ctypes.c_uint16
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_value.restype = _F64
        L.oracle_w4_quantize.argtypes = [_P, _I64, _I64, _P, _P]
        L.oracle_w4_code.argtypes = [_P, _I64, _I64, _I64]
        L.oracle_w4_code.restype = ctypes.c_int
        L.oracle_w4_gemm.argtypes = [_P, _I64, _I64, _P, _P, _I64, _P]
        L.oracle_w4_gemm_at.argtypes = [_P, _I64, _P, _P, _P]
        L.oracle_warp.argtypes = [_P, _I64, _F32, _F32, ctypes.POINTER(WarpStat), _P]
        L.oracle_philox4x64_10.argtypes = [_P, _P, _P]
        L.oracle_verify_uniforms.argtypes = [_U64, _U64, _I32, _P, _P]
        L.oracle_accept_with_uniforms.argtypes = [_P, ctypes.POINTER(WarpStat), _P, _P, _I32, _I64,
                                                  _F32, _P, _P, _P, _P, _P]
        L.oracle_spec_accept.argtypes = [_P, _P, _P, _I32, _I64, _F32, _F32, _U64, _U64,
                                         ctypes.POINTER(WarpStat), _P, _P, _P]
        L.oracle_spec_accept_trials.argtypes = [_P, _P, _P, _I64, _I32, _I64, _F32, _F32, _U64,
                                                _U64, _P, _P, _P]
        L.oracle_rmsnorm.argtypes = [_P, _P, _I64, _I64, _F64, _P]
        L.oracle_swiglu.argtypes = [_P, _P, _I64, _P]
        L.oracle_rope.argtypes = [_P, _I64, _I64, _F64, _P]
        L.oracle_decode_attn.argtypes = [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _P]
        L.oracle_moe_route.argtypes = [_P, _I64, _I64, _I64, _P, _P]
        L.oracle_swiglu_f64.argtypes = [_P, _P, _I64, _P]
        L.oracle_mtp_input.argtypes = [_P, _P, _P, _P, _I64, _F64, _P]
        L.oracle_w8_quantize.argtypes = [_P, _I64, _I64, _P, _P]
        L.oracle_w8_gemm.argtypes = [_P, _I64, _I64, _P, _P, _I64, _P]
        L.oracle_w5_quantize.argtypes = [_P, _I64, _I64, _P, _P]
        L.oracle_w5_gemm.argtypes = [_P, _I64, _I64, _P, _P, _I64, _P]
        L.oracle_f16_gemm.argtypes = [_P, _I64, _I64, _P, _I64, _P]
        L.oracle_b16_gemm.argtypes = [_P, _I64, _I64, _P, _I64, _P]
        L.oracle_w3_quantize.argtypes = [_P, _I64, _I64, _P, _P]
        L.oracle_w3_gemm.argtypes = [_P, _I64, _I64, _P, _P, _I64, _P]
        L.oracle_w2_quantize.argtypes = [_P, _I64, _I64, _P, _P]
        L.oracle_w2_gemm.argtypes = [_P, _I64, _I64, _P, _P, _I64, _P]
        L.oracle_w6_quantize.argtypes = [_P, _I64, _I64, _P, _P]
        L.oracle_w6_gemm.argtypes = [_P, _I64, _I64, _P, _P, _I64, _P]
        L.oracle_embed_rows.argtypes = [_P, _I64, _I64, _P, _I64, _P]
        L.oracle_draft_uniform.argtypes = [_U64, _U64, _I32]
        L.oracle_draft_uniform.restype = _F64
        L.oracle_draft_sample.argtypes = [_P, _I64, _F32, _F32, _U64, _U64, _I32, _P, ctypes.POINTER(WarpStat),
                                          _P, _P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------
def f32_to_f16_bits(x: float) -> int:
    return int(lib().oracle_f32_to_f16(float(np.float32(x))))


def f16_value(bits: int) -> float:
    return float(lib().oracle_f16_value(int(bits)))


def bf16_round(v) -> np.ndarray:
    """Round float64 values to bfloat16 bits (one RNE rounding)."""
    a = np.asarray(v, dtype=np.float64)
    f = lib().oracle_bf16_round
    return np.array([f(float(x)) for x in a.reshape(-1)], dtype=np.uint16).reshape(a.shape)


def bf16_value(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    f = lib().oracle_bf16_value
    return np.array([f(int(x)) for x in b.reshape(-1)], dtype=np.float64).reshape(b.shape)


# --------------------------------------------------------------------------
# (a1) quantizer and (a2/a3) GEMM
# --------------------------------------------------------------------------
def w4_quantize(w: np.ndarray):
    """w: float32 [N][K] (K % 64 == 0) -> (codes u8 [N][K/2], scales u16 [N][K/64])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % 64 == 0
    codes = np.zeros((N, K // 2), dtype=np.uint8)
    scales = np.zeros((N, K // 64), dtype=np.uint16)
    lib().oracle_w4_quantize(_ptr(w), N, K, _ptr(codes), _ptr(scales))
    return codes, scales


def w4_codes_int(codes: np.ndarray) -> np.ndarray:
    """Signed integer codes [N][K] from the canonical packed layout."""
    N, K2 = codes.shape
    out = np.empty((N, K2 * 2), dtype=np.int8)
    L = lib()
    for n in range(N):
        for k in range(K2 * 2):
            out[n, k] = L.oracle_w4_code(_ptr(codes), K2 * 2, n, k)
    return out


def w4_gemm(x_bf16: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """x_bf16: uint16 [M][K]; returns float64 [M][N]."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, K = x_bf16.shape
    N = codes.shape[0]
    assert codes.shape == (N, K // 2) and scales.shape == (N, K // 64)
    y = np.zeros((M, N), dtype=np.float64)
    lib().oracle_w4_gemm(_ptr(x_bf16), M, K, _ptr(np.ascontiguousarray(codes)),
                         _ptr(np.ascontiguousarray(scales)), N, _ptr(y))
    return y


def w4_gemm_at(x_row_bf16: np.ndarray, codes: np.ndarray, scales: np.ndarray, n: int) -> float:
    x = np.ascontiguousarray(x_row_bf16, dtype=np.uint16)
    K = x.shape[0]
    crow = np.ascontiguousarray(codes[n])
    srow = np.ascontiguousarray(scales[n])
    out = np.zeros(1, dtype=np.float64)
    lib().oracle_w4_gemm_at(_ptr(x), K, _ptr(crow), _ptr(srow), _ptr(out))
    return float(out[0])


# --------------------------------------------------------------------------
# (a4) warp, (a5) Philox, (a6/a7) accept/resample
# --------------------------------------------------------------------------
def warp(z: np.ndarray, temperature: float, top_p: float, want_p: bool = False):
    z = np.ascontiguousarray(z, dtype=np.float32)
    V = z.shape[0]
    st = WarpStat()
    p = np.zeros(V, dtype=np.float64) if want_p else None
    lib().oracle_warp(_ptr(z), V, float(temperature), float(top_p), ctypes.byref(st),
                      _ptr(p) if want_p else None)
    return (st, p) if want_p else st


def philox4x64_10(key, ctr):
    k = np.ascontiguousarray(np.array(key, dtype=np.uint64))
    c = np.ascontiguousarray(np.array(ctr, dtype=np.uint64))
    out = np.zeros(4, dtype=np.uint64)
    lib().oracle_philox4x64_10(_ptr(k), _ptr(c), _ptr(out))
    return out


def verify_uniforms(seed: int, step: int, D: int):
    ua = np.zeros(D + 1, dtype=np.float64)
    ur = np.zeros(D + 1, dtype=np.float64)
    lib().oracle_verify_uniforms(int(seed), int(step), int(D), _ptr(ua), _ptr(ur))
    return ua, ur


def accept_with_uniforms(z: np.ndarray, stats, q: np.ndarray, draft: np.ndarray,
                         temperature: float, u_acc: np.ndarray, u_res: np.ndarray):
    z = np.ascontiguousarray(z, dtype=np.float32)
    M, V = z.shape
    D = M - 1
    q = np.ascontiguousarray(q, dtype=np.float32) if D else np.zeros((1, V), np.float32)
    draft = np.ascontiguousarray(np.asarray(draft, dtype=np.int32).reshape(-1)) if D else np.zeros(1, np.int32)
    st = (WarpStat * M)(*stats)
    tok = np.zeros(M, dtype=np.int32)
    nacc = np.zeros(1, dtype=np.int32)
    fl = np.zeros(1, dtype=np.uint32)
    ua = np.ascontiguousarray(u_acc, dtype=np.float64)
    ur = np.ascontiguousarray(u_res, dtype=np.float64)
    lib().oracle_accept_with_uniforms(_ptr(z), st, _ptr(q), _ptr(draft), D, V,
                                      float(temperature), _ptr(ua), _ptr(ur), _ptr(tok),
                                      _ptr(nacc), _ptr(fl))
    return tok, int(nacc[0]), int(fl[0])


def spec_accept(z: np.ndarray, q: np.ndarray, draft: np.ndarray, temperature: float, top_p: float,
                seed: int, step: int):
    """One verify problem. z: float32 [D+1][V], q: float32 [D][V], draft: int32 [D]."""
    z = np.ascontiguousarray(z, dtype=np.float32)
    M, V = z.shape
    D = M - 1
    qq = np.ascontiguousarray(q, dtype=np.float32) if D else np.zeros((1, V), np.float32)
    dr = np.ascontiguousarray(np.asarray(draft, dtype=np.int32).reshape(-1)) if D else np.zeros(1, np.int32)
    st = (WarpStat * M)()
    tok = np.zeros(M, dtype=np.int32)
    nacc = np.zeros(1, dtype=np.int32)
    fl = np.zeros(1, dtype=np.uint32)
    lib().oracle_spec_accept(_ptr(z), _ptr(qq), _ptr(dr), D, V, float(temperature), float(top_p),
                             int(seed), int(step), st, _ptr(tok), _ptr(nacc), _ptr(fl))
    return tok, int(nacc[0]), int(fl[0]), [st[i] for i in range(M)]


def spec_accept_trials(z: np.ndarray, q: np.ndarray, drafts: np.ndarray, temperature: float,
                       top_p: float, seed: int, step0: int):
    """B problems sharing logits z [D+1][V] and q [D][V]; drafts int32 [B][D]."""
    z = np.ascontiguousarray(z, dtype=np.float32)
    M, V = z.shape
    D = M - 1
    drafts = np.ascontiguousarray(drafts, dtype=np.int32).reshape(-1, max(D, 1))
    B = drafts.shape[0]
    qq = np.ascontiguousarray(q, dtype=np.float32) if D else np.zeros((1, V), np.float32)
    tok = np.zeros((B, M), dtype=np.int32)
    nacc = np.zeros(B, dtype=np.int32)
    fl = np.zeros(B, dtype=np.uint32)
    lib().oracle_spec_accept_trials(_ptr(z), _ptr(qq), _ptr(drafts), B, D, V, float(temperature),
                                    float(top_p), int(seed), int(step0), _ptr(tok), _ptr(nacc),
                                    _ptr(fl))
    return tok, nacc, fl


# --------------------------------------------------------------------------
# (a8) glue, (a9) attention, (a10) MoE routing
# --------------------------------------------------------------------------
def rmsnorm(x_bf16: np.ndarray, gamma_bf16: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, D = x.shape
    y = np.zeros((M, D), dtype=np.float64)
    lib().oracle_rmsnorm(_ptr(x), _ptr(np.ascontiguousarray(gamma_bf16, dtype=np.uint16)), M, D,
                         float(eps), _ptr(y))
    return y


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """silu(g) * u; uint16 inputs are bf16 bit patterns, anything else is taken as fp64 values."""
    if np.asarray(g).dtype == np.uint16:
        g = np.ascontiguousarray(g, dtype=np.uint16)
        u = np.ascontiguousarray(u, dtype=np.uint16)
        fn = lib().oracle_swiglu
    else:
        g = np.ascontiguousarray(g, dtype=np.float64)
        u = np.ascontiguousarray(u, dtype=np.float64)
        fn = lib().oracle_swiglu_f64
    assert g.shape == u.shape
    y = np.zeros(g.shape, dtype=np.float64)
    fn(_ptr(g), _ptr(u), g.size, _ptr(y))
    return y


def rope(x: np.ndarray, pos: int, theta: float = 10000.0) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    lib().oracle_rope(_ptr(x), x.shape[0], int(pos), float(theta), _ptr(out))
    return out


def decode_attn(q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, L: int) -> np.ndarray:
    """q float64 [M][Hq][Dh] (rotated); Kc, Vc uint16 bf16 [Hkv][Lc][Dh]."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    M, Hq, Dh = q.shape
    Hkv, Lc, _ = Kc.shape
    out = np.zeros_like(q)
    lib().oracle_decode_attn(_ptr(q), _ptr(np.ascontiguousarray(Kc, dtype=np.uint16)),
                             _ptr(np.ascontiguousarray(Vc, dtype=np.uint16)), M, Hq, Hkv, Dh, L, Lc,
                             _ptr(out))
    return out


def moe_route(logits: np.ndarray, topk: int):
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    M, E = lg.shape
    ex = np.zeros((M, topk), dtype=np.int32)
    wt = np.zeros((M, topk), dtype=np.float64)
    lib().oracle_moe_route(_ptr(lg), M, E, topk, _ptr(ex), _ptr(wt))
    return ex, wt


def moe_block(x_bf16: np.ndarray, router_logits: np.ndarray, topk: int, gate_up, down):
    """Mixture-of-experts FFN of the verify rows, expert by expert in fp64.

    Routing as moe_route (top-k by router logit, softmax weights renormalised
    over the chosen experts).  Expert e: gate|up = gate_up[e] (codes, scales)
    of a [2F][K] W4 matrix whose rows [0, F) are the gate and [F, 2F) the up
    projection; a = bf16(silu(g) * u) on the unrounded products; the expert's
    output is down[e] (a [D][F] W4 matrix) applied to a.  Row m's output is
    sum_t w[m][t] * expert_{experts[m][t]}(x_m), in selection order.
    gate_up / down: (codes [E][N][K/2], scales [E][N][K/64]).
    Returns (experts [M][topk], weights [M][topk], y float64 [M][D]).
    (gist.science, "BaseRT: Best-in-Class LLM Inference on Apple Silicon via
    Native Metal", section "結果": mixture-of-experts models such as
    Qwen3-30B-A3B, 128 experts with 8 active.)"""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M = x.shape[0]
    ex, wt = moe_route(router_logits, topk)
    gu_c, gu_s = gate_up
    dn_c, dn_s = down
    F = gu_c.shape[1] // 2
    D = dn_c.shape[1]
    y = np.zeros((M, D), dtype=np.float64)
    for m in range(M):
        for t in range(topk):
            e = int(ex[m, t])
            gu = w4_gemm(x[m:m + 1], gu_c[e], gu_s[e])
            a = bf16_round(swiglu(gu[:, :F], gu[:, F:]))
            y[m] += wt[m, t] * w4_gemm(a, dn_c[e], dn_s[e])[0]
    return ex, wt, y


# --------------------------------------------------------------------------
# the draft side of the cycle (the MTP head; NEXT row 1 of the hot path)
# --------------------------------------------------------------------------
def mtp_input(h_bf16: np.ndarray, e_bf16: np.ndarray, gamma_h: np.ndarray, gamma_e: np.ndarray,
              eps: float = 1e-6) -> np.ndarray:
    """[rmsnorm(h) * gamma_h ; rmsnorm(e) * gamma_e] in fp64; h, e, gammas: bf16 bits [d]."""
    h = np.ascontiguousarray(h_bf16, dtype=np.uint16).reshape(-1)
    e = np.ascontiguousarray(e_bf16, dtype=np.uint16).reshape(-1)
    d = h.shape[0]
    assert e.shape[0] == d
    out = np.zeros(2 * d, dtype=np.float64)
    lib().oracle_mtp_input(_ptr(h), _ptr(e), _ptr(np.ascontiguousarray(gamma_h, dtype=np.uint16)),
                           _ptr(np.ascontiguousarray(gamma_e, dtype=np.uint16)), d, float(eps), _ptr(out))
    return out


def embed_rows(E: np.ndarray, tokens) -> np.ndarray:
    """Rows E[tokens] of a bf16 [V][d] table; ids outside [0, V) give zero rows."""
    E = np.ascontiguousarray(E, dtype=np.uint16)
    V, d = E.shape
    t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
    out = np.zeros((t.shape[0], d), dtype=np.uint16)
    lib().oracle_embed_rows(_ptr(E), V, d, _ptr(t), t.shape[0], _ptr(out))
    return out


def draft_uniform(seed: int, step: int, depth: int) -> float:
    return float(lib().oracle_draft_uniform(int(seed), int(step), int(depth)))


def draft_sample(z: np.ndarray, temperature: float, top_p: float, seed: int, step: int, depth: int):
    """One draft from logits z [V]: (token, q float32 [V], warp stats, flags)."""
    z = np.ascontiguousarray(z, dtype=np.float32).reshape(-1)
    V = z.shape[0]
    q = np.zeros(V, dtype=np.float32)
    st = WarpStat()
    tok = np.zeros(1, dtype=np.int32)
    fl = np.zeros(1, dtype=np.uint32)
    lib().oracle_draft_sample(_ptr(z), V, float(temperature), float(top_p), int(seed), int(step), int(depth),
                              _ptr(q), ctypes.byref(st), _ptr(tok), _ptr(fl))
    return int(tok[0]), q, st, int(fl[0])


# --------------------------------------------------------------------------
# the W8 weight format (a second format for the skinny GEMM)
# --------------------------------------------------------------------------
def w8_quantize(w: np.ndarray):
    """w: float32 [N][K] (K % 64 == 0) -> (codes u8 [N][K] holding c + 128, scales u16 [N][K/64])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % 64 == 0
    codes = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N, K // 64), dtype=np.uint16)
    lib().oracle_w8_quantize(_ptr(w), N, K, _ptr(codes), _ptr(scales))
    return codes, scales


def w8_gemm(x_bf16: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """x_bf16: uint16 [M][K]; codes u8 [N][K]; returns float64 [M][N]."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, K = x_bf16.shape
    N = codes.shape[0]
    assert codes.shape == (N, K) and scales.shape == (N, K // 64)
    y = np.zeros((M, N), dtype=np.float64)
    lib().oracle_w8_gemm(_ptr(x_bf16), M, K, _ptr(np.ascontiguousarray(codes)), _ptr(np.ascontiguousarray(scales)),
                         N, _ptr(y))
    return y


def w5_quantize(w: np.ndarray):
    """w: float32 [N][K] (K % 64 == 0) -> (codes u8 [N][K] holding c + 16, scales u16 [N][K/64])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % 64 == 0
    codes = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N, K // 64), dtype=np.uint16)
    lib().oracle_w5_quantize(_ptr(w), N, K, _ptr(codes), _ptr(scales))
    return codes, scales


def w5_gemm(x_bf16: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """x_bf16: uint16 [M][K]; codes u8 [N][K] (c + 16); returns float64 [M][N]."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, K = x_bf16.shape
    N = codes.shape[0]
    assert codes.shape == (N, K) and scales.shape == (N, K // 64)
    y = np.zeros((M, N), dtype=np.float64)
    lib().oracle_w5_gemm(_ptr(x_bf16), M, K, _ptr(np.ascontiguousarray(codes)), _ptr(np.ascontiguousarray(scales)),
                         N, _ptr(y))
    return y


def f16_gemm(x_bf16: np.ndarray, w_f16: np.ndarray) -> np.ndarray:
    """x_bf16: uint16 [M][K]; w_f16: uint16 [N][K] (fp16 bit patterns); returns float64 [M][N]."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    w_f16 = np.ascontiguousarray(w_f16, dtype=np.uint16)
    M, K = x_bf16.shape
    N = w_f16.shape[0]
    assert w_f16.shape == (N, K)
    y = np.zeros((M, N), dtype=np.float64)
    lib().oracle_f16_gemm(_ptr(x_bf16), M, K, _ptr(w_f16), N, _ptr(y))
    return y


def b16_gemm(x_bf16: np.ndarray, w_bf16: np.ndarray) -> np.ndarray:
    """x_bf16: uint16 [M][K]; w_bf16: uint16 [N][K] (bf16 bit patterns); returns float64 [M][N]."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    w_bf16 = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    M, K = x_bf16.shape
    N = w_bf16.shape[0]
    assert w_bf16.shape == (N, K)
    y = np.zeros((M, N), dtype=np.float64)
    lib().oracle_b16_gemm(_ptr(x_bf16), M, K, _ptr(w_bf16), N, _ptr(y))
    return y


def w3_quantize(w: np.ndarray):
    """w: float32 [N][K] (K % 64 == 0) -> (codes u8 [N][K] holding c + 4, scales u16 [N][K/64])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % 64 == 0
    codes = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N, K // 64), dtype=np.uint16)
    lib().oracle_w3_quantize(_ptr(w), N, K, _ptr(codes), _ptr(scales))
    return codes, scales


def w3_gemm(x_bf16: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """x_bf16: uint16 [M][K]; codes u8 [N][K] (c + 4); returns float64 [M][N]."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, K = x_bf16.shape
    N = codes.shape[0]
    assert codes.shape == (N, K) and scales.shape == (N, K // 64)
    y = np.zeros((M, N), dtype=np.float64)
    lib().oracle_w3_gemm(_ptr(x_bf16), M, K, _ptr(np.ascontiguousarray(codes)), _ptr(np.ascontiguousarray(scales)),
                         N, _ptr(y))
    return y


def w2_quantize(w: np.ndarray):
    """w: float32 [N][K] (K % 64 == 0) -> (codes u8 [N][K] holding c + 1, scales u16 [N][K/64])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % 64 == 0
    codes = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N, K // 64), dtype=np.uint16)
    lib().oracle_w2_quantize(_ptr(w), N, K, _ptr(codes), _ptr(scales))
    return codes, scales


def w2_gemm(x_bf16: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """x_bf16: uint16 [M][K]; codes u8 [N][K] (c + 1); returns float64 [M][N]."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, K = x_bf16.shape
    N = codes.shape[0]
    assert codes.shape == (N, K) and scales.shape == (N, K // 64)
    y = np.zeros((M, N), dtype=np.float64)
    lib().oracle_w2_gemm(_ptr(x_bf16), M, K, _ptr(np.ascontiguousarray(codes)), _ptr(np.ascontiguousarray(scales)),
                         N, _ptr(y))
    return y


def w6_quantize(w: np.ndarray):
    """w: float32 [N][K] (K % 64 == 0) -> (codes u8 [N][K] holding c + 32, scales u16 [N][K/64])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % 64 == 0
    codes = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N, K // 64), dtype=np.uint16)
    lib().oracle_w6_quantize(_ptr(w), N, K, _ptr(codes), _ptr(scales))
    return codes, scales


def w6_gemm(x_bf16: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """x_bf16: uint16 [M][K]; codes u8 [N][K] (c + 32); returns float64 [M][N]."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, K = x_bf16.shape
    N = codes.shape[0]
    assert codes.shape == (N, K) and scales.shape == (N, K // 64)
    y = np.zeros((M, N), dtype=np.float64)
    lib().oracle_w6_gemm(_ptr(x_bf16), M, K, _ptr(np.ascontiguousarray(codes)), _ptr(np.ascontiguousarray(scales)),
                         N, _ptr(y))
    return y
