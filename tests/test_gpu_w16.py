"""The skinny GEMM on unquantised 16-bit float weights (fp16 and bf16) on the
GPU against the oracle: outputs within the GEMM tolerance for M = 1..8 over
ragged, one-slice and split-K shapes, fp16 weights including subnormals and
the largest finite values; bf16 outputs; partial slices; the packed layout
read back word by word; rows independent of M bit for bit."""
import numpy as np
import pytest

import oracle
from verify_step_w4_amd import binding as B
from verify_step_w4_amd import synth
from verify_step_w4_amd.model import W16Linear

from helpers import GEMM_RTOL, dev, gemm_rel_err, host, log

pytestmark = pytest.mark.gpu

ORACLE = {"f16": oracle.f16_gemm, "bf16": oracle.b16_gemm}


def _weights(kind, seed, N, K, special=False):
    w = synth.normal_f32(synth.rng(seed), (N, K), 0.02)
    if kind == "f16":
        bits = w.astype(np.float16).view(np.uint16).copy()
        if special:   # subnormals, the largest finite values, signed zeros, values with all 11 bits set
            flat = bits.reshape(-1)
            pats = np.array([0x0001, 0x8001, 0x03FF, 0x83FF, 0x7BFF, 0xFBFF, 0x0000, 0x8000, 0x3BFF, 0x07FF],
                            dtype=np.uint16)
            idx = np.linspace(0, flat.size - 1, min(997, flat.size)).astype(np.int64)
            flat[idx] = np.resize(pats, idx.size)
        return bits
    return synth.f32_to_bf16_bits(w)


def _lin(kind, seed, N, K, special=False):
    bits = _weights(kind, seed, N, K, special)
    return bits, W16Linear.from_bits(dev(bits.view(np.int16)), kind)


def _run(kind, x, L, M, N, K, ydtype=None):
    import torch
    y = torch.empty((M, N), dtype=ydtype or torch.float32, device="cuda")
    ws = B.workspace(max(B.w16_workspace_bytes(M, N, K, kind), 256))
    B.w16_skinny_gemm(x, L.packed, y, M, N, K, kind=kind, ws=ws)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("N,K", [(1, 64), (100, 320), (257, 1024), (1000, 2048), (5120, 5120), (64, 17408)])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_gemm_matches_oracle(kind, M, N, K):
    log(f"{kind} gemm M={M} N={N} K={K}")
    bits, L = _lin(kind, 13 * N + K, N, K)
    x = synth.activations_bf16(M * 100 + N + 1, M, K)
    err = gemm_rel_err(_run(kind, dev(x), L, M, N, K), ORACLE[kind](x, bits))
    assert err <= GEMM_RTOL, err


@pytest.mark.parametrize("M,N,K", [(1, 100, 320), (4, 1000, 2048), (8, 257, 1024)])
def test_f16_special_weights(M, N, K):
    """fp16 weights with subnormals, +-65504, signed zeros and full 11-bit
    significands: the exact two-part split keeps every product exact."""
    log(f"f16 special weights M={M} N={N} K={K}")
    bits, L = _lin("f16", 7 * N + K, N, K, special=True)
    x = synth.activations_bf16(N + K, M, K)
    err = gemm_rel_err(_run("f16", dev(x), L, M, N, K), oracle.f16_gemm(x, bits))
    assert err <= GEMM_RTOL, err


@pytest.mark.parametrize("M,N,K", [(4, 1000, 2048), (1, 257, 1024), (6, 5120, 5120)])
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_bf16_output(kind, M, N, K):
    import torch
    from layer_parity import bf16_close
    log(f"{kind} gemm bf16 out M={M} N={N} K={K}")
    bits, L = _lin(kind, 17 * N + K, N, K)
    x = dev(synth.activations_bf16(M + N + 3, M, K))
    y32 = _run(kind, x, L, M, N, K)
    y16 = _run(kind, x, L, M, N, K, ydtype=torch.int16)
    assert np.array_equal(y16, oracle.bf16_round(y32.astype(np.float64)))
    bf16_close(y16, ORACLE[kind](host(x), bits), min_exact=0.9)


@pytest.mark.parametrize("M,N,K", [(4, 5120, 5120), (1, 7168, 5120), (8, 5120, 17408), (3, 100, 320)])
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_partials_sum_to_the_product(kind, M, N, K):
    import torch
    log(f"{kind} partials M={M} N={N} K={K}")
    S, ldp = B.w16_partials_layout(M, N, K, kind)
    assert 1 <= S <= 8 and ldp >= N
    assert all(B.w16_partials_layout(m, N, K, kind) == (S, ldp) for m in range(1, 9))
    bits, L = _lin(kind, 19 * N + K, N, K)
    x = synth.activations_bf16(M + 2 * N, M, K)
    part = torch.full((S * M * ldp,), float("nan"), dtype=torch.float32, device="cuda")
    B.w16_skinny_gemm_partials(dev(x), L.packed, part, M, N, K, kind=kind)
    torch.cuda.synchronize()
    P = host(part).reshape(S, M, ldp)[:, :, :N]
    s = np.zeros((M, N), np.float32)
    for k in range(S):
        s = (s + P[k]).astype(np.float32)
    assert np.isfinite(s).all()
    err = gemm_rel_err(s, ORACLE[kind](x, bits))
    assert err <= GEMM_RTOL, err


def test_packed_layout_reads_back():
    N, K = 100, 320
    log("w16 pack layout")
    bits, L = _lin("f16", 3, N, K)
    words = host(L.packed).view(np.uint16)
    assert words.size == B.lib().vw4_w16_packed_bytes(N, K) // 2
    G = K // 64
    Np = (N + 63) // 64 * 64
    got = np.zeros((Np, K), dtype=np.uint16)
    for n in range(Np):
        t, nb, i = n >> 6, (n >> 4) & 3, n & 15
        for g in range(G):
            for s_ in range(2):
                for kq in range(4):
                    w16 = ((t * G + g) * 8 + 2 * nb + s_) * 64 + 16 * kq + i
                    k = 64 * g + 32 * s_ + 8 * kq
                    got[n, k:k + 8] = words[8 * w16:8 * w16 + 8]
    assert np.array_equal(got[:N], bits) and not got[N:].any()


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_rows_independent_of_m(kind):
    M, N, K = 6, 1000, 2048
    log(f"{kind} row independence")
    bits, L = _lin(kind, 4, N, K)
    x = dev(synth.activations_bf16(5, M, K))
    y = _run(kind, x, L, M, N, K)
    for m in (0, 5):
        assert np.array_equal(_run(kind, x[m:m + 1], L, 1, N, K)[0], y[m])
