"""The W3 and W2 skinny GEMMs (the narrowest weight formats) on the GPU
against the oracle: outputs within the GEMM tolerance for M = 1..8 over
ragged, one-slice and split-K shapes; bf16 outputs; partial slices; the packed
planes decode (from their documented 1-bit and 2-bit layouts; W2's fields in
sign-magnitude) to the oracle's codes; rows are independent of M bit for bit."""
import numpy as np
import pytest

import oracle
from verify_step_w4_amd import binding as B
from verify_step_w4_amd import synth
from verify_step_w4_amd.model import W2Linear, W3Linear

from helpers import GEMM_RTOL, dev, gemm_rel_err, host, log

pytestmark = pytest.mark.gpu

QUANT = {3: oracle.w3_quantize, 2: oracle.w2_quantize}
GEMM = {3: oracle.w3_gemm, 2: oracle.w2_gemm}


def _lin(b, seed, N, K):
    w = synth.normal_f32(synth.rng(seed), (N, K), 0.02)
    codes, scales = QUANT[b](w)
    L = (W3Linear if b == 3 else W2Linear).from_codes(dev(codes), dev(scales))
    return codes, scales, L


def _call(b, x, L, y, M, N, K, ws):
    if b == 3:
        B.w3_skinny_gemm(x, L.hi, L.lo, L.pscales, y, M, N, K, ws=ws)
    else:
        B.w2_skinny_gemm(x, L.packed, L.pscales, y, M, N, K, ws=ws)


def _ws(b, M, N, K):
    return B.workspace(max((B.w3_workspace_bytes if b == 3 else B.w2_workspace_bytes)(M, N, K), 256))


def _run(b, x, L, M, N, K):
    import torch
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    _call(b, x, L, y, M, N, K, _ws(b, M, N, K))
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("N,K", [(1, 64), (100, 320), (257, 1024), (1000, 2048), (5120, 5120), (64, 17408)])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("b", [3, 2])
def test_gemm_matches_oracle(b, M, N, K):
    log(f"w{b} gemm M={M} N={N} K={K}")
    codes, scales, L = _lin(b, 13 * N + K + b, N, K)
    x = synth.activations_bf16(M * 100 + N + 1, M, K)
    err = gemm_rel_err(_run(b, dev(x), L, M, N, K), GEMM[b](x, codes, scales))
    assert err <= GEMM_RTOL, err


@pytest.mark.parametrize("M,N,K", [(4, 1000, 2048), (1, 257, 1024), (6, 5120, 5120)])
@pytest.mark.parametrize("b", [3, 2])
def test_bf16_output(b, M, N, K):
    """bf16 output: the round-to-nearest-even of the call's own fp32 result,
    and within the bf16 bar of the oracle's exact product."""
    import torch
    from layer_parity import bf16_close
    log(f"w{b} gemm bf16 out M={M} N={N} K={K}")
    codes, scales, L = _lin(b, 17 * N + K + b, N, K)
    x = dev(synth.activations_bf16(M + N + 3, M, K))
    y32 = _run(b, x, L, M, N, K)
    y16 = torch.empty((M, N), dtype=torch.int16, device="cuda")
    _call(b, x, L, y16, M, N, K, _ws(b, M, N, K))
    torch.cuda.synchronize()
    assert np.array_equal(host(y16), oracle.bf16_round(y32.astype(np.float64)))
    bf16_close(host(y16), GEMM[b](host(x), codes, scales), min_exact=0.9)


@pytest.mark.parametrize("M,N,K", [(4, 5120, 5120), (1, 7168, 5120), (8, 5120, 17408), (3, 100, 320),
                                   (6, 34816, 5120)])
@pytest.mark.parametrize("b", [3, 2])
def test_partials_sum_to_the_product(b, M, N, K):
    """The partials form: at most 8 slices, a layout that does not depend on M,
    and the S slices summed in slice order give the oracle's product."""
    import torch
    log(f"w{b} partials M={M} N={N} K={K}")
    layout = B.w3_partials_layout if b == 3 else B.w2_partials_layout
    S, ldp = layout(M, N, K)
    assert 1 <= S <= 8 and ldp >= N
    assert all(layout(m, N, K) == (S, ldp) for m in range(1, 9))
    codes, scales, L = _lin(b, 19 * N + K + b, N, K)
    x = synth.activations_bf16(M + 2 * N, M, K)
    part = torch.full((S * M * ldp,), float("nan"), dtype=torch.float32, device="cuda")
    if b == 3:
        B.w3_skinny_gemm_partials(dev(x), L.hi, L.lo, L.pscales, part, M, N, K)
    else:
        B.w2_skinny_gemm_partials(dev(x), L.packed, L.pscales, part, M, N, K)
    torch.cuda.synchronize()
    P = host(part).reshape(S, M, ldp)[:, :, :N]
    s = np.zeros((M, N), np.float32)
    for k in range(S):
        s = (s + P[k]).astype(np.float32)
    assert np.isfinite(s).all()
    err = gemm_rel_err(s, GEMM[b](x, codes, scales))
    assert err <= GEMM_RTOL, err


def _decode_plane2(words, N, K):
    G = K // 64
    out = np.empty((N, K), dtype=np.uint8)
    for n in range(N):
        t, nb, i = n >> 6, (n >> 4) & 3, n & 15
        for k in range(K):
            g, kk = k // 64, k % 64
            s_, kq, j = kk >> 5, (kk >> 3) & 3, kk & 7
            wd = words[((t * G + g) * 64 + kq * 16 + i) * 4 + nb]
            out[n, k] = (wd >> (8 * s_ + 2 * (j >> 1) + 16 * (j & 1))) & 3
    return out


def _decode_plane1(words, N, K):
    G = K // 64
    out = np.empty((N, K), dtype=np.uint8)
    for n in range(N):
        t, nb, i = n >> 6, (n >> 4) & 3, n & 15
        for k in range(K):
            g, kk = k // 64, k % 64
            s_, kq, j = kk >> 5, (kk >> 3) & 3, kk & 7
            wd = words[((t * G + g) * 64 + kq * 16 + i) * 2 + (nb >> 1)]
            out[n, k] = (wd >> (4 * (2 * (nb & 1) + s_) + (j >> 1) + 16 * (j & 1))) & 1
    return out


def _packed_scales(pscales, N, K):
    import torch
    packed = torch.zeros(B.packed_sizes(N, K)[0], dtype=torch.uint8, device="cuda")
    c = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
    s = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
    B.lib().vw4_w4_unpack(packed.data_ptr(), pscales.data_ptr(), N, K, c.data_ptr(), s.data_ptr(), None)
    torch.cuda.synchronize()
    return host(s).view(np.uint16)


@pytest.mark.parametrize("b", [3, 2])
def test_planes_decode_to_the_codes(b):
    N, K = 100, 320
    log(f"w{b} pack round trip")
    codes, scales, L = _lin(b, 3 + b, N, K)
    assert np.array_equal(_packed_scales(L.pscales, N, K), scales)
    if b == 3:
        lo, hi = host(L.lo).view(np.uint32), host(L.hi).view(np.uint32)
        assert lo.size == B.lib().vw4_w3_lo_plane_bytes(N, K) // 4
        assert hi.size == B.lib().vw4_w3_hi_plane_bytes(N, K) // 4
        assert np.array_equal(_decode_plane2(lo, N, K), codes & 3)
        assert np.array_equal(_decode_plane1(hi, N, K), codes >> 2)
    else:
        words = host(L.packed).view(np.uint32)
        assert words.size == B.lib().vw4_w2_packed_bytes(N, K) // 4
        c = codes.astype(np.int64) - 1
        assert np.array_equal(_decode_plane2(words, N, K), (c != 0) | ((c < 0) << 1))


@pytest.mark.parametrize("b", [3, 2])
def test_rows_independent_of_m(b):
    M, N, K = 6, 1000, 2048
    log(f"w{b} row independence")
    codes, scales, L = _lin(b, 4 + b, N, K)
    x = dev(synth.activations_bf16(5, M, K))
    y = _run(b, x, L, M, N, K)
    for m in (0, 5):
        assert np.array_equal(_run(b, x[m:m + 1], L, 1, N, K)[0], y[m])
