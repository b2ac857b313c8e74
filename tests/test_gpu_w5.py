"""The W5 skinny GEMM (a fourth weight format) on the GPU against the oracle:
outputs within the GEMM tolerance for M = 1..8 over ragged, one-slice and
split-K shapes; the packed planes decode (low plane with the W4 unpacker,
high plane from its documented 1-bit layout) to the oracle's codes; rows are
independent of M bit for bit."""
import numpy as np
import pytest

import oracle
from verify_step_w4_amd import binding as B
from verify_step_w4_amd import synth
from verify_step_w4_amd.model import W5Linear

from helpers import GEMM_RTOL, dev, gemm_rel_err, host, log

pytestmark = pytest.mark.gpu


def _w5(seed, N, K):
    w = synth.normal_f32(synth.rng(seed), (N, K), 0.02)
    codes, scales = oracle.w5_quantize(w)
    return codes, scales, W5Linear.from_codes(dev(codes), dev(scales))


def _run(x, lin, M, N, K):
    import torch
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = B.workspace(max(B.w5_workspace_bytes(M, N, K), 256))
    B.w5_skinny_gemm(x, lin.hi, lin.lo, lin.pscales, y, M, N, K, ws=ws)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("N,K", [(1, 64), (100, 320), (257, 1024), (1000, 2048), (5120, 5120), (64, 17408)])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_w5_gemm_matches_oracle(M, N, K):
    log(f"w5 gemm M={M} N={N} K={K}")
    codes, scales, lin = _w5(13 * N + K, N, K)
    x = synth.activations_bf16(M * 100 + N + 1, M, K)
    err = gemm_rel_err(_run(dev(x), lin, M, N, K), oracle.w5_gemm(x, codes, scales))
    assert err <= GEMM_RTOL, err


@pytest.mark.parametrize("M,N,K", [(4, 1000, 2048), (1, 257, 1024), (6, 5120, 5120)])
def test_w5_gemm_bf16_output(M, N, K):
    """bf16 output: the round-to-nearest-even of the call's own fp32 result,
    and within the bf16 bar of the oracle's exact product."""
    import torch
    from layer_parity import bf16_close
    log(f"w5 gemm bf16 out M={M} N={N} K={K}")
    codes, scales, lin = _w5(17 * N + K, N, K)
    x = dev(synth.activations_bf16(M + N + 3, M, K))
    y32 = _run(x, lin, M, N, K)
    y16 = torch.empty((M, N), dtype=torch.int16, device="cuda")
    ws = B.workspace(max(B.w5_workspace_bytes(M, N, K), 256))
    B.w5_skinny_gemm(x, lin.hi, lin.lo, lin.pscales, y16, M, N, K, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(y16), oracle.bf16_round(y32.astype(np.float64)))
    bf16_close(host(y16), oracle.w5_gemm(host(x), codes, scales), min_exact=0.9)


@pytest.mark.parametrize("M,N,K", [(4, 5120, 5120), (1, 7168, 5120), (8, 5120, 17408), (3, 100, 320),
                                   (6, 34816, 5120)])
def test_w5_partials_sum_to_the_product(M, N, K):
    """The partials form: at most 8 slices, a layout that does not depend on M,
    and the S slices summed in slice order give the oracle's product."""
    import torch
    log(f"w5 partials M={M} N={N} K={K}")
    S, ldp = B.w5_partials_layout(M, N, K)
    assert 1 <= S <= 8 and ldp >= N
    assert all(B.w5_partials_layout(m, N, K) == (S, ldp) for m in range(1, 9))
    codes, scales, lin = _w5(19 * N + K, N, K)
    x = synth.activations_bf16(M + 2 * N, M, K)
    part = torch.full((S * M * ldp,), float("nan"), dtype=torch.float32, device="cuda")
    B.w5_skinny_gemm_partials(dev(x), lin.hi, lin.lo, lin.pscales, part, M, N, K)
    torch.cuda.synchronize()
    P = host(part).reshape(S, M, ldp)[:, :, :N]
    s = np.zeros((M, N), np.float32)
    for k in range(S):
        s = (s + P[k]).astype(np.float32)
    assert np.isfinite(s).all()
    err = gemm_rel_err(s, oracle.w5_gemm(x, codes, scales))
    assert err <= GEMM_RTOL, err


def test_w5_planes_decode_to_the_codes():
    import torch
    N, K = 100, 320
    log("w5 pack round trip")
    codes, scales, lin = _w5(3, N, K)
    c = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
    s = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
    B.lib().vw4_w4_unpack(lin.lo.data_ptr(), lin.pscales.data_ptr(), N, K, c.data_ptr(), s.data_ptr(), None)
    torch.cuda.synchronize()
    cc = host(c)
    lo = np.empty((N, K), dtype=np.uint8)
    lo[:, 0::2] = cc & 15
    lo[:, 1::2] = cc >> 4
    assert np.array_equal(lo, codes & 15) and np.array_equal(host(s).view(np.uint16), scales)
    words = host(lin.hi).view(np.uint32)
    assert words.size == B.lib().vw4_w5_hi_plane_bytes(N, K) // 4
    G = K // 64
    hi = np.empty((N, K), dtype=np.uint8)
    for n in range(N):
        t, nb, i = n >> 6, (n >> 4) & 3, n & 15
        for k in range(K):
            g, kk = k // 64, k % 64
            s_, kq, j = kk >> 5, (kk >> 3) & 3, kk & 7
            wd = words[((t * G + g) * 64 + kq * 16 + i) * 2 + (nb >> 1)]
            hi[n, k] = (wd >> (4 * (2 * (nb & 1) + s_) + (j >> 1) + 16 * (j & 1))) & 1
    assert np.array_equal(hi, codes >> 4)


def test_w5_rows_independent_of_m():
    M, N, K = 6, 1000, 2048
    log("w5 row independence")
    codes, scales, lin = _w5(4, N, K)
    x = dev(synth.activations_bf16(5, M, K))
    y = _run(x, lin, M, N, K)
    for m in (0, 5):
        assert np.array_equal(_run(x[m:m + 1], lin, 1, N, K)[0], y[m])
