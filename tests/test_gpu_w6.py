"""The W6 skinny GEMM (a third weight format) on the GPU against the oracle:
outputs within the GEMM tolerance for M = 1..8 over ragged, one-slice and
split-K shapes; the packed planes decode (low plane with the W4 unpacker,
high plane from its documented 2-bit layout) to the oracle's codes; rows are
independent of M bit for bit."""
import numpy as np
import pytest

import oracle
from verify_step_w4_amd import binding as B
from verify_step_w4_amd import synth
from verify_step_w4_amd.model import W6Linear

from helpers import GEMM_RTOL, dev, gemm_rel_err, host, log

pytestmark = pytest.mark.gpu


def _w6(seed, N, K):
    w = synth.normal_f32(synth.rng(seed), (N, K), 0.02)
    codes, scales = oracle.w6_quantize(w)
    return codes, scales, W6Linear.from_codes(dev(codes), dev(scales))


def _run(x, lin, M, N, K):
    import torch
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = B.workspace(max(B.w6_workspace_bytes(M, N, K), 256))
    B.w6_skinny_gemm(x, lin.hi, lin.lo, lin.pscales, y, M, N, K, ws=ws)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("N,K", [(1, 64), (100, 320), (257, 1024), (1000, 2048), (5120, 5120), (64, 17408)])
@pytest.mark.parametrize("M", [1, 4, 8])
def test_w6_gemm_matches_oracle(M, N, K):
    log(f"w6 gemm M={M} N={N} K={K}")
    codes, scales, lin = _w6(13 * N + K, N, K)
    x = synth.activations_bf16(M * 100 + N + 1, M, K)
    err = gemm_rel_err(_run(dev(x), lin, M, N, K), oracle.w6_gemm(x, codes, scales))
    assert err <= GEMM_RTOL, err


def test_w6_planes_decode_to_the_codes():
    import torch
    N, K = 100, 320
    log("w6 pack round trip")
    codes, scales, lin = _w6(3, N, K)
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
    G = K // 64
    hi = np.empty((N, K), dtype=np.uint8)
    for n in range(N):
        t, nb, i = n >> 6, (n >> 4) & 3, n & 15
        for k in range(K):
            g, kk = k // 64, k % 64
            s_, kq, j = kk >> 5, (kk >> 3) & 3, kk & 7
            wd = words[((t * G + g) * 64 + kq * 16 + i) * 4 + nb]
            hi[n, k] = (wd >> (8 * s_ + 2 * (j >> 1) + 16 * (j & 1))) & 3
    assert np.array_equal(hi, codes >> 4)


def test_w6_rows_independent_of_m():
    M, N, K = 6, 1000, 2048
    log("w6 row independence")
    codes, scales, lin = _w6(4, N, K)
    x = dev(synth.activations_bf16(5, M, K))
    y = _run(x, lin, M, N, K)
    for m in (0, 5):
        assert np.array_equal(_run(x[m:m + 1], lin, 1, N, K)[0], y[m])
