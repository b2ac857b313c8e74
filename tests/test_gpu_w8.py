"""The W8 skinny GEMM (a second weight format) on the GPU against the oracle.

* Outputs within the GEMM tolerance of the oracle's exact fp64 product, for
  M = 1..8 and shapes with ragged tiles, one-slice and split-K plans.
* The packed planes unpack (with the W4 unpacker) to the high and low
  nibbles of the oracle's codes; the packed scales are the oracle's.
* Row m of an M-row call equals the one-row call bit for bit; the bf16
  output is the rounded fp32 output.
"""
import numpy as np
import pytest

import oracle
from verify_step_w4_amd import binding as B
from verify_step_w4_amd import synth
from verify_step_w4_amd.model import W8Linear

from helpers import GEMM_RTOL, dev, gemm_rel_err, host, log

pytestmark = pytest.mark.gpu


def _w8(seed, N, K):
    w = synth.normal_f32(synth.rng(seed), (N, K), 0.02)
    codes, scales = oracle.w8_quantize(w)
    lin = W8Linear.from_codes(dev(codes), dev(scales))
    return w, codes, scales, lin


def _run(x, lin, M, N, K, out="f32"):
    import torch
    y = torch.empty((M, N), dtype=torch.float32 if out == "f32" else torch.int16, device="cuda")
    ws = B.workspace(max(B.w8_workspace_bytes(M, N, K), 256))
    B.w8_skinny_gemm(x, lin.hi, lin.lo, lin.pscales, y, M, N, K, ws=ws)
    torch.cuda.synchronize()
    return host(y)


SHAPES = [(1, 64), (100, 320), (257, 1024), (1000, 2048), (5120, 5120), (64, 17408)]


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("M", [1, 4, 6, 8])
def test_w8_gemm_matches_oracle(M, N, K):
    log(f"w8 gemm M={M} N={N} K={K}")
    w, codes, scales, lin = _w8(11 * N + K, N, K)
    x = synth.activations_bf16(M * 100 + N, M, K)
    y = _run(dev(x), lin, M, N, K)
    err = gemm_rel_err(y, oracle.w8_gemm(x, codes, scales))
    assert err <= GEMM_RTOL, err


def test_w8_packed_planes_unpack_to_the_nibbles():
    import torch
    N, K = 100, 320
    log("w8 pack round trip")
    w, codes, scales, lin = _w8(3, N, K)
    got = []
    for plane in (lin.hi, lin.lo):
        c = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
        s = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
        B.lib().vw4_w4_unpack(plane.data_ptr(), lin.pscales.data_ptr(), N, K, c.data_ptr(), s.data_ptr(), None)
        torch.cuda.synchronize()
        cc = host(c)
        nib = np.empty((N, K), dtype=np.uint8)
        nib[:, 0::2] = cc & 15
        nib[:, 1::2] = cc >> 4
        got.append(nib)
        assert np.array_equal(host(s).view(np.uint16), scales)
    assert np.array_equal(got[0], codes >> 4) and np.array_equal(got[1], codes & 15)


def test_w8_rows_independent_of_m_and_bf16_output():
    M, N, K = 6, 1000, 2048
    log("w8 row independence, bf16 output")
    w, codes, scales, lin = _w8(4, N, K)
    x = dev(synth.activations_bf16(5, M, K))
    y = _run(x, lin, M, N, K)
    for m in (0, 3, 5):
        assert np.array_equal(_run(x[m:m + 1], lin, 1, N, K)[0], y[m])
    y16 = _run(x, lin, M, N, K, out="bf16")
    assert np.array_equal(y16, synth.f32_to_bf16_bits(y.astype(np.float32)))


def test_w8_host_quantizer_matches_oracle_on_device_inputs():
    # the library's host quantiser feeds W8Linear.from_fp32: same codes and scales as the oracle
    w = synth.normal_f32(synth.rng(8), (64, 256), 0.02)
    c1, s1 = B.w8_quantize_host(w)
    c2, s2 = oracle.w8_quantize(w)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
