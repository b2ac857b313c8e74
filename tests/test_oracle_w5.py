"""Pins of the oracle's W5 format and W5 GEMM (no GPU): the worked example
in tests/golden/w5_quant_worked_example.txt, a numpy re-implementation bit for
bit, invariants, and the GEMM against numpy's fp64 product with the
dequantised matrix plus a hand-computed output."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "w5_quant_worked_example.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        if line.startswith("#") or "=" not in line:
            continue
        k, v = line.split("=", 1)
        vals[k.strip()] = v.split()
    return vals


def test_worked_example():
    g = _golden()
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, :6] = np.array([float(v) for v in g["weights"]], dtype=np.float32)
    codes, scales = oracle.w5_quantize(w)
    assert int(scales[0, 0]) == int(g["scale_f16_bits"][0], 16)
    assert (codes[0, :6].astype(int) - 16).tolist() == [int(v) for v in g["codes"]]
    assert np.all(codes[0, 6:] == 16)


def _numpy_w5(w):
    N, K = w.shape
    wg = w.reshape(N, K // 64, 64)
    s16 = (np.abs(wg).max(axis=2) / np.float32(15.0)).astype(np.float32).astype(np.float16)
    sf = s16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(wg / sf[:, :, None])
    c = np.where(sf[:, :, None] != 0, np.clip(r, -15, 15), 0).astype(np.int64)
    return (c + 16).astype(np.uint8).reshape(N, K), s16.view(np.uint16)


@pytest.mark.parametrize("seed", range(3))
def test_matches_numpy_reimplementation(seed):
    rng = np.random.default_rng(seed + 50)
    w = rng.normal(0.0, 0.02, (29, 256)).astype(np.float32)
    w[2, 64:128] = 0.0
    w[4, :64] = 1e-9
    w[6, 130] = -2.0
    c1, s1 = oracle.w5_quantize(w)
    c2, s2 = _numpy_w5(w)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_invariants_and_gemm():
    rng = np.random.default_rng(54)
    M, N, K = 3, 40, 384
    w = rng.standard_t(3, (N, K)).astype(np.float32) * 0.02
    codes, scales = oracle.w5_quantize(w)
    c = codes.astype(np.int64) - 16
    assert np.abs(c).max() <= 15
    sf = scales.view(np.float16).astype(np.float64)
    for n in range(N):
        for g in range(K // 64):
            blk = w[n, 64 * g:64 * g + 64].astype(np.float64)
            assert abs(c[n, 64 * g + int(np.argmax(np.abs(blk)))]) == 15
            assert np.all(np.abs(blk - c[n, 64 * g:64 * g + 64] * sf[n, g]) <= sf[n, g] / 2 + 1e-12 * np.abs(blk))
    xb = (rng.normal(0, 1, (M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    deq = c * np.repeat(sf, 64, axis=1)
    np.testing.assert_allclose(oracle.w5_gemm(xb, codes, scales), oracle.bf16_value(xb) @ deq.T, rtol=1e-12,
                               atol=1e-15)
    x1 = (np.arange(1, 65, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16).reshape(1, 64)
    c1 = ((np.arange(64) % 31) - 15 + 16).astype(np.uint8).reshape(1, 64)    # codes -15 .. 15, twice, then -15, -14
    s1 = np.array([[0x3400]], dtype=np.uint16)                             # fp16 0.25
    want = 0.25 * sum((k + 1) * ((k % 31) - 15) for k in range(64))
    assert oracle.w5_gemm(x1, c1, s1)[0, 0] == want
