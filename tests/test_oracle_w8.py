"""Pins of the oracle's W8 format and W8 GEMM (no GPU).

* The worked example in tests/golden/w8_quant_worked_example.txt (half-even
  rounding, the absmax element at +-127, offset-binary storage).
* A numpy re-implementation of the recipe (np.float32 division, np.float16
  cast, np.rint) agrees bit for bit on random and edge-case matrices.
* Invariants: |c| <= 127, the group absmax maps to +-127, |w - c s| <= s / 2.
* The GEMM equals numpy's fp64 product with the dequantised matrix, and a
  hand-computed one-output case exactly.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "w8_quant_worked_example.txt")


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
    codes, scales = oracle.w8_quantize(w)
    assert int(scales[0, 0]) == int(g["scale_f16_bits"][0], 16)
    want = [int(v) for v in g["codes"]]
    assert (codes[0, :6].astype(int) - 128).tolist() == want
    assert np.all(codes[0, 6:] == 128)


def _numpy_w8(w):
    N, K = w.shape
    G = K // 64
    wg = w.reshape(N, G, 64)
    a = np.abs(wg).max(axis=2)
    s16 = (a / np.float32(127.0)).astype(np.float32).astype(np.float16)
    sf = s16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(wg / sf[:, :, None])
    c = np.where(sf[:, :, None] != 0, np.clip(r, -127, 127), 0).astype(np.int64)
    return (c + 128).astype(np.uint8).reshape(N, K), s16.view(np.uint16)


@pytest.mark.parametrize("seed", range(4))
def test_matches_numpy_reimplementation(seed):
    rng = np.random.default_rng(seed)
    w = rng.normal(0.0, 0.02, (37, 256)).astype(np.float32)
    w[3, 64:128] = 0.0                        # zero group
    w[5, :64] = 1e-9                          # underflowing scale
    w[7, 128] = 3.0                           # one large element
    c1, s1 = oracle.w8_quantize(w)
    c2, s2 = _numpy_w8(w)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_invariants():
    rng = np.random.default_rng(9)
    w = rng.standard_t(3, (64, 512)).astype(np.float32) * 0.02
    codes, scales = oracle.w8_quantize(w)
    c = codes.astype(np.int64) - 128
    assert np.abs(c).max() <= 127
    sf = scales.view(np.float16).astype(np.float64)
    for n in range(64):
        for g in range(8):
            blk = w[n, 64 * g:64 * g + 64].astype(np.float64)
            cc = c[n, 64 * g:64 * g + 64]
            j = int(np.argmax(np.abs(blk)))
            assert abs(cc[j]) == 127
            assert np.all(np.abs(blk - cc * sf[n, g]) <= sf[n, g] / 2 + 1e-12 * np.abs(blk))


def test_gemm_matches_numpy_and_hand_case():
    rng = np.random.default_rng(10)
    M, N, K = 5, 33, 320
    w = rng.normal(0.0, 0.02, (N, K)).astype(np.float32)
    codes, scales = oracle.w8_quantize(w)
    xb = (rng.normal(0, 1, (M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = oracle.bf16_value(xb)
    deq = (codes.astype(np.float64) - 128) * np.repeat(scales.view(np.float16).astype(np.float64), 64, axis=1)
    np.testing.assert_allclose(oracle.w8_gemm(xb, codes, scales), x @ deq.T, rtol=1e-12, atol=1e-15)
    # one output by hand: x = 1..64 (bf16 exact), c = k - 64 (k = 0..63 -> -64..-1), s = 0.5
    x1 = (np.arange(1, 65, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16).reshape(1, 64)
    c1 = (np.arange(64) - 64 + 128).astype(np.uint8).reshape(1, 64)
    s1 = np.array([[0x3800]], dtype=np.uint16)          # fp16 0.5
    want = 0.5 * sum((k + 1) * (k - 64) for k in range(64))
    assert oracle.w8_gemm(x1, c1, s1)[0, 0] == want
