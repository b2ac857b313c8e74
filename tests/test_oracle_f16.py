"""Pins of the oracle's fp16- and bf16-weight GEMMs (no GPU): numpy's fp64
product of the bf16 activations with the weights (numpy's own fp16 decoding;
bf16 decoded as the top half of a binary32), the fp16 and bf16 special values
(subnormals, the largest finite values, signed zeros), and hand-computed
outputs."""
import numpy as np

import oracle


def _bf16(a):
    return (np.asarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_matches_numpy_fp64_product():
    rng = np.random.default_rng(81)
    M, N, K = 3, 37, 200
    x = _bf16(rng.normal(0, 1, (M, K)))
    w = rng.normal(0, 0.05, (N, K)).astype(np.float16)
    want = oracle.bf16_value(x) @ w.astype(np.float64).T
    np.testing.assert_allclose(oracle.f16_gemm(x, w.view(np.uint16)), want, rtol=1e-13, atol=1e-15)


def test_special_values():
    K = 8
    w = np.array([[0x0001, 0x8001, 0x03FF, 0x7BFF, 0xFBFF, 0x0000, 0x8000, 0x3C00]], dtype=np.uint16)
    x = _bf16(np.ones((1, K)))
    vals = [2.0 ** -24, -(2.0 ** -24), 1023 * 2.0 ** -24, 65504.0, -65504.0, 0.0, -0.0, 1.0]
    assert oracle.f16_gemm(x, w)[0, 0] == sum(vals)
    x2 = _bf16(np.array([[2.0 ** 20, 1, 1, 1, 1, 1, 1, -3]]))
    want = 2.0 ** 20 * 2.0 ** -24 + sum(vals[1:7]) - 3.0
    assert oracle.f16_gemm(x2, w)[0, 0] == want


def test_hand_computed_output():
    # x = 1 .. 64, w_k = (k - 32) / 8 (all exact in fp16): sum (k + 1) (k - 32) / 8
    x = _bf16(np.arange(1, 65, dtype=np.float32).reshape(1, 64))
    w = ((np.arange(64) - 32) / 8.0).astype(np.float16).view(np.uint16).reshape(1, 64)
    want = sum((k + 1) * (k - 32) for k in range(64)) / 8.0
    assert oracle.f16_gemm(x, w)[0, 0] == want


def test_b16_matches_numpy_fp64_product():
    rng = np.random.default_rng(82)
    M, N, K = 3, 37, 200
    x = _bf16(rng.normal(0, 1, (M, K)))
    w = _bf16(rng.normal(0, 0.05, (N, K)))
    wv = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_allclose(oracle.b16_gemm(x, w), oracle.bf16_value(x) @ wv.T, rtol=1e-13, atol=1e-15)


def test_b16_special_values_and_hand_output():
    # smallest subnormal 2^-133, largest finite (2 - 2^-7) 2^127, signed zeros, 1.0
    w = np.array([[0x0001, 0x8001, 0x7F7F, 0x0000, 0x8000, 0x3F80]], dtype=np.uint16)
    x = _bf16(np.array([[2.0 ** 100, 2.0 ** 100, 2.0 ** -100, 1, 1, -5]]))
    want = 2.0 ** -33 - 2.0 ** -33 + (2 - 2.0 ** -7) * 2.0 ** 27 + 0.0 - 0.0 - 5.0
    assert oracle.b16_gemm(x, w)[0, 0] == want
    x1 = _bf16(np.arange(1, 65, dtype=np.float32).reshape(1, 64))
    w1 = _bf16(((np.arange(64) - 32) / 4.0).reshape(1, 64))
    assert oracle.b16_gemm(x1, w1)[0, 0] == sum((k + 1) * (k - 32) for k in range(64)) / 4.0
