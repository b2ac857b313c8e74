"""Pins of the oracle's fp16-weight GEMM (no GPU): numpy's fp64 product of
the bf16 activations with the fp16 weights (numpy's own fp16 decoding), the
fp16 special values (subnormals, the largest finite value, signed zeros), and
a hand-computed output."""
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
