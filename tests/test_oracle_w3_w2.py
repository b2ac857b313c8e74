"""Pins of the oracle's W3 and W2 formats and GEMMs (no GPU): the worked
examples in tests/golden/w3_quant_worked_example.txt and
w2_quant_worked_example.txt, a numpy re-implementation bit for bit,
invariants, and each GEMM against numpy's fp64 product with the dequantised
matrix plus a hand-computed output."""
import os

import numpy as np
import pytest

import oracle

FMT = {3: (oracle.w3_quantize, oracle.w3_gemm, 3, 4), 2: (oracle.w2_quantize, oracle.w2_gemm, 1, 1)}


def _golden(b):
    vals = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", f"w{b}_quant_worked_example.txt")):
        if line.startswith("#") or "=" not in line:
            continue
        k, v = line.split("=", 1)
        vals[k.strip()] = v.split()
    return vals


@pytest.mark.parametrize("b,suffix", [(3, ""), (2, "_a"), (2, "_b")])
def test_worked_example(b, suffix):
    quant, _, _, bias = FMT[b]
    g = _golden(b)
    wv = [float(v) for v in g["weights" + suffix]]
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, :len(wv)] = np.array(wv, dtype=np.float32)
    codes, scales = quant(w)
    assert int(scales[0, 0]) == int(g["scale" + suffix + "_f16_bits"][0], 16)
    assert (codes[0, :len(wv)].astype(int) - bias).tolist() == [int(v) for v in g["codes" + suffix]]
    assert np.all(codes[0, len(wv):] == bias)


def _numpy_quant(w, qmax, bias):
    N, K = w.shape
    wg = w.reshape(N, K // 64, 64)
    s16 = (np.abs(wg).max(axis=2) / np.float32(qmax)).astype(np.float32).astype(np.float16)
    sf = s16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(wg / sf[:, :, None])
    c = np.where(sf[:, :, None] != 0, np.clip(r, -qmax, qmax), 0).astype(np.int64)
    return (c + bias).astype(np.uint8).reshape(N, K), s16.view(np.uint16)


@pytest.mark.parametrize("b", [3, 2])
@pytest.mark.parametrize("seed", range(3))
def test_matches_numpy_reimplementation(b, seed):
    quant, _, qmax, bias = FMT[b]
    rng = np.random.default_rng(seed + 70 + b)
    w = rng.normal(0.0, 0.02, (29, 256)).astype(np.float32)
    w[2, 64:128] = 0.0
    w[4, :64] = 1e-9
    w[6, 130] = -2.0
    c1, s1 = quant(w)
    c2, s2 = _numpy_quant(w, qmax, bias)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("b", [3, 2])
def test_invariants_and_gemm(b):
    quant, gemm, qmax, bias = FMT[b]
    rng = np.random.default_rng(60 + b)
    M, N, K = 3, 40, 384
    w = rng.standard_t(3, (N, K)).astype(np.float32) * 0.02
    codes, scales = quant(w)
    c = codes.astype(np.int64) - bias
    assert np.abs(c).max() <= qmax and codes.max() <= bias + qmax
    sf = scales.view(np.float16).astype(np.float64)
    for n in range(N):
        for g in range(K // 64):
            blk = w[n, 64 * g:64 * g + 64].astype(np.float64)
            assert abs(c[n, 64 * g + int(np.argmax(np.abs(blk)))]) == qmax
            assert np.all(np.abs(blk - c[n, 64 * g:64 * g + 64] * sf[n, g]) <= sf[n, g] / 2 + 1e-12 * np.abs(blk))
    xb = (rng.normal(0, 1, (M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    deq = c * np.repeat(sf, 64, axis=1)
    np.testing.assert_allclose(gemm(xb, codes, scales), oracle.bf16_value(xb) @ deq.T, rtol=1e-12, atol=1e-15)
    x1 = (np.arange(1, 65, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16).reshape(1, 64)
    period = 2 * qmax + 1
    c1 = ((np.arange(64) % period) - qmax + bias).astype(np.uint8).reshape(1, 64)   # codes -qmax .. qmax, repeated
    s1 = np.array([[0x3400]], dtype=np.uint16)                                      # fp16 0.25
    want = 0.25 * sum((k + 1) * ((k % period) - qmax) for k in range(64))
    assert gemm(x1, c1, s1)[0, 0] == want
