"""Pins of the oracle's number formats, W4 quantiser (a1) and W4 GEMM (a2/a3).

Pins are independent of the oracle's own formulas: numpy's IEEE binary16
conversion, a hand-derived worked example, invariants of the rounding, and
matmuls of weights that the format represents exactly.
"""
import os

import numpy as np
import pytest

import oracle
from verify_step_w4_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_f16_rounding_matches_numpy():
    g = np.random.default_rng(1)
    vals = [0.0, -0.0, 1.0, 65504.0, 65519.99, 65520.0, 1e9, 2.0 ** -14, 2.0 ** -24, 2.0 ** -25,
            3 * 2.0 ** -26, 2.0 ** -25 * 1.0000001, 6.1e-5, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11]
    vals += list(g.standard_normal(3000) * 10.0 ** g.integers(-9, 5, 3000))
    # exact ties between consecutive halves
    h = np.arange(0, 0x7bff, 97, dtype=np.uint16).view(np.float16).astype(np.float64)
    h2 = np.arange(1, 0x7c00, 97, dtype=np.uint16).view(np.float16).astype(np.float64)
    vals += list(((h + h2) / 2)[:len(h2)])
    for v in vals:
        f = np.float32(v)
        for s in (f, -f):
            want = int(np.array([s], dtype=np.float32).astype(np.float16).view(np.uint16)[0])
            assert oracle.f32_to_f16_bits(s) == want, (float(s), hex(want))


def test_f16_decode_all_patterns():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    for b in range(0, 65536, 7):
        r = ref[b]
        v = oracle.f16_value(b)
        if np.isnan(r):
            assert np.isnan(v)
        else:
            assert v == r, hex(b)


def _read_golden(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split("=", 1)
            d[k.strip()] = v.split()
    return d


def test_quant_worked_example():
    d = _read_golden("w4_quant_worked_example.txt")
    w = np.zeros((1, 64), dtype=np.float32)
    vals = np.array([float(x) for x in d["weights"]], dtype=np.float32)
    w[0, :len(vals)] = vals
    codes, scales = oracle.w4_quantize(w)
    assert int(scales[0, 0]) == int(d["scale_f16_bits"][0], 16)
    ci = oracle.w4_codes_int(codes)[0]
    want = [int(x) for x in d["codes"]]
    assert list(ci[:len(want)]) == want
    assert not ci[len(want):].any()


def test_quant_nibble_layout():
    # even k in the low nibble, odd k in the high nibble, stored as c + 8
    w = np.zeros((2, 64), dtype=np.float32)
    w[0, 4] = 1.0     # -> code 7 at k=4 (even): byte 2 low nibble = 15
    w[1, 5] = -1.0    # -> code -7 at k=5 (odd): byte 2 high nibble = 1
    codes, _ = oracle.w4_quantize(w)
    assert codes[0, 2] == (8 << 4) | 15
    assert codes[1, 2] == (1 << 4) | 8
    assert codes[0, 0] == 0x88 and codes[1, 31] == 0x88


def test_quant_invariants_random():
    g = np.random.default_rng(7)
    w = (g.standard_normal((64, 512)) * 0.02).astype(np.float32)
    w[3, 64:128] = 0.0                                   # all-zero group
    w[5, :64] = w[5, :64] * 1e-9                          # tiny group (fp16 subnormal scale)
    codes, scales = oracle.w4_quantize(w)
    ci = oracle.w4_codes_int(codes).astype(np.int64)
    assert ci.min() >= -7 and ci.max() <= 7
    sf = scales.view(np.float16).astype(np.float64)
    assert sf[3, 1] == 0.0 and not ci[3, 64:128].any()
    for n in range(w.shape[0]):
        for gi in range(w.shape[1] // 64):
            s = sf[n, gi]
            wg = w[n, gi * 64:(gi + 1) * 64].astype(np.float64)
            cg = ci[n, gi * 64:(gi + 1) * 64]
            if s == 0.0:
                assert not cg.any()
                continue
            # rounding error bound of round-to-nearest on the rounded scale
            err = np.abs(wg - cg * s)
            unclamped = np.abs(wg / s) <= 7.0
            assert np.all(err[unclamped] <= s / 2 * (1 + 1e-6) + 1e-30)
            # the group's absmax element lands on +-7
            j = int(np.argmax(np.abs(wg)))
            assert abs(cg[j]) == 7 and np.sign(cg[j]) == np.sign(wg[j])


def _numpy_w4(w):
    """The quantiser recipe in numpy's IEEE arithmetic: scale = fp16(absmax / 7)
    (binary32 division, binary16 rounding), codes = clamp(round-half-even(w /
    scale), -7, 7) against the rounded scale, zero codes for a zero scale,
    canonical nibbles c + 8 with even k low."""
    N, K = w.shape
    G = K // 64
    wg = w.reshape(N, G, 64)
    a = np.abs(wg).max(axis=2)
    s16 = (a / np.float32(7.0)).astype(np.float32).astype(np.float16)
    sf = s16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(wg / sf[:, :, None])
    c = np.where(sf[:, :, None] != 0, np.clip(r, -7, 7), 0).astype(np.int64).reshape(N, K)
    u = (c + 8).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8), s16.view(np.uint16)


@pytest.mark.parametrize("seed", range(4))
def test_quant_matches_numpy_reimplementation(seed):
    rng = np.random.default_rng(100 + seed)
    w = rng.normal(0.0, 0.02, (41, 320)).astype(np.float32)
    w[2, 64:128] = 0.0                         # zero group
    w[4, :64] = 1e-9                           # scale underflows to a subnormal fp16 / zero
    w[6, 200] = 2.5                            # one outlier
    w[8, 0:64] = np.float32(7 * 2.0 ** -7) * rng.integers(-1, 2, 64).astype(np.float32)   # ties at +-0.5 ulp
    c1, s1 = oracle.w4_quantize(w)
    c2, s2 = _numpy_w4(w)
    assert np.array_equal(s1, s2)
    assert np.array_equal(c1, c2)


def test_quant_exactly_representable_roundtrip():
    # w = c * 2^-7 with +-7 present in every group: scale must be 2^-7, codes c
    g = np.random.default_rng(3)
    c = g.integers(-7, 8, (16, 256))
    c[:, ::64] = 7
    w = (c * 2.0 ** -7).astype(np.float32)
    codes, scales = oracle.w4_quantize(w)
    assert np.all(scales.view(np.float16).astype(np.float64) == 2.0 ** -7)
    assert np.array_equal(oracle.w4_codes_int(codes), c.astype(np.int8))


def test_gemm_hand_case():
    # one row, one group: codes 1..7 on the first seven k, scale 0.5, x = 1..7
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, :7] = np.arange(1, 8) * 0.5
    codes, scales = oracle.w4_quantize(w)
    assert oracle.f16_value(int(scales[0, 0])) == 0.5
    x = np.zeros((1, 64), dtype=np.float32)
    x[0, :7] = np.arange(1, 8)
    xb = synth.f32_to_bf16_bits(x)
    y = oracle.w4_gemm(xb, codes, scales)
    assert y.shape == (1, 1)
    assert y[0, 0] == 0.5 * sum(k * k for k in range(1, 8))   # 70.0


def test_gemm_matches_numpy_on_representable_weights():
    # weights the W4 format represents exactly => the GEMM is x @ w.T
    g = np.random.default_rng(11)
    M, N, K = 3, 37, 320
    c = g.integers(-7, 8, (N, K))
    c[:, ::64] = -7
    e = g.integers(-9, -4, (N, K // 64))
    w = (c * np.repeat(2.0 ** e, 64, axis=1)).astype(np.float32)
    codes, scales = oracle.w4_quantize(w)
    xb = synth.activations_bf16(5, M, K)
    xf = synth.bf16_bits_to_f32(xb).astype(np.float64)
    y = oracle.w4_gemm(xb, codes, scales)
    ref = xf @ w.astype(np.float64).T
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)
    # single-output entry point agrees bitwise with the full product
    for n in (0, 17, 36):
        assert oracle.w4_gemm_at(xb[1], codes, scales, n) == y[1, n]


def test_gemm_one_hot_codes():
    w = np.zeros((4, 128), dtype=np.float32)
    for n in range(4):
        w[n, 31 * n + 3] = (n + 1) * 0.25
    codes, scales = oracle.w4_quantize(w)
    xb = synth.activations_bf16(9, 2, 128)
    xf = synth.bf16_bits_to_f32(xb).astype(np.float64)
    y = oracle.w4_gemm(xb, codes, scales)
    for n in range(4):
        k = 31 * n + 3
        s = oracle.f16_value(int(scales[n, k // 64]))
        assert np.all(y[:, n] == xf[:, k] * 7 * s)


def test_bf16_rounding_matches_torch_on_fp32_values():
    # for binary32 inputs, one rounding binary64 -> bf16 equals torch's RNE cast
    import torch
    g = np.random.default_rng(2)
    vals = (g.standard_normal(4000) * 10.0 ** g.integers(-30, 30, 4000)).astype(np.float32)
    # exact ties between consecutive bf16 values, and the subnormal range
    b = np.arange(0, 0x7f7f, 37, dtype=np.uint32)
    lo = (b << 16).view(np.float32).astype(np.float64)
    hi = ((b + 1) << 16).view(np.float32).astype(np.float64)
    ties = ((lo + hi) / 2).astype(np.float32)
    sub = (np.arange(1, 300, dtype=np.uint32) << 13).view(np.float32)
    special = np.array([0.0, 1.0, 3.389e38, np.inf, -np.inf, np.finfo(np.float32).max,
                        -np.finfo(np.float32).max], np.float32)
    allv = np.concatenate([vals, ties, sub, -vals[:100], special])
    want = torch.from_numpy(allv).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_round(allv.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_rounding_of_random_fp32_words():
    """One rounding to nearest, ties to even, on random binary32 words (every
    exponent, both signs, infinities; NaN excluded), against torch's cast."""
    import torch
    g = np.random.default_rng(7)
    u = g.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32)
    u = np.concatenate([u, np.array([0x7f800000, 0xff800000, 0x7f7fffff, 0x7f7f8000], np.uint32)])
    f = u.view(np.float32)
    f = f[~np.isnan(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_round(f.astype(np.float64)), want)


def test_bf16_double_rounding_case():
    # a binary64 value just above a bf16 tie: one rounding goes up, rounding
    # through binary32 first would land on the tie and go to even (down)
    tie = 1.0 + 2.0 ** -8
    v = tie + 2.0 ** -40
    assert oracle.bf16_round(np.array([v]))[0] == 0x3F81
    assert oracle.bf16_round(np.array([tie]))[0] == 0x3F80
