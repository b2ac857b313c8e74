"""Gate|up GEMM with the SwiGLU in its epilogue in every weight format other
than W4 (gate/up-interleaved rows): the bf16 output against the oracle's
composition (the format's GEMM on the natural row order, then SwiGLU), at the
bar of the W4 SwiGLU-epilogue tests; nothing written past F."""
import numpy as np
import pytest

import oracle
from verify_step_w4_amd import binding as B
from verify_step_w4_amd import synth
from verify_step_w4_amd.model import LINEAR_FORMATS, W16Linear

from helpers import dev, host, log

pytestmark = pytest.mark.gpu

QG = {"w8": (oracle.w8_quantize, oracle.w8_gemm), "w6": (oracle.w6_quantize, oracle.w6_gemm),
      "w5": (oracle.w5_quantize, oracle.w5_gemm), "w3": (oracle.w3_quantize, oracle.w3_gemm),
      "w2": (oracle.w2_quantize, oracle.w2_gemm)}


def _ref_and_linear(fmt, w):
    """(oracle gate|up product on the natural row order, device matrix of the interleaved rows)."""
    wi = B.interleave_gate_up(w)
    if fmt in ("f16", "bf16"):
        conv = (lambda a: a.astype(np.float16).view(np.uint16)) if fmt == "f16" else \
            (lambda a: oracle.bf16_round(a.astype(np.float64)))
        gemm = oracle.f16_gemm if fmt == "f16" else oracle.b16_gemm
        bits = conv(w)
        return (lambda x: gemm(x, bits)), W16Linear.from_bits(dev(np.ascontiguousarray(conv(wi)).view(np.int16)), fmt)
    quant, gemm = QG[fmt]
    codes, scales = quant(w)
    return (lambda x: gemm(x, codes, scales)), LINEAR_FORMATS[fmt].from_fp32(np.ascontiguousarray(wi))


@pytest.mark.parametrize("M,F,K", [(1, 32, 64), (4, 1024, 2048), (8, 544, 1024), (4, 8704, 5120)])
@pytest.mark.parametrize("fmt", ["w8", "w6", "w5", "w3", "w2", "f16", "bf16"])
def test_swiglu_epilogue_matches_oracle(fmt, M, F, K):
    import torch
    from layer_parity import bf16_close
    log(f"{fmt} gate|up + swiglu M={M} F={F} K={K}")
    w = synth.normal_f32(synth.rng(9 * F + K), (2 * F, K), 0.02)
    ref, lin = _ref_and_linear(fmt, w)
    x = synth.activations_bf16(F + K + M, M, K)
    a = torch.full((M, F + 8), -1, dtype=torch.int16, device="cuda")
    lin.swiglu(dev(x), a, M)
    torch.cuda.synchronize()
    ah = host(a)
    assert (ah[:, F:] == 0xFFFF).all()                  # nothing past F in each row
    gu = ref(x)
    want = oracle.swiglu(gu[:, :F], gu[:, F:])
    bf16_close(np.ascontiguousarray(ah[:, :F]), want, min_exact=0.9)
