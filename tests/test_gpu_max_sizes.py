"""Every weight format at the largest K the GEMM calls accept (65536), with
M = 1 and M = 8 (the largest M) and a ragged N, against the oracle; the
plain call and the partial slices summed in slice order."""
import numpy as np
import pytest

import oracle
from verify_step_w4_amd import binding as B
from verify_step_w4_amd import synth
from verify_step_w4_amd.model import (LINEAR_FORMATS, W4Linear, W16Linear)

from helpers import GEMM_RTOL, dev, gemm_rel_err, host, log

pytestmark = pytest.mark.gpu

K_MAX = 65536
QUANT = {"w4": oracle.w4_quantize, "w8": oracle.w8_quantize, "w6": oracle.w6_quantize, "w5": oracle.w5_quantize,
         "w3": oracle.w3_quantize, "w2": oracle.w2_quantize}
GEMM = {"w4": oracle.w4_gemm, "w8": oracle.w8_gemm, "w6": oracle.w6_gemm, "w5": oracle.w5_gemm,
        "w3": oracle.w3_gemm, "w2": oracle.w2_gemm}


def _case(fmt, N, K, seed):
    w = synth.normal_f32(synth.rng(seed), (N, K), 0.02)
    if fmt == "f16":
        bits = w.astype(np.float16).view(np.uint16)
        return W16Linear.from_bits(dev(bits.view(np.int16)), "f16"), (lambda x: oracle.f16_gemm(x, bits))
    if fmt == "bf16":
        bits = oracle.bf16_round(w.astype(np.float64))
        return W16Linear.from_bits(dev(bits.view(np.int16)), "bf16"), (lambda x: oracle.b16_gemm(x, bits))
    codes, scales = QUANT[fmt](w)
    lin = W4Linear.from_fp32(dev(w)) if fmt == "w4" else LINEAR_FORMATS[fmt].from_fp32(w)
    return lin, (lambda x: GEMM[fmt](x, codes, scales))


@pytest.mark.parametrize("fmt", ["w4", "w8", "w6", "w5", "w3", "w2", "f16", "bf16"])
def test_largest_k(fmt):
    import torch
    N = 65
    log(f"{fmt} gemm at K={K_MAX}, N={N}, M=1 and 8, plain and partials")
    lin, ref = _case(fmt, N, K_MAX, 4100 + len(fmt))
    for M in (1, 8):
        x = synth.activations_bf16(M + 7, M, K_MAX)
        want = ref(x)
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        ws = B.workspace(max(lin.workspace_bytes(M), 256))
        lin.gemm(dev(x), y, M, ws=ws)
        S, ldp = lin.partials_layout(M)
        part = torch.full((S * M * ldp,), float("nan"), dtype=torch.float32, device="cuda")
        lin.partials(dev(x), part, M)
        torch.cuda.synchronize()
        assert gemm_rel_err(host(y), want) <= GEMM_RTOL
        P = host(part).reshape(S, M, ldp)[:, :, :N]
        s = np.zeros((M, N), np.float32)
        for k in range(S):
            s = (s + P[k]).astype(np.float32)
        assert gemm_rel_err(s, want) <= GEMM_RTOL
