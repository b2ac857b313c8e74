"""The allocation-free GEMM entry point (w4_skinny_gemm_noalloc) against the
workspace form (w4_skinny_gemm) through the C ABI: bit for bit, on two calls
in a row on the same GPU (the second with a smaller input, so the scratch
array holds the first call's partials when it starts), on split-K shapes
(partials in the scratch array) and a one-slice shape (none)."""
import numpy as np
import pytest

from verify_step_w4_amd import binding as B
from verify_step_w4_amd import synth

from helpers import dev, host, log

pytestmark = pytest.mark.gpu


def _pair(M, N, K, seed, out="f32"):
    import torch
    w = synth.normal_f32(synth.rng(seed), (N, K), 0.02)
    packed, pscales = B.w4_quantize_packed(dev(w))
    x = dev(synth.activations_bf16(seed + 1, M, K))
    dt = torch.float32 if out == "f32" else torch.int16
    ya = torch.full((M, N), -1, dtype=dt, device="cuda")
    yb = torch.full((M, N), -1, dtype=dt, device="cuda")
    ws = B.workspace(max(B.gemm_workspace_bytes(M, N, K), 256))
    B.w4_skinny_gemm(x, packed, pscales, ya, M, N, K, ws=ws)
    B.w4_skinny_gemm_noalloc(x, packed, pscales, yb, M, N, K)
    torch.cuda.synchronize()
    return host(ya), host(yb)


@pytest.mark.parametrize("first,second", [
    ((8, 5120, 17408), (4, 1024, 5120)),      # split-K both times; the second call uses less of the array
    ((4, 7168, 5120), (1, 300, 1024)),
    ((8, 130958, 1024), (2, 5120, 5120)),     # the largest partials the plan produces (8384512 bytes)
    ((4, 151936, 512), (3, 2000, 640)),       # one-slice plan (no partials), then a split one
])
def test_noalloc_equals_workspace_form_twice(first, second):
    for k, (M, N, K) in enumerate((first, second)):
        log(f"noalloc gemm call {k}: M={M} N={N} K={K}")
        S = B.gemm_workspace_bytes(M, N, K)
        assert S <= B.lib().vw4_noalloc_scratch_bytes()
        ya, yb = _pair(M, N, K, 1000 * k + N % 997 + K)
        assert np.array_equal(ya, yb), (M, N, K)


def test_noalloc_bf16_output():
    log("noalloc gemm bf16 output")
    ya, yb = _pair(4, 5120, 5120, 77, out="bf16")
    assert np.array_equal(ya, yb)


def test_noalloc_rejects_bad_shape():
    import torch
    y = torch.empty((9, 64), dtype=torch.float32, device="cuda")
    x = torch.zeros((9, 64), dtype=torch.int16, device="cuda")
    w = torch.zeros(64 * 32, dtype=torch.uint8, device="cuda")
    s = torch.zeros(64, dtype=torch.int16, device="cuda")
    with pytest.raises(RuntimeError):
        B.w4_skinny_gemm_noalloc(x, w, s, y, 9, 64, 64)
