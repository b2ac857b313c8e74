"""GPU parity of the W4 format (a1) and the W4 skinny GEMM (a2/a3) against the
oracle.  Each side quantises the same fp32 weights itself; codes and scales
must agree bit for bit, GEMM outputs within 1e-3 relative."""
import numpy as np
import pytest

import oracle
from verify_step_w4_amd import binding as B
from verify_step_w4_amd import synth

from helpers import GEMM_RTOL, dev, gemm_rel_err, host, log

pytestmark = pytest.mark.gpu


def _weights(seed, N, K):
    w = synth.linear_weights(seed, N, K)
    return w


@pytest.mark.parametrize("N,K", [(1, 64), (64, 64), (100, 320), (257, 1024), (1000, 2048)])
def test_quantizer_bit_exact(N, K):
    import torch
    log(f"quantize N={N} K={K}")
    w = _weights(N + K, N, K)
    w[0, :64] = 0.0
    codes, scales = B.w4_quantize(dev(w))
    packed, pscales = B.w4_quantize_packed(dev(w))
    torch.cuda.synchronize()
    oc, os_ = oracle.w4_quantize(w)
    assert np.array_equal(host(codes), oc)
    assert np.array_equal(host(scales), os_)
    # packing the canonical form gives the fused packed form; unpacking inverts it
    p2, s2 = B.w4_pack(codes, scales, N, K)
    c3, s3 = B.w4_unpack(packed, pscales, N, K)
    torch.cuda.synchronize()
    assert torch.equal(p2, packed) and torch.equal(s2, pscales)
    assert np.array_equal(host(c3), oc) and np.array_equal(host(s3), os_)


def _gemm(x_bits, packed, pscales, M, N, K, out_dtype="f32"):
    import torch
    y = torch.empty((M, N), dtype=torch.float32 if out_dtype == "f32" else torch.int16, device="cuda")
    ws = B.workspace(B.gemm_workspace_bytes(M, N, K))
    B.w4_skinny_gemm(dev(x_bits) if isinstance(x_bits, np.ndarray) else x_bits, packed, pscales, y, M, N, K, ws=ws)
    torch.cuda.synchronize()
    return y


SHAPES = [(1, 64), (64, 128), (100, 320), (257, 1024), (1000, 2048), (333, 5120), (64, 17408)]


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 6, 8])
def test_gemm_matches_oracle(M, N, K):
    log(f"gemm M={M} N={N} K={K}")
    w = _weights(7 * N + K, N, K)
    x = synth.activations_bf16(M * 1000 + N, M, K)
    packed, pscales = B.w4_quantize_packed(dev(w))
    y = host(_gemm(x, packed, pscales, M, N, K))
    oc, os_ = oracle.w4_quantize(w)
    ref = oracle.w4_gemm(x, oc, os_)
    err = gemm_rel_err(y, ref)
    assert err <= GEMM_RTOL, err


def test_gemm_bf16_output_is_rounded_fp32():
    """The bf16 output is the round-to-nearest-even of the kernel's own fp32
    result (the oracle's rounding applied to the fp32 output), and within the
    bf16 bar of the oracle's exact product."""
    import torch
    M, N, K = 4, 300, 1024
    log(f"gemm bf16 out M={M} N={N} K={K}")
    w = _weights(5, N, K)
    x = synth.activations_bf16(6, M, K)
    packed, pscales = B.w4_quantize_packed(dev(w))
    y32 = host(_gemm(x, packed, pscales, M, N, K))
    y16 = host(_gemm(x, packed, pscales, M, N, K, "bf16"))
    assert np.array_equal(y16, oracle.bf16_round(y32.astype(np.float64)))
    from layer_parity import bf16_close
    oc, os_ = oracle.w4_quantize(w)
    bf16_close(y16, oracle.w4_gemm(x, oc, os_), min_exact=0.9)


@pytest.mark.parametrize("N,K", [(5120, 5120), (1000, 17408), (300, 1024)])
def test_gemm_rows_independent_of_M_and_deterministic(N, K):
    log(f"gemm M-independence N={N} K={K}")
    w = _weights(11, N, K)
    x = synth.activations_bf16(12, 6, K)
    packed, pscales = B.w4_quantize_packed(dev(w))
    y6 = host(_gemm(x, packed, pscales, 6, N, K))
    y6b = host(_gemm(x, packed, pscales, 6, N, K))
    assert np.array_equal(y6, y6b)
    for m in (0, 3, 5):
        y1 = host(_gemm(x[m:m + 1], packed, pscales, 1, N, K))
        assert np.array_equal(y1[0], y6[m])


def test_gemm_strided_rows():
    import torch
    M, N, K = 3, 200, 512
    log("gemm strided x/y")
    w = _weights(21, N, K)
    xfull = synth.activations_bf16(22, M, K + 64)
    packed, pscales = B.w4_quantize_packed(dev(w))
    xd = dev(xfull)
    y = torch.zeros((M, N + 10), dtype=torch.float32, device="cuda")
    ws = B.workspace(B.gemm_workspace_bytes(M, N, K))
    B.w4_skinny_gemm(xd, packed, pscales, y, M, N, K, ws=ws, ldx=K + 64, ldy=N + 10)
    torch.cuda.synchronize()
    yh = host(y)
    oc, os_ = oracle.w4_quantize(w)
    ref = oracle.w4_gemm(np.ascontiguousarray(xfull[:, :K]), oc, os_)
    assert gemm_rel_err(yh[:, :N], ref) <= GEMM_RTOL
    assert np.all(yh[:, N:] == 0)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["qkv", "o", "gate_up", "down"])
def test_gemm_layer_shapes_sampled(name):
    """Dense 27B-layer linears at full size, M=4, in the benchmark's launch
    configuration; 128 sampled outputs per row checked against the oracle."""
    N, K = synth.LAYER27B_LINEARS[name]
    log(f"gemm full-size {name} N={N} K={K}")
    w = _weights(100 + N + K, N, K)
    x = synth.activations_bf16(200 + N, 4, K)
    packed, pscales = B.w4_quantize_packed(dev(w))
    y = host(_gemm(x, packed, pscales, 4, N, K))
    g = np.random.default_rng(N)
    cols = np.unique(np.concatenate([g.integers(0, N, 124), [0, 63, N - 64, N - 1]]))
    oc, os_ = oracle.w4_quantize(np.ascontiguousarray(w[cols]))
    ref = oracle.w4_gemm(x, oc, os_)
    # row-rms floor from the full GPU row (the sampled reference has too few entries)
    rms = np.sqrt((y.astype(np.float64) ** 2).mean(axis=1, keepdims=True))
    err = np.abs(y[:, cols] - ref) / np.maximum(np.abs(ref), rms)
    assert err.max() <= GEMM_RTOL, err.max()


@pytest.mark.parametrize("M,N,K", [(3, 65600, 576), (4, 66000, 640), (1, 70000, 512)])
def test_gemm_many_tiles_split_inside_workgroup(M, N, K):
    """More than 1024 tiles of 64 rows: each workgroup splits K over several
    wavefronts (3 here) and reduces in LDS; every output against the oracle."""
    log(f"gemm many tiles M={M} N={N} K={K}")
    w = _weights(11 * N + K, N, K)
    x = synth.activations_bf16(M * 7 + N, M, K)
    packed, pscales = B.w4_quantize_packed(dev(w))
    y = host(_gemm(x, packed, pscales, M, N, K))
    oc, os_ = oracle.w4_quantize(w)
    assert gemm_rel_err(y, oracle.w4_gemm(x, oc, os_)) <= GEMM_RTOL


@pytest.mark.slow
def test_lm_head_large_vocab_sampled():
    """d=5120, V=151936 LM head at M=4, sampled outputs against the oracle."""
    V, d = synth.LM_LARGE["V"], synth.LM_LARGE["d"]
    log(f"gemm LM head V={V} d={d}")
    w = _weights(31337, V, d)
    x = synth.activations_bf16(31338, 4, d)
    packed, pscales = B.w4_quantize_packed(dev(w))
    y = host(_gemm(x, packed, pscales, 4, V, d))
    g = np.random.default_rng(1)
    cols = np.unique(np.concatenate([g.integers(0, V, 250), [0, V - 1, V - 64]]))
    oc, os_ = oracle.w4_quantize(np.ascontiguousarray(w[cols]))
    ref = oracle.w4_gemm(x, oc, os_)
    rms = np.sqrt((y.astype(np.float64) ** 2).mean(axis=1, keepdims=True))
    err = np.abs(y[:, cols] - ref) / np.maximum(np.abs(ref), rms)
    assert err.max() <= GEMM_RTOL, err.max()


def _rmsnorm_inputs(M, K, seed):
    resid = synth.activations_bf16(seed, M, K, 2.0)
    gamma = synth.f32_to_bf16_bits(1.0 + synth.normal_f32(synth.rng(seed + 1), (K,), 0.02))
    return resid, gamma


@pytest.mark.parametrize("M,N,K", [(4, 7168, 5120), (1, 100, 320), (6, 333, 1024), (8, 64, 5120), (3, 5120, 16384)])
def test_rmsnorm_gemm_equals_norm_then_gemm(M, N, K):
    """The GEMM that normalises its own activations gives bitwise the partials
    of vw4_add_rmsnorm followed by the plain GEMM, and those match the oracle."""
    import torch
    log(f"rmsnorm gemm M={M} N={N} K={K}")
    resid, gamma = _rmsnorm_inputs(M, K, N + K)
    w = _weights(3 * N + K, N, K)
    packed, pscales = B.w4_quantize_packed(dev(w))
    S, ldp = B.gemm_partials_layout(M, N, K)
    rd, gd = dev(resid), dev(gamma)
    nws = B.workspace(B.norm_workspace_bytes(M, K))
    h = torch.empty((M, K), dtype=torch.int16, device="cuda")
    B.add_rmsnorm(rd, None, 1, K, gd, 1e-6, M, K, h, nws)
    p_ref = torch.empty(S * M * ldp, dtype=torch.float32, device="cuda")
    B.w4_skinny_gemm_partials(h, packed, pscales, p_ref, M, N, K)
    nws2 = B.workspace(B.norm_workspace_bytes(M, K))
    B.add_sumsq(rd, None, 1, K, M, K, nws2)
    p = torch.empty(S * M * ldp, dtype=torch.float32, device="cuda")
    B.w4_skinny_gemm_rmsnorm_partials(rd, gd, nws2, 1e-6, packed, pscales, p, M, N, K)
    torch.cuda.synchronize()
    # the defined part of the partials (columns past N are padding)
    assert torch.equal(p.view(S, M, ldp)[:, :, :N], p_ref.view(S, M, ldp)[:, :, :N])
    hh = host(h)
    assert np.array_equal(hh, oracle.bf16_round(oracle.rmsnorm(resid, gamma, 1e-6))) or \
        np.mean(hh == oracle.bf16_round(oracle.rmsnorm(resid, gamma, 1e-6))) > 0.999
    y = host(p).reshape(S, M, ldp).astype(np.float64).sum(axis=0)[:, :N]
    oc, os_ = oracle.w4_quantize(w)
    assert gemm_rel_err(y, oracle.w4_gemm(hh, oc, os_)) <= GEMM_RTOL


def test_rmsnorm_gemm_rejects_more_than_64_chunks():
    """The normalising GEMMs take at most 64 chunk sums per row (K <= 16384):
    K = 16448 is refused on the host, before any launch."""
    import torch
    M, N, K = 2, 64, 16448
    resid = torch.zeros((M, K), dtype=torch.int16, device="cuda")
    gamma = torch.zeros(K, dtype=torch.int16, device="cuda")
    nws = B.workspace(B.norm_workspace_bytes(M, K))
    packed = torch.zeros(N * K // 2, dtype=torch.uint8, device="cuda")
    pscales = torch.zeros(N * K // 64, dtype=torch.int16, device="cuda")
    part = torch.zeros(8 * M * (N + 64), dtype=torch.float32, device="cuda")
    a = torch.zeros((M, 32), dtype=torch.int16, device="cuda")
    with pytest.raises(B.VW4Error, match="K <= 16384"):
        B.w4_skinny_gemm_rmsnorm_partials(resid, gamma, nws, 1e-6, packed, pscales, part, M, N, K)
    with pytest.raises(B.VW4Error, match="K <= 16384"):
        B.w4_skinny_gemm_rmsnorm_swiglu(resid, gamma, nws, 1e-6, packed, pscales, a, 32, M, 32, K)


def _swiglu_ref(h_bits, w_gu, F):
    """Oracle: gate|up products of h (natural row order), SwiGLU on the unrounded sums, bf16."""
    oc, os_ = oracle.w4_quantize(w_gu)
    gu = oracle.w4_gemm(h_bits, oc, os_)
    return oracle.swiglu(gu[:, :F], gu[:, F:])


@pytest.mark.parametrize("M,F,K", [(4, 512, 1024), (1, 96, 320), (6, 2176, 5120), (8, 256, 5120), (4, 17408, 5120)])
def test_rmsnorm_swiglu_gemm_against_oracle(M, F, K):
    """Fused gate|up projection of rmsnorm(resid) * gamma with the SwiGLU in the
    epilogue (gate/up-interleaved weights) against the oracle composition."""
    import torch
    from layer_parity import bf16_close
    log(f"rmsnorm+swiglu gemm M={M} F={F} K={K}")
    resid, gamma = _rmsnorm_inputs(M, K, F + K)
    w = _weights(5 * F + K, 2 * F, K)
    packed, pscales = B.w4_quantize_packed(dev(B.interleave_gate_up(w)))
    rd, gd = dev(resid), dev(gamma)
    nws = B.workspace(B.norm_workspace_bytes(M, K))
    B.add_sumsq(rd, None, 1, K, M, K, nws)
    a = torch.full((M, F + 8), -1, dtype=torch.int16, device="cuda")
    B.w4_skinny_gemm_rmsnorm_swiglu(rd, gd, nws, 1e-6, packed, pscales, a, F + 8, M, F, K)
    torch.cuda.synchronize()
    ah = host(a)
    assert (ah[:, F:] == 0xFFFF).all()                  # nothing past F in each row
    h = oracle.bf16_round(oracle.rmsnorm(resid, gamma, 1e-6))
    if F * K > 20_000_000:                              # full-size FFN: a sample of features
        cols = np.unique(np.random.default_rng(F).integers(0, F, 96))
        wsel = np.ascontiguousarray(np.concatenate([w[cols], w[F + cols]]))
        ref = _swiglu_ref(h, wsel, len(cols))
        bf16_close(np.ascontiguousarray(ah[:, cols]), ref, min_exact=0.9)
    else:
        bf16_close(np.ascontiguousarray(ah[:, :F]), _swiglu_ref(h, w, F), min_exact=0.9)


@pytest.mark.parametrize("M,F,K", [(4, 17408, 5120), (1, 96, 320), (6, 544, 1024), (2, 3200, 512)])
def test_swiglu_gemm_against_oracle(M, F, K):
    """Gate|up GEMM on given activations with the SwiGLU epilogue."""
    import torch
    from layer_parity import bf16_close
    log(f"swiglu gemm M={M} F={F} K={K}")
    x = synth.activations_bf16(F + 3, M, K)
    w = _weights(7 * F + K, 2 * F, K)
    packed, pscales = B.w4_quantize_packed(dev(B.interleave_gate_up(w)))
    a = torch.empty((M, F), dtype=torch.int16, device="cuda")
    B.w4_skinny_gemm_swiglu(dev(x), packed, pscales, a, F, M, F, K)
    torch.cuda.synchronize()
    ah = host(a)
    if F * K > 20_000_000:
        cols = np.unique(np.random.default_rng(F + 1).integers(0, F, 96))
        wsel = np.ascontiguousarray(np.concatenate([w[cols], w[F + cols]]))
        bf16_close(np.ascontiguousarray(ah[:, cols]), _swiglu_ref(x, wsel, len(cols)), min_exact=0.9)
    else:
        bf16_close(ah, _swiglu_ref(x, w, F), min_exact=0.9)


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (4096 * 16 + 16, 7), (10 << 20, 2048), ((3 << 20) + 48, 300)])
def test_stream_read_reads_every_word(nbytes, blocks):
    """The read-ceiling kernel reads the whole buffer: the XOR of its
    per-workgroup words equals the XOR of the buffer's 32-bit words."""
    import torch
    log(f"stream_read bytes={nbytes} blocks={blocks}")
    words = np.random.default_rng(nbytes % 1000 + blocks).integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64)
    buf = torch.from_numpy(words.astype(np.uint32).view(np.int32)).cuda()
    sink = torch.full((blocks + 3,), 12345, dtype=torch.int32, device="cuda")
    B.stream_read(buf, sink, blocks)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(host(sink)[:blocks].view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(words.astype(np.uint32)))
    assert (host(sink)[blocks:] == 12345).all()
