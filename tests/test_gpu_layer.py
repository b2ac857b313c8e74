"""GPU parity of the decoder-layer calls (a8, a9) against the oracle on the
same synthetic bf16/fp32 inputs.

Outputs are stored as bf16, so the bar is the bf16 rounding of the exact
value: |gpu - ref| <= 2^-8 |ref| + 1e-3 * rms(ref) (half an ulp of rounding on
each side plus fp32 accumulation), with almost all elements bit-identical."""
import numpy as np
import pytest

import oracle
from verify_step_w4_amd import binding as B
from verify_step_w4_amd import synth

from helpers import dev, host, log, rows_from_vb, vb_from_rows

pytestmark = pytest.mark.gpu

from layer_parity import BF16_REL, bf16_close  # noqa: F401  (the bf16 bar, shared with the composed tests)


def partials(seed, S, M, N, ldp, std=1.0):
    p = synth.normal_f32(synth.rng(seed), (S, M, ldp), std)
    return p


@pytest.mark.parametrize("M,D,S", [(1, 5120, 1), (4, 5120, 3), (6, 1000, 2), (4, 2048, 1)])
def test_add_rmsnorm(M, D, S):
    import torch
    log(f"add_rmsnorm M={M} D={D} S={S}")
    ldp = (D + 63) // 64 * 64
    resid = synth.activations_bf16(M + D, M, D)
    part = partials(S + D, S, M, D, ldp, 0.5)
    gamma = synth.f32_to_bf16_bits(1.0 + synth.normal_f32(synth.rng(3), (D,), 0.02))
    rd, hd = dev(resid), torch.empty((M, D), dtype=torch.int16, device="cuda")
    B.add_rmsnorm(rd, dev(part), S, ldp, dev(gamma), 1e-6, M, D, hd, B.workspace(B.norm_workspace_bytes(M, D)))
    torch.cuda.synchronize()
    # oracle: exact sum and one bf16 rounding for the residual; h is the
    # RMSNorm of the residual as stored (the kernels sum the partials in fp32,
    # so a residual within 1e-7 of a bf16 rounding midpoint may land one ulp
    # from the exact rounding; the residual check covers that ulp, and h is
    # judged on the residual it was computed from)
    exact = synth.bf16_bits_to_f32(resid).astype(np.float64) + part[:, :, :D].astype(np.float64).sum(axis=0)
    bf16_close(host(rd), exact)
    h_ref = oracle.rmsnorm(host(rd), gamma, 1e-6)
    bf16_close(host(hd), h_ref)


def test_bf16_rounding_of_fp32_bit_patterns():
    """The kernels' fp32 -> bf16 conversion is round to nearest even: with a
    zero residual and one partial, vw4_add_sumsq stores bf16(0 + p) = bf16(p).
    2^20 patterns: random words plus ties (low half 0x8000, both parities),
    carries into the exponent, overflow to infinity, subnormals and NaNs; each
    finite one against the oracle's rounding of the same value, NaN -> NaN."""
    import torch
    M, D = 16, 65536
    g = np.random.default_rng(20261203)
    u = g.integers(0, 2 ** 32, size=M * D, dtype=np.uint64).astype(np.uint32)
    hi = g.integers(0, 2 ** 16, size=M * D // 8, dtype=np.uint64).astype(np.uint32)
    n = len(hi)
    u[:n] = (hi << 16) | 0x8000                           # exact ties
    u[n:2 * n] = (hi << 16) | g.integers(0x7f00, 0x8100, n).astype(np.uint32)   # near ties
    u[2 * n:3 * n] = g.integers(0, 0x00800000, n).astype(np.uint32) | (hi & 0x8000) << 16   # subnormals
    special = np.array([0x7f7fffff, 0x7f7f8000, 0x7f7f7fff, 0xff7fffff, 0x7f800000, 0xff800000, 0x7fc00000,
                        0x7f800001, 0xffffffff, 0x00000001, 0x00008000, 0x00018000, 0x3f808000, 0x3f818000,
                        0x3fffffff, 0x00000000], dtype=np.uint32)
    u[3 * n:3 * n + len(special)] = special
    u[u == 0x80000000] = 0                               # -0 + (+0) is +0: left out
    f = u.view(np.float32).reshape(M, D)
    resid = torch.zeros((M, D), dtype=torch.int16, device="cuda")
    B.add_sumsq(resid, dev(f.reshape(1, M, D)), 1, D, M, D, B.workspace(B.norm_workspace_bytes(M, D)))
    torch.cuda.synchronize()
    got = host(resid).view(np.uint16).reshape(-1)
    nan = np.isnan(f.reshape(-1))
    assert np.all(((got & 0x7fff) > 0x7f80)[nan])
    ref = oracle.bf16_round(f.reshape(-1)[~nan].astype(np.float64)).view(np.uint16)
    assert np.array_equal(got[~nan], ref), int((got[~nan] != ref).sum())


@pytest.mark.parametrize("M,D,S", [(4, 5120, 8), (1, 5120, 1), (6, 1000, 3), (4, 2048, 0), (3, 8192, 8),
                                   (2, 4, 1), (64, 260, 2), (4, 3072, 4), (5, 2304, 8), (2, 4100, 5)])
def test_add_rmsnorm_out_equals_two_launch_path(M, D, S):
    """The one-launch, out-of-place add + RMSNorm gives bitwise the residual
    and h of vw4_add_rmsnorm (same chunk sums, same order), and matches the
    oracle; resid_in is left unchanged."""
    import torch
    log(f"add_rmsnorm_out M={M} D={D} S={S}")
    ldp = (D + 63) // 64 * 64
    resid = synth.activations_bf16(M * 3 + D, M, D)
    part = partials(S + D + 1, max(S, 1), M, D, ldp, 0.5)
    gamma = synth.f32_to_bf16_bits(1.0 + synth.normal_f32(synth.rng(D + 5), (D,), 0.02))
    pd = dev(part) if S else None
    r1, h1 = dev(resid), torch.empty((M, D), dtype=torch.int16, device="cuda")
    B.add_rmsnorm(r1, pd, max(S, 1), ldp, dev(gamma), 1e-6, M, D, h1, B.workspace(B.norm_workspace_bytes(M, D)))
    rin = dev(resid)
    r2, h2 = torch.full((M, D), 7, dtype=torch.int16, device="cuda"), torch.empty((M, D), dtype=torch.int16,
                                                                                   device="cuda")
    B.add_rmsnorm_out(rin, pd, max(S, 1), ldp, dev(gamma), 1e-6, M, D, r2, h2)
    torch.cuda.synchronize()
    assert np.array_equal(host(rin), resid)
    assert np.array_equal(host(r2), host(r1))
    assert np.array_equal(host(h2), host(h1))
    exact = synth.bf16_bits_to_f32(resid).astype(np.float64)
    if S:
        exact = exact + part[:, :, :D].astype(np.float64).sum(axis=0)
    bf16_close(host(r2), exact)
    bf16_close(host(h2), oracle.rmsnorm(host(r2), gamma, 1e-6))   # h of the stored residual


def test_add_rmsnorm_out_rejects_bad_arguments():
    import torch
    M, D = 2, 1024
    a = torch.zeros((M, 8200), dtype=torch.int16, device="cuda")
    b = torch.zeros((M, 8200), dtype=torch.int16, device="cuda")
    hh = torch.zeros((M, 8200), dtype=torch.int16, device="cuda")
    g = torch.zeros(8200, dtype=torch.int16, device="cuda")
    p = torch.zeros(9 * M * 8256, dtype=torch.float32, device="cuda")
    with pytest.raises(B.VW4Error, match="D % 4 == 0"):
        B.add_rmsnorm_out(a, None, 1, 1024, g, 1e-6, M, 1022, b, hh)
    with pytest.raises(B.VW4Error, match="D <= 8192"):
        B.add_rmsnorm_out(a, None, 1, 8196, g, 1e-6, M, 8196, b, hh)
    with pytest.raises(B.VW4Error, match="S <= 8"):
        B.add_rmsnorm_out(a, p, 9, 1024, g, 1e-6, M, D, b, hh)
    with pytest.raises(B.VW4Error, match="must not overlap"):
        B.add_rmsnorm_out(a, p, 1, 1024, g, 1e-6, M, D, a, hh)


def test_rmsnorm_without_add():
    import torch
    M, D = 3, 5120
    resid = synth.activations_bf16(5, M, D, 2.0)
    gamma = synth.f32_to_bf16_bits(1.0 + synth.normal_f32(synth.rng(6), (D,), 0.02))
    rd, hd = dev(resid), torch.empty((M, D), dtype=torch.int16, device="cuda")
    B.add_rmsnorm(rd, None, 1, D, dev(gamma), 1e-6, M, D, hd, B.workspace(B.norm_workspace_bytes(M, D)))
    torch.cuda.synchronize()
    assert np.array_equal(host(rd), resid)
    bf16_close(host(hd), oracle.rmsnorm(resid, gamma, 1e-6))


@pytest.mark.parametrize("M,L,S", [(4, 0, 1), (4, 8191, 2), (1, 32767, 3)])
def test_rope_kv_append(M, L, S):
    import torch
    nq, nkv, hd = 40, 8, 128
    N = (nq + 2 * nkv) * hd
    ldp = N
    Lmax = (L + M + 3 + 31) // 32 * 32                # the value cache is kept in 32-position blocks
    log(f"rope_kv M={M} L={L} S={S}")
    part = partials(L + S, S, M, N, ldp)
    qd = torch.empty((M, nq, hd), dtype=torch.int16, device="cuda")
    Kc = torch.zeros((nkv, Lmax, hd), dtype=torch.int16, device="cuda")
    Vc = torch.zeros((nkv, Lmax // 32, hd, 32), dtype=torch.int16, device="cuda")   # blocked values
    B.rope_kv_append(dev(part), S, ldp, M, nq, nkv, hd, L, 10000.0, qd, Kc, Vc, Lmax)
    torch.cuda.synchronize()
    x = part.astype(np.float64).sum(axis=0)          # exact sum of the partials
    q_ref = np.zeros((M, nq, hd))
    k_ref = np.zeros((M, nkv, hd))
    for m in range(M):
        for h in range(nq):
            q_ref[m, h] = oracle.rope(x[m, h * hd:(h + 1) * hd], L + m)
        for h in range(nkv):
            k_ref[m, h] = oracle.rope(x[m, (nq + h) * hd:(nq + h + 1) * hd], L + m)
    v_ref = x[:, (nq + nkv) * hd:].reshape(M, nkv, hd)
    bf16_close(host(qd), q_ref)
    Kh, Vh = host(Kc), rows_from_vb(host(Vc))
    bf16_close(np.stack([Kh[:, L + m] for m in range(M)]), k_ref)
    bf16_close(np.stack([Vh[:, L + m] for m in range(M)]), v_ref)
    # nothing else of the cache is touched
    mask = np.ones(Lmax, bool)
    mask[L:L + M] = False
    assert not Kh[:, mask].any() and not Vh[:, mask].any()


@pytest.mark.parametrize("M,F,S", [(4, 17408, 2), (1, 768, 1), (6, 300, 3)])
def test_swiglu(M, F, S):
    import torch
    log(f"swiglu M={M} F={F} S={S}")
    ldp = (2 * F + 63) // 64 * 64
    part = partials(F + S, S, M, 2 * F, ldp, 1.5)
    ad = torch.empty((M, F), dtype=torch.int16, device="cuda")
    B.swiglu(dev(part), S, ldp, M, F, ad)
    torch.cuda.synchronize()
    x = part.astype(np.float64).sum(axis=0)
    g, u = x[:, :F], x[:, F:2 * F]
    ref = g / (1.0 + np.exp(-g)) * u
    bf16_close(host(ad), ref)


def _attn_case(M, nq, nkv, L, seed, Lmax=None):
    import torch
    hd = 128
    Lmax = Lmax or (L + M + 5 + 31) // 32 * 32
    q = synth.activations_bf16(seed, M * nq, hd).reshape(M, nq, hd)
    Kc = synth.activations_bf16(seed + 1, nkv * Lmax, hd).reshape(nkv, Lmax, hd)
    Vc = synth.activations_bf16(seed + 2, nkv * Lmax, hd).reshape(nkv, Lmax, hd)
    out = torch.empty((M, nq * hd), dtype=torch.int16, device="cuda")
    ws = B.workspace(B.attn_workspace_bytes(M, nq, nkv, hd, L + M))
    B.decode_attn(dev(q), dev(Kc), dev(vb_from_rows(Vc)), Lmax, L, M, nq, nkv, hd, out, ws)
    torch.cuda.synchronize()
    return q, Kc, Vc, host(out).reshape(M, nq, hd)


@pytest.mark.parametrize("M,nq,nkv,L", [(4, 40, 8, 0), (4, 40, 8, 100), (1, 40, 8, 1023), (4, 40, 8, 1024),
                                        (2, 8, 2, 777), (6, 10, 2, 300), (4, 40, 8, 8192), (8, 40, 8, 777),
                                        (3, 40, 8, 31), (6, 40, 8, 2049), (1, 40, 8, 0), (4, 40, 8, 32764),
                                        (4, 40, 8, 1051), (1, 40, 8, 30), (4, 40, 4, 4000), (2, 8, 2, 6000)])
def test_decode_attn(M, nq, nkv, L):
    log(f"attn M={M} nq={nq} nkv={nkv} L={L}")
    q, Kc, Vc, out = _attn_case(M, nq, nkv, L, 1000 + L + M)
    ref = oracle.decode_attn(synth.bf16_bits_to_f32(q).astype(np.float64), Kc, Vc, L)
    bf16_close(out, ref)


def test_decode_attn_context_ends_at_cache_end():
    """L + M == Lmax: the last tile's rows run past the cache and must be masked."""
    M, nq, nkv, L = 4, 40, 8, 1020
    q, Kc, Vc, out = _attn_case(M, nq, nkv, L, 55, Lmax=1024)
    ref = oracle.decode_attn(synth.bf16_bits_to_f32(q).astype(np.float64), Kc, Vc, L)
    bf16_close(out, ref)


def test_decode_attn_ignores_cache_past_context():
    """NaN in every cache position at or past L + M (stale memory) changes
    nothing: 31 positions past the last whole tile (merge pass) and a partial
    8-position piece."""
    import torch
    M, nq, nkv, L, hd = 4, 40, 8, 1051, 128
    q, Kc, Vc, out = _attn_case(M, nq, nkv, L, 17)
    Lmax = Kc.shape[1]
    Kc2, Vc2 = Kc.copy(), Vc.copy()
    Kc2[:, L + M:] = 0x7fc0
    Vc2[:, L + M:] = 0xffc0
    out2 = torch.empty((M, nq * hd), dtype=torch.int16, device="cuda")
    ws = B.workspace(B.attn_workspace_bytes(M, nq, nkv, hd, L + M))
    B.decode_attn(dev(q), dev(Kc2), dev(vb_from_rows(Vc2)), Lmax, L, M, nq, nkv, hd, out2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(out2).reshape(M, nq, hd), out)


def test_decode_attn_causal_rows():
    """Row m must not see positions beyond L + m: perturbing them leaves it unchanged."""
    import torch
    M, nq, nkv, L, hd = 4, 40, 8, 500, 128
    q, Kc, Vc, out = _attn_case(M, nq, nkv, L, 7)
    Lmax = Kc.shape[1]
    Kc2, Vc2 = Kc.copy(), Vc.copy()
    Kc2[:, L + 1:] = synth.activations_bf16(99, nkv * (Lmax - L - 1), hd).reshape(nkv, Lmax - L - 1, hd)
    Vc2[:, L + 1:] = 0
    out2 = torch.empty((M, nq * hd), dtype=torch.int16, device="cuda")
    ws = B.workspace(B.attn_workspace_bytes(M, nq, nkv, hd, L + M))
    B.decode_attn(dev(q), dev(Kc2), dev(vb_from_rows(Vc2)), Lmax, L, M, nq, nkv, hd, out2, ws)
    torch.cuda.synchronize()
    o2 = host(out2).reshape(M, nq, hd)
    assert np.array_equal(o2[0], out[0])
    assert not np.array_equal(o2[1], out[1])
