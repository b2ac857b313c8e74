"""Pins of the oracle's decoder-layer pieces: RMSNorm, SwiGLU, RoPE (a8),
GQA decode attention (a9) and the MoE router (a10).

Independent references: closed forms (unit RMS, scale invariance, rotation
norm, relative-position property), torch's CPU silu and softmax, and special
cases of attention whose answer is fixed (equal keys give the mean of V, a
single position gives v0, future positions do not matter).
"""
import numpy as np
import torch

import oracle
from verify_step_w4_amd import synth


def test_rmsnorm_closed_forms():
    x = synth.activations_bf16(1, 3, 256, 3.0)
    ones = synth.f32_to_bf16_bits(np.ones(256, np.float32))
    y = oracle.rmsnorm(x, ones, eps=0.0)
    assert np.allclose(np.sqrt((y ** 2).mean(axis=1)), 1.0, rtol=1e-13)
    # scale invariance under an exact power-of-two scaling of the input
    x2 = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(x) * np.float32(4.0))
    np.testing.assert_allclose(oracle.rmsnorm(x2, ones, 0.0), y, rtol=1e-13)
    gam = synth.activations_bf16(2, 1, 256)[0]
    yg = oracle.rmsnorm(x, gam, 0.0)
    np.testing.assert_allclose(yg, y * synth.bf16_bits_to_f32(gam).astype(np.float64), rtol=1e-13)


def test_swiglu_against_torch():
    g = synth.activations_bf16(3, 1, 4096, 3.0)[0]
    u = synth.activations_bf16(4, 1, 4096)[0]
    y = oracle.swiglu(g, u)
    gt = torch.from_numpy(synth.bf16_bits_to_f32(g).astype(np.float64))
    ut = torch.from_numpy(synth.bf16_bits_to_f32(u).astype(np.float64))
    ref = (torch.nn.functional.silu(gt) * ut).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-300)


def test_swiglu_f64_against_torch():
    g = synth.normal_f32(synth.rng(13), (2048,), 4.0).astype(np.float64) / 3.0
    u = synth.normal_f32(synth.rng(14), (2048,), 1.0).astype(np.float64) * 1.1
    y = oracle.swiglu(g, u)
    ref = (torch.nn.functional.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-300)


def _dequant(codes, scales):
    """fp64 weights from the canonical format: code c (u - 8) times the fp16 scale of its group."""
    c = oracle.w4_codes_int(codes).astype(np.float64)
    s = np.vectorize(oracle.f16_value)(scales).astype(np.float64)
    return c * np.repeat(s, 64, axis=1)


def _moe_bank(seed, E, F, D):
    gu = [oracle.w4_quantize(synth.linear_weights(seed + e, 2 * F, D)) for e in range(E)]
    dn = [oracle.w4_quantize(synth.linear_weights(seed + 100 + e, D, F)) for e in range(E)]
    stack = lambda L: (np.stack([a for a, _ in L]), np.stack([b for _, b in L]))
    return stack(gu), stack(dn)


def test_moe_block_brute_force():
    """Expert-by-expert against numpy: dequantised fp64 matrices, argsort routing,
    softmax weights, gate = first F rows, SwiGLU, down projection."""
    E, F, D, topk, M = 6, 64, 128, 3, 3
    gate_up, down = _moe_bank(300, E, F, D)
    x = synth.activations_bf16(301, M, D)
    lg = synth.synthetic_logits(302, M, E, 1.0)
    ex, wt, y = oracle.moe_block(x, lg, topk, gate_up, down)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    ref = np.zeros((M, D))
    for m in range(M):
        order = np.argsort(-lg[m].astype(np.float64), kind="stable")[:topk]
        p = np.exp(lg[m].astype(np.float64) - lg[m].max())
        w = p[order] / p[order].sum()
        for e, we in zip(order, w):
            W1 = _dequant(gate_up[0][e], gate_up[1][e])
            h = W1 @ xf[m]
            g, u = h[:F], h[F:]
            a = synth.bf16_bits_to_f32(oracle.bf16_round(g / (1 + np.exp(-g)) * u)).astype(np.float64)
            ref[m] += we * (_dequant(down[0][e], down[1][e]) @ a)
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())
    assert (ex == np.stack([np.argsort(-lg[m].astype(np.float64), kind="stable")[:topk] for m in range(M)])).all()


def test_moe_block_identical_experts_is_dense():
    """With every expert equal, the renormalised weights sum to one and the
    block is the single expert's FFN whatever the routing."""
    E, F, D, topk, M = 5, 64, 128, 2, 2
    gate_up, down = _moe_bank(400, 1, F, D)
    gate_up = tuple(np.repeat(a, E, axis=0) for a in gate_up)
    down = tuple(np.repeat(a, E, axis=0) for a in down)
    x = synth.activations_bf16(401, M, D)
    _, _, y = oracle.moe_block(x, synth.synthetic_logits(402, M, E, 1.0), topk, gate_up, down)
    _, _, y1 = oracle.moe_block(x, np.zeros((M, 1), np.float32), 1, tuple(a[:1] for a in gate_up),
                                tuple(a[:1] for a in down))
    np.testing.assert_allclose(y, y1, rtol=1e-13, atol=1e-15)


def test_rope_rotation_properties():
    g = np.random.default_rng(5)
    q = g.standard_normal(128)
    k = g.standard_normal(128)
    assert np.allclose(oracle.rope(q, 0), q, rtol=0, atol=0)
    for pos in (1, 77, 4099):
        assert abs(np.linalg.norm(oracle.rope(q, pos)) - np.linalg.norm(q)) < 1e-10
    # <R(a) q, R(b) k> depends only on a - b
    d1 = oracle.rope(q, 1030) @ oracle.rope(k, 1000)
    d2 = oracle.rope(q, 40) @ oracle.rope(k, 10)
    assert abs(d1 - d2) < 1e-9
    # pair d = 0 (the highest frequency) rotates by exactly pos radians
    e = np.zeros(128)
    e[0] = 1.0
    r = oracle.rope(e, 3)
    assert abs(r[0] - np.cos(3)) < 1e-15 and abs(r[64] - np.sin(3)) < 1e-15


def test_rope_frequency_schedule_hand_values():
    """Pair d of a head of H dims turns by pos * theta^(-2d/H): at H = 128 and
    theta = 10000 that is pos * 10^(-d/16), so pair 16 turns by pos / 10,
    pair 32 by pos / 100 and pair 48 by pos / 1000 (rotate-half: dims d and
    d + H/2).  These values hold for no other exponent (theta^(-d/H) would
    give pos / 10^(d/32)), so a wrong schedule fails here."""
    H = 128
    cases = [(32, 100, 1.0), (16, 10, 1.0), (48, 2500, 2.5), (8, 4, 4 * 10 ** -0.5), (63, 7, 7 * 10 ** (-63 / 16))]
    for d, pos, ang in cases:
        e = np.zeros(H)
        e[d] = 1.0
        r = oracle.rope(e, pos)
        assert abs(r[d] - np.cos(ang)) < 1e-12 and abs(r[d + H // 2] - np.sin(ang)) < 1e-12, (d, pos)
        # every other entry stays zero: the pair turns only within itself
        rest = np.delete(r, [d, d + H // 2])
        assert np.all(rest == 0.0)
        # the second half of the pair turns the other way round: (0, 1) -> (-sin, cos)
        f = np.zeros(H)
        f[d + H // 2] = 1.0
        r2 = oracle.rope(f, pos)
        assert abs(r2[d] + np.sin(ang)) < 1e-12 and abs(r2[d + H // 2] - np.cos(ang)) < 1e-12, (d, pos)
    # another head size and base: H = 64, theta = 1e6, pair 16 turns by pos / 1000
    e = np.zeros(64)
    e[16] = 1.0
    r = oracle.rope(e, 1000, theta=1e6)
    assert abs(r[16] - np.cos(1.0)) < 1e-12 and abs(r[48] - np.sin(1.0)) < 1e-12


def _kv(seed, Hkv, Lc, Dh):
    return (synth.activations_bf16(seed, Hkv * Lc, Dh).reshape(Hkv, Lc, Dh),
            synth.activations_bf16(seed + 1, Hkv * Lc, Dh).reshape(Hkv, Lc, Dh))


def test_attention_special_cases():
    M, Hq, Hkv, Dh, L = 3, 10, 2, 64, 20
    Lc = L + M
    Kc, Vc = _kv(7, Hkv, Lc, Dh)
    q = np.random.default_rng(1).standard_normal((M, Hq, Dh))
    # equal keys -> uniform weights -> mean of the visible values
    Keq = np.repeat(Kc[:, :1, :], Lc, axis=1).copy()
    out = oracle.decode_attn(q, Keq, Vc, L)
    Vf = synth.bf16_bits_to_f32(Vc).astype(np.float64)
    for i in range(M):
        for h in range(Hq):
            np.testing.assert_allclose(out[i, h], Vf[h // 5, :L + i + 1].mean(axis=0), rtol=1e-12)
    # a single visible position returns v0
    out1 = oracle.decode_attn(q[:1], Kc, Vc, 0)
    for h in range(Hq):
        np.testing.assert_allclose(out1[0, h], Vf[h // 5, 0], rtol=1e-15)
    # causality: changing positions beyond L+i does not change row i
    Vc2 = Vc.copy()
    Vc2[:, L + 1:, :] = 0
    ref = oracle.decode_attn(q, Kc, Vc, L)
    out2 = oracle.decode_attn(q, Kc, Vc2, L)
    np.testing.assert_array_equal(out2[0], ref[0])
    assert not np.array_equal(out2[1], ref[1])


def test_attention_matches_torch_softmax():
    M, Hq, Hkv, Dh, L = 2, 8, 2, 32, 50
    Kc, Vc = _kv(9, Hkv, L + M, Dh)
    q = np.random.default_rng(2).standard_normal((M, Hq, Dh))
    out = oracle.decode_attn(q, Kc, Vc, L)
    Kf = torch.from_numpy(synth.bf16_bits_to_f32(Kc).astype(np.float64))
    Vf = torch.from_numpy(synth.bf16_bits_to_f32(Vc).astype(np.float64))
    for i in range(M):
        for h in range(Hq):
            s = Kf[h // 4, :L + i + 1] @ torch.from_numpy(q[i, h]) / np.sqrt(Dh)
            ref = torch.softmax(s, 0) @ Vf[h // 4, :L + i + 1]
            np.testing.assert_allclose(out[i, h], ref.numpy(), rtol=1e-12, atol=1e-14)


def test_moe_route_against_sort_and_softmax():
    lg = synth.synthetic_logits(4, 4, 128, 1.0)
    lg[2, 5] = lg[2, 9] = lg[2].max() + 1          # tie -> lower index first
    ex, wt = oracle.moe_route(lg, 8)
    for m in range(4):
        order = np.argsort(-lg[m].astype(np.float64), kind="stable")[:8]
        assert list(ex[m]) == list(order)
        pr = torch.softmax(torch.from_numpy(lg[m].astype(np.float64)), 0).numpy()
        np.testing.assert_allclose(wt[m], pr[order] / pr[order].sum(), rtol=1e-13)
        assert abs(wt[m].sum() - 1) < 1e-14
    assert ex[2, 0] == 5 and ex[2, 1] == 9
