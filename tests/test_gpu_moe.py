"""GPU parity of the MoE calls (a10) against the oracle: router top-k and
slot list, grouped W4 GEMM, grouped gate|up GEMM with the SwiGLU epilogue,
down + combine (the whole expert layer), and the MoE-shaped verify step.

Routing is integer work and must match bit for bit (experts, slot list);
the routing weights are fp64 on both sides, stored fp32 (relative 2^-24).
Expert outputs follow the GEMM bar (1e-3 relative to max(|ref|, row rms)).
The expert layer and the whole MoE step are checked op by op, teacher forced:
each op is recomputed by the oracle from the GPU's own input to it (its
SwiGLU activations per slot, the fp32 sums of its split-K partials, its
residual rows) and held to its own bar; the end-to-end difference from the
oracle's own composition is reported as a statistic."""
import numpy as np
import pytest

import oracle
from verify_step_w4_amd import binding as B
from verify_step_w4_amd import synth
from verify_step_w4_amd.model import MOE_30B, ExpertBank, MoEVerify, W4Linear

from helpers import GEMM_RTOL, dev, gemm_rel_err, host, log
from layer_parity import bf16_close, slice_sum_f32

pytestmark = pytest.mark.gpu


def _route(lg, topk):
    import torch
    M, E = lg.shape
    ms = min(E, M * topk)
    ex = torch.empty((M, topk), dtype=torch.int32, device="cuda")
    wt = torch.empty((M, topk), dtype=torch.float32, device="cuda")
    se = torch.full((ms,), -7, dtype=torch.int32, device="cuda")
    ns = torch.zeros(1, dtype=torch.int32, device="cuda")
    rs = torch.empty((M, topk), dtype=torch.int32, device="cuda")
    B.moe_route(dev(lg), M, E, topk, ex, wt, se, ns, rs)
    torch.cuda.synchronize()
    return host(ex), host(wt), host(se), int(host(ns)[0]), host(rs)


def _check_route(lg, topk):
    ex, wt, se, ns, rs = _route(lg, topk)
    ex_o, wt_o = oracle.moe_route(lg, topk)
    assert np.array_equal(ex, ex_o)
    np.testing.assert_allclose(wt.astype(np.float64), wt_o, rtol=1.2e-7, atol=0)
    uniq = np.unique(ex_o)
    assert ns == len(uniq) and np.array_equal(se[:ns], uniq)
    assert (se[ns:] == -7).all()                      # nothing beyond the live slots is written
    assert np.array_equal(se[rs], ex)                 # row_slot names the slot of each choice
    return ns


@pytest.mark.parametrize("M,E,topk,seed", [(4, 128, 8, 1), (1, 128, 8, 2), (6, 128, 8, 3), (16, 1024, 64, 4),
                                           (3, 5, 5, 5), (2, 64, 1, 6)])
def test_moe_route(M, E, topk, seed):
    log(f"moe_route M={M} E={E} topk={topk}")
    lg = synth.synthetic_logits(seed, M, E, 1.0)
    _check_route(lg, topk)


def test_moe_route_ties_and_signed_zero():
    M, E, topk = 4, 128, 8
    lg = synth.synthetic_logits(9, M, E, 1.0)
    lg[0, 10] = lg[0, 3] = lg[0, 77] = lg[0].max() + 0.5     # three-way tie at the top -> 3, 10, 77
    lg[1] = 0.0
    lg[1, 5] = -0.0                                           # -0 == +0: index order decides
    lg[2, :] = np.float32(-1.0)
    lg[2, 100] = np.float32(-1.0) + np.float32(2.0 ** -23)    # one ulp above the rest
    lg[3, ::2] = lg[3, 1::2]                                  # pairs of equal logits
    ns = _check_route(lg, topk)
    ex, _, _, _, _ = _route(lg, topk)
    assert list(ex[0, :3]) == [3, 10, 77]
    assert list(ex[1]) == list(range(8))
    assert ex[2, 0] == 100 and list(ex[2, 1:]) == list(range(7))
    assert ns <= M * topk


def _host_bank(seed, E, F, d):
    g = synth.rng(seed)
    gu = synth.normal_f32(g, (E, 2 * F, d), 0.02)
    dn = synth.normal_f32(g, (E, d, F), 0.02)
    return gu, dn


def _oracle_bank(gu, dn):
    q_gu = [oracle.w4_quantize(w) for w in gu]
    q_dn = [oracle.w4_quantize(w) for w in dn]
    st = lambda L: (np.stack([a for a, _ in L]), np.stack([b for _, b in L]))
    return st(q_gu), st(q_dn)


@pytest.mark.parametrize("M,N,K,E,slots,max_slots", [(4, 1536, 2048, 6, [5, 0, 3], 5), (1, 192, 320, 4, [3], 1),
                                                     (6, 2048, 768, 3, [0, 1, 2], 8)])
def test_grouped_gemm_against_oracle(M, N, K, E, slots, max_slots):
    """Given slot list: live slots equal the oracle's per-expert GEMM; slots at
    or beyond n_slots are not written."""
    import torch
    log(f"grouped gemm M={M} N={N} K={K} E={E} slots={slots}")
    w = synth.normal_f32(synth.rng(N + K), (E, N, K), 0.02)
    bank = W4Linear.from_fp32(dev(w.reshape(E * N, K)))
    x = synth.activations_bf16(K + M, M, K)
    S, ldp = B.grouped_gemm_layout(M, N, K, max_slots)
    sst = S * M * ldp
    part = torch.full((max_slots * sst,), float("nan"), dtype=torch.float32, device="cuda")
    se = torch.zeros(max_slots, dtype=torch.int32, device="cuda")
    se[:len(slots)] = torch.tensor(slots, dtype=torch.int32)
    ns = torch.tensor([len(slots)], dtype=torch.int32, device="cuda")
    B.w4_grouped_gemm(dev(x), K, 0, bank.packed, N * K // 2, bank.pscales, N * K // 64, se, ns, max_slots, part, sst,
                      M, N, K)
    torch.cuda.synchronize()
    P = host(part).reshape(max_slots, S, M, ldp)
    for s, e in enumerate(slots):
        codes, scales = oracle.w4_quantize(w[e])
        ref = oracle.w4_gemm(x, codes, scales)
        y = P[s].astype(np.float64).sum(axis=0)[:, :N]
        err = gemm_rel_err(y, ref)
        assert err <= GEMM_RTOL, (s, e, err)
    assert np.isnan(P[len(slots):]).all()


@pytest.mark.parametrize("M,F,K,E,slots,max_slots", [(4, 768, 2048, 5, [4, 1, 2], 6), (1, 96, 320, 3, [2], 1)])
def test_grouped_gemm_swiglu_against_oracle(M, F, K, E, slots, max_slots):
    """Grouped gate|up projection with the SwiGLU in the epilogue: live slots
    equal the oracle's per-expert composition, the others are not written."""
    import torch
    log(f"grouped gemm+swiglu M={M} F={F} K={K} slots={slots}")
    w = synth.normal_f32(synth.rng(F + K + 1), (E, 2 * F, K), 0.02)
    wi = np.stack([B.interleave_gate_up(w[e]) for e in range(E)])
    bank = W4Linear.from_fp32(dev(wi.reshape(E * 2 * F, K)))
    x = synth.activations_bf16(K + M + 1, M, K)
    a = torch.full((max_slots, M, F), -1, dtype=torch.int16, device="cuda")
    se = torch.zeros(max_slots, dtype=torch.int32, device="cuda")
    se[:len(slots)] = torch.tensor(slots, dtype=torch.int32)
    ns = torch.tensor([len(slots)], dtype=torch.int32, device="cuda")
    B.w4_grouped_gemm_swiglu(dev(x), K, 0, bank.packed, 2 * F * K // 2, bank.pscales, 2 * F * K // 64, se, ns,
                             max_slots, a, M * F, M, F, K)
    torch.cuda.synchronize()
    ah = host(a)
    for s, e in enumerate(slots):
        oc, os_ = oracle.w4_quantize(w[e])
        gu = oracle.w4_gemm(x, oc, os_)
        bf16_close(np.ascontiguousarray(ah[s]), oracle.swiglu(gu[:, :F], gu[:, F:]), min_exact=0.9)
    assert (ah[len(slots):] == 0xFFFF).all()


def _moe_device(cfg, M, gu, dn, lm_w, gamma):
    bank = ExpertBank.from_fp32(dev(gu), dev(dn))
    mv = MoEVerify(cfg, M, W4Linear.from_fp32(dev(lm_w)), dev(gamma))
    return bank, mv


class MoECapture:
    """gemm_hook of MoEVerify.moe / forward: host copies of the routing, the
    per-slot SwiGLU activations and the per-slot down partials."""

    def __init__(self, mv):
        self.mv, self.c = mv, {}

    def __call__(self, when, name):
        import torch
        torch.cuda.synchronize()
        mv, c = self.mv, self.c
        if when == "post" and name == "gate_up":
            c["n_slots"] = int(host(mv.n_slots)[0])
            c["slot_expert"] = host(mv.slot_expert).copy()
            c["row_slot"] = host(mv.row_slot).copy()
            c["experts"] = host(mv.experts).copy()
            c["weights"] = host(mv.weights).copy()
            c["a"] = host(mv.a).copy()
        elif when == "post" and name == "down":
            P = host(mv.part_dn).reshape(mv.max_slots, mv.dn_S, mv.M, mv.dn_ldp)
            c["down"] = P[:, :, :, :mv.d].copy()


def check_moe_layer(cap, x, lg, topk, gu, dn, y_gpu):
    """Routing bit-exact; per live slot the SwiGLU activations (bf16 bar) and
    the down projection of the GPU's activations (1e-3); the weighted combine
    of the GPU's expert outputs (1e-3).  Returns the worst fp32 error."""
    c = cap.c
    ex_o, wt_o = oracle.moe_route(lg, topk)
    assert np.array_equal(c["experts"], ex_o)
    np.testing.assert_allclose(c["weights"].astype(np.float64), wt_o, rtol=1.2e-7, atol=0)
    F = gu.shape[1] // 2
    worst = 0.0
    outs = {}
    for s in range(c["n_slots"]):
        e = int(c["slot_expert"][s])
        g = oracle.w4_gemm(x, *oracle.w4_quantize(gu[e]))
        bf16_close(np.ascontiguousarray(c["a"][s]), oracle.swiglu(g[:, :F], g[:, F:]), min_exact=0.9,
                   what=f"slot {s} swiglu")
        o = slice_sum_f32(c["down"][s])
        err = gemm_rel_err(o, oracle.w4_gemm(np.ascontiguousarray(c["a"][s]), *oracle.w4_quantize(dn[e])))
        assert err <= GEMM_RTOL, (s, e, err)
        worst = max(worst, err)
        outs[s] = o.astype(np.float64)
    M = x.shape[0]
    y_ref = np.zeros((M, dn.shape[1]))
    for m in range(M):
        for t in range(topk):
            y_ref[m] += float(c["weights"][m, t]) * outs[int(c["row_slot"][m, t])][m]
    err = gemm_rel_err(y_gpu, y_ref)
    assert err <= GEMM_RTOL, ("combine", err)
    return max(worst, err)


@pytest.mark.parametrize("E,topk,d,F,M", [(16, 4, 512, 256, 4), (8, 8, 2048, 768, 4), (12, 3, 256, 128, 6),
                                          (128, 8, 256, 64, 1)])
def test_moe_layer_against_oracle(E, topk, d, F, M):
    """Route + grouped gate|up + grouped SwiGLU + grouped down + combine vs the
    oracle's expert-by-expert block on the same weights and router logits."""
    import torch
    log(f"moe layer E={E} topk={topk} d={d} F={F} M={M}")
    cfg = dict(n_exp=E, topk=topk, d=d, F=F, V=64, eps=1e-6)
    gu, dn = _host_bank(E + d, E, F, d)
    lm_w = synth.linear_weights(7, 64, d)
    gamma = synth.f32_to_bf16_bits(1 + synth.normal_f32(synth.rng(8), (d,), 0.02))
    bank, mv = _moe_device(cfg, M, gu, dn, lm_w, gamma)
    x = synth.activations_bf16(E + F, M, d)
    lg = synth.synthetic_logits(E + M, M, E, 1.0)
    cap = MoECapture(mv)
    y = host(mv.moe(dev(x), dev(lg), bank, gemm_hook=cap)).astype(np.float64)
    torch.cuda.synchronize()
    worst = check_moe_layer(cap, x, lg, topk, gu, dn, y)
    ex, wt, ref = oracle.moe_block(x, lg, topk, *_oracle_bank(gu, dn))
    assert np.array_equal(host(mv.experts), ex)
    print(f"[moe] n_slots {int(host(mv.n_slots)[0])} per op worst {worst:.2e}; "
          f"end to end (statistic) {gemm_rel_err(y, ref):.3e}", flush=True)


def test_moe_step_logits_against_oracle():
    """The whole MoE-shaped forward to the logits: x + moe(x), final RMSNorm, LM head."""
    import torch
    E, topk, d, F, M, V = 16, 4, 512, 256, 4, 3000
    log("moe step logits vs oracle")
    cfg = dict(n_exp=E, topk=topk, d=d, F=F, V=V, eps=1e-6)
    gu, dn = _host_bank(31, E, F, d)
    lm_w = synth.linear_weights(32, V, d)
    gamma = synth.f32_to_bf16_bits(1 + synth.normal_f32(synth.rng(33), (d,), 0.02))
    bank, mv = _moe_device(cfg, M, gu, dn, lm_w, gamma)
    x = synth.activations_bf16(34, M, d)
    lg = synth.synthetic_logits(35, M, E, 1.0)
    cap = MoECapture(mv)
    logits = host(mv.forward(dev(x), dev(lg), bank, gemm_hook=cap)).astype(np.float64)
    torch.cuda.synchronize()
    _check_moe_step(cap, mv, x, lg, topk, gu, dn, gamma, lm_w, logits)
    # end to end from the oracle's own chain: a statistic
    _, _, y = oracle.moe_block(x, lg, topk, *_oracle_bank(gu, dn))
    resid = oracle.bf16_round(synth.bf16_bits_to_f32(x).astype(np.float64) + y)
    h = oracle.bf16_round(oracle.rmsnorm(resid, gamma, 1e-6))
    ref = oracle.w4_gemm(h, *oracle.w4_quantize(lm_w))
    rms = np.sqrt((ref ** 2).mean(axis=1, keepdims=True))
    rel = np.abs(logits - ref) / np.maximum(np.abs(ref), rms)
    print(f"[moe step] end to end (statistic): max rel {rel.max():.3e} median {np.median(rel):.3e}", flush=True)


def _check_moe_step(cap, mv, x, lg, topk, gu, dn, gamma, lm_w, logits):
    """The expert layer (check_moe_layer), then the residual add, the final
    RMSNorm and the LM head, each from the GPU's own input.  With the combine
    fused into the final norm (MoEVerify.fuse_combine), the forward keeps only
    the experts' partials; y is formed from them by vw4_moe_combine, whose
    values the fused launch uses bit for bit."""
    if mv.fuse_combine:
        import torch
        B.moe_combine(mv.part_dn, mv.dn_S, mv.dn_ldp, mv.dn_sstride, mv.row_slot, mv.weights, mv.M, mv.topk, mv.d,
                      mv.y, mv.d)
        torch.cuda.synchronize()
    y = host(mv.y).astype(np.float64)
    check_moe_layer(cap, x, lg, topk, gu, dn, y)
    resid = host(mv.resid).copy()
    bf16_close(resid, synth.bf16_bits_to_f32(x).astype(np.float64) + y, what="moe residual")
    h = host(mv.h).copy()
    bf16_close(h, oracle.rmsnorm(resid, gamma, 1e-6), what="moe final norm")
    err = gemm_rel_err(logits, oracle.w4_gemm(h, *oracle.w4_quantize(lm_w)))
    assert err <= GEMM_RTOL, ("moe lm head", err)


def _full_moe(seed):
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    c = MOE_30B
    bank = ExpertBank.random(c["n_exp"], c["d"], c["F"], 0.02, gen)
    lm = W4Linear.random(c["V"], c["d"], 0.02, gen)
    gamma = (1 + 0.02 * torch.randn(c["d"], generator=gen, device="cuda")).to(torch.bfloat16).view(torch.int16)
    return bank, MoEVerify(c, 4, lm, gamma)


def test_moe_full_size_grouped_equals_per_expert_dense():
    """At 128 experts x (2048 -> 768 -> 2048): the grouped expert layer equals
    the same experts run one by one through the dense W4 GEMM calls and
    combined on the host in fp64 with the router's weights."""
    import torch
    log("moe full size: grouped == per-expert dense")
    bank, mv = _full_moe(21)
    c = MOE_30B
    M, d, F = 4, c["d"], c["F"]
    x = dev(synth.activations_bf16(22, M, d))
    lg = synth.synthetic_logits(23, M, c["n_exp"], 1.0)
    y = host(mv.moe(x, dev(lg), bank)).astype(np.float64)
    torch.cuda.synchronize()
    ex_o, wt_o = oracle.moe_route(lg, c["topk"])
    assert np.array_equal(host(mv.experts), ex_o)
    ref = np.zeros((M, d))
    gus, gul = bank.gu_estride
    dns, dnl = bank.dn_estride
    a = torch.empty((M, F), dtype=torch.int16, device="cuda")
    out = torch.empty((M, d), dtype=torch.float32, device="cuda")
    ws = B.workspace(max(B.gemm_workspace_bytes(M, d, F), 256))
    # gate/up-interleaved rows -> columns [gate f | up f] for the unfused SwiGLU
    inter = B.interleave_gate_up(np.arange(2 * F).reshape(2 * F, 1))[:, 0]
    natural = torch.as_tensor(np.argsort(inter), device="cuda")
    for e in sorted(set(ex_o.reshape(-1).tolist())):
        S, ldp = B.gemm_partials_layout(M, 2 * F, d)
        part = torch.empty(S * M * ldp, dtype=torch.float32, device="cuda")
        B.w4_skinny_gemm_partials(x, bank.gate_up.packed[e * gus:(e + 1) * gus],
                                  bank.gate_up.pscales[e * gul:(e + 1) * gul], part, M, 2 * F, d)
        pn = part.view(S, M, ldp)[:, :, :2 * F][:, :, natural].contiguous()
        B.swiglu(pn, S, 2 * F, M, F, a)
        B.w4_skinny_gemm(a, bank.down.packed[e * dns:(e + 1) * dns], bank.down.pscales[e * dnl:(e + 1) * dnl], out,
                         M, d, F, ws=ws)
        o = host(out).astype(np.float64)
        for m in range(M):
            for t in range(c["topk"]):
                if ex_o[m, t] == e:
                    ref[m] += wt_o[m, t] * o[m]
    err = gemm_rel_err(y, ref)
    print(f"[moe full] rel err {err:.3e}", flush=True)
    assert err <= GEMM_RTOL


def test_moe_fused_add_rmsnorm_equals_combine_then_norm():
    """The expert combine inside the final add + RMSNorm launch
    (vw4_moe_add_rmsnorm) against vw4_moe_combine then vw4_add_rmsnorm_out:
    the residual and normalised rows bitwise equal, on the full-size MoE step
    (top-8 of 128, d = 2048) and through MoEVerify.forward with and without
    the fusion (logits bitwise equal too)."""
    import torch
    log("moe fused combine + add + rmsnorm == the two calls")
    bank, mv = _full_moe(31)
    c = MOE_30B
    M, d = 4, c["d"]
    x = dev(synth.activations_bf16(32, M, d))
    lg = dev(synth.synthetic_logits(33, M, c["n_exp"], 1.0))
    outs = []
    for fused in (False, True):
        mv.fuse_combine = fused
        logits = host(mv.forward(x, lg, bank)).copy()
        torch.cuda.synchronize()
        outs.append((logits, host(mv.resid).copy(), host(mv.h).copy()))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)
    # the call itself on the same partials, against the two calls
    mv.moe(x, lg, bank)
    torch.cuda.synchronize()
    r1 = torch.empty_like(mv.resid)
    h1 = torch.empty_like(mv.h)
    B.add_rmsnorm_out(x[:M], mv.y, 1, d, mv.final_gamma, c["eps"], M, d, r1, h1)
    r2 = torch.full_like(mv.resid, -1)
    h2 = torch.full_like(mv.h, -1)
    B.moe_add_rmsnorm(x[:M], mv.part_dn, mv.dn_S, mv.dn_ldp, mv.dn_sstride, mv.row_slot, mv.weights, c["topk"],
                      mv.final_gamma, c["eps"], M, d, r2, h2)
    torch.cuda.synchronize()
    assert np.array_equal(host(r1), host(r2)) and np.array_equal(host(h1), host(h2))


@pytest.mark.parametrize("S,D", [(1, 2048), (2, 2048), (3, 2048), (4, 2048), (1, 4096), (2, 4096), (3, 1028),
                                 (2, 2500), (4, 4), (1, 3840)])
@pytest.mark.parametrize("M,topk", [(1, 1), (4, 8), (7, 5)])
def test_moe_fused_add_rmsnorm_every_instance(S, D, M, topk):
    """Every built (slices, chunks per wavefront) form of vw4_moe_add_rmsnorm,
    ragged widths (D not a multiple of 256) and padded partial layouts, against
    vw4_moe_combine then vw4_add_rmsnorm_out: bitwise equal."""
    import torch
    log(f"moe fused norm S={S} D={D} M={M} topk={topk}")
    n_slots, ldp = 11, D + 12
    sstride = S * M * ldp + 20
    g = synth.rng(1000 * S + D + 17 * M + topk)
    part = dev(synth.normal_f32(g, (n_slots * sstride,), 0.5))
    rs = np.stack([g.permutation(n_slots)[:topk] for _ in range(M)]).astype(np.int32)
    wt = g.random((M, topk)).astype(np.float32)
    wt /= wt.sum(axis=1, keepdims=True)
    row_slot, weights = dev(rs), dev(wt)
    x = dev(synth.activations_bf16(D + M, M, D))
    gamma = dev(synth.f32_to_bf16_bits(1 + synth.normal_f32(g, (D,), 0.1)))
    y = torch.full((M, D), float("nan"), dtype=torch.float32, device="cuda")
    B.moe_combine(part, S, ldp, sstride, row_slot, weights, M, topk, D, y, D)
    r1 = torch.full((M, D), -1, dtype=torch.int16, device="cuda")
    h1 = torch.full_like(r1, -1)
    B.add_rmsnorm_out(x, y, 1, D, gamma, 1e-6, M, D, r1, h1)
    r2 = torch.full_like(r1, -1)
    h2 = torch.full_like(r1, -1)
    B.moe_add_rmsnorm(x, part, S, ldp, sstride, row_slot, weights, topk, gamma, 1e-6, M, D, r2, h2)
    torch.cuda.synchronize()
    assert np.array_equal(host(r1), host(r2))
    assert np.array_equal(host(h1), host(h2))


def test_moe_fused_add_rmsnorm_rejects_unsupported():
    import torch
    M, d = 4, 2048
    part = torch.zeros(4 * 9 * M * d, dtype=torch.float32, device="cuda")
    rs = torch.zeros((M, 16), dtype=torch.int32, device="cuda")
    wt = torch.zeros((M, 16), dtype=torch.float32, device="cuda")
    g = torch.zeros(d, dtype=torch.int16, device="cuda")
    x = torch.zeros((M, d), dtype=torch.int16, device="cuda")
    r, h = torch.zeros_like(x), torch.zeros_like(x)
    with pytest.raises(B.VW4Error, match="built"):
        B.moe_add_rmsnorm(x, part, 2, d, 2 * M * d, rs, wt, 9, g, 1e-6, M, d, r, h)
    with pytest.raises(B.VW4Error, match="built"):
        B.moe_add_rmsnorm(x, part, 5, d, 5 * M * d, rs, wt, 8, g, 1e-6, M, d, r, h)
    with pytest.raises(B.VW4Error, match="overlap"):
        B.moe_add_rmsnorm(x, part, 2, d, 2 * M * d, rs, wt, 8, g, 1e-6, M, d, x, h)


def test_moe_step_graph_replay_matches_eager():
    """Full-size MoE verify step as a HIP graph: new router logits copied into
    the captured buffer before each replay; tokens and logits equal the eager
    step with the same inputs and Philox step."""
    import torch
    log("moe full size: graph replay == eager")
    bank, mv = _full_moe(24)
    c = MOE_30B
    M = 4
    x = dev(synth.activations_bf16(25, M, c["d"]))
    pool = [dev(synth.synthetic_logits(26 + k, M, c["n_exp"], 1.0)) for k in range(3)]
    q, drafts = synth.q_and_drafts(27, M - 1, c["V"], 3.0, B=1)
    qd, dd = dev(q), dev(drafts[0])
    seed, T, top_p = 0x5EED0006, 0.6, 0.95
    eager = []
    for k in range(3):
        tok, nacc, _ = mv.run(x, pool[k], bank, qd, dd, T, top_p, seed, k)
        torch.cuda.synchronize()
        eager.append((host(tok).copy(), host(nacc).copy(), host(mv.logits).copy(), int(host(mv.n_slots)[0])))
    lg_buf = pool[0].clone()
    step_dev = torch.zeros(1, dtype=torch.int64, device="cuda")
    g = mv.capture(x, lg_buf, bank, qd, dd, T, top_p, seed, step_dev)
    step_dev.zero_()
    torch.cuda.synchronize()
    for k in range(3):
        lg_buf.copy_(pool[k])
        g.replay()
        torch.cuda.synchronize()
        _ = torch.ones(1000, device="cuda").sum().item()
        assert np.array_equal(host(mv.logits), eager[k][2]), k
        assert np.array_equal(host(mv.tokens), eager[k][0]) and np.array_equal(host(mv.n_acc), eager[k][1]), k
        assert int(host(mv.n_slots)[0]) == eager[k][3]
    n = int(eager[0][1][0])
    assert 0 <= n <= M - 1


def test_moe_step_graph_replays_match_oracle():
    """The MoE-shaped verify step (16 experts, top-4, d 512, FFN 256, V 3000)
    captured as a HIP graph and replayed with fresh router logits copied into
    the captured buffer each time.  Every replay is checked op by op against
    the oracle on its own inputs (routing, expert activations and outputs,
    combine, residual, final norm, LM head), and its tokens and n_acc against
    oracle.spec_accept on its own logits with that Philox step (outside
    flagged near-ties)."""
    import torch
    E, topk, d, F, M, V = 16, 4, 512, 256, 4, 3000
    log("moe graph replays vs oracle")
    cfg = dict(n_exp=E, topk=topk, d=d, F=F, V=V, eps=1e-6)
    gu, dn = _host_bank(41, E, F, d)
    lm_w = synth.linear_weights(42, V, d)
    gamma = synth.f32_to_bf16_bits(1 + synth.normal_f32(synth.rng(43), (d,), 0.02))
    bank, mv = _moe_device(cfg, M, gu, dn, lm_w, gamma)
    x = synth.activations_bf16(44, M, d)
    xd = dev(x)
    pool = [synth.synthetic_logits(45 + k, M, E, 1.0) for k in range(3)]
    q, drafts = synth.q_and_drafts(49, M - 1, V, 3.0, B=1)
    qd, dd = dev(q), dev(drafts[0])
    seed, T, top_p = 0x5EED0008, 0.6, 0.95
    lg_buf = dev(pool[0])
    step_dev = torch.zeros(1, dtype=torch.int64, device="cuda")
    g = mv.capture(xd, lg_buf, bank, qd, dd, T, top_p, seed, step_dev)
    step_dev.zero_()
    torch.cuda.synchronize()
    ties = B.FLAG_TOPP_TIE | B.FLAG_ACCEPT_TIE | B.FLAG_CDF_TIE
    flagged = 0
    for k in range(3):
        lg_buf.copy_(dev(pool[k]))
        g.replay()
        torch.cuda.synchronize()
        _ = torch.ones(1000, device="cuda").sum().item()
        cap = MoECapture(mv)
        cap("post", "gate_up")
        cap("post", "down")
        logits = host(mv.logits).astype(np.float64)
        _check_moe_step(cap, mv, x, pool[k], topk, gu, dn, gamma, lm_w, logits)
        otok, onacc, oflags, _ = oracle.spec_accept(host(mv.logits), q, drafts[0], T, top_p, seed, k)
        if (int(host(mv.flags)[0]) | oflags) & ties:
            flagged += 1
            continue
        assert int(host(mv.n_acc)[0]) == onacc and list(host(mv.tokens)[0]) == list(otok), (k, otok, onacc)
    assert flagged <= 1
    assert int(step_dev.item()) == 3
