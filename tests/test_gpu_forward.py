"""The whole verify forward (a2-a9, a11) on the GPU.

* Op by op against the oracle, teacher forced (tests/layer_parity.py): every
  op of a small decoder (2 layers, d=256, GQA 4/2 heads of 128, FFN 512,
  V=1000) and of one full-size 27B-shaped layer is recomputed by the oracle
  from the GPU's own input to that op and held to its own bar -- fp32 GEMM
  sums and logits within 1e-3, bf16 outputs within their rounding and >= 97 %
  bit-identical.  The end-to-end difference of the logits from the oracle's
  own composition is reported as a statistic (one-ulp bf16 flips propagate
  through random layers).
* Verify row i of an M-row pass equals the autoregressive M=1 step at position
  L + i (teacher forced: rows 0..i-1 already in the KV cache), bit for bit,
  at the full layer width.  This is the property behind "the verify pass
  changes nothing but speed".
* Bitwise determinism of the verify step.
"""
import numpy as np
import pytest

import oracle
from verify_step_w4_amd import binding as B
from verify_step_w4_amd import synth
from verify_step_w4_amd.model import DENSE_27B, LINEAR_FORMATS, Decoder, VerifyStep, W4Linear, W16Linear

from helpers import GEMM_RTOL, dev, gemm_rel_err, host, log, rows_from_vb, vb_from_rows
from layer_parity import DecoderCapture, bf16_close, check_decoder_ops, end_to_end

pytestmark = pytest.mark.gpu

TINY = dict(d=256, nq=4, nkv=2, hd=128, F=512, layers=2, V=1000, eps=1e-6, theta=10000.0)


def _host_model(cfg, seed):
    g = synth.rng(seed)
    d, nq, nkv, hd, F, V = (cfg[k] for k in ("d", "nq", "nkv", "hd", "F", "V"))
    layers = []
    for _ in range(cfg["layers"]):
        layers.append(dict(qkv=synth.normal_f32(g, ((nq + 2 * nkv) * hd, d), 0.02),
                           o=synth.normal_f32(g, (d, nq * hd), 0.02),
                           gate_up=synth.normal_f32(g, (2 * F, d), 0.02),
                           down=synth.normal_f32(g, (d, F), 0.02),
                           g1=synth.f32_to_bf16_bits(1 + synth.normal_f32(g, (d,), 0.02)),
                           g2=synth.f32_to_bf16_bits(1 + synth.normal_f32(g, (d,), 0.02))))
    return dict(layers=layers, final_gamma=synth.f32_to_bf16_bits(1 + synth.normal_f32(g, (d,), 0.02)),
                lm_head=synth.normal_f32(g, (V, d), 0.02))


def _f16_bits(w):
    return (w.astype(np.float16).view(np.uint16),)


def _bf16_bits(w):
    return (oracle.bf16_round(w.astype(np.float64)),)


# the oracle's (quantiser, GEMM) of each format other than W4; a quantiser
# returns the arguments the GEMM takes after x
ORACLE_FORMATS = {"w8": (oracle.w8_quantize, oracle.w8_gemm), "w6": (oracle.w6_quantize, oracle.w6_gemm),
                  "w5": (oracle.w5_quantize, oracle.w5_gemm), "w3": (oracle.w3_quantize, oracle.w3_gemm),
                  "w2": (oracle.w2_quantize, oracle.w2_gemm), "f16": (_f16_bits, oracle.f16_gemm),
                  "bf16": (_bf16_bits, oracle.b16_gemm)}


def _linear(v, fmt):
    """A device matrix in format fmt from host fp32 weights (rows as given)."""
    if fmt in ("f16", "bf16"):
        bits = ORACLE_FORMATS[fmt][0](v)[0]
        return W16Linear.from_bits(dev(bits.view(np.int16)), fmt)
    return LINEAR_FORMATS[fmt].from_fp32(v)


def _device_weights(hm, fmt="w4"):
    layers = []
    for l in hm["layers"]:
        d = {}
        for k, v in l.items():
            if k in ("g1", "g2"):
                d[k] = dev(v)
            elif k == "gate_up":   # the fused SwiGLU GEMM takes gate/up-interleaved rows
                vi = B.interleave_gate_up(v)
                d[k] = W4Linear.from_fp32(dev(vi)) if fmt == "w4" else _linear(vi, fmt)
            elif fmt != "w4":
                d[k] = _linear(v, fmt)
            else:
                d[k] = W4Linear.from_fp32(dev(v))
        layers.append(d)
    lm = _linear(hm["lm_head"], fmt) if fmt != "w4" else W4Linear.from_fp32(dev(hm["lm_head"]))
    return dict(layers=layers, final_gamma=dev(hm["final_gamma"]), lm_head=lm)


def _oracle_forward(cfg, hm, Kc, Vc, x, L, quant=None, gemm=None):
    """Oracle composition of the layer ops; Kc/Vc: per-layer uint16 arrays (modified)."""
    d, nq, nkv, hd, F, eps = (cfg[k] for k in ("d", "nq", "nkv", "hd", "F", "eps"))
    quant = quant or oracle.w4_quantize
    gemm = gemm or oracle.w4_gemm
    M = x.shape[0]
    q4 = {}
    for li, l in enumerate(hm["layers"]):
        q4[li] = {k: quant(l[k]) for k in ("qkv", "o", "gate_up", "down")}
    lm = quant(hm["lm_head"])
    resid = x.copy()
    for li, l in enumerate(hm["layers"]):
        Q = q4[li]
        h = oracle.bf16_round(oracle.rmsnorm(resid, l["g1"], eps))
        qkv = gemm(h, *Q["qkv"])
        q = np.zeros((M, nq, hd))
        for m in range(M):
            for hh in range(nq):
                q[m, hh] = oracle.bf16_value(oracle.bf16_round(oracle.rope(qkv[m, hh * hd:(hh + 1) * hd], L + m)))
            for hh in range(nkv):
                kk = oracle.rope(qkv[m, (nq + hh) * hd:(nq + hh + 1) * hd], L + m)
                Kc[li][hh, L + m] = oracle.bf16_round(kk)
                Vc[li][hh, L + m] = oracle.bf16_round(qkv[m, (nq + nkv + hh) * hd:(nq + nkv + hh + 1) * hd])
        att = oracle.bf16_round(oracle.decode_attn(q, Kc[li], Vc[li], L).reshape(M, nq * hd))
        o = gemm(att, *Q["o"])
        resid = oracle.bf16_round(oracle.bf16_value(resid) + o)
        h = oracle.bf16_round(oracle.rmsnorm(resid, l["g2"], eps))
        gu = gemm(h, *Q["gate_up"])
        a = oracle.bf16_round(oracle.swiglu(gu[:, :F], gu[:, F:]))
        dn = gemm(a, *Q["down"])
        resid = oracle.bf16_round(oracle.bf16_value(resid) + dn)
    h = oracle.bf16_round(oracle.rmsnorm(resid, hm["final_gamma"], eps))
    return gemm(h, *lm)


def test_forward_matches_oracle_small_decoder():
    cfg = TINY
    M, L = 4, 37
    Lmax = 64                                           # >= L + M, a multiple of 32 (blocked value cache)
    log("forward vs oracle, small decoder")
    hm = _host_model(cfg, 4242)
    dec = Decoder(cfg, M, Lmax, weights=_device_weights(hm), kv_fill=False)
    g = synth.rng(77)
    Kh = [synth.f32_to_bf16_bits(synth.normal_f32(g, (cfg["nkv"], Lmax, cfg["hd"]), 1.0)) for _ in range(cfg["layers"])]
    Vh = [synth.f32_to_bf16_bits(synth.normal_f32(g, (cfg["nkv"], Lmax, cfg["hd"]), 1.0)) for _ in range(cfg["layers"])]
    for li in range(cfg["layers"]):
        dec.Kc[li].copy_(dev(Kh[li]))
        dec.Vc[li].copy_(dev(vb_from_rows(Vh[li])).view(dec.Vc[li].shape))   # blocked values
    x = synth.activations_bf16(78, M, cfg["d"])
    import torch
    cap = DecoderCapture(dec, M)
    logits = host(dec.forward(dev(x), L, M, gemm_hook=cap)).copy()
    torch.cuda.synchronize()
    worst, ident = check_decoder_ops(cap, hm, cfg, x, L)
    Ko, Vo = [k.copy() for k in Kh], [v.copy() for v in Vh]
    ref = _oracle_forward(cfg, hm, Ko, Vo, x, L)
    mx, med = end_to_end(logits, ref)
    print(f"[forward] per op: worst fp32 rel {worst:.2e}, bf16 identical >= {ident:.4f}; "
          f"end to end (statistic): max rel {mx:.3e}, median {med:.3e}", flush=True)
    # the KV rows the verify pass appended: layer 0 sees identical inputs on
    # both sides (bit-exact up to rare one-ulp rounding flips); later layers
    # inherit the flips of earlier ones, so only closeness is required there
    for li in range(cfg["layers"]):
        for gpu_c, ora_c in ((host(dec.Kc[li]), Ko[li]), (rows_from_vb(host(dec.Vc[li])), Vo[li])):
            kg = gpu_c[:, L:L + M]
            ko = ora_c[:, L:L + M]
            if li == 0:
                assert np.mean(kg == ko) > 0.95
            a = synth.bf16_bits_to_f32(kg).astype(np.float64)
            b = synth.bf16_bits_to_f32(ko).astype(np.float64)
            assert np.abs(a - b).max() <= 3e-2 * np.sqrt((b ** 2).mean())


def _dense_cfg(layers, V):
    c = dict(DENSE_27B)
    c["layers"] = layers
    c["V"] = V
    return c


@pytest.mark.parametrize("fmt", ["w8", "w6", "w5", "w3", "w2", "f16", "bf16"])
def test_forward_matches_oracle_small_decoder_other_format(fmt):
    """The same small decoder with every linear and the LM head in another
    weight format (gate|up with the SwiGLU in its epilogue) against the
    oracle's composition in that format: each op on the GPU's own inputs
    at its bar, then the verify rows equal to the one-row steps bit for bit."""
    import torch
    cfg = TINY
    M, L, Lmax = 4, 37, 64
    log(f"forward vs oracle, small decoder, {fmt}")
    hm = _host_model(cfg, 4243)
    dec = Decoder(cfg, M, Lmax, weights=_device_weights(hm, fmt), kv_fill=False)
    g = synth.rng(79)
    Kh = [synth.f32_to_bf16_bits(synth.normal_f32(g, (cfg["nkv"], Lmax, cfg["hd"]), 1.0)) for _ in range(cfg["layers"])]
    Vh = [synth.f32_to_bf16_bits(synth.normal_f32(g, (cfg["nkv"], Lmax, cfg["hd"]), 1.0)) for _ in range(cfg["layers"])]
    for li in range(cfg["layers"]):
        dec.Kc[li].copy_(dev(Kh[li]))
        dec.Vc[li].copy_(dev(vb_from_rows(Vh[li])).view(dec.Vc[li].shape))
    x = synth.activations_bf16(80, M, cfg["d"])
    cap = DecoderCapture(dec, M)
    logits = host(dec.forward(dev(x), L, M, gemm_hook=cap)).copy()
    torch.cuda.synchronize()
    quant, gemm = ORACLE_FORMATS[fmt]
    worst, ident = check_decoder_ops(cap, hm, cfg, x, L, quant=quant, gemm=gemm)
    ref = _oracle_forward(cfg, hm, [k.copy() for k in Kh], [v.copy() for v in Vh], x, L, quant=quant, gemm=gemm)
    mx, med = end_to_end(logits, ref)
    print(f"[forward {fmt}] per op: worst fp32 rel {worst:.2e}, bf16 identical >= {ident:.4f}; "
          f"end to end (statistic): max rel {mx:.3e}, median {med:.3e}", flush=True)
    # verify rows equal the one-row steps bit for bit in this format too
    for li in range(cfg["layers"]):
        dec.Kc[li].copy_(dev(Kh[li]))
        dec.Vc[li].copy_(dev(vb_from_rows(Vh[li])).view(dec.Vc[li].shape))
    xd = dev(x)
    verify = host(dec.forward(xd, L, M)).copy()
    for li in range(cfg["layers"]):
        dec.Kc[li].copy_(dev(Kh[li]))
        dec.Vc[li].copy_(dev(vb_from_rows(Vh[li])).view(dec.Vc[li].shape))
    for i in range(M):
        assert np.array_equal(host(dec.forward(xd[i:i + 1], L + i, 1))[0], verify[i]), i


def test_full_size_layer_matches_oracle():
    """One decoder layer at the 27B shapes (d 5120, GQA 40/8 x 128, FFN 17408)
    over a context of 8192 positions at M = 4 -- the launch configuration of
    the benchmark -- against the oracle's composition of the same layer (LM
    head cut to 2048 rows; it is tested at full width elsewhere)."""
    import torch
    cfg = _dense_cfg(1, 2048)
    M, L = 4, 8192
    Lmax = L + M + 28                                   # a multiple of 32
    log("full-size layer vs oracle (L=8192, M=4)")
    hm = _host_model(cfg, 4343)
    dec = Decoder(cfg, M, Lmax, weights=_device_weights(hm), kv_fill=False)
    g = synth.rng(79)
    Kh = [synth.f32_to_bf16_bits(synth.normal_f32(g, (cfg["nkv"], Lmax, cfg["hd"]), 1.0))]
    Vh = [synth.f32_to_bf16_bits(synth.normal_f32(g, (cfg["nkv"], Lmax, cfg["hd"]), 1.0))]
    dec.Kc[0].copy_(dev(Kh[0]))
    dec.Vc[0].copy_(dev(vb_from_rows(Vh[0])).view(dec.Vc[0].shape))
    x = synth.activations_bf16(80, M, cfg["d"])
    cap = DecoderCapture(dec, M)
    logits = host(dec.forward(dev(x), L, M, gemm_hook=cap)).copy()
    torch.cuda.synchronize()
    worst, ident = check_decoder_ops(cap, hm, cfg, x, L)
    Ko, Vo = [k.copy() for k in Kh], [v.copy() for v in Vh]
    ref = _oracle_forward(cfg, hm, Ko, Vo, x, L)
    mx, med = end_to_end(logits, ref)
    print(f"[full-size layer] per op: worst fp32 rel {worst:.2e}, bf16 identical >= {ident:.4f}; "
          f"end to end (statistic): max rel {mx:.3e}, median {med:.3e}", flush=True)
    # the K and V rows the pass appended (identical inputs on both sides:
    # bit-exact up to rare one-ulp rounding flips)
    for gpu_c, ora_c in ((host(dec.Kc[0]), Ko[0]), (rows_from_vb(host(dec.Vc[0])), Vo[0])):
        assert np.mean(gpu_c[:, L:L + M] == ora_c[:, L:L + M]) > 0.95
        assert np.array_equal(gpu_c[:, :L], ora_c[:, :L])          # the context is untouched


def test_verify_rows_equal_autoregressive_steps():
    import torch
    cfg = _dense_cfg(2, 4096)
    M, L = 4, 1000
    Lmax = L + M + 4
    log("verify rows == AR steps (full width, 2 layers)")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    dec = Decoder(cfg, M, Lmax, gen=gen)
    K0 = [k.clone() for k in dec.Kc]
    V0 = [v.clone() for v in dec.Vc]
    x = dev(synth.activations_bf16(9, M, cfg["d"]))
    verify = host(dec.forward(x, L, M)).copy()
    # sequential single-row steps on a fresh copy of the cache
    for li in range(cfg["layers"]):
        dec.Kc[li].copy_(K0[li])
        dec.Vc[li].copy_(V0[li])
    for i in range(M):
        ar = host(dec.forward(x[i:i + 1], L + i, 1))
        assert np.array_equal(ar[0], verify[i]), f"row {i} differs"


def test_verify_step_deterministic_and_accepts():
    import torch
    cfg = _dense_cfg(2, 151936)
    M, L = 4, 512
    Lmax = L + M + 4
    log("verify step determinism (full width, 2 layers, V=151936)")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(6)
    dec = Decoder(cfg, M, Lmax, gen=gen)
    vs = VerifyStep(dec, M)
    x = dev(synth.activations_bf16(10, M, cfg["d"]))
    q, drafts = synth.q_and_drafts(11, M - 1, cfg["V"], 3.0, B=1)
    qd, dd = dev(q), dev(drafts[0])
    K0 = [k.clone() for k in dec.Kc]
    outs = []
    for rep in range(2):
        for li in range(cfg["layers"]):
            dec.Kc[li].copy_(K0[li])
        tok, nacc, fl = vs.run(x, L, qd, dd, 0.6, 0.95, 0x5EED0004, 0)
        torch.cuda.synchronize()
        outs.append((host(tok).copy(), host(nacc).copy(), host(dec.logits[:M]).copy(), B.rowstats_to_numpy(vs.stats)))
    assert np.array_equal(outs[0][2], outs[1][2])
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    assert outs[0][3].tobytes() == outs[1][3].tobytes()
    n = int(outs[0][1][0])
    assert 0 <= n <= M - 1 and 0 <= int(outs[0][0][0, n]) < cfg["V"]


def test_graph_replay_matches_eager_steps():
    """The verify step captured as a HIP graph: every replay (with eager work in
    between) equals the eager step with the same Philox step number."""
    import torch
    cfg = _dense_cfg(2, 8192)
    M, L = 4, 300
    log("graph replay == eager (full width, 2 layers)")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(8)
    dec = Decoder(cfg, M, L + M + 4, gen=gen)
    vs = VerifyStep(dec, M)
    x = dev(synth.activations_bf16(12, M, cfg["d"]))
    q, drafts = synth.q_and_drafts(13, M - 1, cfg["V"], 1.0, B=1)
    qd, dd = dev(q), dev(drafts[0])
    seed, T, top_p = 0x5EED0005, 0.6, 0.95
    eager = []
    for k in range(3):
        tok, nacc, fl = vs.run(x, L, qd, dd, T, top_p, seed, k)
        torch.cuda.synchronize()
        eager.append((host(tok).copy(), host(nacc).copy(), host(dec.logits[:M]).copy()))
    step_dev = torch.zeros(1, dtype=torch.int64, device="cuda")
    g = vs.capture(x, L, qd, dd, T, top_p, seed, step_dev)   # the warm-up run inside uses step 0
    step_dev.zero_()
    torch.cuda.synchronize()
    for k in range(3):
        g.replay()
        torch.cuda.synchronize()
        _ = torch.ones(1000, device="cuda").sum().item()          # eager work between replays
        assert np.array_equal(host(dec.logits[:M]), eager[k][2]), k
        assert np.array_equal(host(vs.tokens), eager[k][0]) and np.array_equal(host(vs.n_acc), eager[k][1]), k
    assert int(step_dev.item()) == 3


@pytest.mark.parametrize("fmt", ["w4", "w8", "w2", "bf16"])
def test_graph_replays_match_oracle_small_decoder(fmt):
    """The verify step of the small decoder (weights in format fmt) captured
    as a HIP graph (the form
    the benchmark times) and replayed three times, with eager work and a new
    Philox step each time.  Every replay: its logits equal those of an eager
    forward whose every op passed the teacher-forced oracle checks; its LM
    head matches the oracle on the replay's own final hidden rows (1e-3), its
    final RMSNorm on its own residual rows, its last layer's attention on its
    own q and KV cache (bf16 bar); its tokens and n_acc equal
    oracle.spec_accept on its own logits with that Philox step (outside
    flagged near-ties)."""
    import torch
    cfg = TINY
    M, L, Lmax = 4, 37, 64
    d, nq, hd, V, eps = cfg["d"], cfg["nq"], cfg["hd"], cfg["V"], cfg["eps"]
    log(f"graph replays vs oracle, small decoder, {fmt}")
    hm = _host_model(cfg, 4244)
    dec = Decoder(cfg, M, Lmax, weights=_device_weights(hm, fmt), kv_fill=False)
    quant, gemm = (oracle.w4_quantize, oracle.w4_gemm) if fmt == "w4" else ORACLE_FORMATS[fmt]
    g = synth.rng(83)
    for li in range(cfg["layers"]):
        dec.Kc[li].copy_(dev(synth.f32_to_bf16_bits(synth.normal_f32(g, (cfg["nkv"], Lmax, hd), 1.0))))
        vr = synth.f32_to_bf16_bits(synth.normal_f32(g, (cfg["nkv"], Lmax, hd), 1.0))
        dec.Vc[li].copy_(dev(vb_from_rows(vr)).view(dec.Vc[li].shape))
    vs = VerifyStep(dec, M)
    x = synth.activations_bf16(84, M, d)
    xd = dev(x)
    q, drafts = synth.q_and_drafts(85, M - 1, V, 3.0, B=1)
    qd, dd = dev(q), dev(drafts[0])
    seed, T, top_p = 0x5EED0007, 0.6, 0.95
    # eager step, every op checked against the oracle on its own inputs
    cap = DecoderCapture(dec, M)
    vs.run(xd, L, qd, dd, T, top_p, seed, 0, gemm_hook=cap)
    torch.cuda.synchronize()
    check_decoder_ops(cap, hm, cfg, x, L, quant=quant, gemm=gemm)
    eager = host(dec.logits[:M]).copy()
    step_dev = torch.zeros(1, dtype=torch.int64, device="cuda")
    gr = vs.capture(xd, L, qd, dd, T, top_p, seed, step_dev)
    step_dev.zero_()
    torch.cuda.synchronize()
    lm_q = quant(hm["lm_head"])
    ties = B.FLAG_TOPP_TIE | B.FLAG_ACCEPT_TIE | B.FLAG_CDF_TIE
    last = cfg["layers"] - 1
    flagged = 0
    for k in range(3):
        gr.replay()
        torch.cuda.synchronize()
        _ = torch.ones(1000, device="cuda").sum().item()          # eager work between replays
        z = host(dec.logits[:M]).copy()
        assert np.array_equal(z, eager), k
        hfin = host(dec.h[:M]).copy()
        assert gemm_rel_err(z, gemm(hfin, *lm_q)) <= GEMM_RTOL, k
        bf16_close(hfin, oracle.rmsnorm(host(dec.last_resid[:M]), hm["final_gamma"], eps), what=f"final norm {k}")
        att_ref = oracle.decode_attn(oracle.bf16_value(host(dec.q[:M])), host(dec.Kc[last]),
                                     rows_from_vb(host(dec.Vc[last])), L).reshape(M, nq * hd)
        bf16_close(host(dec.attn[:M]), att_ref, what=f"last-layer attention {k}")
        otok, onacc, oflags, _ = oracle.spec_accept(z, q, drafts[0], T, top_p, seed, k)
        gflags = int(host(vs.flags)[0])
        if (gflags | oflags) & ties:
            flagged += 1
            continue
        assert int(host(vs.n_acc)[0]) == onacc and list(host(vs.tokens)[0]) == list(otok), (k, otok, onacc)
    assert flagged <= 1
    assert int(step_dev.item()) == 3
