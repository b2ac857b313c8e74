"""The draft side of the cycle and the closed loop on the GPU.

* Embedding rows and the MTP projection input against the oracle (bit-exact
  rows; the normalised halves up to rare one-ulp bf16 flips).
* draft_sample against the oracle on the same logits: the token bit-exact
  outside the CDF-boundary flag, q within binary32 rounding; the device-step
  form equals the host-step form.
* One MTP-head draft step (projection, one decoder layer, final norm, LM head)
  against the oracle's composition on a small model.
* The closed loop at T = 0 emits exactly the greedy autoregressive sequence,
  with the head's drafts (mostly rejected on random weights) and with drafts
  that are the greedy continuation (all accepted); at T = 0.6 it is
  deterministic and every cycle emits 1 .. D + 1 tokens.
"""
import numpy as np
import pytest

import oracle
from verify_step_w4_amd import binding as B
from verify_step_w4_amd import synth
from verify_step_w4_amd.model import DENSE_27B, Decoder, MTPHead, SpecLoop, W4Linear

from helpers import dev, host, log, rows_from_vb, vb_from_rows
from layer_parity import DecoderCapture, bf16_close, check_decoder_ops, end_to_end
from test_gpu_forward import TINY, _device_weights, _host_model, _oracle_forward

pytestmark = pytest.mark.gpu
SEED = 0x5EED0007


def _stats_dev(logits_dev, T, top_p):
    import torch
    rows, V = logits_dev.shape
    st = torch.zeros(rows * B.ROWSTAT_BYTES, dtype=torch.uint8, device="cuda")
    ws = B.workspace(B.verify_workspace_bytes(rows, V), "cuda")
    B.verify_logits(None, None, None, rows, V, 64, T, top_p, logits_dev, st, ws)
    return st


def test_embed_rows_match_oracle():
    import torch
    V, d = 1000, 256
    E = synth.f32_to_bf16_bits(synth.normal_f32(synth.rng(5), (V, d), 1.0))
    tok = np.array([3, 0, V - 1, -1, V, 3, 517], dtype=np.int32)
    out = torch.zeros((len(tok), d), dtype=torch.int16, device="cuda")
    log("embed rows")
    B.embed_rows(dev(E), dev(tok), len(tok), out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out), oracle.embed_rows(E, tok))


@pytest.mark.parametrize("d", [8, 264, 256, 5120, 8192])
@pytest.mark.parametrize("row,token", [(2, 7), (-1, 0), (9, -3), (3, 999)])
def test_mtp_input_matches_oracle(d, row, token):
    import torch
    V, rows = 1000, 4
    g = synth.rng(d + 17)
    E = synth.f32_to_bf16_bits(synth.normal_f32(g, (V, d), 1.0))
    h = synth.f32_to_bf16_bits(synth.normal_f32(g, (rows, d), 3.0))
    gh = synth.f32_to_bf16_bits(1 + synth.normal_f32(g, (d,), 0.02))
    ge = synth.f32_to_bf16_bits(1 + synth.normal_f32(g, (d,), 0.02))
    out = torch.zeros((1, 2 * d), dtype=torch.int16, device="cuda")
    log(f"mtp input d={d} row={row} token={token}")
    B.mtp_input(dev(h), rows, dev(np.array([row], np.int32)), dev(E), dev(np.array([token], np.int32)), dev(gh),
                dev(ge), 1e-6, out)
    torch.cuda.synchronize()
    r = min(max(row, 0), rows - 1)
    e = oracle.embed_rows(E, [token])[0]
    ref = oracle.bf16_round(oracle.mtp_input(h[r], e, gh, ge, 1e-6))
    got = host(out)[0]
    a = synth.bf16_bits_to_f32(got).astype(np.float64)
    b = synth.bf16_bits_to_f32(ref).astype(np.float64)
    assert np.mean(got == ref) > 0.99
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.abs(b) + 1e-30)       # at most one bf16 ulp apart
    if not 0 <= token < V:
        assert not got[d:].any()                                      # zero embedding row


@pytest.mark.parametrize("V", [1000, 151936])
@pytest.mark.parametrize("T,top_p", [(0.0, 0.95), (0.6, 0.95), (1.0, 1.0), (0.6, 0.5)])
def test_draft_sample_matches_oracle(V, T, top_p):
    import torch
    z = synth.normal_f32(synth.rng(V + int(10 * T)), (V,), 3.0)
    zd = dev(z.reshape(1, V))
    st = _stats_dev(zd, T, top_p)
    ws = B.workspace(B.draft_workspace_bytes(V), "cuda")
    q = torch.zeros(V, dtype=torch.float32, device="cuda")
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")
    step_dev = torch.zeros(1, dtype=torch.int64, device="cuda")
    log(f"draft_sample V={V} T={T} top_p={top_p}")
    mism = flagged = 0
    for step, depth in [(0, 0), (1, 0), (5, 2), (2 ** 33 + 1, 6), (77, 1), (78, 1), (79, 3), (1000, 0)]:
        B.draft_sample(zd, st, V, T, SEED, step, depth, q, tok, fl, ws)
        torch.cuda.synchronize()
        t_ref, q_ref, _, f_ref = oracle.draft_sample(z, T, top_p, SEED, step, depth)
        if (int(host(fl)[0]) | f_ref) & 8:
            flagged += 1
        elif int(host(tok)[0]) != t_ref:
            mism += 1
        np.testing.assert_allclose(host(q).astype(np.float64), q_ref.astype(np.float64), rtol=1e-6, atol=0)
        # the device-step form draws the same token
        step_dev.fill_(step)
        tok2 = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        B.draft_sample(zd, st, V, T, SEED, 0, depth, None, tok2, fl, ws, step_dev=step_dev)
        torch.cuda.synchronize()
        assert int(host(tok2)[0]) == int(host(tok)[0])
    assert mism == 0 and flagged <= 1


def test_draft_sample_single_token_vocab_and_max_depth():
    import torch
    V = 1
    zd = dev(np.array([[0.25]], dtype=np.float32))
    st = _stats_dev(zd, 0.6, 0.95)
    ws = B.workspace(B.draft_workspace_bytes(V), "cuda")
    q = torch.zeros(V, dtype=torch.float32, device="cuda")
    tok = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")
    log("draft_sample V=1, depth 1023")
    B.draft_sample(zd, st, V, 0.6, SEED, 3, 1023, q, tok, fl, ws)
    torch.cuda.synchronize()
    assert int(host(tok)[0]) == 0 and host(q).tolist() == [1.0]
    assert oracle.draft_sample(np.array([0.25], np.float32), 0.6, 0.95, SEED, 3, 1023)[0] == 0


def _head_host(cfg, seed):
    g = synth.rng(seed)
    d = cfg["d"]
    lay = _host_model(dict(cfg, layers=1), seed + 1)["layers"][0]
    return dict(proj=synth.normal_f32(g, (d, 2 * d), 0.02), layer=lay,
                gamma_h=synth.f32_to_bf16_bits(1 + synth.normal_f32(g, (d,), 0.02)),
                gamma_e=synth.f32_to_bf16_bits(1 + synth.normal_f32(g, (d,), 0.02)),
                final_gamma=synth.f32_to_bf16_bits(1 + synth.normal_f32(g, (d,), 0.02)))


def test_mtp_draft_step_matches_oracle():
    import torch
    cfg = TINY
    d, V, Lmax, pos = cfg["d"], cfg["V"], 64, 29
    log("MTP head draft step vs oracle, small model")
    hm = _host_model(cfg, 4242)
    target = Decoder(cfg, 4, Lmax, weights=_device_weights(hm), kv_fill=False)
    E = synth.f32_to_bf16_bits(synth.normal_f32(synth.rng(91), (V, d), 1.0))
    hh = _head_host(cfg, 93)
    dl = _device_weights(dict(layers=[hh["layer"]], final_gamma=hh["final_gamma"], lm_head=hm["lm_head"]))
    head = MTPHead(target, dev(E), kv_fill=False,
                   weights=dict(gamma_h=dev(hh["gamma_h"]), gamma_e=dev(hh["gamma_e"]),
                                final_gamma=dl["final_gamma"], layer=dl["layers"][0],
                                proj=W4Linear.from_fp32(dev(hh["proj"]))))
    g = synth.rng(95)
    Kh = synth.f32_to_bf16_bits(synth.normal_f32(g, (cfg["nkv"], Lmax, cfg["hd"]), 1.0))
    Vh = synth.f32_to_bf16_bits(synth.normal_f32(g, (cfg["nkv"], Lmax, cfg["hd"]), 1.0))
    head.block.Kc[0].copy_(dev(Kh))
    head.block.Vc[0].copy_(dev(vb_from_rows(Vh)).view(head.block.Vc[0].shape))
    h = synth.activations_bf16(96, 3, d)
    token = 411
    q = torch.zeros(V, dtype=torch.float32, device="cuda")
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    T, top_p = 0.6, 0.95
    cap = DecoderCapture(head.block, 1)
    logits = host(head.draft(dev(h), 3, dev(np.array([1], np.int32)), dev(np.array([token], np.int32)), pos, T,
                             top_p, SEED, 12, 2, q, tok, gemm_hook=cap)).copy()
    torch.cuda.synchronize()
    # teacher forced, op by op: the projection input, the projection (bf16
    # output) from the GPU's input, then every op of the head's decoder layer
    # and the LM head from the GPU's own inputs (tests/layer_parity.py)
    inp_gpu = host(head.inp).reshape(1, -1)
    bf16_close(inp_gpu[0], oracle.mtp_input(h[1], E[token], hh["gamma_h"], hh["gamma_e"], cfg["eps"]),
               min_exact=0.99, what="projection input")
    x_gpu = host(head.x).reshape(1, -1).copy()
    bf16_close(x_gpu, oracle.w4_gemm(inp_gpu, *oracle.w4_quantize(hh["proj"])), what="projection")
    bm = dict(layers=[hh["layer"]], final_gamma=hh["final_gamma"], lm_head=hm["lm_head"])
    worst, ident = check_decoder_ops(cap, bm, dict(cfg, layers=1), x_gpu, pos)
    # end to end from the oracle's own chain: a statistic
    inp = oracle.bf16_round(oracle.mtp_input(h[1], E[token], hh["gamma_h"], hh["gamma_e"], cfg["eps"]))
    x = oracle.bf16_round(oracle.w4_gemm(inp.reshape(1, -1), *oracle.w4_quantize(hh["proj"])))
    ref = _oracle_forward(dict(cfg, layers=1), bm, [Kh.copy()], [Vh.copy()], x, pos)
    mx, med = end_to_end(logits, ref)
    print(f"[mtp draft] per op: worst fp32 rel {worst:.2e}, bf16 identical >= {ident:.4f}; "
          f"end to end (statistic): max rel {mx:.3e}, median {med:.3e}", flush=True)
    # the draw, from the GPU's own logits, is the oracle's
    t_ref, q_ref, _, f_ref = oracle.draft_sample(logits[0], T, top_p, SEED, 12, 2)
    assert (f_ref & 8) or int(host(tok)[0]) == t_ref
    np.testing.assert_allclose(host(q).astype(np.float64), q_ref.astype(np.float64), rtol=1e-6, atol=0)


def _loop_setup(seed, D, L0, fmt="w4"):
    import torch
    cfg = dict(DENSE_27B, layers=2, V=4096)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    target = Decoder(cfg, D + 1, L0 + 64, gen=gen, fmt=fmt)
    E = torch.randn((cfg["V"], cfg["d"]), generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
    # a target in another format gets a draft-only W4 LM head
    lm = W4Linear.random(cfg["V"], cfg["d"], 0.02, gen) if fmt != "w4" else None
    head = MTPHead(target, E, gen=gen, lm_head=lm)
    kv = ([k.clone() for k in target.Kc], [v.clone() for v in target.Vc],
          [k.clone() for k in head.block.Kc], [v.clone() for v in head.block.Vc])
    return target, head, kv


def _reset(target, head, kv):
    for dst, src in zip((target.Kc, target.Vc, head.block.Kc, head.block.Vc), kv):
        for a, b in zip(dst, src):
            a.copy_(b)


def _ar_sequence(target, head, kv, L0, t0, n, T, top_p):
    _reset(target, head, kv)
    loop = SpecLoop(target, head, 1)
    seq = [loop.start(L0, t0, T, top_p, SEED, 0)]
    while len(seq) < n:
        loop.tokens_in[:1].fill_(seq[-1])
        B.embed_rows(head.embed, loop.tokens_in, 1, loop.x)
        tok, _, _ = loop.ar_vs.run(loop.x, loop.L, None, None, T, top_p, SEED, len(seq))
        seq.append(int(tok.view(-1)[0].item()))
        loop.L += 1
    return seq


@pytest.mark.parametrize("D,fmt", [(1, "w4"), (3, "w4"), (5, "w4"), (3, "w8"), (2, "w5"), (2, "w2"), (2, "bf16")])
def test_spec_loop_greedy_equals_autoregressive(D, fmt):
    import torch
    L0, t0, n = 700, 123, 14
    log(f"closed loop at T = 0 vs greedy AR (2 layers, full width), D = {D}, {fmt} target")
    target, head, kv = _loop_setup(21, D, L0, fmt)
    ar = _ar_sequence(target, head, kv, L0, t0, n + D + 1, 0.0, 0.95)
    # the head's drafts
    _reset(target, head, kv)
    loop = SpecLoop(target, head, D)
    seq = [loop.start(L0, t0, 0.0, 0.95, SEED, 0)]
    cycles = 0
    while len(seq) < n:
        seq += loop.cycle(0.0, 0.95, SEED, cycles + 1)
        cycles += 1
    assert seq[:n] == ar[:n], (seq, ar)
    assert loop.L == L0 + len(seq)
    # drafts that are the greedy continuation: every cycle accepts all D
    _reset(target, head, kv)
    loop = SpecLoop(target, head, D)
    seq = [loop.start(L0, t0, 0.0, 0.95, SEED, 0)]
    while len(seq) + D + 1 <= len(ar):
        drafts = torch.tensor(ar[len(seq):len(seq) + D], dtype=torch.int32, device="cuda")
        out = loop.cycle(0.0, 0.95, SEED, len(seq), drafts=drafts)
        assert len(out) == D + 1
        seq += out
    assert seq == ar[:len(seq)] and len(seq) >= n


def test_spec_loop_sampling_deterministic():
    D, L0, t0 = 3, 500, 77
    log("closed loop at T = 0.6: determinism and cycle invariants")
    target, head, kv = _loop_setup(22, D, L0)
    runs = []
    for rep in range(2):
        _reset(target, head, kv)
        loop = SpecLoop(target, head, D)
        seq = [loop.start(L0, t0, 0.6, 0.95, SEED, 0)]
        for c in range(6):
            out = loop.cycle(0.6, 0.95, SEED, c + 1)
            assert 1 <= len(out) <= D + 1 and all(0 <= t < 4096 for t in out)
            seq += out
        assert loop.L == L0 + len(seq)
        runs.append(seq)
    assert runs[0] == runs[1]


PER_WEIGHT = {"w4": 0.53125, "w8": 1.03125, "w6": 0.78125, "w5": 0.65625, "w3": 0.40625, "w2": 0.28125,
              "f16": 2.0, "bf16": 2.0}


@pytest.mark.parametrize("fmt", ["w4", "w8", "w6", "w5", "w3", "w2", "f16", "bf16"])
def test_gemm_pass_counts_and_bytes(fmt):
    """The GEMM-only pass the bench times issues one launch per linear plus the
    LM head, and its algorithmic bytes are the weights' bytes plus activations."""
    import torch
    cfg = dict(DENSE_27B, layers=2, V=4096)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(31)
    log(f"gemm pass counts, {fmt}")
    dec = Decoder(cfg, 4, 128, gen=gen, fmt=fmt)
    n = dec.gemm_pass(4)
    torch.cuda.synchronize()
    assert n == 4 * cfg["layers"] + 1
    wb = dec.weight_bytes()
    alg = dec.gemm_alg_bytes(4)
    per_w = PER_WEIGHT[fmt]
    M, d, F, nqkv = 4, cfg["d"], cfg["F"], (cfg["nq"] + 2 * cfg["nkv"]) * cfg["hd"]
    nw = cfg["layers"] * (nqkv * d + d * d + 2 * F * d + d * F) + cfg["V"] * d
    assert wb == int(round(nw * per_w))
    # activations in (bf16) and outputs out (fp32 partial sums; gate|up writes
    # the bf16 SwiGLU of its epilogue instead)
    gate_up_out = M * F * 2
    act = cfg["layers"] * (M * d * 2 + M * nqkv * 4 + M * d * 2 + M * d * 4 + M * d * 2 + gate_up_out
                           + M * F * 2 + M * d * 4) + M * d * 2 + M * cfg["V"] * 4
    assert alg == wb + act


def test_depth_autotune():
    """The draft-depth autotune (DepthTuner) on the 2-layer full-width model:
    * random weights at T = 0.6: the head's drafts are independent of the
      target and almost never accepted, so every depth emits about one token
      per cycle at a higher cost than the AR step -- AR is locked;
    * T = 0 with drafts that are the target's greedy continuation: every
      draft is accepted (D + 1 tokens per cycle, alpha = 1), and the pick is
      the depth with the most (D + 1) / cycle time among the measured ones;
    * at T = 0 the sequence decode() emits equals greedy autoregressive
      decoding token for token whatever depth is locked (AR, 1, 2, 3)."""
    import torch
    from verify_step_w4_amd.model import DepthTuner
    L0, t0 = 600, 321
    log("draft-depth autotune (2 layers, full width)")
    target, head, kv = _loop_setup(23, 3, L0)
    tuner = DepthTuner(target, head, (1, 2, 3))
    _reset(target, head, kv)
    rep = tuner.tune(L0, t0, 0.6, 0.95, SEED, cycles=6, reps=5)
    print(f"[autotune, random head] {rep}", flush=True)
    assert rep["depth"] == 0 and rep["pick"] == "ar"
    assert all(1.0 <= rep["tokens_per_cycle"][f"D{D}"] <= D + 1 for D in (1, 2, 3))
    # greedy continuation drafts: alpha = 1
    cycles = 4
    ar = _ar_sequence(target, head, kv, L0, t0, cycles * 4 + 4, 0.0, 0.95)

    def greedy_drafts(loop, emitted):
        return torch.tensor(ar[len(emitted):len(emitted) + loop.D], dtype=torch.int32, device="cuda")

    _reset(target, head, kv)
    rep = tuner.tune(L0, t0, 0.0, 0.95, SEED, cycles=cycles, reps=5, drafts_fn=greedy_drafts)
    print(f"[autotune, greedy drafts] {rep}", flush=True)
    for D in (1, 2, 3):
        assert rep["tokens_per_cycle"][f"D{D}"] == D + 1
    tps = rep["tokens_per_s"]
    for D in (1, 2, 3):
        assert abs(tps[f"D{D}"] - (D + 1) * 1e3 / rep["ms"][f"D{D}"]) < 1e-9 * tps[f"D{D}"]
    assert abs(tps["ar"] - 1e3 / rep["ms"]["ar"]) < 1e-9 * tps["ar"]
    want = DepthTuner.choose({0: tps["ar"], 1: tps["D1"], 2: tps["D2"], 3: tps["D3"]})
    assert rep["depth"] == want and want == max((0, 1, 2, 3), key=lambda D: (tps["ar" if D == 0 else f"D{D}"], -D))
    # whatever depth is locked, T = 0 decoding is greedy decoding
    n = 13
    for D in (0, 1, 2, 3):
        _reset(target, head, kv)
        tuner.depth = D
        seq, loop = tuner.decode(L0, t0, n, 0.0, 0.95, SEED)
        assert seq[:n] == ar[:n], (D, seq, ar)
        assert loop.L == L0 + len(seq)
