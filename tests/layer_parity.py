"""Teacher-forced parity of a decoder forward, op by op.

A forward of the GPU decoder is run with a hook that snapshots its buffers
around every GEMM launch.  Each op is then recomputed by the oracle from the
GPU's own input to that op (its bf16 activations, the fp32 sums of its split-K
partials taken in slice order, its KV cache) and only that op's output is
compared:

* fp32 outputs (GEMM sums, logits): the GEMM bar, max |y - ref| / max(|ref|,
  row rms) <= GEMM_RTOL (1e-3);
* bf16 outputs (norms, RoPE, attention, SwiGLU, residual adds): within the
  bf16 rounding of the exact value (2^-8 |ref| + 1e-3 rms) and at least 97 %
  bit-identical to the oracle's rounding.

One-ulp bf16 flips therefore cannot accumulate from layer to layer, and every
op is held to its own bar; the end-to-end error of the logits is reported as
a statistic by the callers.
"""
import numpy as np

import oracle
from verify_step_w4_amd import binding as B
from verify_step_w4_amd import synth

from helpers import GEMM_RTOL, gemm_rel_err, host, rows_from_vb

BF16_REL = 2.0 ** -8


def bf16_close(gpu_bits, ref, rms_axis=-1, min_exact=0.97, what=""):
    """bf16 results against the exact value: within its bf16 rounding (plus
    1e-3 of the row rms for fp32 accumulation) and mostly bit-identical."""
    g = synth.bf16_bits_to_f32(gpu_bits).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt((ref ** 2).mean(axis=rms_axis, keepdims=True))
    err = np.abs(g - ref)
    assert np.all(err <= BF16_REL * np.abs(ref) + 1e-3 * rms), (what, float((err / (np.abs(ref) + rms)).max()))
    exact = float((np.asarray(gpu_bits) == oracle.bf16_round(ref)).mean())
    assert exact >= min_exact, (what, exact)
    return exact


def slice_sum_f32(parts):
    """The consumers' reduction of split-K partials: fp32 adds in slice order."""
    s = np.zeros(parts.shape[1:], dtype=np.float32)
    for k in range(parts.shape[0]):
        s = (s + parts[k]).astype(np.float32)
    return s


class DecoderCapture:
    """gemm_hook of Decoder.forward: host copies of the buffers each op reads
    and writes, per layer.  Before layer l's qkv the current residual is
    dec.resid, before its gate|up it is dec.resid2 (the out-of-place add +
    RMSNorm alternates between the two)."""

    def __init__(self, dec, M):
        self.dec, self.M = dec, M
        self.layers = []
        self.final = {}

    def _parts(self, name):
        dec, M = self.dec, self.M
        N, K = dec.shapes[name]
        S, ldp = dec.layers[0][name].partials_layout(M)
        return host(dec.parts[name][:S * M * ldp]).reshape(S, M, ldp)[:, :, :N].copy()

    def __call__(self, when, name):
        import torch
        torch.cuda.synchronize()
        dec, M = self.dec, self.M
        if when == "pre" and name == "qkv":
            li = len(self.layers)
            self.layers.append(dict(h1=host(dec.h[:M]).copy(), resid1=host(dec.resid[:M]).copy()))
            if li > 0:   # the add + RMSNorm that closed the previous layer
                self.layers[li - 1]["resid_next"] = self.layers[li]["resid1"]
                self.layers[li - 1]["h_next"] = self.layers[li]["h1"]
        cur = self.layers[-1] if self.layers else None
        if when == "post" and name == "qkv":
            cur["qkv"] = self._parts("qkv")
        elif when == "pre" and name == "o":
            li = len(self.layers) - 1
            cur["q"] = host(dec.q[:M]).copy()
            cur["attn"] = host(dec.attn[:M]).copy()
            cur["Kc"] = host(dec.Kc[li]).copy()
            cur["Vc"] = rows_from_vb(host(dec.Vc[li]))
        elif when == "post" and name == "o":
            cur["o"] = self._parts("o")
        elif when == "pre" and name == "gate_up":
            cur["resid2"] = host(dec.resid2[:M]).copy()
            cur["h2"] = host(dec.h[:M]).copy()
        elif when == "post" and name == "gate_up":
            cur["a"] = host(dec.a[:M]).copy()
        elif when == "post" and name == "down":
            cur["down"] = self._parts("down")
        elif when == "pre" and name == "lm_head":
            self.final = dict(resid=host(dec.resid[:M]).copy(), h=host(dec.h[:M]).copy())
            cur["resid_next"], cur["h_next"] = self.final["resid"], self.final["h"]
        elif when == "post" and name == "lm_head":
            self.final["logits"] = host(dec.logits[:M]).copy()


def check_decoder_ops(cap, hm, cfg, x, L, quant=None, gemm=None, report=None):
    """Every op of the captured forward against the oracle on the GPU's own
    inputs (see the module docstring).  hm: the host fp32 weights the device
    model was quantised from; x: the input rows (bf16 bits).  Returns the worst
    fp32 error and the lowest bf16 identity fraction seen."""
    quant = quant or oracle.w4_quantize
    gemm = gemm or oracle.w4_gemm
    d, nq, nkv, hd, F, eps = (cfg[k] for k in ("d", "nq", "nkv", "hd", "F", "eps"))
    M = x.shape[0]
    worst, ident = 0.0, 1.0

    def gem(name, y, ref):
        nonlocal worst
        e = gemm_rel_err(y, ref)
        assert e <= GEMM_RTOL, (name, e)
        worst = max(worst, e)

    def b16(name, bits, ref, **kw):
        nonlocal ident
        ident = min(ident, bf16_close(bits, ref, what=name, **kw))

    assert len(cap.layers) == len(hm["layers"])
    # the first RMSNorm reads the input rows unchanged
    assert np.array_equal(cap.layers[0]["resid1"], x)
    for li, (c, l) in enumerate(zip(cap.layers, hm["layers"])):
        tag = f"layer {li}"
        Q = {k: quant(l[k]) for k in ("qkv", "o", "gate_up", "down")}
        b16(f"{tag} rmsnorm 1", c["h1"], oracle.rmsnorm(c["resid1"], l["g1"], eps))
        qkv = slice_sum_f32(c["qkv"])
        gem(f"{tag} qkv", qkv, gemm(c["h1"], *Q["qkv"]))
        # RoPE of q and the new k at positions L + m, v appended as is
        q_ref = np.zeros((M, nq, hd))
        k_ref = np.zeros((M, nkv, hd))
        for m in range(M):
            row = qkv[m].astype(np.float64)
            for h in range(nq):
                q_ref[m, h] = oracle.rope(row[h * hd:(h + 1) * hd], L + m, cfg["theta"])
            for h in range(nkv):
                k_ref[m, h] = oracle.rope(row[(nq + h) * hd:(nq + h + 1) * hd], L + m, cfg["theta"])
        b16(f"{tag} rope q", c["q"], q_ref)
        b16(f"{tag} rope k", np.stack([c["Kc"][:, L + m] for m in range(M)]), k_ref)
        v_new = np.stack([c["Vc"][:, L + m] for m in range(M)])
        v_ref = qkv[:, (nq + nkv) * hd:].astype(np.float64).reshape(M, nkv, hd)
        assert np.array_equal(v_new, oracle.bf16_round(v_ref)), f"{tag} v append"
        # attention over the cache as the GPU left it (context + appended rows)
        att_ref = oracle.decode_attn(oracle.bf16_value(c["q"]), c["Kc"], c["Vc"], L).reshape(M, nq * hd)
        b16(f"{tag} attention", c["attn"], att_ref)
        o = slice_sum_f32(c["o"])
        gem(f"{tag} o", o, gemm(c["attn"], *Q["o"]))
        b16(f"{tag} residual 1", c["resid2"], oracle.bf16_value(c["resid1"]) + o.astype(np.float64))
        b16(f"{tag} rmsnorm 2", c["h2"], oracle.rmsnorm(c["resid2"], l["g2"], eps))
        # the SwiGLU runs in the gate|up GEMM's epilogue on its fp32 sums, which
        # the oracle cannot be handed; it starts from the exact products, so
        # the GEMM's own rounding (about 1e-5 of the row rms from the folded
        # offset) moves a few more values across a bf16 rounding boundary: at
        # least 90 % bit-identical, as in the dedicated SwiGLU-epilogue tests
        gu = gemm(c["h2"], *Q["gate_up"])
        b16(f"{tag} swiglu", c["a"], oracle.swiglu(gu[:, :F], gu[:, F:]), min_exact=0.9)
        dn = slice_sum_f32(c["down"])
        gem(f"{tag} down", dn, gemm(c["a"], *Q["down"]))
        b16(f"{tag} residual 2", c["resid_next"], oracle.bf16_value(c["resid2"]) + dn.astype(np.float64))
        g_next = hm["layers"][li + 1]["g1"] if li + 1 < len(hm["layers"]) else hm["final_gamma"]
        b16(f"{tag} rmsnorm next", c["h_next"], oracle.rmsnorm(c["resid_next"], g_next, eps))
    gem("lm head", cap.final["logits"], gemm(cap.final["h"], *quant(hm["lm_head"])))
    if report is not None:
        report["worst_fp32_rel"], report["min_bf16_identical"] = worst, ident
    return worst, ident


def end_to_end(logits, ref):
    """(max, median) of |logits - ref| / max(|ref|, row rms): a statistic."""
    rms = np.sqrt((ref ** 2).mean(axis=1, keepdims=True))
    rel = np.abs(logits - ref) / np.maximum(np.abs(ref), rms)
    return float(rel.max()), float(np.median(rel))
