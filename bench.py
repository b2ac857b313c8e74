#!/usr/bin/env python3
"""Benchmark of the batched verify step on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line (rank 0): verify steps/s for the workload, plus the
roofline of the dominant kernel (the W4 skinny GEMM) measured with HIP
events on the stream it runs on, and the CPU oracle timed on a bounded
sample of the same workload.

Workloads (synthetic, seeded; the weights are random, drawn on the device):
  lm_head_verify  LM-head verify step: hidden rows bf16 ~N(0,1) [4][5120],
                  W4 group-64 LM head [151936][5120] (~N(0,0.02), three copies
                  rotated so the 256 MB Infinity Cache cannot hold the working
                  set), temperature 0.6 / top_p 0.95 statistics, Leviathan–Chen
                  acceptance of 3 drafts drawn from q = softmax(N(0,3)).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verify steps/s and achieved HBM GB/s (W4 skinny GEMM, M=4) vs peak"
HBM_PEAK_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# --------------------------------------------------------------------------
# LM-head verify workload
# --------------------------------------------------------------------------
def lm_head_workload(args):
    import numpy as np
    import torch

    from verify_step_w4_amd import binding as B
    from verify_step_w4_amd.model import BYTES_PER_WEIGHT, LMHeadVerify, W4Linear

    V, d, M, D = 151936, 5120, 4, 3
    T, top_p = 0.6, 0.95
    seed = 0x5EED0003
    ncopies = 3
    nsteps_inputs = 64
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261203)
    log(f"generating {ncopies} W4 LM heads [{V}][{d}]")
    heads = [W4Linear.random(V, d, 0.02, gen) for _ in range(ncopies)]
    xs = (torch.randn((nsteps_inputs, M, d), generator=gen, device=dev)).to(torch.bfloat16).view(torch.int16)
    qs = torch.softmax(torch.randn((nsteps_inputs, D, V), generator=gen, device=dev, dtype=torch.float64) * 3.0,
                       dim=-1).to(torch.float32)
    drafts = torch.multinomial(qs.reshape(-1, V).double(), 1, generator=gen).reshape(nsteps_inputs, D).to(torch.int32)
    vs = LMHeadVerify(V, d, M)
    K, W = args.steps, args.warmup
    tok_all = torch.empty((K, M), dtype=torch.int32, device=dev)
    nacc_all = torch.empty(K, dtype=torch.int32, device=dev)
    flag_all = torch.empty(K, dtype=torch.int32, device=dev)

    def one(i, timed=False, ev=None):
        j = i % nsteps_inputs
        head = heads[i % ncopies]
        if ev is not None:
            ev[0].record()
        vs.gemm(xs[j], head)
        if ev is not None:
            ev[1].record()
        out = {}
        if timed:
            out = dict(tokens=tok_all[i:i + 1], n_acc=nacc_all[i:i + 1], flags=flag_all[i:i + 1])
        vs.stats_and_accept(qs[j], drafts[j], T, top_p, seed, i, **out)

    for i in range(W):
        one(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(K):
        one(i, timed=True, ev=evs[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    gemm_ms = [a.elapsed_time(b) for a, b in evs]
    gemm_avg = float(np.mean(gemm_ms))
    alg_bytes = V * d * BYTES_PER_WEIGHT + M * d * 2 + M * V * 4
    achieved = alg_bytes / (gemm_avg * 1e-3) / 1e9
    nacc = nacc_all.cpu().numpy()
    flags = flag_all.cpu().numpy()
    hist = np.bincount(np.clip(nacc, 0, D), minlength=D + 1).tolist()
    res = dict(
        ms_per_step=total_ms / K,
        value=K / (total_ms * 1e-3),
        wall_s=wall,
        config={"workload": "lm_head_verify", "d": d, "V": V, "M": M, "draft_depth": D, "temperature": T,
                "top_p": top_p, "weights": "int4 group-64 symmetric, fp16 scales", "lm_head_copies": ncopies},
        roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                  "kernel": "w4_gemm_kernel<4>", "alg_bytes_per_launch": int(alg_bytes),
                  "avg_launch_us": round(gemm_avg * 1e3, 2)},
        stages_us={"w4_gemm_lm_head": round(gemm_avg * 1e3, 2),
                   "stats_and_accept": round(total_ms / K * 1e3 - gemm_avg * 1e3, 2)},
        accepted_length_hist=hist,
        flagged_steps=int(((flags & ~B.FLAG_NONFINITE) != 0).sum()),
    )
    return res


def lm_head_cpu_baseline(nsteps=3):
    """The CPU oracle on a bounded sample: nsteps full LM-head verify steps
    (fp64 W4 GEMM over all 151936 rows, sorted-vocab top-p, scalar accept)."""
    import numpy as np

    import oracle
    from verify_step_w4_amd import synth
    V, d, D = 151936, 5120, 3
    g = synth.rng(synth.SEED_BASE + 3)
    w = synth.normal_f32(g, (V, d), 0.02)
    codes, scales = oracle.w4_quantize(w)
    del w
    xs = [synth.f32_to_bf16_bits(synth.normal_f32(g, (D + 1, d), 1.0)) for _ in range(nsteps)]
    q, drafts = synth.q_and_drafts(synth.SEED_BASE + 33, D, V, 3.0, B=nsteps)
    t0 = time.perf_counter()
    for s in range(nsteps):
        z = oracle.w4_gemm(xs[s], codes, scales).astype(np.float32)
        oracle.spec_accept(z, q, drafts[s], 0.6, 0.95, 0x5EED0003, s)
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(nsteps / dt, 4), "unit": "verify steps/s", "cores": cores, "kind": "oracle",
            "sample": f"{nsteps} LM-head verify steps (d=5120, V=151936, M=4), quantisation untimed"}


# --------------------------------------------------------------------------
# Full verify step of the 27B-shaped dense decoder
# --------------------------------------------------------------------------
def verify27b_workload(args):
    import numpy as np
    import torch

    from verify_step_w4_amd import binding as B
    from verify_step_w4_amd.model import DENSE_27B, Decoder, VerifyStep

    cfg = dict(DENSE_27B)
    M, D, L = 4, 3, args.context
    T, top_p, seed = 0.6, 0.95, 0x5EED0004
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261204)
    t0 = time.perf_counter()
    log(f"generating the 64-layer W4 decoder (d=5120, GQA 40/8x128, FFN 17408) + LM head, KV context L={L}")
    dec = Decoder(cfg, M, L + M + 8, gen=gen)
    torch.cuda.synchronize()
    log(f"weights ready in {time.perf_counter() - t0:.1f} s ({dec.weight_bytes() / 1e9:.2f} GB W4)")
    V, d = cfg["V"], cfg["d"]
    npool = 8
    xs = torch.randn((npool, M, d), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
    qs = torch.softmax(torch.randn((npool, D, V), generator=gen, device=dev, dtype=torch.float64) * 3.0,
                       dim=-1).to(torch.float32)
    drafts = torch.multinomial(qs.reshape(-1, V).double(), 1, generator=gen).reshape(npool, D).to(torch.int32)
    vs = VerifyStep(dec, M)
    ar = VerifyStep(dec, 1)
    K, W = args.steps, args.warmup
    nacc_all = torch.empty(K, dtype=torch.int32, device=dev)
    tok_all = torch.empty((K, M), dtype=torch.int32, device=dev)
    flag_all = torch.empty(K, dtype=torch.int32, device=dev)
    gemm_events = []

    def hook(when, name):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        gemm_events.append(e)

    # (a) eager pass: every W4 GEMM launch bracketed by HIP events on its stream
    for i in range(W):
        vs.run(xs[i % npool], L, qs[i % npool], drafts[i % npool], T, top_p, seed, i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        j = i % npool
        vs.run(xs[j], L, qs[j], drafts[j], T, top_p, seed, i, gemm_hook=hook)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / K
    gemm_ms = sum(gemm_events[2 * k].elapsed_time(gemm_events[2 * k + 1]) for k in range(len(gemm_events) // 2))
    n_gemm = len(gemm_events) // 2
    # (b) the timed region: the verify step captured once as a HIP graph and
    # replayed; each replay is preceded by copying the next step's inputs
    # into the captured buffers (counted in the time)
    x_s, q_s, d_s = xs[0].clone(), qs[0].clone(), drafts[0].clone()
    step_dev = torch.zeros(1, dtype=torch.int64, device=dev)
    graph = vs.capture(x_s, L, q_s, d_s, T, top_p, seed, step_dev)
    for i in range(W):
        graph.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(K):
        j = i % npool
        x_s.copy_(xs[j])
        q_s.copy_(qs[j])
        d_s.copy_(drafts[j])
        graph.replay()
        tok_all[i:i + 1].copy_(vs.tokens)
        nacc_all[i:i + 1].copy_(vs.n_acc)
        flag_all[i:i + 1].copy_(vs.flags)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    # (c) the M = 1 autoregressive step on the same weights and context, same way
    x1 = xs[0][:1].clone()
    step1 = torch.zeros(1, dtype=torch.int64, device=dev)
    g1 = ar.capture(x1, L, None, None, T, top_p, seed, step1)
    for i in range(W):
        g1.replay()
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for i in range(K):
        x1.copy_(xs[i % npool][:1])
        g1.replay()
    a1.record()
    torch.cuda.synchronize()
    ar_ms = a0.elapsed_time(a1) / K
    step_ms = total_ms / K
    alg_gemm = dec.gemm_alg_bytes(M)            # per step, all GEMM launches
    gemm_launch_us = gemm_ms * 1e3 / n_gemm
    per_launch_bytes = alg_gemm / (n_gemm / K)
    achieved = per_launch_bytes / (gemm_launch_us * 1e-6) / 1e9
    step_bytes = dec.weight_bytes() + dec.kv_bytes(L, M)
    nacc = nacc_all.cpu().numpy()
    flags = flag_all.cpu().numpy()
    res = dict(
        ms_per_step=step_ms,
        value=K / (total_ms * 1e-3),
        wall_s=wall,
        config={"workload": "verify27b", "layers": 64, "d_model": d, "heads_q_kv_dim": [40, 8, 128],
                "ffn": cfg["F"], "V": V, "context": L, "M": M, "draft_depth": D, "temperature": T, "top_p": top_p,
                "weights": "int4 group-64 symmetric, fp16 scales", "kv_cache": "bf16"},
        roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                  "kernel": "w4_gemm_kernel<4> (all 257 W4 GEMM launches of a step)",
                  "alg_bytes_per_launch": int(per_launch_bytes), "avg_launch_us": round(gemm_launch_us, 2)},
        stages_us={"w4_gemm_total": round(gemm_ms * 1e3 / K, 1),
                   "eager_step": round(eager_ms * 1e3, 1),
                   "rest_of_eager_step": round(eager_ms * 1e3 - gemm_ms * 1e3 / K, 1)},
        m1_ar_step_ms=round(ar_ms, 4),
        verify_over_ar=round(step_ms / ar_ms, 4),
        step_hbm_gbs=round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
        accepted_length_hist=np.bincount(np.clip(nacc, 0, D), minlength=D + 1).tolist(),
        flagged_steps=int(((flags & ~B.FLAG_NONFINITE) != 0).sum()),
    )
    return res


def verify27b_cpu_baseline():
    """The CPU oracle on a bounded sample of the same step: one decoder layer
    of the 27B-class shapes (4 W4 GEMMs over its 175 MB of weights, fp64),
    scaled by 64 layers, plus the LM head (sampled 1/16 of the rows, scaled).
    Attention/glue are O(L * d) and small next to the GEMMs at L = 8192;
    they are left out of the sample (said so in `sample`)."""
    import numpy as np

    import oracle
    from verify_step_w4_amd import synth
    g = synth.rng(synth.SEED_BASE + 4)
    shapes = [(7168, 5120), (5120, 5120), (34816, 5120), (5120, 17408)]
    x = {K: synth.f32_to_bf16_bits(synth.normal_f32(g, (4, K), 1.0)) for _, K in shapes}
    tot = 0.0
    for N, K in shapes:
        w = synth.normal_f32(g, (N, K), 0.02)
        codes, scales = oracle.w4_quantize(w)
        del w
        t0 = time.perf_counter()
        oracle.w4_gemm(x[K], codes, scales)
        tot += time.perf_counter() - t0
    V16 = 151936 // 16
    w = synth.normal_f32(g, (V16, 5120), 0.02)
    codes, scales = oracle.w4_quantize(w)
    t0 = time.perf_counter()
    oracle.w4_gemm(x[5120], codes, scales)
    lm = (time.perf_counter() - t0) * 16
    step_s = 64 * tot + lm
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(1.0 / step_s, 5), "unit": "verify steps/s", "cores": cores, "kind": "oracle",
            "sample": "one 27B-class layer's four W4 GEMMs at M=4 (x64 layers) + 1/16 of the LM head (x16); "
                      "attention and glue not in the sample"}


WORKLOADS = {"lm_head_verify": (lm_head_workload, lm_head_cpu_baseline),
             "verify27b": (verify27b_workload, verify27b_cpu_baseline)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="lm_head_verify", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--context", type=int, default=8192, help="KV context length L of the verify27b workload")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    run, cpu = WORKLOADS[args.workload]
    res = run(args)
    out = {"metric": METRIC, "value": round(res["value"], 3), "unit": "verify steps/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": res["config"], "roofline": res["roofline"]}
    for k in ("stages_us", "accepted_length_hist", "flagged_steps", "m1_ar_step_ms", "verify_over_ar",
              "step_hbm_gbs"):
        if k in res:
            out[k] = res[k]
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
