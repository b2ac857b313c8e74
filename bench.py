#!/usr/bin/env python3
"""Benchmark of the batched verify step on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line (rank 0): verify steps/s for the workload, plus the
roofline of the dominant kernel (the W4 skinny GEMM) measured with HIP
events on the stream it runs on, and the CPU oracle timed on a bounded
sample of the same workload.

Workloads (synthetic, seeded; the weights are random, drawn on the device):
  verify27b       (default) the whole verify step of a 27B-shaped dense
                  decoder: 64 layers (d=5120, GQA 40/8 heads of 128, SwiGLU FFN
                  17408, all linears W4 group-64), RMSNorm, RoPE, decode
                  attention of the 4 verify rows over a bf16 KV cache of
                  --context positions, the W4 LM head [151936][5120],
                  temperature 0.6 / top_p 0.95 statistics and Leviathan–Chen
                  acceptance of 3 drafts; captured as one HIP graph.  Also
                  times the M = 1 autoregressive step on the same state.
  moe_verify      MoE-shaped verify step: 128 SwiGLU experts (2048 -> 768 ->
                  2048) with top-8 routing of each row on fresh N(0,1) router
                  logits, grouped W4 GEMMs over the chosen experts, LM head
                  [151936][2048], same acceptance; 4 expert banks and LM heads
                  rotated.
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
# bytes per weight (codes + one fp16 scale per 64, or the 16-bit weight) and a
# description of each weight format the decoder takes
WEIGHT_FORMATS = ("w4", "w8", "w6", "w5", "w3", "w2", "f16", "bf16")
WEIGHT_BYTES = {"w4": 0.53125, "w8": 1.03125, "w6": 0.78125, "w5": 0.65625, "w3": 0.40625, "w2": 0.28125,
                "f16": 2.0, "bf16": 2.0}
WEIGHT_DESC = {"w4": "int4 group-64 symmetric, fp16 scales", "w8": "int8 group-64 symmetric, fp16 scales",
               "w6": "6-bit group-64 symmetric, fp16 scales", "w5": "5-bit group-64 symmetric, fp16 scales",
               "w3": "3-bit group-64 symmetric, fp16 scales", "w2": "2-bit group-64 symmetric, fp16 scales",
               "f16": "fp16, unquantised", "bf16": "bf16, unquantised"}
CALIB_COPY_BYTES = 256 << 20


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w4_gemm_hbm_traffic.md")


def measured_traffic(workload):
    """HBM bytes per W4 GEMM launch of a workload's step, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (scaled by the plain-copy
    calibration there), or None if there is none or the GEMM sources have
    changed since the counters were taken."""
    import hashlib
    import re
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    h = hashlib.sha256()
    for name in ("w4_gemm.hip", "skinny_gemm.h"):
        h.update(open(os.path.join(ROOT, "verify_step_w4_amd", "csrc", name), "rb").read())
    digest = h.hexdigest()
    m = re.search(r"W4 GEMM sources sha256 \(w4_gemm\.hip, then skinny_gemm\.h\): ([0-9a-f]{64})", text)
    if not m or m.group(1) != digest:
        return None
    m = re.search(r"^\| " + re.escape(workload) + r" \| ([0-9.]+) \| ([0-9.]+) \| ([0-9.]+) \|", text, re.M)
    if not m:
        return None
    return int(float(m.group(3)))


def time_graphs(issue_fns, reps):
    """Capture each issue_fn() (which launches work and returns its launch
    count) into its own HIP graph, then replay the graphs in turn reps times
    between two HIP events on the replay stream.  Returns (ms per launch,
    launches per round)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graphs, n = [], 0
    with torch.cuda.stream(s):
        for fn in issue_fns:
            fn()
    torch.cuda.synchronize()
    for fn in issue_fns:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            n += fn()
        graphs.append(g)
    torch.cuda.synchronize()
    for g in graphs:
        g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        for g in graphs:
            g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * n), n


def read_ceiling_gbs(nbytes=1 << 30, reps=10):
    """The plain streaming-read ceiling of this part: vw4_stream_read over a
    1 GiB buffer (four times the Infinity Cache) at several grid sizes, the
    best mean over `reps` back-to-back calls timed with HIP events on the
    current stream.  Returns (GB/s, workgroups)."""
    import torch

    from verify_step_w4_amd import binding as B
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1 << 14, dtype=torch.int32, device="cuda")
    best = (0.0, 0)
    for blocks in (1024, 2048, 4096, 8192):
        for _ in range(2):
            B.stream_read(buf, sink, blocks)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            B.stream_read(buf, sink, blocks)
        e1.record()
        torch.cuda.synchronize()
        gbs = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        if gbs > best[0]:
            best = (gbs, blocks)
    del buf, sink
    return best


class InputStage:
    """The per-step inputs of a captured step packed in one device byte
    buffer: views into `stage` are what the graph reads, and `pool` holds
    npool input sets in the same layout, so one copy (pool[j] -> stage)
    refreshes every input of a step.  specs: (name, shape, torch dtype)."""

    def __init__(self, specs, npool, device="cuda"):
        import torch
        self.offs, off = {}, 0
        for name, shape, dt in specs:
            n = int(torch.tensor([], dtype=dt).element_size())
            for v in shape:
                n *= v
            self.offs[name] = (off, n, tuple(shape), dt)
            off += (n + 255) // 256 * 256
        self.nbytes = off
        self.stage = torch.empty(off, dtype=torch.uint8, device=device)
        self.pool = torch.empty((npool, off), dtype=torch.uint8, device=device)

    def _view(self, buf, name):
        off, n, shape, dt = self.offs[name]
        return buf[off:off + n].view(dt).view(shape)

    def view(self, name):
        return self._view(self.stage, name)

    def slot(self, j, name):
        return self._view(self.pool[j], name)

    def load(self, j):
        self.stage.copy_(self.pool[j])


class Telemetry:
    """Samples the GPU's clocks, temperatures and power through amdsmi in a
    background thread (every `period` s) while the GPU works.  summary()
    gives min / median / max of each metric and the change of the firmware's
    throttle-residency counters over the run; if amdsmi is unavailable it
    says why instead."""

    FIELDS = (("gfxclk_mhz", "current_gfxclk", "current_gfxclks"), ("uclk_mhz", "current_uclk", None),
              ("hotspot_c", "temperature_hotspot", None), ("hbm_c", "temperature_mem", None),
              ("socket_power_w", "current_socket_power", None))
    RESIDENCY = ("prochot_residency_acc", "ppt_residency_acc", "socket_thm_residency_acc",
                 "vr_thm_residency_acc", "hbm_thm_residency_acc")

    def __init__(self, period=0.25):
        import threading
        self.period, self.samples, self.error = period, [], None
        self.first = self.last = None
        self.stop_evt = threading.Event()
        self.thread = None
        try:
            import amdsmi
            import torch
            amdsmi.amdsmi_init()
            self.smi = amdsmi
            handles = amdsmi.amdsmi_get_processor_handles()
            p = torch.cuda.get_device_properties(0)
            want = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}"
            self.handle = next((h for h in handles
                                if amdsmi.amdsmi_get_gpu_device_bdf(h).lower().startswith(want)), None)
            if self.handle is None:
                raise RuntimeError(f"no amdsmi device at PCI {want}")
            self.first = self.last = amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
        except Exception as e:  # telemetry is a report, never a reason to fail the bench
            self.error = f"{type(e).__name__}: {e}"

    @staticmethod
    def _num(v):
        if isinstance(v, (list, tuple)):
            vals = [x for x in (Telemetry._num(y) for y in v) if x is not None]
            return max(vals) if vals else None
        return float(v) if isinstance(v, (int, float)) else None

    def _run(self):
        while not self.stop_evt.wait(self.period):
            try:
                m = self.smi.amdsmi_get_gpu_metrics_info(self.handle)
            except Exception as e:
                self.error = f"{type(e).__name__}: {e}"
                return
            self.last = m
            row = {}
            for name, key, alt in self.FIELDS:
                v = self._num(m.get(key))
                if v is None and alt:
                    v = self._num(m.get(alt))
                row[name] = v
            self.samples.append(row)

    def start(self):
        import threading
        if self.error is None:
            self.thread = threading.Thread(target=self._run, daemon=True)
            self.thread.start()
        return self

    def stop(self):
        if self.thread is not None:
            self.stop_evt.set()
            self.thread.join()
        return self

    def summary(self):
        if not self.samples:
            return {"unavailable": self.error or "no samples"}
        import statistics
        out = {"samples": len(self.samples), "period_s": self.period}
        for name, _, _ in self.FIELDS:
            vals = [s[name] for s in self.samples if s[name] is not None]
            if vals:
                out[name] = {"min": min(vals), "median": statistics.median(vals), "max": max(vals)}
        n0, n1 = self._num(self.first.get("accumulation_counter")), self._num(self.last.get("accumulation_counter"))
        if n0 is not None and n1 is not None and n1 > n0:
            res = {}
            for key in self.RESIDENCY:
                a, b = self._num(self.first.get(key)), self._num(self.last.get(key))
                if a is not None and b is not None:
                    res[key.replace("_residency_acc", "")] = round((b - a) / (n1 - n0), 4)
            out["throttle_residency_frac"] = res
        if self.error:
            out["error"] = self.error
        return out


def sustained_run(issue_step, ms_per_step, seconds, group=2):
    """Replay one step (issue_step(i) enqueues step i) back to back for at
    least `seconds` on the current stream while Telemetry samples the GPU.
    A HIP event after every `group` steps gives samples of >= 10 ms each;
    returns the median, p10 and p90 of ms per step over those samples, the
    step rate of the first and last second, and the telemetry summary."""
    import numpy as np
    import torch
    n = max(group * 30, int(np.ceil(seconds * 1e3 / ms_per_step / group)) * group)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n // group + 1)]
    tel = Telemetry().start()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(n):
        issue_step(i)
        if (i + 1) % group == 0:
            evs[(i + 1) // group].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tel.stop()
    ms = np.array([evs[k].elapsed_time(evs[k + 1]) / group for k in range(len(evs) - 1)])
    t_end = np.cumsum(ms * group)  # ms since the start, at the end of each sample

    def rate(lo, hi):
        sel = (t_end > lo) & (t_end <= hi)
        return round(float(group * sel.sum() / (ms[sel] * group).sum() * 1e3), 2) if sel.any() else None

    total = float(t_end[-1])
    return {"steps": n, "seconds": round(total / 1e3, 2), "wall_s": round(wall, 2),
            "ms_per_step": {"median": round(float(np.median(ms)), 4), "p10": round(float(np.percentile(ms, 10)), 4),
                            "p90": round(float(np.percentile(ms, 90)), 4), "samples": len(ms),
                            "steps_per_sample": group},
            "steps_per_s_first_second": rate(0, 1000), "steps_per_s_last_second": rate(total - 1000, total),
            "gpu_telemetry": tel.summary()}


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
    # the statistics + acceptance stage at every (temperature, top_p) of the
    # workload: its time as a replayed graph (verify_logits, spec_accept_ex,
    # step advance on one set of logits, q and drafts; 8 stages per graph),
    # and the accepted-length
    # histogram of 256 steps with fresh inputs (logits of the rotated heads)
    sweep = {}
    step_dev = torch.zeros(1, dtype=torch.int64, device=dev)
    for Ts in (0.0, 0.6, 1.0):
        for ps in (0.95, 1.0):
            vs.gemm(xs[0], heads[0])
            s_ = torch.cuda.Stream()
            s_.wait_stream(torch.cuda.current_stream())

            def stage(Ts=Ts, ps=ps):
                B.verify_logits(None, None, None, M, V, d, Ts, ps, vs.logits, vs.stats, vs.stat_ws)
                B.spec_accept_ex(vs.logits, 0, vs.stats, 0, qs[0], 0, drafts[0], 1, D, V, Ts, seed, step_dev,
                                 vs.tokens, vs.n_acc, vs.flags, vs.acc_ws)
                B.step_advance(step_dev, 1)

            with torch.cuda.stream(s_):
                stage()
            torch.cuda.current_stream().wait_stream(s_)
            torch.cuda.synchronize()
            # 8 stages per graph, so that the cost of launching a graph from
            # the host does not show in the per-stage time
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(8):
                    stage()
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record()
            for _ in range(10):
                g.replay()
            a1.record()
            torch.cuda.synchronize()
            us = a0.elapsed_time(a1) / 80 * 1e3
            na = torch.empty(256, dtype=torch.int32, device=dev)
            fl = torch.empty(256, dtype=torch.int32, device=dev)
            for i in range(256):
                j = i % nsteps_inputs
                vs.gemm(xs[j], heads[i % ncopies])
                vs.stats_and_accept(qs[j], drafts[j], Ts, ps, seed + 1, i, n_acc=na[i:i + 1], flags=fl[i:i + 1])
            nh = na.cpu().numpy()
            flh = fl.cpu().numpy()
            sweep[f"T={Ts},top_p={ps}"] = {
                "stats_and_accept_us": round(us, 2),
                "accepted_length_hist_256": np.bincount(np.clip(nh, 0, D), minlength=D + 1).tolist(),
                "flagged_steps": int(((flh & ~B.FLAG_NONFINITE) != 0).sum())}
            log(f"T={Ts} top_p={ps}: {sweep[f'T={Ts},top_p={ps}']}")
    res = dict(
        ms_per_step=total_ms / K,
        value=K / (total_ms * 1e-3),
        wall_s=wall,
        config={"workload": "lm_head_verify", "d": d, "V": V, "M": M, "draft_depth": D, "temperature": T,
                "top_p": top_p, "weights": "int4 group-64 symmetric, fp16 scales", "lm_head_copies": ncopies},
        roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                  "kernel": "w4_gemm_kernel (M=4)", "alg_bytes_per_launch": int(alg_bytes),
                  "avg_launch_us": round(gemm_avg * 1e3, 2)},
        stages_us={"w4_gemm_lm_head": round(gemm_avg * 1e3, 2),
                   "stats_and_accept": round(total_ms / K * 1e3 - gemm_avg * 1e3, 2)},
        accepted_length_hist=hist,
        flagged_steps=int(((flags & ~B.FLAG_NONFINITE) != 0).sum()),
        stats_accept_sweep=sweep,
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
    from verify_step_w4_amd.model import BYTES_PER_WEIGHT, DENSE_27B, Decoder, VerifyStep

    cfg = dict(DENSE_27B)
    M, D, L = 4, 3, args.context
    T, top_p, seed = 0.6, 0.95, 0x5EED0004
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261204)
    t0 = time.perf_counter()
    sweep_L = [] if args.no_context_sweep else [c for c in (1024, 8192, 32768) if c != L]
    Lcap = max([L] + sweep_L)
    fmt = args.weights
    log(f"generating the 64-layer {fmt.upper()} decoder (d=5120, GQA 40/8x128, FFN 17408) + LM head, KV cache for "
        f"{Lcap} positions, timed context L={L}")
    dec = Decoder(cfg, M, Lcap + M + 8, gen=gen, fmt=fmt)
    bpw = WEIGHT_BYTES[fmt]
    torch.cuda.synchronize()
    log(f"weights ready in {time.perf_counter() - t0:.1f} s ({dec.weight_bytes() / 1e9:.2f} GB {fmt.upper()})")
    V, d = cfg["V"], cfg["d"]
    npool = 8
    xs = torch.randn((npool, M, d), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
    qs = torch.softmax(torch.randn((npool, D, V), generator=gen, device=dev, dtype=torch.float64) * 3.0,
                       dim=-1).to(torch.float32)
    drafts = torch.multinomial(qs.reshape(-1, V).double(), 1, generator=gen).reshape(npool, D).to(torch.int32)
    vs = VerifyStep(dec, M)
    ar = VerifyStep(dec, 1)
    K, W = args.steps, args.warmup
    out_all = torch.empty((K, M + 2), dtype=torch.int32, device=dev)   # tokens, n_acc, flags per step
    nacc_all, flag_all = out_all[:, M], out_all[:, M + 1]
    gemm_events = []

    gemm_names = []

    def hook(when, name):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        gemm_events.append(e)
        if when == "pre":
            gemm_names.append(name)

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
    per_gemm = [gemm_events[2 * k].elapsed_time(gemm_events[2 * k + 1]) for k in range(len(gemm_events) // 2)]
    gemm_ms = sum(per_gemm)
    n_gemm = len(per_gemm)
    by_name = {}
    for nm, t in zip(gemm_names, per_gemm):
        by_name.setdefault(nm, []).append(t)
    # (b) the timed region: the verify step captured once as a HIP graph and
    # replayed; each replay is preceded by copying the next step's inputs
    # into the captured buffers (counted in the time)
    stage = InputStage([("x", (M, d), torch.int16), ("q", (D, V), torch.float32), ("d", (D,), torch.int32)], npool)
    for j in range(npool):
        stage.slot(j, "x").copy_(xs[j])
        stage.slot(j, "q").copy_(qs[j])
        stage.slot(j, "d").copy_(drafts[j])
    stage.load(0)
    x_s, q_s, d_s = stage.view("x"), stage.view("q"), stage.view("d")
    step_dev = torch.zeros(1, dtype=torch.int64, device=dev)
    graph = vs.capture(x_s, L, q_s, d_s, T, top_p, seed, step_dev)
    for i in range(W):
        graph.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(K):
        stage.load(i % npool)
        graph.replay()
        out_all[i].copy_(vs.outputs)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    sustained = None
    if args.sustain > 0:
        # the same replays for >= args.sustain seconds: spread of the step
        # time, and the GPU's clocks / temperatures / power meanwhile

        def issue(i):
            stage.load(i % npool)
            graph.replay()

        sustained = sustained_run(issue, total_ms / K, args.sustain)
        log(f"sustained: {sustained}")
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
    # (d) the W4 GEMM kernel by itself: the 257 GEMM launches of a step, same
    # shapes, weights and buffers, captured as a graph and replayed
    ms_launch, n_launch = time_graphs([lambda: dec.gemm_pass(M)], 20)
    alg_gemm = dec.gemm_alg_bytes(M)            # per step, all GEMM launches
    gemm_launch_us = ms_launch * 1e3
    per_launch_bytes = alg_gemm / n_launch
    achieved = per_launch_bytes / (gemm_launch_us * 1e-6) / 1e9
    step_bytes = dec.weight_bytes() + dec.kv_bytes(L, M)
    # (e) the same step (graph, inputs copied in) and the M = 1 step at the
    # other context lengths of the workload
    ctx_sweep = {}
    for Ls in sweep_L:
        gs = vs.capture(x_s, Ls, q_s, d_s, T, top_p, seed, step_dev)
        g1s = ar.capture(x1, Ls, None, None, T, top_p, seed, step1)
        Ks = max(10, K // 4)
        res_ms = []
        for g_, one in ((gs, False), (g1s, True)):
            for i in range(3):
                g_.replay()
            torch.cuda.synchronize()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record()
            for i in range(Ks):
                j = i % npool
                if one:
                    x1.copy_(xs[j][:1])
                else:
                    stage.load(j)
                g_.replay()
            c1.record()
            torch.cuda.synchronize()
            res_ms.append(c0.elapsed_time(c1) / Ks)
        sb = dec.weight_bytes() + dec.kv_bytes(Ls, M)
        ctx_sweep[Ls] = {"ms_per_step": round(res_ms[0], 4), "steps_per_s": round(1e3 / res_ms[0], 2),
                         "m1_ar_step_ms": round(res_ms[1], 4), "verify_over_ar": round(res_ms[0] / res_ms[1], 4),
                         "step_hbm_gbs": round(sb / (res_ms[0] * 1e-3) / 1e9, 1)}
        log(f"context {Ls}: {ctx_sweep[Ls]}")
        del gs, g1s
    nacc = nacc_all.cpu().numpy()
    flags = flag_all.cpu().numpy()
    shapes = dict(dec.shapes)
    shapes["lm_head"] = (V, d)
    linears = {}
    for nm in by_name:
        N, Kd = shapes[nm]
        b = N * Kd * bpw + M * Kd * 2 + (M * (N // 2) * 2 if nm == "gate_up" else M * N * 4)
        us = time_graphs([lambda nm=nm: dec.gemm_pass(M, names=(nm,))], 20 if nm != "lm_head" else 200)[0] * 1e3
        linears[nm] = {"N": N, "K": Kd, "avg_us": round(us, 2), "GBs": round(b / (us * 1e-6) / 1e9, 1),
                       "frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    # (f) the decode attention (tile kernel + merge) by itself, one call per
    # layer over that layer's cache, captured as a graph and replayed, at each
    # context of the workload: K and V of L + M positions read once
    attention = {}
    nq, nkv, hd = 40, 8, 128
    for Ls in sorted(set([L] + sweep_L)):

        def attn_pass(Ls=Ls):
            for li in range(cfg["layers"]):
                B.decode_attn(dec.q, dec.Kc[li], dec.Vc[li], dec.Lmax, Ls, M, nq, nkv, hd, dec.attn, dec.attn_ws)
            return cfg["layers"]

        us = time_graphs([attn_pass], 10)[0] * 1e3
        kv = 2 * nkv * (Ls + M) * hd * 2
        attention[Ls] = {"us_per_layer": round(us, 2), "kv_bytes": kv, "GBs": round(kv / (us * 1e-6) / 1e9, 1),
                         "frac": round(kv / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    res = dict(
        ms_per_step=step_ms,
        value=K / (total_ms * 1e-3),
        wall_s=wall,
        attention_by_context=attention,
        config={"workload": "verify27b", "layers": 64, "d_model": d, "heads_q_kv_dim": [40, 8, 128],
                "ffn": cfg["F"], "V": V, "context": L, "M": M, "draft_depth": D, "temperature": T, "top_p": top_p,
                "weights": WEIGHT_DESC[fmt],
                "kv_cache": "bf16"},
        roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(achieved / HBM_PEAK_GBS, 4),
                  "traffic": measured_traffic("verify27b") if fmt == "w4" else None,
                  "kernel": f"{fmt}_gemm_kernel (the 257 {fmt.upper()} GEMM launches of a step at M=4, replayed "
                            "as a graph)",
                  "alg_bytes_per_launch": int(per_launch_bytes), "avg_launch_us": round(gemm_launch_us, 2)},
        stages_us={"w4_gemm_total_eager": round(gemm_ms * 1e3 / K, 1),
                   "w4_gemm_total_graph": round(gemm_launch_us * n_launch, 1),
                   "eager_step": round(eager_ms * 1e3, 1),
                   "rest_of_eager_step": round(eager_ms * 1e3 - gemm_ms * 1e3 / K, 1)},
        m1_ar_step_ms=round(ar_ms, 4),
        verify_over_ar=round(step_ms / ar_ms, 4),
        step_hbm_gbs=round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
        accepted_length_hist=np.bincount(np.clip(nacc, 0, D), minlength=D + 1).tolist(),
        flagged_steps=int(((flags & ~B.FLAG_NONFINITE) != 0).sum()),
        context_sweep=ctx_sweep,
    )
    res[f"{fmt}_gemm_by_linear"] = linears
    if sustained is not None:
        res["sustained"] = sustained
    return res


def tokens_per_cycle(alpha: float, D: int) -> float:
    """Expected tokens a cycle emits when each of the D drafts is accepted
    with probability alpha independently (Leviathan, Kalman, Matias, ICML
    2023): the accepted prefix plus the corrected or bonus token,
    (1 - alpha^(D+1)) / (1 - alpha)."""
    return D + 1.0 if alpha >= 1.0 else (1.0 - alpha ** (D + 1)) / (1.0 - alpha)


def spec_loop_workload(args):
    """The closed cycle on the 27B-shaped model: D drafts of the MTP head (one
    decoder layer + projection + the shared W4 LM head each), one verify pass
    over D + 1 rows, acceptance.  Each cycle (and the M = 1 AR step) is
    captured as a HIP graph at context L and replayed; acceptance is measured
    on an eager run of real cycles (random weights: the head's drafts are
    independent of the target, so few are accepted), and the tokens/s of each
    depth follow for per-draft acceptance rates alpha from
    E[tokens per cycle] = (1 - alpha^(D+1)) / (1 - alpha)."""
    import numpy as np
    import torch

    from verify_step_w4_amd import binding as B
    from verify_step_w4_amd.model import DENSE_27B, Decoder, DepthTuner, MTPHead, SpecLoop, W4Linear

    cfg = dict(DENSE_27B)
    L = args.context
    T, top_p, seed = 0.6, 0.95, 0x5EED0008
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261208)
    V, d = cfg["V"], cfg["d"]
    fmt = args.weights
    log(f"generating the 64-layer {fmt.upper()} decoder, the MTP head and a {V} x {d} bf16 embedding table; "
        f"context {L}")
    dec = Decoder(cfg, 4, L + 72, gen=gen, fmt=fmt)
    E = torch.randn((V, d), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
    # a target in another format drafts with a draft-only W4 LM head (the
    # pages' design); its shared-head cost is timed too
    draft_lm = W4Linear.random(V, d, 0.02, gen) if fmt != "w4" else None
    head = MTPHead(dec, E, gen=gen, lm_head=draft_lm)
    torch.cuda.synchronize()
    K, W = max(10, args.steps // 4), max(3, args.warmup // 4)

    def time_graph(g, reps):
        for _ in range(W):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    depths = {}
    step_dev = torch.zeros(1, dtype=torch.int64, device=dev)
    for D in (1, 2, 3):
        loop = SpecLoop(dec, head, D)
        loop.start(L - 1, 123, T, top_p, seed, 0)
        g_cycle = loop.capture(lambda: loop.run_graphable(T, top_p, seed, step_dev))
        g_draft = loop.capture(lambda: loop.draft(T, top_p, seed, step_dev))
        t_cycle, t_draft = time_graph(g_cycle, K), time_graph(g_draft, K)
        depths[D] = {"cycle_ms": round(t_cycle, 4), "draft_ms": round(t_draft, 4),
                     "verify_ms": round(t_cycle - t_draft, 4), "draft_ms_per_depth": round(t_draft / D, 4)}
        log(f"D={D}: {depths[D]}")
        del g_cycle, g_draft
    shared = None
    if draft_lm is not None:
        # the same drafts through the target's own (W8) LM head, for comparison
        head_shared = MTPHead(dec, E, gen=gen)
        loop_s = SpecLoop(dec, head_shared, 3)
        loop_s.start(L - 1, 123, T, top_p, seed, 0)
        t_s = time_graph(loop_s.capture(lambda: loop_s.draft(T, top_p, seed, step_dev)), K)
        shared = {"draft_ms_d3_shared_target_head": round(t_s, 4),
                  "draft_only_head_speedup": round(t_s / depths[3]["draft_ms"], 3)}
        log(f"drafts with the target's W8 head: {shared}")
        del loop_s, head_shared
    ar_loop = SpecLoop(dec, head, 1)
    ar_loop.start(L - 1, 123, T, top_p, seed, 0)

    def ar_step():
        B.embed_rows(E, ar_loop.tokens_in, 1, ar_loop.x)
        ar_loop.ar_vs.run_graphable(ar_loop.x, ar_loop.L, None, None, T, top_p, seed, step_dev)

    t_ar = time_graph(ar_loop.capture(ar_step), K)
    # real cycles, eagerly launched (one host sync per cycle for n_acc)
    D = 3
    loop = SpecLoop(dec, head, D)
    emitted = [loop.start(L - 1, 123, T, top_p, seed, 0)]
    ncyc = 8
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    acc = []
    for c in range(ncyc):
        out = loop.cycle(T, top_p, seed, c + 1)
        acc.append(len(out) - 1)
        emitted += out
    eager_s = (time.perf_counter() - t0) / ncyc
    alpha_meas = float(np.mean(acc)) / D

    # the draft-depth autotune: every depth and the AR step measured on the
    # device (graph-timed cycles, real cycles for the yield), the best locked
    tuner = DepthTuner(dec, head, (1, 2, 3))
    tune = tuner.tune(L - 1, 123, T, top_p, seed, cycles=8, reps=K)
    autotune = {"pick": tune["pick"], "tokens_per_s": {k: round(v, 2) for k, v in tune["tokens_per_s"].items()},
                "ms": {k: round(v, 4) for k, v in tune["ms"].items()},
                "tokens_per_cycle": {k: round(v, 4) for k, v in tune["tokens_per_cycle"].items()}}
    log(f"autotune: {autotune}")
    # the same rule on modelled yields, for acceptance rates the random head cannot reach
    model = {}
    for a in (round(alpha_meas, 4), 0.5, 0.6, 0.7, 0.8, 0.9):
        tps = {0: 1e3 / t_ar}
        for D_, r in depths.items():
            tps[D_] = tokens_per_cycle(a, D_) * 1e3 / r["cycle_ms"]
        pick = DepthTuner.choose(tps)
        model[str(a)] = {"tokens_per_s": {("ar" if k == 0 else f"D{k}"): round(v, 2) for k, v in tps.items()},
                         "autotune_pick": "ar" if pick == 0 else f"D{pick}"}
    # the dominant kernel: the W4 GEMM launches of the verify pass at M = 4
    ms_launch, n_launch = time_graphs([lambda: dec.gemm_pass(4)], 10)
    per_launch = dec.gemm_alg_bytes(4) / n_launch
    achieved = per_launch / (ms_launch * 1e-3) / 1e9
    t3 = depths[3]["cycle_ms"]
    return dict(
        ms_per_step=t3,
        value=1e3 / t3,
        unit="spec cycles/s",
        config={"workload": "spec_loop_27b", "layers": 64, "d_model": d, "V": V, "context": L, "draft_depth": 3,
                "weights": fmt, "draft_lm_head": "w4 (draft-only)" if draft_lm is not None else "shared",
                "mtp_head": "rmsnorm(h) | rmsnorm(embed) -> W4 2d->d -> 1 decoder layer -> final norm -> W4 LM head",
                "temperature": T, "top_p": top_p},
        roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(achieved / HBM_PEAK_GBS, 4),
                  "traffic": measured_traffic("verify27b") if fmt == "w4" else None,
                  "kernel": f"{fmt}_gemm_kernel (the GEMM launches of the verify pass at M=4, replayed as a graph)",
                  "alg_bytes_per_launch": int(per_launch), "avg_launch_us": round(ms_launch * 1e3, 2)},
        spec_loop={"by_depth": depths, "m1_ar_step_ms": round(t_ar, 4), "eager_cycle_ms": round(eager_s * 1e3, 2),
                   "measured_accepted_per_cycle": acc, "measured_alpha": round(alpha_meas, 4),
                   "autotune": autotune, "tokens_per_s_by_alpha": model, "draft_only_head": shared},
    )


def verify27b_cpu_baseline_layer(reps=8):
    """The CPU oracle on the four linears of one layer at M=4 (fp64), reps row sets."""
    import oracle
    from verify_step_w4_amd import synth
    g = synth.rng(synth.SEED_BASE + 2)
    tot = 0.0
    for N, K in [(7168, 5120), (5120, 5120), (34816, 5120), (5120, 17408)]:
        codes, scales = oracle.w4_quantize(synth.normal_f32(g, (N, K), 0.02))
        for r in range(reps):
            x = synth.f32_to_bf16_bits(synth.normal_f32(g, (4, K), 1.0))
            t0 = time.perf_counter()
            oracle.w4_gemm(x, codes, scales)
            tot += time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(reps / tot, 4), "unit": "layer passes/s", "cores": cores, "kind": "oracle",
            "sample": f"one 27B-class layer's four W4 GEMMs at M=4 on {reps} row sets; quantisation untimed"}


def layer_linears_w8_cpu_baseline(reps=4, fmt="w8"):
    """The CPU oracle's W8 (or W6, W5, W3, W2) GEMM on the four linears of one layer at M=4 (fp64), reps row sets."""
    import oracle
    from verify_step_w4_amd import synth
    if fmt in ("f16", "bf16"):
        return layer_linears_w16_cpu_baseline(fmt, reps)
    quant, gemm = {"w8": (oracle.w8_quantize, oracle.w8_gemm), "w6": (oracle.w6_quantize, oracle.w6_gemm),
                   "w5": (oracle.w5_quantize, oracle.w5_gemm), "w3": (oracle.w3_quantize, oracle.w3_gemm),
                   "w2": (oracle.w2_quantize, oracle.w2_gemm)}[fmt]
    g = synth.rng(synth.SEED_BASE + 9)
    tot = 0.0
    for N, K in [(7168, 5120), (5120, 5120), (34816, 5120), (5120, 17408)]:
        codes, scales = quant(synth.normal_f32(g, (N, K), 0.02))
        for r in range(reps):
            x = synth.f32_to_bf16_bits(synth.normal_f32(g, (4, K), 1.0))
            t0 = time.perf_counter()
            gemm(x, codes, scales)
            tot += time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(reps / tot, 4), "unit": "layer passes/s", "cores": cores, "kind": "oracle",
            "sample": f"one 27B-class layer's four {fmt.upper()} GEMMs at M=4 on {reps} row sets; "
                      "quantisation untimed"}


def layer_linears_w16_cpu_baseline(fmt, reps=4):
    """The CPU oracle's fp16 (or bf16) weight GEMM on the four linears of one layer at M=4 (fp64)."""
    import numpy as np

    import oracle
    from verify_step_w4_amd import synth
    g = synth.rng(synth.SEED_BASE + 9)
    tot = 0.0
    for N, K in [(7168, 5120), (5120, 5120), (34816, 5120), (5120, 17408)]:
        w = synth.normal_f32(g, (N, K), 0.02)
        bits = w.astype(np.float16).view(np.uint16) if fmt == "f16" else synth.f32_to_bf16_bits(w)
        for r in range(reps):
            x = synth.f32_to_bf16_bits(synth.normal_f32(g, (4, K), 1.0))
            t0 = time.perf_counter()
            (oracle.f16_gemm if fmt == "f16" else oracle.b16_gemm)(x, bits)
            tot += time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(reps / tot, 4), "unit": "layer passes/s", "cores": cores, "kind": "oracle",
            "sample": f"one 27B-class layer's four {fmt.upper()}-weight GEMMs at M=4 on {reps} row sets"}


def verify27b_cpu_baseline(context=8192, M=4):
    """The CPU oracle on the whole verify step, sampled by layer count only:
    one decoder layer at the 27B-class shapes composed as the oracle forward
    of the tests (RMSNorm, W4 qkv GEMM, RoPE of q and the new k, KV append,
    GQA attention of the M rows over `context` positions, W4 o GEMM, residual
    add, RMSNorm, W4 gate|up GEMM, SwiGLU, W4 down GEMM, residual add, with the
    bf16 rounding after each op), timed once and scaled to 64 layers; then the
    final RMSNorm, the whole LM head [151936][5120], the temperature / top-p
    statistics of the M rows and the acceptance of 3 drafts, timed once.  The
    weight codes and fp16 scales are random (the oracle's arithmetic costs the
    same for any values), so no quantiser runs."""
    import numpy as np

    import oracle
    from verify_step_w4_amd import synth
    g = np.random.default_rng(synth.SEED_BASE + 4)
    d, nq, nkv, hd, F, V = 5120, 40, 8, 128, 17408, 151936
    L = context

    def lin(N, K):
        codes = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
        scales = (np.float16(2.0 ** -9) * (1 + g.random((N, K // 64)))).astype(np.float16).view(np.uint16)
        return codes, scales

    W = {"qkv": lin((nq + 2 * nkv) * hd, d), "o": lin(d, nq * hd), "gate_up": lin(2 * F, d), "down": lin(d, F)}
    lm = lin(V, d)
    gam = synth.f32_to_bf16_bits(1 + 0.02 * g.standard_normal(d).astype(np.float32))
    Kc = synth.f32_to_bf16_bits(g.standard_normal((nkv, L + M, hd)).astype(np.float32))
    Vc = synth.f32_to_bf16_bits(g.standard_normal((nkv, L + M, hd)).astype(np.float32))
    x = synth.f32_to_bf16_bits(g.standard_normal((M, d)).astype(np.float32))
    q_d, drafts = synth.q_and_drafts(synth.SEED_BASE + 5, M - 1, V, 3.0, B=1)

    t0 = time.perf_counter()
    resid = x
    h = oracle.bf16_round(oracle.rmsnorm(resid, gam))
    qkv = oracle.w4_gemm(h, *W["qkv"])
    q = np.zeros((M, nq, hd))
    for m in range(M):
        for hh in range(nq):
            q[m, hh] = oracle.bf16_value(oracle.bf16_round(oracle.rope(qkv[m, hh * hd:(hh + 1) * hd], L + m)))
        for hh in range(nkv):
            Kc[hh, L + m] = oracle.bf16_round(oracle.rope(qkv[m, (nq + hh) * hd:(nq + hh + 1) * hd], L + m))
            Vc[hh, L + m] = oracle.bf16_round(qkv[m, (nq + nkv + hh) * hd:(nq + nkv + hh + 1) * hd])
    att = oracle.bf16_round(oracle.decode_attn(q, Kc, Vc, L).reshape(M, nq * hd))
    resid = oracle.bf16_round(oracle.bf16_value(resid) + oracle.w4_gemm(att, *W["o"]))
    h = oracle.bf16_round(oracle.rmsnorm(resid, gam))
    gu = oracle.w4_gemm(h, *W["gate_up"])
    a = oracle.bf16_round(oracle.swiglu(gu[:, :F], gu[:, F:]))
    resid = oracle.bf16_round(oracle.bf16_value(resid) + oracle.w4_gemm(a, *W["down"]))
    t_layer = time.perf_counter() - t0

    t0 = time.perf_counter()
    h = oracle.bf16_round(oracle.rmsnorm(resid, gam))
    z = oracle.w4_gemm(h, *lm).astype(np.float32)
    oracle.spec_accept(z, q_d, drafts[0], 0.6, 0.95, 0x5EED0004, 0)
    t_head = time.perf_counter() - t0
    step_s = 64 * t_layer + t_head
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(1.0 / step_s, 5), "unit": "verify steps/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole verify step at context {L}, M={M}: one full decoder layer (norms, W4 GEMMs, "
                      f"RoPE + KV append, attention over {L} positions, SwiGLU, residual adds) timed once "
                      f"({t_layer:.2f} s) and scaled to 64 layers (the only extrapolation), plus the final norm, "
                      f"the whole 151936 x 5120 LM head, statistics and acceptance timed once ({t_head:.2f} s); "
                      f"random weight codes, no quantiser"}

# --------------------------------------------------------------------------
# MoE-shaped verify step
# --------------------------------------------------------------------------
def moe_workload(args):
    import numpy as np
    import torch

    from verify_step_w4_amd import binding as B
    from verify_step_w4_amd.model import BYTES_PER_WEIGHT, MOE_30B, ExpertBank, MoEVerify, W4Linear

    cfg = dict(MOE_30B)
    E, topk, d, F, V = (cfg[k] for k in ("n_exp", "topk", "d", "F", "V"))
    M, D = 4, 3
    T, top_p, seed = 0.6, 0.95, 0x5EED0005
    nrot = 4                      # expert banks and LM heads rotated: 4 x 486 MB working set
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261205)
    log(f"generating {nrot} expert banks ({E} x SwiGLU {d}->{F}->{d}) and {nrot} LM heads [{V}][{d}], W4")
    banks = [ExpertBank.random(E, d, F, 0.02, gen) for _ in range(nrot)]
    heads = [W4Linear.random(V, d, 0.02, gen) for _ in range(nrot)]
    gamma = (1 + 0.02 * torch.randn(d, generator=gen, device=dev)).to(torch.bfloat16).view(torch.int16)
    mvs = [MoEVerify(cfg, M, heads[k], gamma) for k in range(nrot)]
    ar = [MoEVerify(cfg, 1, heads[k], gamma) for k in range(nrot)]
    K, W = args.steps, args.warmup
    npool = 8
    router = torch.randn((K + W, M, E), generator=gen, device=dev, dtype=torch.float32)   # fresh per step
    xs = torch.randn((npool, M, d), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
    qs = torch.softmax(torch.randn((npool, D, V), generator=gen, device=dev, dtype=torch.float64) * 3.0,
                       dim=-1).to(torch.float32)
    drafts = torch.multinomial(qs.reshape(-1, V).double(), 1, generator=gen).reshape(npool, D).to(torch.int32)
    torch.cuda.synchronize()
    ev = {"gate_up": [], "down": [], "lm_head": []}
    cur = {}

    def hook(when, name):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        if when == "pre":
            cur[name] = e
        else:
            ev[name].append((cur[name], e))

    # (a) eager pass with the W4 GEMM launches bracketed by events
    nsl_eager = torch.empty(K, dtype=torch.int32, device=dev)
    for i in range(W):
        k, j = i % nrot, i % npool
        mvs[k].run(xs[j], router[i], banks[k], qs[j], drafts[j], T, top_p, seed, i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        k, j = i % nrot, i % npool
        mvs[k].run(xs[j], router[W + i], banks[k], qs[j], drafts[j], T, top_p, seed, i, gemm_hook=hook)
        nsl_eager[i:i + 1].copy_(mvs[k].n_slots)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / K
    t_us = {nm: np.array([a.elapsed_time(b) for a, b in v]) * 1e3 for nm, v in ev.items()}
    nsl = nsl_eager.cpu().numpy().astype(np.float64)
    eb_gu = 2 * F * d * BYTES_PER_WEIGHT
    eb_dn = d * F * BYTES_PER_WEIGHT
    gu_bytes = nsl * eb_gu + M * d * 2 + nsl * M * F * 2
    dn_bytes = nsl * eb_dn + nsl * M * F * 2 + nsl * M * d * 4
    lm_bytes = V * d * BYTES_PER_WEIGHT + M * d * 2 + M * V * 4
    grouped = float((gu_bytes + dn_bytes).sum() / ((t_us["gate_up"] + t_us["down"]).sum() * 1e-6) / 1e9)
    # (b) timed region: one graph per (bank, LM head) pair, replayed in turn;
    # each replay is preceded by one copy of the step's inputs (packed: rows,
    # router logits, q, drafts) into the captured buffers
    stage = InputStage([("x", (M, d), torch.int16), ("lg", (M, E), torch.float32), ("q", (D, V), torch.float32),
                        ("d", (D,), torch.int32)], K)
    for i in range(K):
        j = i % npool
        stage.slot(i, "x").copy_(xs[j])
        stage.slot(i, "lg").copy_(router[W + i])
        stage.slot(i, "q").copy_(qs[j])
        stage.slot(i, "d").copy_(drafts[j])
    stage.stage.zero_()
    stage.view("x").copy_(xs[0])
    stage.view("lg").copy_(router[0])
    stage.view("q").copy_(qs[0])
    stage.view("d").copy_(drafts[0])
    x_s, lg_s, q_s, d_s = stage.view("x"), stage.view("lg"), stage.view("q"), stage.view("d")
    step_dev = torch.zeros(1, dtype=torch.int64, device=dev)
    graphs = [mvs[k].capture(x_s, lg_s, banks[k], q_s, d_s, T, top_p, seed, step_dev) for k in range(nrot)]
    for i in range(W):
        graphs[i % nrot].replay()
    step_dev.zero_()
    out_all = torch.empty((K, M + 3), dtype=torch.int32, device=dev)   # tokens, n_acc, flags, experts per step
    nacc_all, flag_all, nsl_all = out_all[:, M], out_all[:, M + 1], out_all[:, M + 2]
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(K):
        k = i % nrot
        stage.load(i)
        graphs[k].replay()
        out_all[i].copy_(mvs[k].outputs)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    step_ms = total_ms / K
    # (c) the M = 1 step (one row, D = 0) on the same weights, same way
    stage1 = InputStage([("x", (1, d), torch.int16), ("lg", (1, E), torch.float32)], K)
    for i in range(K):
        stage1.slot(i, "x").copy_(xs[i % npool][:1])
        stage1.slot(i, "lg").copy_(router[W + i][:1])
    stage1.load(0)
    x1, lg1 = stage1.view("x"), stage1.view("lg")
    step1 = torch.zeros(1, dtype=torch.int64, device=dev)
    g1 = [ar[k].capture(x1, lg1, banks[k], None, None, T, top_p, seed, step1) for k in range(nrot)]
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for i in range(K):
        stage1.load(i)
        g1[i % nrot].replay()
    a1.record()
    torch.cuda.synchronize()
    ar_ms = a0.elapsed_time(a1) / K
    # (d) the W4 GEMM kernel by itself: each bank's 3 GEMM launches on its
    # last routing, banks in turn, four rounds, captured as one graph (so that
    # the per-replay cost of a graph is spread over many launches) and replayed
    def gemm_rounds(rounds=4):
        return sum(mvs[k].gemm_pass(banks[k]) for _ in range(rounds) for k in range(nrot))

    ms_launch, n_launch = time_graphs([gemm_rounds], 12)
    n_launch //= 4
    ns_last = np.array([int(mv.n_slots.item()) for mv in mvs], dtype=np.float64)
    pass_bytes = float((ns_last * (eb_gu + eb_dn + M * F * 2 + M * F * 2 + M * d * 4)).sum()
                       + nrot * (M * d * 2 + lm_bytes))
    per_launch_bytes = pass_bytes / n_launch
    achieved = per_launch_bytes / (ms_launch * 1e-3) / 1e9
    nacc = nacc_all.cpu().numpy()
    flags = flag_all.cpu().numpy()
    ns = nsl_all.cpu().numpy()
    step_bytes = float(np.mean(ns)) * 3 * d * F * BYTES_PER_WEIGHT + V * d * BYTES_PER_WEIGHT
    return dict(
        ms_per_step=step_ms,
        value=K / (total_ms * 1e-3),
        wall_s=wall,
        config={"workload": "moe_verify", "experts": E, "top_k": topk, "d_model": d, "expert_ffn": F, "V": V,
                "M": M, "draft_depth": D, "temperature": T, "top_p": top_p,
                "weights": "int4 group-64 symmetric, fp16 scales", "rotated_banks": nrot},
        roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic("moe_verify"),
                  "kernel": "w4_gemm_kernel (grouped gate|up + SwiGLU, grouped down, LM head: the 3 W4 GEMM launches "
                            "of a step, replayed as graphs)",
                  "alg_bytes_per_launch": int(per_launch_bytes),
                  "avg_launch_us": round(ms_launch * 1e3, 2)},
        grouped_gemm_gbs=round(grouped, 1),
        experts_per_step={"mean": round(float(np.mean(ns)), 2), "min": int(ns.min()), "max": int(ns.max())},
        stages_us={"grouped_gate_up": round(float(t_us["gate_up"].mean()), 2),
                   "grouped_down": round(float(t_us["down"].mean()), 2),
                   "lm_head": round(float(t_us["lm_head"].mean()), 2),
                   "eager_step": round(eager_ms * 1e3, 1)},
        m1_ar_step_ms=round(ar_ms, 4),
        verify_over_ar=round(step_ms / ar_ms, 4),
        step_hbm_gbs=round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
        accepted_length_hist=np.bincount(np.clip(nacc, 0, D), minlength=D + 1).tolist(),
        flagged_steps=int(((flags & ~B.FLAG_NONFINITE) != 0).sum()),
    )


def moe_cpu_baseline(nsteps=4):
    """The CPU oracle on a bounded sample: nsteps whole MoE verify steps
    (routing, the chosen experts expert by expert in fp64, the full LM head,
    sorted-vocab top-p and the scalar accept loop).  Weight generation and
    quantisation are untimed; only the experts a step routes to are built
    (the router logits are restricted to them, which leaves the choice and the
    renormalised weights unchanged)."""
    import numpy as np

    import oracle
    from verify_step_w4_amd import synth
    E, topk, d, F, V, M, D = 128, 8, 2048, 768, 151936, 4, 3
    g = synth.rng(synth.SEED_BASE + 5)
    lm = oracle.w4_quantize(synth.normal_f32(g, (V, d), 0.02))
    gamma = synth.f32_to_bf16_bits(1 + synth.normal_f32(g, (d,), 0.02))
    q, drafts = synth.q_and_drafts(synth.SEED_BASE + 55, D, V, 3.0, B=nsteps)
    dt = 0.0
    for s in range(nsteps):
        x = synth.f32_to_bf16_bits(synth.normal_f32(g, (M, d), 1.0))
        lg = synth.normal_f32(g, (M, E), 1.0)
        chosen = np.unique(oracle.moe_route(lg, topk)[0])
        mask = np.full((M, E), -np.inf, dtype=np.float32)
        for m, row in enumerate(oracle.moe_route(lg, topk)[0]):
            mask[m, row] = lg[m, row]
        sub = np.ascontiguousarray(mask[:, chosen])
        gu = [oracle.w4_quantize(synth.normal_f32(g, (2 * F, d), 0.02)) for _ in chosen]
        dn = [oracle.w4_quantize(synth.normal_f32(g, (d, F), 0.02)) for _ in chosen]
        st = lambda L: (np.stack([a for a, _ in L]), np.stack([b for _, b in L]))
        t0 = time.perf_counter()
        _, _, y = oracle.moe_block(x, sub, topk, st(gu), st(dn))
        resid = oracle.bf16_round(synth.bf16_bits_to_f32(x).astype(np.float64) + y)
        h = oracle.bf16_round(oracle.rmsnorm(resid, gamma, 1e-6))
        z = oracle.w4_gemm(h, *lm).astype(np.float32)
        oracle.spec_accept(z, q, drafts[s], 0.6, 0.95, 0x5EED0005, s)
        dt += time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(nsteps / dt, 4), "unit": "verify steps/s", "cores": cores, "kind": "oracle",
            "sample": f"{nsteps} whole MoE verify steps (128 experts top-8, d=2048, FFN 768, V=151936, M=4); "
                      "weight generation and quantisation untimed"}


# --------------------------------------------------------------------------
# One 27B-class decoder layer's linears, M swept
# --------------------------------------------------------------------------
def layer_linears_workload(args):
    """The fused qkv [7168][5120], o [5120][5120], gate|up [34816][5120] (SwiGLU
    epilogue) and down [5120][17408] W4 GEMMs of one layer; 8 layers' weights
    rotated (1.4 GB).  A step is one pass over a layer's four linears at M=4;
    the M sweep times the same passes at M = 1, 2, 3, 4, 6."""
    import numpy as np
    import torch

    from verify_step_w4_amd import binding as B
    from verify_step_w4_amd.model import BYTES_PER_WEIGHT, W4Linear

    d, F, nqkv = 5120, 17408, 7168
    nlay = 8
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261202)
    log(f"generating {nlay} layers of W4 linears (175.5 MB each)")
    layers = [dict(qkv=W4Linear.random(nqkv, d, 0.02, gen), o=W4Linear.random(d, d, 0.02, gen),
                   gate_up=W4Linear.random(2 * F, d, 0.02, gen), down=W4Linear.random(d, F, 0.02, gen))
              for _ in range(nlay)]
    Mmax = 6
    xs = {K: torch.randn((Mmax, K), generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
          for K in (d, F)}
    parts = {nm: torch.empty(8 * Mmax * (N + 64), dtype=torch.float32, device="cuda")
             for nm, N in (("qkv", nqkv), ("o", d), ("down", d))}
    a = torch.empty((Mmax, F), dtype=torch.int16, device="cuda")
    shapes = {"qkv": (nqkv, d), "o": (d, d), "gate_up": (2 * F, d), "down": (d, F)}

    def issue(M, names=("qkv", "o", "gate_up", "down")):
        n = 0
        for L in layers:
            for nm in names:
                N, K = shapes[nm]
                if nm == "gate_up":
                    B.w4_skinny_gemm_swiglu(xs[K][:M], L[nm].packed, L[nm].pscales, a, F, M, F, K)
                else:
                    B.w4_skinny_gemm_partials(xs[K][:M], L[nm].packed, L[nm].pscales, parts[nm], M, N, K)
                n += 1
        return n

    def alg(M, nm):
        N, K = shapes[nm]
        out = M * (N // 2) * 2 if nm == "gate_up" else M * N * 4
        return N * K * BYTES_PER_WEIGHT + M * K * 2 + out

    reps = max(1, args.steps // nlay)
    sweep = {}
    for M in (1, 2, 3, 4, 6):
        ms_launch, n_launch = time_graphs([lambda M=M: issue(M)], reps)
        per_layer_us = ms_launch * 1e3 * 4
        layer_bytes = sum(alg(M, nm) for nm in shapes)
        sweep[M] = {"layer_us": round(per_layer_us, 2),
                    "layer_GBs": round(layer_bytes / (per_layer_us * 1e-6) / 1e9, 1)}
        for nm in shapes:
            us = time_graphs([lambda M=M, nm=nm: issue(M, (nm,))], reps)[0] * 1e3
            sweep[M][nm + "_GBs"] = round(alg(M, nm) / (us * 1e-6) / 1e9, 1)
        log(f"M={M}: {sweep[M]}")
    s4 = sweep[4]
    ms4 = s4["layer_us"] * 1e-3
    layer_bytes4 = sum(alg(4, nm) for nm in shapes)
    return dict(
        ms_per_step=ms4,
        value=1.0 / (ms4 * 1e-3),
        config={"workload": "layer_linears", "d_model": d, "qkv": [nqkv, d], "o": [d, d], "gate_up": [2 * F, d],
                "down": [d, F], "M": 4, "rotated_layers": nlay,
                "weights": "int4 group-64 symmetric, fp16 scales"},
        roofline={"bound": "hbm", "achieved": round(layer_bytes4 / 4 / (ms4 / 4 * 1e-3) / 1e9, 1),
                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(layer_bytes4 / (ms4 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                  "kernel": "w4_gemm_kernel (the four linears of a layer at M=4, replayed as a graph)",
                  "alg_bytes_per_launch": int(layer_bytes4 / 4), "avg_launch_us": round(s4["layer_us"] / 4, 2)},
        m_sweep=sweep,
        unit_note="value = layer passes (four W4 GEMM launches) per second at M=4",
    )


def layer_linears_w6_workload(args):
    return layer_linears_w8_workload(args, fmt="w6")


def layer_linears_w5_workload(args):
    return layer_linears_w8_workload(args, fmt="w5")


def layer_linears_w3_workload(args):
    return layer_linears_w8_workload(args, fmt="w3")


def layer_linears_w2_workload(args):
    return layer_linears_w8_workload(args, fmt="w2")


def layer_linears_f16_workload(args):
    return layer_linears_w8_workload(args, fmt="f16")


def layer_linears_bf16_workload(args):
    return layer_linears_w8_workload(args, fmt="bf16")


def layer_linears_w8_workload(args, fmt="w8"):
    """The same four linears of one 27B-shaped layer in the W8 format (int8
    codes, fp16 scale per 64 K: 1.03125 bytes per weight, 351 MB per layer),
    or the W6 (0.78125 bytes per weight), W5 (0.65625), W3 (0.40625) or W2
    (0.28125) format, or unquantised fp16 / bf16 (2 bytes, no scales; 2
    layers rotated, 1.5 GB); plain GEMM
    outputs (gate|up as one [34816][5120] product); 4 layers' weights rotated.
    A step is one pass over a layer's four linears at M = 4."""
    import torch

    from verify_step_w4_amd import binding as B
    from verify_step_w4_amd.model import W2Linear, W3Linear, W5Linear, W6Linear, W8Linear, W16Linear

    d, F, nqkv = 5120, 17408, 7168
    w16 = fmt in ("f16", "bf16")
    nlay = 2 if w16 else 4
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261209)
    shapes = {"qkv": (nqkv, d), "o": (d, d), "gate_up": (2 * F, d), "down": (d, F)}
    Lin = {"w8": W8Linear, "w6": W6Linear, "w5": W5Linear, "w3": W3Linear, "w2": W2Linear}.get(fmt)
    code_bytes = {"w8": 1.0, "w6": 0.75, "w5": 0.625, "w3": 0.375, "w2": 0.25, "f16": 2.0, "bf16": 2.0}[fmt]
    two_plane = {"w8": B.w8_skinny_gemm, "w6": B.w6_skinny_gemm, "w5": B.w5_skinny_gemm, "w3": B.w3_skinny_gemm}

    def gemm(x, L, y, M, N, K, ws):
        if w16:
            B.w16_skinny_gemm(x, L.packed, y, M, N, K, kind=fmt, ws=ws)
        elif fmt == "w2":
            B.w2_skinny_gemm(x, L.packed, L.pscales, y, M, N, K, ws=ws)
        else:
            two_plane[fmt](x, L.hi, L.lo, L.pscales, y, M, N, K, ws=ws)
    wsb = {"w8": B.w8_workspace_bytes, "w6": B.w6_workspace_bytes, "w5": B.w5_workspace_bytes,
           "w3": B.w3_workspace_bytes, "w2": B.w2_workspace_bytes,
           "f16": lambda M, N, K: B.w16_workspace_bytes(M, N, K, "f16"),
           "bf16": lambda M, N, K: B.w16_workspace_bytes(M, N, K, "bf16")}[fmt]
    log(f"generating {nlay} layers of {fmt.upper()} linears")
    mk = (lambda N, K: W16Linear.random(N, K, gen, fmt)) if w16 else (lambda N, K: Lin.random(N, K, gen))
    layers = [{nm: mk(N, K) for nm, (N, K) in shapes.items()} for _ in range(nlay)]
    M = 4
    xs = {K: torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16) for K in (d, F)}
    ys = {nm: torch.empty((M, N), dtype=torch.float32, device="cuda") for nm, (N, K) in shapes.items()}
    ws = {nm: B.workspace(max(wsb(M, N, K), 256)) for nm, (N, K) in shapes.items()}

    def issue(names=tuple(shapes)):
        n = 0
        for L in layers:
            for nm in names:
                N, K = shapes[nm]
                gemm(xs[K], L[nm], ys[nm], M, N, K, ws[nm])
                n += 1
        return n

    def alg(nm):
        N, K = shapes[nm]
        return int(N * K * code_bytes) + (0 if w16 else N * (K // 64) * 2) + M * K * 2 + M * N * 4

    reps = max(1, args.steps // nlay)
    ms_launch, n_launch = time_graphs([issue], reps)
    layer_us = ms_launch * 1e3 * 4
    per = {}
    for nm in shapes:
        us = time_graphs([lambda nm=nm: issue((nm,))], reps)[0] * 1e3
        per[nm] = {"avg_us": round(us, 2), "GBs": round(alg(nm) / (us * 1e-6) / 1e9, 1),
                   "frac": round(alg(nm) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    log(f"{fmt.upper()} layer {layer_us:.2f} us: {per}")
    lb = sum(alg(nm) for nm in shapes)
    return dict(
        ms_per_step=layer_us * 1e-3,
        value=1.0 / (layer_us * 1e-6),
        unit="layer passes/s",
        config={"workload": f"layer_linears_{fmt}", "d_model": d, "qkv": [nqkv, d], "o": [d, d], "gate_up": [2 * F, d],
                "down": [d, F], "M": M, "rotated_layers": nlay,
                "weights": {"w8": "int8 group-64 symmetric, fp16 scales (two nibble planes)",
                            "w6": "6-bit group-64 symmetric, fp16 scales (2-bit + 4-bit planes)",
                            "w5": "5-bit group-64 symmetric, fp16 scales (1-bit + 4-bit planes)",
                            "w3": "3-bit group-64 symmetric, fp16 scales (1-bit + 2-bit planes)",
                            "w2": "2-bit group-64 symmetric (codes -1..1), fp16 scales (one 2-bit plane)",
                            "f16": "fp16, unquantised (exact two-part bf16 split on the matrix cores)",
                            "bf16": "bf16, unquantised"}[fmt]},
        roofline={"bound": "hbm", "achieved": round(lb / (layer_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                  "unit": "GB/s", "frac": round(lb / (layer_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                  "kernel": f"{fmt}_gemm_kernel (+ {fmt}_reduce_kernel; the four linears of a layer at M=4, "
                            "graph-replayed)",
                  "alg_bytes_per_launch": int(lb / 4), "avg_launch_us": round(layer_us / 4, 2)},
        **{f"{fmt}_gemm_by_linear": per},
    )


# --------------------------------------------------------------------------
# Single small LM-head verify step (d=1024, V=8192)
# --------------------------------------------------------------------------
def lm_small_workload(args):
    """x [4][1024] -> W4 LM head [8192][1024] -> temperature 0.6 / top_p 0.95
    statistics -> acceptance of 3 drafts from q = softmax(N(0, 2)); 240 copies
    of the 4.46 MB head rotated (1.07 GB), one copy per step."""
    import numpy as np
    import torch

    from verify_step_w4_amd import binding as B
    from verify_step_w4_amd.model import BYTES_PER_WEIGHT, LMHeadVerify, W4Linear

    V, d, M, D = 8192, 1024, 4, 3
    T, top_p, seed = 0.6, 0.95, 0x5EED0001
    ncopy = 240
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261201)
    log(f"generating {ncopy} W4 LM heads [{V}][{d}]")
    heads = [W4Linear.random(V, d, 0.02, gen) for _ in range(ncopy)]
    npool = 64
    xs = torch.randn((npool, M, d), generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
    qs = torch.softmax(torch.randn((npool, D, V), generator=gen, device="cuda", dtype=torch.float64) * 2.0,
                       dim=-1).to(torch.float32)
    drafts = torch.multinomial(qs.reshape(-1, V).double(), 1, generator=gen).reshape(npool, D).to(torch.int32)
    vs = LMHeadVerify(V, d, M)
    step_dev = torch.zeros(1, dtype=torch.int64, device="cuda")

    def issue_step(k):
        j = k % npool
        vs.gemm(xs[j], heads[k % ncopy])
        B.verify_logits(None, None, None, M, V, d, T, top_p, vs.logits, vs.stats, vs.stat_ws)
        B.spec_accept_ex(vs.logits, 0, vs.stats, 0, qs[j], 0, drafts[j], 1, D, V, T, seed, step_dev, vs.tokens,
                         vs.n_acc, vs.flags, vs.acc_ws)
        B.step_advance(step_dev, 1)

    # one graph per group of 240 steps (all copies once), replayed
    ms_step, n = time_graphs([lambda: [issue_step(k) for k in range(ncopy)] and ncopy], max(1, args.steps // ncopy))
    gemm_ms, _ = time_graphs([lambda: [vs.gemm(xs[k % npool], heads[k]) for k in range(ncopy)] and ncopy], 2)
    alg = V * d * BYTES_PER_WEIGHT + M * d * 2 + M * V * 4
    return dict(
        ms_per_step=ms_step,
        value=1.0 / (ms_step * 1e-3),
        config={"workload": "lm_small", "d": d, "V": V, "M": M, "draft_depth": D, "temperature": T, "top_p": top_p,
                "weights": "int4 group-64 symmetric, fp16 scales", "lm_head_copies": ncopy},
        roofline={"bound": "hbm", "achieved": round(alg / (gemm_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                  "unit": "GB/s", "frac": round(alg / (gemm_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                  "kernel": "w4_gemm_kernel (M=4, 4.46 MB head: launch-latency bound)",
                  "alg_bytes_per_launch": int(alg), "avg_launch_us": round(gemm_ms * 1e3, 2)},
        stages_us={"w4_gemm": round(gemm_ms * 1e3, 2), "stats_and_accept": round((ms_step - gemm_ms) * 1e3, 2)},
    )


def lm_small_cpu_baseline(nsteps=200):
    """The CPU oracle on nsteps whole small LM-head verify steps."""
    import oracle
    from verify_step_w4_amd import synth
    V, d, D = 8192, 1024, 3
    g = synth.rng(synth.SEED_BASE + 1)
    codes, scales = oracle.w4_quantize(synth.normal_f32(g, (V, d), 0.02))
    q, drafts = synth.q_and_drafts(synth.SEED_BASE + 11, D, V, 2.0, B=nsteps)
    xs = [synth.f32_to_bf16_bits(synth.normal_f32(g, (D + 1, d), 1.0)) for _ in range(nsteps)]
    t0 = time.perf_counter()
    for s in range(nsteps):
        z = oracle.w4_gemm(xs[s], codes, scales).astype("float32")
        oracle.spec_accept(z, q, drafts[s], 0.6, 0.95, 0x5EED0001, s)
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(nsteps / dt, 3), "unit": "verify steps/s", "cores": cores, "kind": "oracle",
            "sample": f"{nsteps} whole small LM-head verify steps (d=1024, V=8192, M=4)"}


def oracle_one_core(fn_name, **kw):
    """Run the CPU-oracle baseline `fn_name(**kw)` of this file in a child
    process limited to one host thread (OMP_NUM_THREADS=1); the child touches
    no GPU.  Returns its result, or a note of why there is none."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    code = f"import json, bench; print(json.dumps(bench.{fn_name}(**{kw!r})))"
    try:
        r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=600)
        return json.loads(r.stdout.strip().splitlines()[-1])
    except Exception as e:
        return {"unavailable": f"{type(e).__name__}: {e}"}


WORKLOADS = {"lm_head_verify": (lm_head_workload, lm_head_cpu_baseline),
             "verify27b": (verify27b_workload, lambda: verify27b_cpu_baseline()),
             "moe_verify": (moe_workload, moe_cpu_baseline),
             "layer_linears": (layer_linears_workload, lambda: verify27b_cpu_baseline_layer()),
             "lm_small": (lm_small_workload, lm_small_cpu_baseline),
             "spec_loop_27b": (spec_loop_workload, lambda: verify27b_cpu_baseline()),
             "layer_linears_w8": (layer_linears_w8_workload, lambda: layer_linears_w8_cpu_baseline()),
             "layer_linears_w6": (layer_linears_w6_workload, lambda: layer_linears_w8_cpu_baseline(fmt="w6")),
             "layer_linears_w5": (layer_linears_w5_workload, lambda: layer_linears_w8_cpu_baseline(fmt="w5")),
             "layer_linears_w3": (layer_linears_w3_workload, lambda: layer_linears_w8_cpu_baseline(fmt="w3")),
             "layer_linears_w2": (layer_linears_w2_workload, lambda: layer_linears_w8_cpu_baseline(fmt="w2")),
             "layer_linears_f16": (layer_linears_f16_workload, lambda: layer_linears_w8_cpu_baseline(fmt="f16")),
             "layer_linears_bf16": (layer_linears_bf16_workload, lambda: layer_linears_w8_cpu_baseline(fmt="bf16"))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="verify27b", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--weights", default="w4", choices=WEIGHT_FORMATS,
                    help="verify27b: weight format of the decoder's linears and LM head")
    ap.add_argument("--context", type=int, default=8192, help="KV context length L of the verify27b workload")
    ap.add_argument("--no-context-sweep", action="store_true",
                    help="verify27b: skip the extra timings at the other context lengths (1024, 8192, 32768)")
    ap.add_argument("--sustain", type=float, default=10.0,
                    help="verify27b: seconds of back-to-back steps sampled for the step-time spread and the GPU's "
                         "clocks / temperatures / power (0 = skip)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    run, cpu = WORKLOADS[args.workload]
    # A plain copy kernel of known size (256 MiB read, 256 MiB written), run
    # once before the workload: HBM byte counters read in the same process
    # are calibrated against it.
    src = torch.ones(CALIB_COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    res = run(args)
    ceil, ceil_blocks = read_ceiling_gbs()
    log(f"streaming-read ceiling: {ceil:.0f} GB/s ({ceil_blocks} workgroups of 256)")
    if res.get("roofline") and res["roofline"].get("unit") == "GB/s":
        res["roofline"]["measured_ceiling_gbs"] = round(ceil, 1)
        res["roofline"]["frac_of_ceiling"] = round(res["roofline"]["achieved"] / ceil, 4)
    out = {"metric": METRIC, "value": round(res["value"], 3),
           "unit": res.get("unit", "layer passes/s" if args.workload == "layer_linears" else "verify steps/s"),
           "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": res["config"], "roofline": res["roofline"]}
    for k in ("stages_us", "w4_gemm_by_linear", "accepted_length_hist", "flagged_steps", "m1_ar_step_ms",
              "verify_over_ar", "step_hbm_gbs", "experts_per_step", "grouped_gemm_gbs", "m_sweep", "unit_note",
              "context_sweep", "stats_accept_sweep", "sustained", "attention_by_context", "spec_loop",
              "w8_gemm_by_linear", "w6_gemm_by_linear", "w5_gemm_by_linear", "w3_gemm_by_linear",
              "w2_gemm_by_linear", "f16_gemm_by_linear", "bf16_gemm_by_linear"):
        if k in res:
            out[k] = res[k]
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = verify27b_cpu_baseline(context=args.context) if args.workload == "verify27b" else cpu()
        if args.workload == "verify27b":
            log("timing the CPU oracle on one host thread")
            one = oracle_one_core("verify27b_cpu_baseline", context=args.context)
            out["cpu_baseline"]["one_core"] = {k: one[k] for k in ("value", "cores", "sample", "unavailable")
                                               if k in one}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
