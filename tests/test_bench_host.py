"""Host logic of bench.py (no GPU): the packed per-step input buffer, the
telemetry summary and the lookup of the committed HBM-traffic figures."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_input_stage_layout_and_copy():
    import torch
    specs = [("x", (4, 5120), torch.int16), ("q", (3, 1001), torch.float32), ("d", (3,), torch.int32)]
    st = bench.InputStage(specs, npool=5, device="cpu")
    # 256-byte aligned offsets, in spec order, each region large enough
    offs = [st.offs[n][0] for n, _, _ in specs]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert offs[1] >= 4 * 5120 * 2 and offs[2] >= offs[1] + 3 * 1001 * 4
    assert st.nbytes % 256 == 0 and st.nbytes >= offs[2] + 12
    # views alias the staging bytes and have the requested shapes and types
    for name, shape, dt in specs:
        v = st.view(name)
        assert tuple(v.shape) == shape and v.dtype == dt
        assert v.data_ptr() == st.stage.data_ptr() + st.offs[name][0]
    # one load copies every input of a slot
    g = torch.Generator().manual_seed(3)
    for j in range(5):
        st.slot(j, "x").copy_(torch.randint(-2**15, 2**15, (4, 5120), generator=g, dtype=torch.int16))
        st.slot(j, "q").copy_(torch.rand((3, 1001), generator=g))
        st.slot(j, "d").copy_(torch.tensor([j, j + 1, j + 2], dtype=torch.int32))
    st.load(3)
    for name, _, _ in specs:
        assert torch.equal(st.view(name), st.slot(3, name))
    assert st.view("d").tolist() == [3, 4, 5]


def test_telemetry_summary_from_samples():
    t = bench.Telemetry.__new__(bench.Telemetry)
    t.period, t.error = 0.25, None
    t.samples = [{"gfxclk_mhz": 2400.0, "uclk_mhz": 2000.0, "hotspot_c": 50.0, "hbm_c": 48.0, "socket_power_w": p}
                 for p in (800.0, 900.0, 850.0)]
    t.first = {"accumulation_counter": 100, "ppt_residency_acc": 10, "socket_thm_residency_acc": 0}
    t.last = {"accumulation_counter": 300, "ppt_residency_acc": 60, "socket_thm_residency_acc": 0}
    s = t.summary()
    assert s["samples"] == 3 and s["socket_power_w"] == {"min": 800.0, "median": 850.0, "max": 900.0}
    assert s["gfxclk_mhz"]["median"] == 2400.0
    assert s["throttle_residency_frac"]["ppt"] == 0.25 and s["throttle_residency_frac"]["socket_thm"] == 0.0
    # a list-valued clock (one per partition) reads as its maximum; "N/A" as missing
    assert bench.Telemetry._num([2100, "N/A", 2390]) == 2390.0
    assert bench.Telemetry._num("N/A") is None
    empty = bench.Telemetry.__new__(bench.Telemetry)
    empty.samples, empty.error = [], "no device"
    assert empty.summary() == {"unavailable": "no device"}


def test_measured_traffic_follows_the_committed_digest():
    text = open(bench.TRAFFIC_FILE).read()
    import re
    m = re.search(r"^\| verify27b \| ([0-9]+) \| ([0-9]+) \| ([0-9]+) \|", text, re.M)
    assert m, "the traffic summary lists verify27b"
    # the reported figure is the per-launch total while the GEMM sources have
    # the digest the counters were taken with, and None otherwise
    import hashlib
    h = hashlib.sha256()
    for name in ("w4_gemm.hip", "skinny_gemm.h"):
        h.update(open(os.path.join(ROOT, "verify_step_w4_amd", "csrc", name), "rb").read())
    digest = h.hexdigest()
    recorded = re.search(r"W4 GEMM sources sha256 \(w4_gemm\.hip, then skinny_gemm\.h\): ([0-9a-f]{64})",
                         text).group(1)
    got = bench.measured_traffic("verify27b")
    assert got == (int(m.group(3)) if digest == recorded else None)
    assert bench.measured_traffic("no_such_workload") is None


@pytest.mark.parametrize("argv", [["--gpus", "2"]])
def test_more_than_one_gpu_is_refused(argv, monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py"] + argv)
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2


@pytest.mark.parametrize("D", [1, 2, 3, 7])
@pytest.mark.parametrize("alpha", [0.0, 0.3, 0.7, 0.95, 1.0])
def test_tokens_per_cycle_by_enumeration(alpha, D):
    # P(k drafts accepted) = alpha^k (1 - alpha) for k < D, alpha^D for k = D;
    # the cycle emits k + 1 tokens
    e = sum((k + 1) * alpha ** k * (1 - alpha) for k in range(D)) + (D + 1) * alpha ** D
    assert abs(bench.tokens_per_cycle(alpha, D) - e) < 1e-12


def test_depth_choice_rule():
    """The autotune's decision: the most tokens per second wins, AR (depth 0)
    is kept on ties and whenever no depth beats it."""
    from verify_step_w4_amd.model import DepthTuner
    assert DepthTuner.choose({0: 216.0, 1: 201.6, 2: 186.6, 3: 173.0}) == 0      # alpha ~ 0: AR
    assert DepthTuner.choose({0: 216.0, 1: 343.0, 2: 409.0, 3: 438.0}) == 3      # alpha 0.7
    assert DepthTuner.choose({0: 216.0, 1: 303.0, 2: 327.0, 3: 324.0}) == 2      # alpha 0.5
    assert DepthTuner.choose({0: 300.0, 1: 300.0, 2: 299.0}) == 0                # tie: the smaller depth
    assert DepthTuner.choose({0: 100.0, 2: 150.0, 3: 150.0}) == 2
