"""GPU parity of the temperature/top-p statistics (a4) and of spec_accept
(a5-a7) against the oracle, stage-isolated: both sides read the same
synthetic fp32 logits, q and drafts.  Integer results (argmax, n_kept,
accepted counts, tokens) must agree exactly outside flagged near-ties."""
import numpy as np
import pytest

import oracle
from verify_step_w4_amd import binding as B
from verify_step_w4_amd import synth

from helpers import GEMM_RTOL, dev, gemm_rel_err, host, log

pytestmark = pytest.mark.gpu


def gpu_stats(z: np.ndarray, T: float, top_p: float):
    import torch
    rows, V = z.shape
    zd = dev(np.ascontiguousarray(z, dtype=np.float32))
    st = torch.zeros(rows * 32, dtype=torch.uint8, device="cuda")
    ws = B.workspace(B.verify_workspace_bytes(rows, V))
    B.verify_logits(None, None, None, rows, V, 64, T, top_p, zd, st, ws)
    torch.cuda.synchronize()
    return B.rowstats_to_numpy(st), zd, st


def check_stats(z, T, top_p):
    s, _, _ = gpu_stats(z, T, top_p)
    flagged = 0
    for r in range(z.shape[0]):
        o = oracle.warp(z[r], T, top_p)
        g = s[r]
        assert int(g["argmax"]) == o.argmax
        assert float(g["max_logit"]) == o.m
        if (g["flags"] & B.FLAG_TOPP_TIE) or (o.flags & 2):
            flagged += 1
            continue
        assert int(g["n_kept"]) == o.n_kept, (r, int(g["n_kept"]), o.n_kept)
        assert float(g["tau"]) == o.tau
        assert abs(float(g["log_z"]) - o.log_z) <= 1e-12 * max(1.0, abs(o.log_z))
    return flagged


@pytest.mark.parametrize("V", [1, 16, 1000, 8192, 16384, 16385, 151936])
@pytest.mark.parametrize("T,top_p", [(0.0, 0.95), (0.6, 0.95), (1.0, 0.95), (0.6, 1.0), (1.0, 0.5)])
def test_stats_match_oracle(V, T, top_p):
    log(f"stats V={V} T={T} top_p={top_p}")
    z = synth.synthetic_logits(V + int(100 * T), 4, V, 3.0)
    flagged = check_stats(z, T, top_p)
    assert flagged <= 1


def test_stats_ties_and_signed_zero():
    V = 5000
    z = synth.synthetic_logits(77, 4, V, 1.0)
    z[0, :] = np.round(z[0, :] * 4) / 4          # heavy ties everywhere
    z[1, ::2] = 0.0
    z[1, 1::2] = -0.0                              # signed zeros share one key
    z[2, 10] = z[2, 20] = z[2].max() + 1            # tied maximum
    z[3, :] = 0.5                                   # constant row
    log("stats ties")
    for T, p in ((0.6, 0.95), (1.0, 0.5), (0.0, 0.9)):
        check_stats(z, T, p)


def test_stats_crowded_cutoff_bin():
    """Level 3 publishes a chunk's non-empty bins of the cutoff's 22-bit key
    prefix as a record of at most 59 entries, and its dense counts when it
    has more.  Here the cutoff falls among up to 1024 consecutive floats just
    above 1.0 (one prefix, every one its own bin); row 0 has chunks with 600
    and 384 of them (dense) and one with 40 (record), row 1 50 per chunk in
    9 chunks (records only), row 2 one chunk with 60 (dense) and one with
    exactly 59 (record).  The other logits are -30, far below the cutoff."""
    V = 40000                                       # chunked path: 10 chunks of 4096
    rng = np.random.default_rng(31)
    near = (np.float32(1.0) + np.arange(1024, dtype=np.float32) * np.float32(2.0 ** -23)).astype(np.float32)
    z = np.full((3, V), -30.0, dtype=np.float32)
    pos0 = np.concatenate([rng.choice(4096, 600, replace=False), 4096 + rng.choice(4096, 40, replace=False),
                           5 * 4096 + rng.choice(4096, 384, replace=False)])
    z[0, pos0] = rng.permutation(near)
    pos1 = np.concatenate([c * 4096 + rng.choice(4096, 50, replace=False) for c in range(9)])
    z[1, pos1] = rng.permutation(near)[:450]
    pos2 = np.concatenate([2 * 4096 + rng.choice(4096, 60, replace=False),
                           7 * 4096 + rng.choice(4096, 59, replace=False)])
    z[2, pos2] = rng.permutation(near)[:119]
    log("stats crowded cutoff bin")
    for T, p in ((0.6, 0.95), (1.0, 0.5)):
        for r in range(3):                          # the construction puts tau among the crowded values
            assert near[0] <= oracle.warp(z[r], T, p).tau <= near[-1]
        assert check_stats(z, T, p) == 0


def test_stats_flag_non_finite():
    z = synth.synthetic_logits(5, 2, 300, 1.0)
    z[1, 7] = np.inf
    log("stats non-finite")
    s, _, _ = gpu_stats(z, 0.6, 0.95)
    assert s[1]["flags"] & B.FLAG_NONFINITE
    assert not (s[0]["flags"] & B.FLAG_NONFINITE)


def test_stats_deterministic():
    z = synth.synthetic_logits(9, 4, 151936, 3.0)
    log("stats determinism")
    a, _, _ = gpu_stats(z, 0.6, 0.95)
    b, _, _ = gpu_stats(z, 0.6, 0.95)
    assert a.tobytes() == b.tobytes()


def run_accept(z, q, drafts, T, top_p, seed, step0, shared=False):
    """GPU stats + spec_accept for B problems.  z: [B][M][V] (or [M][V] if shared)."""
    import torch
    if shared:
        M, V = z.shape
        Bn = drafts.shape[0]
        s, zd, st = gpu_stats(z, T, top_p)
        lstride = sstride = qstride = 0
        qd = dev(np.ascontiguousarray(q, dtype=np.float32)) if M > 1 else None
    else:
        Bn, M, V = z.shape
        zf = z.reshape(Bn * M, V)
        # statistics row by row in chunks of 64 rows (one call handles <= 64 rows)
        zd = dev(np.ascontiguousarray(zf, dtype=np.float32))
        st = torch.zeros(Bn * M * 32, dtype=torch.uint8, device="cuda")
        ws = B.workspace(B.verify_workspace_bytes(64, V))
        for r0 in range(0, Bn * M, 64):
            rows = min(64, Bn * M - r0)
            B.verify_logits(None, None, None, rows, V, 64, T, top_p, zd[r0:r0 + rows], st[r0 * 32:(r0 + rows) * 32],
                            ws)
        lstride, sstride, qstride = M * V, M, (M - 1) * V
        qd = dev(np.ascontiguousarray(q, dtype=np.float32)) if M > 1 else None
    D = M - 1
    dd = dev(np.ascontiguousarray(drafts, dtype=np.int32)) if D else None
    tok = torch.empty((Bn, M), dtype=torch.int32, device="cuda")
    nacc = torch.empty(Bn, dtype=torch.int32, device="cuda")
    fl = torch.empty(Bn, dtype=torch.int32, device="cuda")
    ws = B.workspace(B.accept_workspace_bytes(Bn, V))
    B.spec_accept(zd, lstride, st, sstride, qd, qstride, dd, Bn, D, V, T, seed, step0, tok, nacc, fl, ws)
    torch.cuda.synchronize()
    return host(tok), host(nacc), host(fl).view(np.uint32)


@pytest.mark.parametrize("V,D,T,top_p", [
    (16, 3, 0.6, 0.95), (1000, 3, 0.6, 0.95), (8192, 3, 0.6, 0.95), (8192, 1, 1.0, 1.0),
    (8192, 3, 0.0, 0.95), (151936, 3, 0.6, 0.95), (151936, 3, 1.0, 0.95), (151936, 0, 0.6, 0.95),
    (5000, 7, 1.0, 0.95), (151936, 3, 0.0, 0.95), (1000, 7, 0.0, 1.0), (16384, 3, 0.6, 0.95), (16385, 2, 1.0, 0.95),
])
def test_accept_matches_oracle(V, D, T, top_p):
    Bn = 48 if V > 10000 else 200
    log(f"accept V={V} D={D} T={T} top_p={top_p} B={Bn}")
    M = D + 1
    z = synth.synthetic_logits(V + D, Bn * M, V, 1.5).reshape(Bn, M, V)
    g = synth.rng(V * 7 + D)
    # q: softmax of draft logits; make some drafts agree with the target so
    # that all acceptance lengths occur
    ql = synth.normal_f32(g, (Bn, max(D, 1), V), 3.0)
    ql[: Bn // 2, :, :] = z[: Bn // 2, :max(D, 1), :] / np.float32(max(T, 0.6))
    q = synth.softmax_f32(ql)[:, :D, :] if D else np.zeros((Bn, 0, V), np.float32)
    drafts = np.stack([synth.sample_drafts(g, q[b], 1)[0] for b in range(Bn)]) if D else np.zeros((Bn, 0), np.int32)
    if T == 0.0 and D:
        # greedy targets: half of the problems draft the argmax, so that
        # acceptances occur whatever q is
        drafts[: Bn // 2] = np.argmax(z[: Bn // 2, :D, :], axis=2).astype(np.int32)
    seed, step0 = synth.PHILOX_SEED_BASE + 3, 1000
    tok, nacc, fl = run_accept(z, q, drafts, T, top_p, seed, step0)
    mism = flagged = 0
    ties = B.FLAG_TOPP_TIE | B.FLAG_ACCEPT_TIE | B.FLAG_CDF_TIE
    for b in range(Bn):
        ot, on, of = oracle.spec_accept(z[b], q[b] if D else np.zeros((0, V), np.float32),
                                        drafts[b] if D else np.zeros(0, np.int32), T, top_p, seed, step0 + b)[:3]
        if (of | int(fl[b])) & ties:
            flagged += 1
            continue
        # away from every threshold both sides raise the same flags (R = 0
        # fallback, non-finite input) and draw the same tokens
        assert int(fl[b]) == of, (b, int(fl[b]), of)
        assert int(nacc[b]) == on, (b, int(nacc[b]), on)
        if not np.array_equal(tok[b], ot):
            mism += 1
    assert mism == 0
    # near-ties are rare (the bands are 1e-5 for the accept test and 1e-9 of
    # the mass elsewhere): a flagging fault that skipped most problems would
    # leave the token check nearly empty
    assert flagged <= max(2, Bn // 20), (flagged, Bn)
    if D:
        assert len(set(nacc.tolist())) >= 2   # more than one acceptance length occurred


@pytest.mark.parametrize("V,D,T,top_p,case", [
    (151936, 3, 0.6, 0.95, "mixed"), (151936, 0, 0.6, 0.95, "mixed"), (20000, 2, 1.0, 1.0, "mixed"),
    (151936, 2, 1.0, 0.95, "r_zero"),
])
def test_accept_kept_masses_equal_recomputed(V, D, T, top_p, case):
    """Above 16384 entries, batches of at most 8 problems keep the chunk pass's
    residual masses for the sampling pass, larger batches recompute them: the
    same 24 problems as three batches of 8 and as one batch of 24 give the same
    tokens, counts and flags, and the kept form matches the oracle outside
    flagged near-ties.  "r_zero": q >= p on the rejected row, so R = 0 and the
    sampler falls back to p (the kept masses are not used there)."""
    Bn, M = 24, D + 1
    log(f"accept kept vs recomputed masses V={V} D={D} T={T} top_p={top_p} {case}")
    z = synth.synthetic_logits(V + 31 * D, Bn * M, V, 1.5).reshape(Bn, M, V)
    g = synth.rng(V * 11 + D)
    if case == "r_zero":
        # row 0: q slightly above p everywhere and the draft outside the top-p set
        # (p = 0 there, q > 0): certain rejection at k = 0 with R = 0
        q = np.zeros((Bn, D, V), np.float32)
        drafts = np.zeros((Bn, D), np.int32)
        for b in range(Bn):
            for i in range(D):
                _, pi = oracle.warp(z[b, i], T, top_p, want_p=True)
                q[b, i] = (pi * (1 + 1e-6)).astype(np.float32)
                out = np.flatnonzero(pi == 0.0)
                drafts[b, i] = int(out[b % len(out)])
                q[b, i, drafts[b, i]] = 1e-3
    else:
        ql = synth.normal_f32(g, (Bn, max(D, 1), V), 3.0)
        ql[: Bn // 2, :, :] = z[: Bn // 2, :max(D, 1), :] / np.float32(T)
        q = synth.softmax_f32(ql)[:, :D, :] if D else np.zeros((Bn, 0, V), np.float32)
        drafts = (np.stack([synth.sample_drafts(g, q[b], 1)[0] for b in range(Bn)]) if D
                  else np.zeros((Bn, 0), np.int32))
    seed, step0 = synth.PHILOX_SEED_BASE + 5, 77
    assert B.accept_workspace_bytes(8, V) > B.accept_workspace_bytes(9, V)    # the two layouts
    tok, nacc, fl = run_accept(z, q, drafts, T, top_p, seed, step0)
    parts = [run_accept(z[i:i + 8], q[i:i + 8], drafts[i:i + 8], T, top_p, seed, step0 + i) for i in range(0, Bn, 8)]
    assert np.array_equal(np.concatenate([p[0] for p in parts]), tok)
    assert np.array_equal(np.concatenate([p[1] for p in parts]), nacc)
    assert np.array_equal(np.concatenate([p[2] for p in parts]), fl)
    ties = B.FLAG_TOPP_TIE | B.FLAG_ACCEPT_TIE | B.FLAG_CDF_TIE
    flagged = 0
    for b in range(Bn):
        ot, on, of = oracle.spec_accept(z[b], q[b] if D else np.zeros((0, V), np.float32),
                                        drafts[b] if D else np.zeros(0, np.int32), T, top_p, seed, step0 + b)[:3]
        if (of | int(fl[b])) & ties:
            flagged += 1
            continue
        assert int(fl[b]) == of and int(nacc[b]) == on and np.array_equal(tok[b], ot), b
    assert flagged <= 2
    if case == "r_zero":
        assert np.all(nacc == 0) and np.all(fl & B.FLAG_R_ZERO)


@pytest.mark.parametrize("V", [1_000_000, 1 << 20])
def test_stats_and_accept_at_the_chunk_cap(V):
    """Vocabularies past 64 chunks of 4096: the chunks grow (15872 or 16384
    entries, 63 or 64 of them), so the statistics passes run several tiles per
    chunk and steer with the largest coarse and fine stagings, and the
    acceptance rescans multi-tile chunks (its masses recomputed).  Statistics
    and acceptance against the oracle, outside flagged near-ties."""
    log(f"stats + accept at V={V}")
    z = synth.synthetic_logits(V % 997 + 3, 4, V, 2.0)
    for T, top_p in ((0.6, 0.95), (1.0, 0.5), (0.6, 1.0)):
        assert check_stats(z, T, top_p) <= 1
    Bn, D, T, top_p = 3, 1, 0.6, 0.95
    zb = synth.synthetic_logits(V % 991 + 7, Bn * (D + 1), V, 2.0).reshape(Bn, D + 1, V)
    g = synth.rng(V % 983)
    ql = synth.normal_f32(g, (Bn, D, V), 3.0)
    ql[0] = zb[0, :D] / np.float32(T)           # one problem whose draft law is the target's
    q = synth.softmax_f32(ql)
    drafts = np.stack([synth.sample_drafts(g, q[b], 1)[0] for b in range(Bn)])
    seed, step0 = synth.PHILOX_SEED_BASE + 9, 31
    tok, nacc, fl = run_accept(zb, q, drafts, T, top_p, seed, step0)
    ties = B.FLAG_TOPP_TIE | B.FLAG_ACCEPT_TIE | B.FLAG_CDF_TIE
    checked = 0
    for b in range(Bn):
        ot, on, of = oracle.spec_accept(zb[b], q[b], drafts[b], T, top_p, seed, step0 + b)[:3]
        if (of | int(fl[b])) & ties:
            continue
        assert int(fl[b]) == of and int(nacc[b]) == on and np.array_equal(tok[b], ot), b
        checked += 1
    assert checked >= Bn - 1


def test_accept_special_cases():
    V, D = 2000, 3
    M = D + 1
    log("accept special cases")
    z = synth.synthetic_logits(3, M, V, 1.0)
    # q <= p everywhere: every draft is accepted
    _, p0 = oracle.warp(z[0], 1.0, 1.0, want_p=True)
    ps = np.stack([oracle.warp(z[i], 1.0, 1.0, want_p=True)[1] for i in range(D)])
    q = (ps * (1 - 1e-6)).astype(np.float32)
    g = synth.rng(4)
    drafts = np.stack([synth.sample_drafts(g, q, 1)[0] for _ in range(64)])
    tok, nacc, fl = run_accept(z, q, drafts, 1.0, 1.0, 7, 0, shared=True)
    assert np.all(nacc == D)
    assert np.array_equal(tok[:, :D], drafts)
    # greedy: tokens are the argmax of each row
    am = np.argmax(z, axis=1)
    drafts2 = np.tile(am[:D], (64, 1)).astype(np.int32)
    drafts2[32:, 1] = (am[1] + 1) % V
    qu = np.full((D, V), 1.0 / V, dtype=np.float32)
    tok, nacc, fl = run_accept(z, qu, drafts2, 0.0, 0.95, 7, 0, shared=True)
    assert np.all(nacc[:32] == D) and np.all(nacc[32:] == 1)
    assert np.all(tok[:32] == am) and np.all(tok[32:, :2] == am[:2])


def test_accept_greedy_residual_zero_and_cdf_ends():
    """T = 0 (one-hot targets): a rejected draft whose row's q puts all its mass
    on the argmax leaves R = 0, so the token falls back to the argmax with the
    R-zero flag; the same step without that q gives the argmax unflagged.
    Both against the oracle."""
    V, D = 64, 2
    M = D + 1
    z = synth.synthetic_logits(11, M, V, 1.0)
    am = np.argmax(z, axis=1)
    q = np.zeros((D, V), dtype=np.float32)
    q[0, am[0]] = 1.0
    q[1, am[1]] = 1.0                               # all of row 1's mass on its argmax
    drafts = np.tile(np.array([am[0], (am[1] + 5) % V], dtype=np.int32), (16, 1))
    tok, nacc, fl = run_accept(z, q, drafts, 0.0, 0.95, 21, 0, shared=True)
    assert np.all(nacc == 1)
    assert np.all(tok[:, 0] == am[0]) and np.all(tok[:, 1] == am[1]) and np.all(tok[:, 2] == -1)
    assert np.all(fl & B.FLAG_R_ZERO)
    qu = np.full((D, V), 1.0 / V, dtype=np.float32)
    tok2, nacc2, fl2 = run_accept(z, qu, drafts, 0.0, 0.95, 21, 0, shared=True)
    assert np.all(nacc2 == 1) and np.all(tok2[:, 1] == am[1])
    assert not np.any(fl2 & B.FLAG_R_ZERO)
    for b in range(16):
        otok, onacc, ofl, _ = oracle.spec_accept(z, q, drafts[b], 0.0, 0.95, 21, b)
        assert onacc == int(nacc[b]) and list(otok) == list(tok[b]) and ofl == int(fl[b])


def test_accept_non_finite_rows():
    V, D = 500, 2
    z = synth.synthetic_logits(8, 3, V, 1.0)
    z[1, 5] = np.nan
    q, drafts = synth.q_and_drafts(9, D, V, 2.0, B=8)
    log("accept non-finite")
    tok, nacc, fl = run_accept(z, q, drafts, 0.6, 0.95, 1, 0, shared=True)
    assert np.all(nacc == -1) and np.all(tok == -1) and np.all(fl & B.FLAG_NONFINITE)


@pytest.mark.slow
def test_tiny_vocab_distribution_1e6_trials():
    """V=16 LM-head recipe: 1e6 trials in one spec_accept call.  Trial-by-trial
    equality with the oracle on identical (synthetic-weight GEMM) logits, and
    a per-position chi-square of the GPU samples against p."""
    import scipy.stats
    import torch
    Bn = 1_000_000
    log("tiny-vocab 1e6 trials")
    prob = synth.lm_verify_problem(synth.LM_TINY, synth.SEED_BASE + 1, B=Bn)
    T, top_p = 0.6, 0.95
    # logits from the GPU LM head; the oracle computes its own and both must agree
    packed, pscales = B.w4_quantize_packed(dev(prob["w"]))
    z = torch.empty((4, 16), dtype=torch.float32, device="cuda")
    st = torch.zeros(4 * 32, dtype=torch.uint8, device="cuda")
    ws = B.workspace(B.verify_workspace_bytes(4, 16, 1024))
    B.verify_logits(dev(prob["x"]), packed, pscales, 4, 16, 1024, T, top_p, z, st, ws)
    torch.cuda.synchronize()
    oc, os_ = oracle.w4_quantize(prob["w"])
    z_or = oracle.w4_gemm(prob["x"], oc, os_)
    assert gemm_rel_err(host(z), z_or) <= GEMM_RTOL
    # stage-isolated trials on the oracle's own fp32 logits (same input both sides)
    zs = z_or.astype(np.float32)
    seed = synth.PHILOX_SEED_BASE + 1
    tok, nacc, fl = run_accept(zs, prob["q"], prob["drafts"], T, top_p, seed, 0, shared=True)
    otok, onacc, ofl = oracle.spec_accept_trials(zs, prob["q"], prob["drafts"], T, top_p, seed, 0)
    ok = ((ofl | fl) & (B.FLAG_TOPP_TIE | B.FLAG_ACCEPT_TIE | B.FLAG_CDF_TIE)) == 0
    assert ok.mean() > 0.99
    assert np.array_equal(nacc[ok], onacc[ok])
    assert np.array_equal(tok[ok], otok[ok])
    p = np.stack([oracle.warp(zs[i], T, top_p, want_p=True)[1] for i in range(4)])
    for i in range(4):
        reached = nacc >= i
        obs = np.bincount(tok[reached, i], minlength=16).astype(np.float64)
        sup = p[i] > 0
        assert obs[~sup].sum() == 0
        res = scipy.stats.chisquare(obs[sup], p[i][sup] * obs.sum())
        assert res.pvalue > 1e-4 / 4, (i, res)
