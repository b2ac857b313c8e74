"""Pins of the oracle's Leviathan–Chen accept / residual-resample loop (a6/a7).

* Special cases with a forced answer: q <= p (always accept), T = 0 (argmax),
  q(x) > 0 = p(x) (certain rejection), one-hot q, D = 0 (plain sampling).
* Decision boundaries driven by chosen uniforms: accept iff u < p/q; the
  residual sampler maps the middle of each CDF interval to its token.
* The exact law in rational arithmetic: the procedure's output law equals p
  ("max_diff = 0.0" in the numbers table of hazakura.dev's mtplx page).
* Pearson chi-square of 1e6 oracle trials on the V=16 LM-head recipe, per
  position, conditional on reaching it; tokens outside top-p never appear.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.stats

import oracle
from oracle import exact_law
from verify_step_w4_amd import synth


def _stats(z, T, top_p):
    return [oracle.warp(z[i], T, top_p) for i in range(z.shape[0])]


def _p_rows(z, T, top_p):
    return np.stack([oracle.warp(z[i], T, top_p, want_p=True)[1] for i in range(z.shape[0])])


def test_q_below_p_always_accepts():
    z = synth.synthetic_logits(10, 4, 64, 1.0)
    T, top_p = 1.0, 1.0
    p = _p_rows(z, T, top_p)
    q = (p[:3] * (1 - 1e-6)).astype(np.float32)        # q <= p everywhere
    for step in range(200):
        dr = np.array([step % 64, (7 * step) % 64, (13 * step) % 64], dtype=np.int32)
        tok, nacc, fl = oracle.spec_accept(z, q, dr, T, top_p, 99, step)[:3]
        assert nacc == 3 and list(tok[:3]) == list(dr)
        assert 0 <= tok[3] < 64


def test_greedy_emits_argmax():
    z = synth.synthetic_logits(11, 4, 100, 1.0)
    q, drafts = synth.q_and_drafts(12, 3, 100, 2.0, B=300)
    am = np.argmax(z, axis=1)
    drafts[:100, 0] = am[0]
    drafts[:50, 1] = am[1]
    for b in range(300):
        tok, nacc, fl = oracle.spec_accept(z, q, drafts[b], 0.0, 0.95, 5, b)[:3]
        lead = 0
        while lead < 3 and drafts[b, lead] == am[lead]:
            lead += 1
        assert nacc == lead
        assert list(tok[:nacc + 1]) == list(am[:nacc + 1])


def test_draft_outside_top_p_is_rejected():
    z = synth.synthetic_logits(13, 2, 200, 1.0)
    st0, p0 = oracle.warp(z[0], 0.6, 0.5, want_p=True)
    outside = int(np.nonzero(p0 == 0)[0][0])
    q = np.full((1, 200), 1.0 / 200, dtype=np.float32)
    for step in range(100):
        tok, nacc, fl = oracle.spec_accept(z, q, np.array([outside], np.int32), 0.6, 0.5, 1, step)[:3]
        assert nacc == 0 and p0[tok[0]] > 0


def test_one_hot_q_residual_excludes_draft():
    z = synth.synthetic_logits(14, 2, 32, 0.5)
    p0 = _p_rows(z, 1.0, 1.0)[0]
    x = int(np.argmax(p0))
    q = np.zeros((1, 32), dtype=np.float32)
    q[0, x] = 1.0
    rejected = 0
    for step in range(400):
        tok, nacc, fl = oracle.spec_accept(z, q, np.array([x], np.int32), 1.0, 1.0, 2, step)[:3]
        if nacc == 0:
            rejected += 1
            assert tok[0] != x
    assert rejected > 0


def test_accept_decision_boundary():
    z = synth.synthetic_logits(15, 2, 16, 1.0)
    st = _stats(z, 1.0, 1.0)
    p = _p_rows(z, 1.0, 1.0)
    q = np.full((1, 16), 1.0 / 16, dtype=np.float32)
    for x in range(16):
        ratio = p[0, x] / np.float64(q[0, x])
        if ratio >= 1.0:
            continue
        below = np.nextafter(ratio, 0) * (1 - 1e-12)
        above = ratio * (1 + 1e-12)
        ur = np.array([0.5, 0.5])
        t1, n1, _ = oracle.accept_with_uniforms(z, st, q, [x], 1.0, np.array([below, 0.5]), ur)
        t2, n2, _ = oracle.accept_with_uniforms(z, st, q, [x], 1.0, np.array([above, 0.5]), ur)
        assert n1 == 1 and t1[0] == x
        assert n2 == 0


@pytest.mark.parametrize("D", [0, 1])
def test_residual_sampler_interval_midpoints(D):
    V = 24
    z = synth.synthetic_logits(16, D + 1, V, 1.0)
    T, top_p = 0.8, 0.9
    st = _stats(z, T, top_p)
    p = _p_rows(z, T, top_p)
    if D:
        q = synth.softmax_f32(synth.synthetic_logits(17, 1, V, 2.0))
        x = int(np.argmax(q[0] - p[0]))                 # q(x) > p(x): force rejection via u ~ 1
        r = np.maximum(0.0, p[0] - q[0].astype(np.float64))
        ua = np.array([1.0 - 2.0 ** -53, 0.5])
    else:
        q = np.zeros((1, V), dtype=np.float32)
        x = 0
        r = p[0]
        ua = np.array([0.5])
    C = np.cumsum(r)
    R = C[-1]
    for v in range(V):
        if r[v] <= 0:
            continue
        lo = C[v - 1] if v else 0.0
        mid = (lo + C[v]) / 2 / R
        ur = np.array([mid] * (D + 1))
        tok, nacc, fl = oracle.accept_with_uniforms(z, st, q, [x] if D else [], T, ua, ur)
        assert nacc == 0 and tok[0] == v


def test_exact_law_small_rationals():
    g = np.random.default_rng(21)
    for trial in range(300):
        V = int(g.integers(1, 7))
        pn = g.integers(0, 6, V)
        qn = g.integers(0, 6, V)
        if pn.sum() == 0:
            pn[0] = 1
        if qn.sum() == 0:
            qn[-1] = 1
        p = [Fraction(int(a), int(pn.sum())) for a in pn]
        q = [Fraction(int(a), int(qn.sum())) for a in qn]
        law = exact_law.law_first_token(p, q)
        assert exact_law.max_diff(law, p) == 0


def test_exact_law_lm_head_tiny_vocab():
    prob = synth.lm_verify_problem(synth.LM_TINY, synth.SEED_BASE + 1)
    codes, scales = oracle.w4_quantize(prob["w"])
    z = oracle.w4_gemm(prob["x"], codes, scales).astype(np.float32)
    for i in range(3):
        _, p = oracle.warp(z[i], 0.6, 0.95, want_p=True)
        pf = exact_law.to_fractions(p)
        qf = exact_law.to_fractions(prob["q"][i])
        assert exact_law.max_diff(exact_law.law_first_token(pf, qf), pf) == 0


@pytest.mark.slow
def test_oracle_distribution_chi_square_tiny_vocab():
    """1e6 accept/resample trials at V=16, T=0.6, top_p=0.95."""
    B = 1_000_000
    prob = synth.lm_verify_problem(synth.LM_TINY, synth.SEED_BASE + 1, B=B)
    codes, scales = oracle.w4_quantize(prob["w"])
    z = oracle.w4_gemm(prob["x"], codes, scales).astype(np.float32)
    T, top_p = 0.6, 0.95
    tok, nacc, fl = oracle.spec_accept_trials(z, prob["q"], prob["drafts"], T, top_p,
                                              synth.PHILOX_SEED_BASE + 1, 0)
    assert np.all(nacc >= 0)
    p = _p_rows(z, T, top_p)
    for i in range(4):
        reached = nacc >= i
        obs = np.bincount(tok[reached, i], minlength=16).astype(np.float64)
        support = p[i] > 0
        assert obs[~support].sum() == 0, "token outside the top-p set emitted"
        n = obs.sum()
        assert n > 1000
        exp = p[i][support] * n
        res = scipy.stats.chisquare(obs[support], exp)
        assert res.pvalue > 1e-4 / 4, (i, res)
