"""Pins of the oracle's temperature/top-p warp (a4) and Philox generator (a5).

Independent references: scipy's softmax (top_p = 1), numpy's argmax (T = 0),
a brute-force nucleus over all subsets of a tiny vocabulary (the textbook
definition: the smallest set of tokens whose probability reaches top_p), and
numpy's own Philox4x64-10 bit generator.
"""
import itertools

import numpy as np
import pytest
import scipy.special

import oracle
from verify_step_w4_amd import synth


@pytest.mark.parametrize("T", [0.6, 1.0, 2.5])
def test_warp_top_p_one_is_softmax(T):
    z = synth.synthetic_logits(1, 1, 4096, 1.5)[0]
    st, p = oracle.warp(z, T, 1.0, want_p=True)
    ref = scipy.special.softmax(z.astype(np.float64) / np.float64(np.float32(T)))
    np.testing.assert_allclose(p, ref, rtol=1e-12, atol=1e-300)
    assert st.n_kept == 4096 and st.flags == 0
    assert abs(p.sum() - 1.0) < 1e-12


def test_warp_greedy_is_argmax_lowest_index():
    z = synth.synthetic_logits(2, 1, 1000, 1.0)[0]
    z[[10, 500, 900]] = z.max() + 1.0          # three-way tie for the max
    st, p = oracle.warp(z, 0.0, 0.95, want_p=True)
    assert st.argmax == int(np.argmax(z)) == 10
    assert p[10] == 1.0 and p.sum() == 1.0


def test_warp_tiny_temperature_limit_is_argmax():
    z = (np.arange(50, dtype=np.float32) * 0.25)[::-1].copy()
    np.random.default_rng(0).shuffle(z)
    st, p = oracle.warp(z, 1e-4, 0.95, want_p=True)
    assert p[int(np.argmax(z))] == 1.0 and st.n_kept == 1


def _brute_force_nucleus(z, T, top_p):
    """Smallest set S (by size) with mass(S) >= top_p * E, choosing the
    heaviest set of that size; then widened by ties with its smallest logit."""
    e = np.exp((z.astype(np.float64) - z.max()) / np.float64(np.float32(T)))
    E = e.sum()
    P = np.float64(np.float32(top_p)) * E
    V = len(z)
    for k in range(1, V + 1):
        best, best_mass = None, -1.0
        for S in itertools.combinations(range(V), k):
            m = sum(e[list(S)])
            if m > best_mass:
                best, best_mass = S, m
        if best_mass >= P * (1 - 1e-12):
            tau = min(z[list(best)])
            return set(np.nonzero(z >= tau)[0].tolist())
    return set(range(V))


@pytest.mark.parametrize("seed", range(12))
def test_warp_top_p_matches_brute_force(seed):
    g = np.random.default_rng(seed)
    V = int(g.integers(2, 11))
    z = (g.standard_normal(V) * 2).astype(np.float32)
    if seed % 3 == 0:
        z[g.integers(0, V)] = z[g.integers(0, V)]     # a tie
    for top_p in (0.3, 0.8, 0.95):
        for T in (0.6, 1.0):
            st, p = oracle.warp(z, T, top_p, want_p=True)
            if st.flags & 2:
                continue                                # boundary near-tie: set not unique
            kept = set(np.nonzero(p > 0)[0].tolist())
            assert kept == _brute_force_nucleus(z, T, top_p), (z, T, top_p)


@pytest.mark.parametrize("T,top_p", [(0.6, 0.95), (1.0, 0.95), (0.6, 0.5)])
def test_warp_invariants_large(T, top_p):
    z = synth.synthetic_logits(3, 1, 151936, 3.0)[0]
    st, p = oracle.warp(z, T, top_p, want_p=True)
    e = np.exp((z.astype(np.float64) - z.max()) / np.float64(np.float32(T)))
    kept = p > 0
    assert kept.sum() == st.n_kept
    mass = e[kept].sum()
    Pt = np.float64(np.float32(top_p)) * e.sum()
    assert mass >= Pt * (1 - 1e-12)
    # dropping the cutoff logit's tokens leaves less than top_p
    assert e[z > st.tau].sum() < Pt * (1 + 1e-12)
    assert abs(p.sum() - 1.0) < 1e-12
    assert np.all(z[kept] >= st.tau) and np.all(z[~kept] < st.tau)


def test_warp_non_finite_flag():
    z = np.zeros(8, dtype=np.float32)
    z[3] = np.nan
    st = oracle.warp(z, 0.6, 0.95)
    assert st.flags & 1


# ------------------------------- Philox ----------------------------------
def _numpy_philox_block(key, ctr):
    """First block numpy's Philox(key, counter) emits.  numpy advances the
    counter by one before producing a block, so ask it for ctr - 1."""
    c = list(ctr)
    # subtract one with borrow across the 4 words
    for i in range(4):
        if c[i] > 0:
            c[i] -= 1
            break
        c[i] = 2 ** 64 - 1
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(c, dtype=np.uint64))
    return bg.random_raw(4)


@pytest.mark.parametrize("key,ctr", [
    ((0, 0), (0, 0, 0, 0)), ((5, 0), (7, 1, 0, 0)), ((0x5EED0001, 0), (123456789, 3, 0, 0)),
    ((2 ** 64 - 1, 2 ** 63), (2 ** 64 - 1, 2 ** 64 - 1, 5, 9)), ((1, 2), (0, 0, 0, 1)),
])
def test_philox_matches_numpy(key, ctr):
    ours = oracle.philox4x64_10(key, ctr)
    ref = _numpy_philox_block(key, ctr)
    assert [int(v) for v in ours] == [int(v) for v in ref]


def test_philox_counter_alignment_documented():
    # numpy's first block is produced from counter + 1 (pins which of the two
    # alignments numpy uses, so the comparison above is not vacuous)
    key, ctr = (9, 0), (40, 2, 0, 0)
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(ctr, dtype=np.uint64))
    first = [int(v) for v in bg.random_raw(4)]
    assert first == [int(v) for v in oracle.philox4x64_10(key, (41, 2, 0, 0))]
    assert first != [int(v) for v in oracle.philox4x64_10(key, ctr)]


def test_uniforms_range_and_uniformity():
    import scipy.stats
    us = []
    for step in range(4000):
        ua, ur = oracle.verify_uniforms(0x5EED0001, step, 3)
        us.extend(ua)
        us.extend(ur)
    us = np.array(us)
    assert us.min() >= 0.0 and us.max() < 1.0
    assert scipy.stats.kstest(us, "uniform").pvalue > 1e-4
    # 53-bit grid
    assert np.all((us * 2.0 ** 53) == np.floor(us * 2.0 ** 53))
