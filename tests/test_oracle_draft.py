"""Pins of the oracle's draft side (the MTP head's sampling and input; no GPU).

* The draft uniform is the Philox4x64-10 block numpy's generator gives for
  counter (step, depth, 1, 0), second word, 53 bits, and it is not the verify
  stream's uniform of the same step and row.
* A draft at T = 0 is the argmax (lowest index on ties) with a one-hot q.
* At top_p = 1 the draft is the inverse-CDF sample of scipy's softmax(z / T)
  at that uniform, and q is that softmax.
* At top_p < 1 every draw lies in the brute-force kept set and the draw
  frequencies follow q (Pearson chi-square).
* The projection input is scale-free in h and e separately, each half has
  unit mean square with unit gains and eps = 0, and the h half comes first.
* Embedding rows are the table rows of the ids, zero rows for ids outside
  [0, V).
"""
import numpy as np
import pytest

import oracle

SEED = 0x5EED0006


def _numpy_block(key, ctr):
    c = list(ctr)
    for i in range(4):          # numpy emits the block of counter + 1
        if c[i] > 0:
            c[i] -= 1
            break
        c[i] = 2 ** 64 - 1
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(c, dtype=np.uint64))
    return [int(v) for v in bg.random_raw(4)]


@pytest.mark.parametrize("seed,step,depth", [(SEED, 0, 0), (SEED, 17, 2), (1, 2 ** 40 + 3, 6), (2 ** 64 - 1, 5, 1)])
def test_draft_uniform_is_philox_stream_one(seed, step, depth):
    r1 = _numpy_block((seed, 0), (step, depth, 1, 0))[1]
    assert oracle.draft_uniform(seed, step, depth) == (r1 >> 11) * 2.0 ** -53
    # the verify stream (third counter word 0) gives a different number
    _, u_res = oracle.verify_uniforms(seed, step, depth)
    assert oracle.draft_uniform(seed, step, depth) != u_res[depth]


def test_draft_greedy_is_argmax_one_hot():
    z = np.array([0.5, 3.0, -1.0, 3.0, 2.0], dtype=np.float32)
    for step in range(5):
        tok, q, st, fl = oracle.draft_sample(z, 0.0, 0.95, SEED, step, 0)
        assert tok == 1 and fl == 0
        assert q.tolist() == [0.0, 1.0, 0.0, 0.0, 0.0]


@pytest.mark.parametrize("T", [0.6, 1.0])
def test_draft_top_p_one_is_inverse_cdf_of_softmax(T):
    import scipy.special
    rng = np.random.default_rng(31)
    V = 50
    z = rng.normal(0.0, 2.0, V).astype(np.float32)
    p = scipy.special.softmax(z.astype(np.float64) / T)
    cdf = np.cumsum(p)
    checked = 0
    for step in range(300):
        r1 = _numpy_block((SEED, 0), (step, 3, 1, 0))[1]
        u = (r1 >> 11) * 2.0 ** -53
        if np.min(np.abs(cdf - u)) < 1e-12:
            continue
        y_ref = int(np.argmax(cdf > u)) if u < cdf[-1] else V - 1
        tok, q, st, fl = oracle.draft_sample(z, T, 1.0, SEED, step, 3)
        assert tok == y_ref, step
        checked += 1
    assert checked > 290
    np.testing.assert_allclose(q.astype(np.float64), p, rtol=1e-6, atol=0)


def test_draft_top_p_support_and_frequencies():
    import scipy.stats
    rng = np.random.default_rng(32)
    V, T, top_p = 12, 0.6, 0.8
    z = rng.normal(0.0, 1.0, V).astype(np.float32)
    # brute-force kept set: smallest prefix of (z desc, index asc) reaching top_p of the mass
    e = np.exp((z.astype(np.float64) - z.max()) / T)
    order = sorted(range(V), key=lambda j: (-z[j], j))
    acc, kept = 0.0, []
    for j in order:
        kept.append(j)
        acc += e[j]
        if acc >= top_p * e.sum():
            break
    tau = z[kept[-1]]
    kept = {j for j in range(V) if z[j] >= tau}
    n = 20000
    counts = np.zeros(V)
    for step in range(n):
        tok, q, st, fl = oracle.draft_sample(z, T, top_p, SEED, step, 0)
        counts[tok] += 1
    assert set(np.nonzero(counts)[0].tolist()) <= kept
    assert set(np.nonzero(q)[0].tolist()) == kept
    idx = sorted(kept)
    pk = e[idx] / e[idx].sum()
    assert scipy.stats.chisquare(counts[idx], n * pk).pvalue > 1e-4


def _bf16_bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_mtp_input_properties():
    rng = np.random.default_rng(33)
    d = 256
    h = _bf16_bits(rng.normal(0.0, 3.0, d))
    e = _bf16_bits(rng.normal(0.0, 0.02, d))
    one = _bf16_bits(np.ones(d))
    two = _bf16_bits(np.full(d, 2.0))
    base = oracle.mtp_input(h, e, one, one, eps=0.0)
    # scale-free in each input (doubling is exact in bf16)
    h2 = _bf16_bits(oracle.bf16_value(h) * 2.0)
    e4 = _bf16_bits(oracle.bf16_value(e) * 4.0)
    assert np.array_equal(oracle.mtp_input(h2, e4, one, one, eps=0.0), base)
    # unit mean square per half
    assert abs(np.mean(base[:d] ** 2) - 1.0) < 1e-12 and abs(np.mean(base[d:] ** 2) - 1.0) < 1e-12
    # the halves are independent, h first (its gain doubles only the first half)
    other = oracle.mtp_input(h, _bf16_bits(rng.normal(0.0, 1.0, d)), two, one, eps=0.0)
    assert np.array_equal(other[:d], 2.0 * base[:d]) and not np.array_equal(other[d:], base[d:])
    # eps enters as in RMSNorm: a constant row c gives c / sqrt(c^2 + eps)
    c = 0.5
    cst = oracle.mtp_input(_bf16_bits(np.full(d, c)), _bf16_bits(np.full(d, -c)), one, one, eps=1e-2)
    assert np.allclose(cst[:d], c / np.sqrt(c * c + 1e-2), rtol=1e-15)
    assert np.allclose(cst[d:], -c / np.sqrt(c * c + 1e-2), rtol=1e-15)


def test_embed_rows_gathers_ids():
    V, d = 37, 16
    E = (np.arange(V, dtype=np.uint16)[:, None] * 64 + np.arange(d, dtype=np.uint16)[None, :]).astype(np.uint16)
    tok = [3, 0, V - 1, -1, V, 3]
    out = oracle.embed_rows(E, tok)
    assert np.array_equal(out[0], E[3]) and np.array_equal(out[1], E[0]) and np.array_equal(out[2], E[V - 1])
    assert not out[3].any() and not out[4].any() and np.array_equal(out[5], E[3])
