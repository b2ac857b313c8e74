"""Exact law of the accept/resample procedure, in rational arithmetic.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

hazakura.dev, "mtplx——M5 Maxで63tok/s…", section "mtplxの数字——本当なの？": the
table reports the output distribution of the speculative cycle matching the
target exactly ("max_diff = 0.0"); devtrends.cc, "…MTPLX", section
"2つ目のモデル不要！MTPの裏技": exact rejection sampling with residual
correction gives the same distribution as plain step-by-step sampling.

For one position with target p and draft distribution q (both summing to one),
the procedure emits
    v  with probability  q(v) * min(1, p(v)/q(v))                (draft accepted)
     + (1 - sum_x q(x) min(1, p(x)/q(x))) * r(v)                  (rejected, resampled)
with r = max(0, p - q) / sum max(0, p - q).  The law of the bonus position is
p itself.  Everything here is fractions.Fraction: no rounding anywhere.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Sequence


def to_fractions(v: Sequence[float], renormalize: bool = True):
    f = [Fraction(float(x)) for x in v]
    if renormalize:
        s = sum(f)
        f = [x / s for x in f]
    return f


def law_first_token(p: Sequence[Fraction], q: Sequence[Fraction]):
    """Exact probability of each emitted token at a draft position."""
    V = len(p)
    acc = [Fraction(0)] * V
    for x in range(V):
        if q[x] > 0:
            acc[x] = q[x] * min(Fraction(1), p[x] / q[x])
    p_reject = 1 - sum(acc)
    res = [max(Fraction(0), p[v] - q[v]) for v in range(V)]
    R = sum(res)
    out = []
    for v in range(V):
        r = res[v] / R if R > 0 else p[v]
        out.append(acc[v] + p_reject * r)
    return out


def max_diff(a: Sequence[Fraction], b: Sequence[Fraction]) -> Fraction:
    return max(abs(x - y) for x, y in zip(a, b))


def accept_probability(p: Sequence[Fraction], q: Sequence[Fraction]) -> Fraction:
    """Probability that a draft drawn from q is accepted: sum_x min(p(x), q(x))."""
    return sum(min(px, qx) for px, qx in zip(p, q))
