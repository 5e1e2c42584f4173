"""Seeded trials for the statistical checks of stochastic verification (test helper).

An order-1 Markov "model" over a tiny vocabulary: the target and draft
distributions of a tree node depend only on that node's token, through fixed
tables P[a] and Q[a].  A round's tree has a fixed shape, and every child's token
is an independent draw from Q[token of its parent] (Gumbel-max), so the i.i.d.
proposal precondition of rejection sampling holds.  This module only draws;
none of the method's arithmetic is here.
"""
from __future__ import annotations

import numpy as np

# the guide's mask-figure tree: root with two children, two grandchildren under
# the first and one under the second
SHAPE = np.array([-1, 0, 0, 1, 1, 2], dtype=np.int32)


def markov_tables(seed: int, V: int):
    """Target and draft logit tables (float32), rows indexed by the context token."""
    rng = np.random.default_rng(seed)
    P = rng.dirichlet(np.ones(V) * 0.8, size=V)
    Q = rng.dirichlet(np.ones(V) * 0.8, size=V)
    return np.log(P).astype(np.float32), np.log(Q).astype(np.float32)


def softmax_rows(logits):
    """The distributions the float32 tables define (float64), for expected counts."""
    x = np.asarray(logits, dtype=np.float64)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def draw_round(rng, LT, LQ, roots, shape=SHAPE):
    """One round per trial: tokens [T][n] grown from `roots` by Gumbel-max on
    the parent's draft row, logit rows [T][n][V], and the uniforms [T][n]."""
    T, n, V = len(roots), len(shape), LT.shape[1]
    tok = np.zeros((T, n), dtype=np.int32)
    tok[:, 0] = roots
    for c in range(1, n):
        g = rng.gumbel(size=(T, V))
        tok[:, c] = np.argmax(LQ[tok[:, shape[c]]].astype(np.float64) + g, axis=1)
    tl = np.ascontiguousarray(LT[tok])
    dl = np.ascontiguousarray(LQ[tok])
    ua = rng.random((T, n), dtype=np.float32)
    us = rng.random((T, n), dtype=np.float32)
    return tok, tl, dl, ua, us


def chi_square_pvalue(counts, expected, min_expected=5.0):
    from scipy import stats
    keep = expected > min_expected
    chi2 = float(((counts - expected) ** 2 / np.where(keep, expected, 1.0))[keep].sum())
    return chi2, float(stats.chi2.sf(chi2, int(keep.sum()) - 1))
