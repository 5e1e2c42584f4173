"""Pins of the oracle's tree-budget calibration (CPU only).

The expected acceptance length is pinned by:
  - the values the pages print for a chain: [chapter]'s E[T] for four
    (alpha, gamma) pairs, its cost 1.32 and speedup 2.10 for gamma = 4,
    alpha = 0.7, c = 0.08, and [guide]'s decay P(K >= k) = 0.7^k;
  - brute force: every accept/reject outcome of every drafted node is
    enumerated, the walk is run on each, and the outcome probabilities are
    summed (no recursion);
  - special cases: the root alone, a star, probabilities of 0 and 1;
  - the verification rule itself: on fixed small trees, the oracle's
    stochastic verifier is run on 20 000 seeded uniforms and its mean emitted
    count and per-node path frequencies must match AL and reach, with each
    node's acceptance probability taken from its rows (min(1, p'/q) along the
    recursive residual).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import BAD_NNODES, BAD_PARENT, BAD_PROB
from oracle.budget import chain_cost, expected_length, expected_length_request, goodput, select_budget
from oracle.verify import verify_stochastic_request


def random_tree(rng, n, max_children=None):
    par = [-1]
    kids = [0]
    for i in range(1, n):
        ok = [j for j in range(i) if max_children is None or kids[j] < max_children]
        p = int(rng.choice(ok))
        par.append(p)
        kids[p] += 1
        kids.append(0)
    return par


def brute_force(par, n, a):
    """Enumerate o in {0,1}^(n-1): o[v] = 1 if v would pass its test."""
    al = 0.0
    reach = [0.0] * n
    for bits in itertools.product((0, 1), repeat=n - 1):
        o = (1,) + bits
        w = 1.0
        for v in range(1, n):
            w *= a[v] if o[v] else 1.0 - a[v]
        if w == 0.0:
            continue
        u, on_path = 0, [0]
        while True:
            nxt = next((c for c in range(u + 1, n) if par[c] == u and o[c]), None)
            if nxt is None:
                break
            u = nxt
            on_path.append(u)
        al += w * len(on_path)          # accepted nodes + 1 emitted token = len(path)
        for v in on_path:
            reach[v] += w
    return reach, al


def test_chain_matches_printed_expected_tokens(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "expected_tokens.json")))
    for row in g["expected_tokens_per_round"]:
        gamma, alpha = row["gamma"], row["alpha"]
        n = gamma + 1
        _, al = expected_length_request(list(range(-1, n - 1)), n, [0.0] + [alpha] * gamma)
        decimals = len(str(row["E_T"]).split(".")[1])
        assert abs(al - row["E_T"]) <= 0.5 * 10 ** -decimals, (row, al)


def test_chain_reach_matches_printed_decay(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "expected_tokens.json")))
    alpha = g["decay_alpha"]
    n = 8
    reach, _ = expected_length_request(list(range(-1, n - 1)), n, [0.0] + [alpha] * (n - 1))
    for row in g["decay"]:
        assert abs(reach[row["k"]] - row["P_accept_at_least_k"]) <= 5e-4


def test_printed_cost_and_speedup():
    # [chapter]: gamma = 4, alpha = 0.7, c = 0.08 -> cost 1.32, speedup ~2.10x
    _, al = expected_length_request([-1, 0, 1, 2, 3], 5, [0.0, 0.7, 0.7, 0.7, 0.7])
    assert abs(chain_cost(4, 0.08) - 1.32) < 1e-12
    assert abs(goodput(al, chain_cost(4, 0.08)) - 2.10) < 5e-3


@pytest.mark.parametrize("n", range(1, 7))
def test_every_small_tree_brute_force(n):
    rng = np.random.default_rng(70 + n)
    for par in itertools.product(*[range(i) for i in range(1, n)]):
        par = [-1] + list(par)
        a = [0.0] + list(rng.random(n - 1))
        reach, al = expected_length_request(par, n, a)
        rb, ab = brute_force(par, n, a)
        assert abs(al - ab) <= 1e-12 * ab
        assert np.allclose(reach, rb, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("seed", range(12))
def test_random_trees_brute_force_with_certain_outcomes(seed):
    rng = np.random.default_rng(500 + seed)
    n = int(rng.integers(7, 12))
    par = random_tree(rng, n, max_children=int(rng.integers(1, 4)))
    a = [0.0] + [float(x) for x in rng.choice([0.0, 1.0, 0.3, 0.85, rng.random()], size=n - 1)]
    reach, al = expected_length_request(par, n, a)
    rb, ab = brute_force(par, n, a)
    assert abs(al - ab) <= 1e-12 * ab
    assert np.allclose(reach, rb, rtol=1e-12, atol=1e-15)


def test_special_cases():
    assert expected_length_request([-1], 1, [0.5]) == ([1.0], 1.0)
    # star with k children of acceptance a: AL = 1 + (1 - (1 - a)^k)
    for k, a in ((1, 0.3), (4, 0.5), (7, 0.9)):
        _, al = expected_length_request([-1] + [0] * k, k + 1, [0.0] + [a] * k)
        assert abs(al - (2.0 - (1.0 - a) ** k)) < 1e-14
    # all ones: the walk follows first children to the end
    par = [-1, 0, 1, 1, 0, 2, 5, 4]
    reach, al = expected_length_request(par, 8, [0.0] + [1.0] * 7)
    assert al == 5.0 and reach == [1, 1, 1, 0, 0, 1, 1, 0]
    # all zeros: only the root's correction token
    assert expected_length_request(par, 8, [0.0] * 8)[1] == 1.0


def test_batched_status_and_padding():
    par = [[-1, 0, 0, 1], [-1, 0, 0, 1], [0, 0, 0, 1], [-1, 0, 0, 1], [-1, 0, 2, 1]]
    a = [[0.3, 0.5, 0.5, 0.5], [0.0, 0.5, 1.5, 0.5], [0.0, 0.5, 0.5, 0.5], [0.0, float("nan"), 0.5, 0.5],
         [0.0, 0.5, 0.5, 0.5]]
    reach, al, st = expected_length(par, [3, 3, 4, 2, 4], a, 4)
    assert st == [0, BAD_PROB, BAD_PARENT, BAD_PROB, BAD_PARENT]
    assert al[0] == pytest.approx(1.75) and reach[0] == [1.0, 0.5, 0.25, 0.0]
    assert al[1:] == [0.0] * 4
    _, _, st = expected_length(par[:1], [5], a[:1], 4)
    assert st == [BAD_NNODES]
    # a probability past n_nodes is never read
    _, al, st = expected_length([[-1, 0, 0, 1]], [2], [[0.0, 0.5, 7.0, float("nan")]], 4)
    assert st == [0] and al == [1.5]


def test_select_budget():
    al = [1.0, 2.0, 3.0]
    itl = [[1.0, 1.0, 1.0],       # flat latency: the largest tree
           [1.0, 3.0, 9.0],       # latency grows faster than AL: the smallest
           [2.0, 4.0, 6.0],       # equal goodputs: the lowest index
           [0.0, float("nan"), -1.0],
           [0.0, 4.0, float("inf")]]
    assert select_budget(al, itl) == [2, 0, 0, -1, 1]


def softmax(z):
    e = np.exp(z - z.max())
    return e / e.sum()


def acceptance_from_rows(tl, dl, tok, par, n):
    """a[v] = min(1, p'(x_v) / q(x_v)), p' the parent's target distribution
    after the earlier siblings' residual updates (q(x) = 0 accepts)."""
    a = [0.0] * n
    for u in range(n):
        kids = [c for c in range(u + 1, n) if par[c] == u]
        p, q = softmax(tl[u]), softmax(dl[u])
        for c in kids:
            x = tok[c]
            a[c] = 1.0 if q[x] == 0 else min(1.0, p[x] / q[x])
            r = np.maximum(p - q, 0.0)
            if r.sum() > 0:
                p = r / r.sum()
    return a


@pytest.mark.parametrize("seed", range(3))
def test_model_matches_the_stochastic_verifier(seed):
    rng = np.random.default_rng(900 + seed)
    n, V = 9, 4
    par = random_tree(rng, n, max_children=3)
    tl = rng.standard_normal((n, V)) * 1.5
    dl = tl + rng.standard_normal((n, V)) * 0.8
    tok = np.array([0] + [int(rng.integers(0, V)) for _ in range(n - 1)])
    a = acceptance_from_rows(tl, dl, tok, par, n)
    reach, al = expected_length_request(par, n, a)
    trials = 20000
    emitted = np.empty(trials)
    hits = np.zeros(n)
    for t in range(trials):
        path, out, _ = verify_stochastic_request(tl, dl, tok, par, n, rng.random(n), rng.random(n))
        emitted[t] = len(out)
        hits[list(path)] += 1
    se = emitted.std(ddof=1) / math.sqrt(trials)
    assert abs(emitted.mean() - al) < 5 * se + 1e-9, (emitted.mean(), al, se)
    freq = hits / trials
    for v in range(n):
        sd = math.sqrt(max(reach[v] * (1 - reach[v]), 1e-12) / trials)
        assert abs(freq[v] - reach[v]) < 5 * sd + 1e-9, (v, freq[v], reach[v])
