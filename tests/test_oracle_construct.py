"""Pins of the oracle's token-tree construction (CPU only).

Merge (Method B) is pinned by a hand-worked example, by the merge condition
itself (every candidate prefix is the token sequence of a node), by a count of
distinct prefixes taken with a set, and by the shape of a depth-first
preorder.  Expansion (Method A) is pinned by numpy's argmax (k = 1), by a
brute-force sort, by the schedule example's level sizes and by the parent and
level structure of the result.
"""
import json
import os
import random

import numpy as np
import pytest

from oracle import NONFINITE, TREE_OVERFLOW
from oracle.construct import expand_level, expand_tree, merge_candidates, topk_tokens


def root_path_tokens(tokens, parent, v):
    out = []
    while v > 0:
        out.append(tokens[v])
        v = parent[v]
    return out[::-1]


def random_candidates(rng, m, lmax, vocab):
    """Candidates that share prefixes often: each continues a random earlier one."""
    cands = []
    for i in range(m):
        L = rng.randint(0, lmax)
        if cands and rng.random() < 0.7:
            base = rng.choice(cands)
            cut = rng.randint(0, len(base))
            seq = list(base[:cut])
        else:
            seq = []
        while len(seq) < L:
            seq.append(rng.randrange(vocab))
        cands.append(seq[:L])
    return cands


def test_merge_hand_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "construct_examples.json")))["merge"]
    tokens, parent, n, node_of, st = merge_candidates(g["root_token"], g["candidates"], 64)
    assert st == 0 and n == len(g["tokens"])
    assert tokens == g["tokens"] and parent == g["parent"] and node_of == g["node_of"]


@pytest.mark.parametrize("seed", range(40))
def test_merge_condition_and_shape(seed):
    rng = random.Random(seed)
    cands = random_candidates(rng, rng.randint(1, 12), 9, rng.choice([2, 3, 50]))
    tokens, parent, n, node_of, st = merge_candidates(5, cands, 4096)
    assert st == 0
    # merge condition: S_v = S_u for every candidate prefix
    for i, seq in enumerate(cands):
        assert len(node_of[i]) == len(seq)
        for j in range(len(seq)):
            assert root_path_tokens(tokens, parent, node_of[i][j]) == seq[:j + 1]
    # no redundancy: one node per distinct prefix, plus the root
    prefixes = {tuple(seq[:j + 1]) for seq in cands for j in range(len(seq))}
    assert n == 1 + len(prefixes)
    # depth-first preorder: parent first, every subtree a contiguous id range
    assert parent[0] == -1 and tokens[0] == 5
    size = [1] * n
    for v in range(n - 1, 0, -1):
        assert 0 <= parent[v] < v
        size[parent[v]] += size[v]
    for v in range(1, n):
        p = parent[v]
        # v's subtree ends where the next sibling or an ancestor's sibling starts
        assert v + size[v] <= p + size[p]
    for u in range(n):
        kids = [v for v in range(n) if parent[v] == u]
        # consecutive children: each starts right after the previous one's subtree
        for a, b in zip(kids, kids[1:]):
            assert b == a + size[a]
        # siblings: distinct tokens, ordered by the first candidate holding them
        assert len({tokens[v] for v in kids}) == len(kids)
        first = [min(i for i in range(len(cands)) if v in node_of[i]) for v in kids]
        assert first == sorted(first)


def test_merge_special_cases():
    t, p, n, no, st = merge_candidates(1, [[4, 5, 6, 7]], 16)
    assert (t, p, n, no) == ([1, 4, 5, 6, 7], [-1, 0, 1, 2, 3], 5, [[1, 2, 3, 4]])
    t2 = merge_candidates(1, [[4, 5, 6, 7], [4, 5, 6, 7], []], 16)
    assert t2[:3] == (t, p, n) and t2[3] == [[1, 2, 3, 4], [1, 2, 3, 4], []]
    t, p, n, no, st = merge_candidates(9, [], 4)
    assert (t, p, n, st) == ([9], [-1], 1, 0)
    t, p, n, no, st = merge_candidates(9, [[1, 2], [3, 4]], 4)
    assert st == TREE_OVERFLOW and n == 0
    assert merge_candidates(9, [[1, 2], [1, 3]], 4)[4] == 0


@pytest.mark.parametrize("seed", range(20))
def test_topk_against_argmax_and_sort(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(1, 60))
    row = rng.integers(-3, 4, size=V).astype(np.float32)   # many ties
    assert topk_tokens(row, 1) == [int(np.argmax(row))]
    for k in range(1, V + 1):
        want = sorted(range(V), key=lambda i: (-float(row[i]), i))[:k]
        assert topk_tokens(row, k) == want


def test_topk_ties_and_order():
    assert topk_tokens([1.0, 3.0, 3.0, 2.0], 2) == [1, 2]
    assert topk_tokens([1.0, 3.0, 3.0, 2.0], 4) == [1, 2, 3, 0]
    assert topk_tokens([-0.5, -0.25, -1.0], 3) == [1, 0, 2]


def test_expansion_schedule_level_sizes(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "construct_examples.json")))
    rng = np.random.default_rng(3)
    V = 40
    table = {}

    def draft_row(tokens, parent, u):
        key = tuple(root_path_tokens(tokens, parent, u))
        if key not in table:
            table[key] = rng.normal(size=V)
        return table[key]

    tokens, parent, n, st = expand_tree(0, g["schedule"], draft_row, 256)
    assert st == 0
    depth = [0] * n
    for v in range(1, n):
        depth[v] = depth[parent[v]] + 1
    sizes = [sum(1 for v in range(n) if depth[v] == d) for d in range(1, len(g["schedule"]) + 1)]
    assert sizes == g["level_sizes"] and n == 1 + sum(sizes)
    # level order, parents first, each node's children = top-k of its own row, best first
    assert depth == sorted(depth)
    for u in range(n):
        kids = [v for v in range(n) if parent[v] == u]
        if kids:
            row = table[tuple(root_path_tokens(tokens, parent, u))]
            k = g["schedule"][depth[u]]
            assert [tokens[v] for v in kids] == list(np.argsort(-row, kind="stable")[:k])


def test_expand_level_errors():
    t, p, n, fr, st = expand_level([0], [-1], 1, [0], [np.zeros(5)], 3, 3)
    assert st == TREE_OVERFLOW and n == 1 and fr == []
    t, p, n, fr, st = expand_level([0], [-1], 1, [0], [np.array([0.0, np.nan, 1.0])], 1, 8)
    assert st == NONFINITE and n == 1
    t, p, n, fr, st = expand_level([0, 4], [-1, 0], 2, [1, 0], [np.array([0.0, 2.0, 1.0]), np.array([5.0, 1.0, 1.0])], 2, 8)
    assert st == 0 and t == [0, 4, 1, 2, 0, 1] and p == [-1, 0, 1, 1, 0, 0] and fr == [2, 3, 4, 5]
