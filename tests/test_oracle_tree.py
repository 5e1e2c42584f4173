"""Pins of the oracle's tree mask (CPU only)."""
import itertools
import os

import numpy as np
import pytest

from oracle import BAD_NNODES, BAD_PARENT
from oracle.tree import ancestors_walk, children, depth, topology_mask, validate



def closure_mask(parent, n):
    """Ancestor-or-self relation by Warshall transitive closure of the child->parent
    edge relation (an algorithm independent of the oracle's parent walk)."""
    R = np.eye(n, dtype=bool)
    for c in range(1, n):
        R[c, parent[c]] = True
    for k in range(n):
        R = R | (R[:, [k]] & R[[k], :])
    return R


def all_parent_arrays(n):
    ranges = [range(i) for i in range(1, n)]
    for tail in itertools.product(*ranges):
        yield np.array((-1,) + tail, dtype=np.int64)


def test_mask_matches_page_figure(golden_dir):
    lines = [l.split() for l in open(os.path.join(golden_dir, "mask_figure.txt"))
             if l.strip() and not l.startswith("#")]
    assert lines[0][0] == "parent"
    parent = np.array([int(x) for x in lines[0][1:]])
    want = np.array([[0.0 if x == "0" else -np.inf for x in row] for row in lines[1:]])
    got = topology_mask(parent, len(parent))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7])
def test_mask_bruteforce_all_trees(n):
    count = 0
    for parent in all_parent_arrays(n):
        M = topology_mask(parent, n)
        R = closure_mask(parent, n)
        assert np.array_equal(M == 0, R), parent
        # allowed set of u is its root path: depth(u) + 1 entries, lower triangular
        for u in range(n):
            assert (M[u] == 0).sum() == depth(parent, u) + 1
            assert M[u, 0] == 0 and M[u, u] == 0
        assert np.all(np.triu(M == 0, 1) == False)  # noqa: E712
        count += 1
    assert count == max(1, int(np.prod(range(1, n))))


def test_children_ascending_and_walk():
    parent = np.array([-1, 0, 0, 1, 1, 2])
    assert children(parent, 6, 0) == [1, 2]
    assert children(parent, 6, 1) == [3, 4]
    assert children(parent, 6, 5) == []
    assert ancestors_walk(parent, 4) == [4, 1, 0]


def test_validate_flags():
    assert validate(np.array([-1, 0, 1]), 3, 4) == 0
    assert validate(np.array([-1, 0, 1]), 0, 4) == BAD_NNODES
    assert validate(np.array([-1, 0, 1, 0, 0]), 5, 4) == BAD_NNODES
    assert validate(np.array([0, 0, 1]), 3, 4) == BAD_PARENT
    assert validate(np.array([-1, 2, 1]), 3, 4) == BAD_PARENT
    assert validate(np.array([-1, 0, -1]), 3, 4) == BAD_PARENT
