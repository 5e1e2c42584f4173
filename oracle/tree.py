"""Token-tree helpers of the oracle (test infrastructure only).

A tree of n nodes is a parent array: parent[0] = -1 is the root (the last
token already emitted), and every other node u has one parent p_u with
0 <= p_u < u.  [guide] "Mathematical Formulation of the Token Tree" defines
S_u = S_{p_u} followed by t_u; the ordering constraint p_u < u is this
project's reading of "Depth-First Flattening" (any topological order,
depth-first preorder in generated inputs).
"""
from __future__ import annotations

import numpy as np

from . import BAD_NNODES, BAD_PARENT


def validate(parent, n: int, n_max: int) -> int:
    """Status flags for one request's tree description (0 when well formed)."""
    if n < 1 or n > n_max:
        return BAD_NNODES
    if int(parent[0]) != -1:
        return BAD_PARENT
    for i in range(1, n):
        p = int(parent[i])
        if p < 0 or p >= i:
            return BAD_PARENT
    return 0


def ancestors_walk(parent, u: int) -> list[int]:
    """u, then its parent, grandparent, ... up to the root.

    [guide] "The Topology-Aware 2D Causal Mask" and the mask builder of its
    PyTorch section: start at the node, mark it, then follow parent pointers
    until the root has been marked.
    """
    out = []
    cur = int(u)
    while cur != -1:
        out.append(cur)
        cur = int(parent[cur])
    return out


def topology_mask(parent, n: int) -> np.ndarray:
    """Dense n x n mask M of [guide] "The Topology-Aware 2D Causal Mask".

    M[u, v] = 0 when v is u itself or one of u's ancestors, else -inf (the
    case split of the mask equation; the page's rendering drops the braces of
    {u} and the line break before -inf).
    """
    M = np.full((n, n), -np.inf)
    for u in range(n):
        for v in ancestors_walk(parent, u):
            M[u, v] = 0.0
    return M


def children(parent, n: int, u: int) -> list[int]:
    """Children of u in ascending node index (the order siblings are tried in)."""
    return [c for c in range(n) if int(parent[c]) == u]


def depth(parent, u: int) -> int:
    return len(ancestors_walk(parent, u)) - 1
