"""Token-tree construction (test infrastructure only).

[guide] "Token Tree Construction: Expansion vs. Merge" gives two ways to build
the tree that the verifier later checks:

  Method A, expansion within one draft model: a schedule <k_1, ..., k_m>; at
  depth i every node of the previous level receives the k_i most probable
  next tokens of the draft model at that node.
  Method B, merge of several draft models' candidates: every candidate
  sequence is merged into one tree M such that each prefix of each candidate
  is the token sequence S_v of some node v of M (the merge condition), with
  identical prefixes sharing one node.

Readings (the pages are silent on these; the design notes list them):
  - The root, node 0, is the last token already emitted; drafted tokens hang
    below it (the page's listing makes level 1 a forest of roots instead).
  - Merge numbering: depth-first preorder of the trie, siblings in the order
    of the first candidate (lowest index) that contains them.
  - Expansion numbering: level by level, within a level in frontier order and
    then by rank (the order in which the page's listing appends children);
    parents therefore always precede children.
  - "Most probable" = largest logit (softmax at any temperature keeps the
    order); equal logits rank the lower token index first.
  - A tree that would exceed n_max nodes is not built: status TREE_OVERFLOW.
"""
from __future__ import annotations

import numpy as np

from . import NONFINITE, TREE_OVERFLOW


# ---------------------------------------------------------------------------
# Method B: merge
# ---------------------------------------------------------------------------

def merge_candidates(root_token: int, cands, n_max: int):
    """Merge candidate token sequences into one tree (Method B).

    cands: list of token lists (the drafted continuations, root excluded).
    Returns (tokens, parent, n, node_of, status): tokens and parent are lists
    of length n; node_of[i][j] is the node whose token sequence is
    cands[i][:j + 1] (S_v = S_u in the merge condition).  status is 0 or
    TREE_OVERFLOW (then n = 0 and every list is empty).

    Built as an explicit trie: a node's children are kept in a dict, which
    remembers the order in which they were first inserted, i.e. the index of
    the first candidate that contains them.  A depth-first walk of that trie
    then numbers the nodes.
    """
    kids = [dict()]          # trie node -> {token: trie child}
    tok = [int(root_token)]
    trie_of = []
    for seq in cands:
        cur, row = 0, []
        for t in seq:
            t = int(t)
            if t not in kids[cur]:
                kids[cur][t] = len(tok)
                kids.append(dict())
                tok.append(t)
            cur = kids[cur][t]
            row.append(cur)
        trie_of.append(row)
    if len(tok) > n_max:
        return [], [], 0, [[] for _ in cands], TREE_OVERFLOW
    order, tparent = [], {0: None}
    stack = [0]
    while stack:             # depth-first preorder, children in insertion order
        v = stack.pop()
        order.append(v)
        ch = list(kids[v].values())
        for c in ch:
            tparent[c] = v
        stack.extend(reversed(ch))
    rank = {v: r for r, v in enumerate(order)}
    tokens = [tok[v] for v in order]
    parent = [-1 if tparent[v] is None else rank[tparent[v]] for v in order]
    node_of = [[rank[v] for v in row] for row in trie_of]
    return tokens, parent, len(order), node_of, 0


# ---------------------------------------------------------------------------
# Method A: expansion
# ---------------------------------------------------------------------------

def topk_tokens(row, k: int) -> list[int]:
    """The k tokens with the largest logits, best first; ties: lower index first."""
    row = np.asarray(row, dtype=np.float64)
    order = np.lexsort((np.arange(row.size), -row))   # primary: -logit, then index
    return [int(x) for x in order[:k]]


def expand_level(tokens, parent, n: int, frontier, rows, k: int, n_max: int):
    """One expansion step: every frontier node (in order) receives the top-k
    tokens of its draft row as children, appended after node n - 1.

    tokens, parent: lists holding the current tree (length >= n).
    rows[f]: draft logits of frontier[f].  Returns (tokens, parent, n,
    new_frontier, status); on TREE_OVERFLOW or a non-finite logit the tree is
    returned unchanged with an empty frontier.
    """
    tokens, parent = list(tokens[:n]), list(parent[:n])
    if n + len(frontier) * k > n_max:
        return tokens, parent, n, [], TREE_OVERFLOW
    for r in rows:
        if not np.all(np.isfinite(np.asarray(r, dtype=np.float64))):
            return tokens, parent, n, [], NONFINITE
    new = []
    for f, u in enumerate(frontier):
        for t in topk_tokens(rows[f], k):
            tokens.append(t)
            parent.append(int(u))
            new.append(len(tokens) - 1)
    return tokens, parent, len(tokens), new, 0


def expand_tree(root_token: int, schedule, draft_row, n_max: int):
    """A whole tree by Method A with schedule <k_1, ..., k_m>.

    draft_row(tokens, parent, u) -> the draft model's logits at node u (in the
    pages, a forward pass over the prompt followed by u's ancestral tokens).
    Returns (tokens, parent, n, status).
    """
    tokens, parent, n = [int(root_token)], [-1], 1
    frontier = [0]
    for k in schedule:
        rows = [draft_row(tokens, parent, u) for u in frontier]
        tokens, parent, n, frontier, st = expand_level(tokens, parent, n, frontier, rows, int(k), n_max)
        if st:
            return tokens, parent, n, st
    return tokens, parent, n, 0
