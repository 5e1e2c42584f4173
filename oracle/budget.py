"""Tree-budget calibration (test infrastructure only).

What is computed, and where the pages state it:
  - [chapter] "Worked Example: How Many Tokens Land Per Expensive Pass?":
    acceptance events are modelled as independent draws; a round emits the K
    accepted drafts plus one more token (a correction or a bonus), T = K + 1,
    and for a chain of gamma drafts with acceptance alpha
    E[T] = (1 - alpha^(gamma + 1)) / (1 - alpha).  A round's cost in
    target-pass equivalents is gamma * c + 1 and the speedup is E[T] / cost.
  - [cohere] "Dynamic speculative decoding": goodput = AL / ITL (acceptance
    length over inter-token latency); the best number of drafts per batch
    size is found offline from measured AL and ITL and kept as a lookup table.
  - [guide] "Dynamic Tree Budget Calibration": tree size should follow the
    batch size (large trees at low concurrency, small ones at high).

Readings (the pages leave these open; the design notes list them):
  - The independence model of [chapter] is applied per tree node: a drafted
    node v, when it is tested, is accepted with probability a[v],
    independently of every other test.  Children are tested in ascending node
    id, and the first accepted child continues the walk; this is the order of
    the verification walk ([guide] "Stochastic Verification Algorithm").
    For a chain with a[v] = alpha this is [chapter]'s model exactly.
  - AL is the expected number of tokens a round emits, E[T] = 1 + E[accepted
    nodes], so a tree of the root alone has AL = 1.
  - Goodput is AL / ITL.  A batch of B requests emits B * AL tokens per step,
    so per batch size the table keeps the tree shape with the largest AL / ITL;
    equal goodputs keep the lower shape index (shapes listed smallest first).
  - accept_prob[0] (the root is never tested) is ignored; a probability that
    is NaN or outside [0, 1] flags the request BAD_PROB.
"""
from __future__ import annotations

import math

from . import BAD_PROB
from .tree import children, validate


def _prob_status(a, n: int) -> int:
    for v in range(1, n):
        x = float(a[v])
        if not (0.0 <= x <= 1.0):     # also false for NaN
            return BAD_PROB
    return 0


def expected_length_request(parent, n: int, a):
    """(reach, AL) of one tree under the per-node independence model.

    reach[v] = probability that v lies on the accepted path (reach[0] = 1).
    The walk is taken literally, node by node from the root: at node u the
    children are tried in ascending id; child c is reached when every earlier
    sibling was rejected and c itself is accepted.  AL is written as the
    recursion E(u) = sum over children c of P(c is the first accepted child)
    * (1 + E(c)), AL = 1 + E(root), computed from the leaves up; reach is a
    separate walk from the root down.  Both are float64.
    """
    kids = [children(parent, n, u) for u in range(n)]
    # AL: expected accepted nodes below each node, leaves first (children have larger ids)
    below = [0.0] * n
    for u in range(n - 1, -1, -1):
        all_rejected = 1.0
        e = 0.0
        for c in kids[u]:
            e += all_rejected * float(a[c]) * (1.0 + below[c])
            all_rejected *= 1.0 - float(a[c])
        below[u] = e
    # reach: from the root down
    reach = [0.0] * n
    reach[0] = 1.0
    for u in range(n):
        all_rejected = 1.0
        for c in kids[u]:
            reach[c] = reach[u] * all_rejected * float(a[c])
            all_rejected *= 1.0 - float(a[c])
    return reach, 1.0 + below[0]


def expected_length(parent, n_nodes, accept_prob, n_max: int):
    """Batched form.  Returns (reach [B][n_max] with 0 in padding, AL [B],
    status [B]); a failed request has AL = 0 and reach all 0."""
    B = len(n_nodes)
    reach = [[0.0] * n_max for _ in range(B)]
    al = [0.0] * B
    status = [0] * B
    for b in range(B):
        n = int(n_nodes[b])
        st = validate(parent[b], n, n_max)
        if st == 0:
            st = _prob_status(accept_prob[b], n)
        status[b] = st
        if st:
            continue
        r, e = expected_length_request(parent[b], n, accept_prob[b])
        reach[b][:n] = r
        al[b] = e
    return reach, al, status


def chain_cost(gamma: int, c: float) -> float:
    """[chapter]'s cost of one round in target-pass equivalents: gamma draft
    passes at relative cost c, plus one verification pass."""
    return gamma * c + 1.0


def goodput(al: float, itl: float) -> float:
    """[cohere]: acceptance length over inter-token latency."""
    return al / itl


def select_budget(al, itl):
    """Best shape per batch size.

    al[s]: acceptance length of shape s; itl[i][s]: measured latency of one
    step of batch size i with shape s (> 0).  Returns, per batch size, the
    index of the shape with the largest goodput al[s] / itl[i][s] (ties keep
    the lower index), or -1 when no latency is positive and finite.
    """
    best = []
    for row in itl:
        pick, top = -1, -math.inf
        for s, t in enumerate(row):
            t = float(t)
            if not (t > 0.0 and math.isfinite(t)):
                continue
            g = goodput(float(al[s]), t)
            if g > top:
                pick, top = s, g
        best.append(pick)
    return best
