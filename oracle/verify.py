"""Token-tree verification oracle (test infrastructure only).

Conventions (readings of the pages, see the design notes):
  * Node 0 is the root: the last token already emitted.  Logit row u is the
    target (or draft) distribution of the token that follows S_u.
  * Verification emits path_len = L + 1 tokens: the tokens of the L accepted
    nodes, then one correction/bonus token ([chapter] "Worked Example: How
    Many Tokens Land Per Expensive Pass?": every round emits T = K + 1).
  * Siblings are tried in ascending node index.

Everything is float64; logits are widened exactly from their stored type.
"""
from __future__ import annotations

import numpy as np

from . import BAD_TOKEN, NONFINITE
from .tree import children, validate


def softmax(z, temperature: float = 1.0) -> np.ndarray:
    """Vocabulary-wide softmax of logits / temperature, max-subtracted."""
    x = np.asarray(z, dtype=np.float64) / float(temperature)
    x = x - x.max()
    e = np.exp(x)
    return e / e.sum()


def inverse_cdf(weights: np.ndarray, u: float) -> tuple[int, float, float]:
    """Draw from unnormalised non-negative weights with uniform u in [0, 1).

    Returns (token, lo, hi): the smallest token whose cumulative weight exceeds
    u * total (strictly, so zero-weight tokens are never chosen), and the
    normalised CDF interval [lo, hi) that u fell in.  If rounding leaves no
    cumulative value above u * total, the last positive-weight token is taken.
    """
    cum = np.cumsum(weights)
    total = cum[-1]
    thr = float(u) * total
    idx = np.nonzero(cum > thr)[0]
    if len(idx):
        y = int(idx[0])
    else:
        y = int(np.nonzero(weights > 0)[0][-1])
    lo = float(cum[y - 1] / total) if y > 0 else 0.0
    hi = float(cum[y] / total)
    return y, lo, hi


# --------------------------------------------------------------------------
# greedy
# --------------------------------------------------------------------------

def verify_greedy_request(target_logits, tokens, parent, n: int):
    """[guide] "Greedy Verification Algorithm", steps 1-5, walked literally.

    Start at the root; t_pred = argmax_w P_target(w | S_u) (lowest index among
    equal maxima); descend into the first child (ascending index) whose token
    equals t_pred; otherwise emit t_pred as the final token and stop.  At a
    leaf the argmax is still emitted (step 5; the page's harness calls the
    leaf's forced token a correction).
    Returns (path, out_tokens).
    """
    path = [0]
    out = []
    u = 0
    while True:
        t_pred = int(np.argmax(np.asarray(target_logits[u], dtype=np.float64)))
        match = None
        for c in children(parent, n, u):
            if int(tokens[c]) == t_pred:
                match = c
                break
        out.append(t_pred)
        if match is None:
            return path, out
        path.append(match)
        u = match


def verify_greedy(target_logits, tokens, parent, n_nodes, n_max: int):
    """Batched greedy verification: (paths, outs, status) per request."""
    B = len(n_nodes)
    paths, outs = [None] * B, [None] * B
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = int(n_nodes[b])
        st = validate(parent[b], n, n_max)
        if st == 0 and not np.all(np.isfinite(target_logits[b, :n])):
            st = NONFINITE
        status[b] = st
        if st:
            continue
        paths[b], outs[b] = verify_greedy_request(target_logits[b], tokens[b], parent[b], n)
    return paths, outs, status


# --------------------------------------------------------------------------
# stochastic
# --------------------------------------------------------------------------

def verify_stochastic_request(target_logits, draft_logits, tokens, parent, n: int,
                              u_accept, u_sample, temperature: float = 1.0):
    """Tree rejection sampling driven by the given uniforms.

    [guide] "Stochastic Verification Algorithm" and [chapter] "Misconception:
    ..." (the min(1, p/q) acceptance rule and the residual max(p - q, 0) / Z).
    At node u, with p = softmax(target_u / T) and q = softmax(draft_u / T):
      p' := p.  For each child c of u in ascending index, proposal x = t_c:
        accept when u_accept[c] * q(x) <= p'(x)  (the chapter's u <= p/q test,
        multiplied out so that q(x) = 0 accepts);  then emit x, move to c and
        start over with c's own distributions;
        otherwise p' := max(p' - q, 0) / Z with Z = sum(max(p' - q, 0)) when
        Z > 0 (p' is kept when Z = 0), and the next sibling is tried against
        the residual.  This is the chapter's exactness argument applied
        recursively: after a rejection the round must emit a draw from the
        residual, and that draw may itself be proposed by the next i.i.d.
        sibling and tested against the residual.
      If no child is accepted (a leaf included), draw the final token from p'
      with u_sample[u] by inverse CDF and stop.
    Returns (path, out_tokens, trace); trace lists every decision as
    ("accept", node, child, u, p'(x)/q(x)) or ("sample", node, token, u, lo, hi).
    """
    V = np.asarray(target_logits[0]).shape[0]
    path = [0]
    out = []
    trace = []
    u = 0
    while True:
        p = softmax(target_logits[u], temperature)
        kids = children(parent, n, u)
        p_cur = p
        accepted = None
        if kids:
            q = softmax(draft_logits[u], temperature)
            for c in kids:
                x = int(tokens[c])
                ratio = p_cur[x] / q[x] if q[x] > 0 else np.inf
                ua = float(u_accept[c])
                trace.append(("accept", u, c, ua, float(ratio)))
                if ua * q[x] <= p_cur[x]:
                    accepted = c
                    break
                r = np.maximum(p_cur - q, 0.0)
                Z = r.sum()
                if Z > 0:
                    p_cur = r / Z
        if accepted is not None:
            path.append(accepted)
            out.append(int(tokens[accepted]))
            u = accepted
            continue
        y, lo, hi = inverse_cdf(p_cur, float(u_sample[u]))
        trace.append(("sample", u, y, float(u_sample[u]), lo, hi))
        out.append(y)
        assert 0 <= y < V
        return path, out, trace


def verify_stochastic(target_logits, draft_logits, tokens, parent, n_nodes, u_accept, u_sample,
                      n_max: int, temperature: float = 1.0):
    """Batched stochastic verification: (paths, outs, traces, status)."""
    B = len(n_nodes)
    V = target_logits.shape[-1]
    paths, outs, traces = [None] * B, [None] * B, [None] * B
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = int(n_nodes[b])
        st = validate(parent[b], n, n_max)
        if st == 0:
            internal = sorted(set(int(parent[b][c]) for c in range(1, n)))
            if np.any((tokens[b][1:n] < 0) | (tokens[b][1:n] >= V)):
                st |= BAD_TOKEN
            if not np.all(np.isfinite(target_logits[b, :n])):
                st |= NONFINITE
            if internal and not np.all(np.isfinite(draft_logits[b, internal])):
                st |= NONFINITE
        status[b] = st
        if st:
            continue
        paths[b], outs[b], traces[b] = verify_stochastic_request(
            target_logits[b], draft_logits[b], tokens[b], parent[b], n,
            u_accept[b], u_sample[b], temperature)
    return paths, outs, traces, status


def divergence_in_band(trace, path, out, other_path, other_out, band: float = 1e-6) -> bool:
    """Whether another verifier's result may differ from this oracle's (reading C18).

    `trace`, `path` and `out` are this oracle's decision trace and result for
    one request; `other_path` and `other_out` are the other result.  Equal
    results are accepted.  Otherwise the oracle's decisions are replayed in
    trace order and the first one whose outcome the other result does not
    share is located:
      * an accept test of child c at node u diverges when the other path
        enters c after u and the oracle's does not, or the other way round;
        it lies in the band when |u_accept - p'(x)/q(x)| < band (a test with
        q(x) = 0 always accepts and is never in the band);
      * the draw at the node where both walks stop diverges when the emitted
        tokens differ; it lies in the band when u_sample is within `band` of
        either end of the CDF interval the oracle's draw fell in.
    Only that first divergent decision may lie in the band; later decisions
    are not looked at (after it the two walks follow different subtrees).  A
    difference that no decision explains (a path that leaves the oracle's
    walk without a divergent test, or tokens that differ on agreed nodes)
    returns False.
    """
    path, out = list(path), list(out)
    other_path, other_out = list(other_path), list(other_out)
    if path == other_path and out == other_out:
        return True
    pos = 0                                   # index of the current node in both paths
    for rec in trace:
        node = rec[1]
        if pos >= len(path) or path[pos] != node:
            return False                      # the trace does not follow the oracle's path
        if pos >= len(other_path) or other_path[pos] != node:
            return False                      # the other walk left earlier without a divergent test
        mine_next = path[pos + 1] if pos + 1 < len(path) else None
        other_next = other_path[pos + 1] if pos + 1 < len(other_path) else None
        if rec[0] == "accept":
            child, ua, ratio = rec[2], rec[3], rec[4]
            mine = mine_next == child
            other = other_next == child
            if mine != other:
                return bool(np.isfinite(ratio) and abs(ua - ratio) < band)
            if mine:
                if pos >= len(other_out) or other_out[pos] != out[pos]:
                    return False              # same accepted node, different token
                pos += 1
        else:
            token, us, lo, hi = rec[2], rec[3], rec[4], rec[5]
            if other_next is not None:
                return False                  # the other walk went on past the oracle's last node
            if pos >= len(other_out):
                return False
            if other_out[pos] != token:
                return bool(abs(us - lo) < band or abs(us - hi) < band)
            return len(other_path) == len(path) and other_out[:pos + 1] == out[:pos + 1]
    return False


# --------------------------------------------------------------------------
# linear speculative decoding (the chain special case)
# --------------------------------------------------------------------------

def linear_speculative(p_rows, q_rows, drafts, u_accept, u_sample):
    """[chapter] "The Mechanism" + the acceptance rule of "Misconception: ...".

    The draft proposed x_1..x_gamma; p_rows[i] is the target distribution at the
    position of x_{i+1} (i = 0..gamma, the last one is the bonus position) and
    q_rows[i] the draft distribution x_{i+1} was drawn from.  For i = 1..gamma:
    accept x_i when u_i <= min(1, p(x_i) / q(x_i)) (the traced example's
    `u <= accept_prob`); on the first rejection emit a draw from the
    normalised residual max(p - q, 0) and stop; if all are accepted emit a
    bonus draw from the last target distribution.
    u_accept[i] is the uniform for x_{i+1}; u_sample[i] the draw at position i.
    Returns the emitted tokens (K accepted drafts + 1).
    """
    gamma = len(drafts)
    out = []
    for i in range(gamma):
        p, q = np.asarray(p_rows[i], np.float64), np.asarray(q_rows[i], np.float64)
        x = int(drafts[i])
        a = min(1.0, p[x] / q[x]) if q[x] > 0 else 1.0
        if float(u_accept[i]) <= a:
            out.append(x)
            continue
        res = np.maximum(p - q, 0.0)
        res = res / res.sum()
        out.append(inverse_cdf(res, float(u_sample[i]))[0])
        return out
    out.append(inverse_cdf(np.asarray(p_rows[gamma], np.float64), float(u_sample[gamma]))[0])
    return out


def linear_greedy(target_rows, drafts):
    """Greedy linear speculation ([guide] "The Linear Speculation Dilemma"
    figure): keep drafts while each equals the target's argmax at its position;
    at the first mismatch emit the target's argmax and stop; if all match emit
    the argmax at the bonus position."""
    out = []
    for i, x in enumerate(drafts):
        t = int(np.argmax(np.asarray(target_rows[i], np.float64)))
        if int(x) != t:
            out.append(t)
            return out
        out.append(int(x))
    out.append(int(np.argmax(np.asarray(target_rows[len(drafts)], np.float64))))
    return out
