"""Tree attention oracle (test infrastructure only).

[guide] "Generalizing Attention to Tree Topologies": node u attends with
weights alpha_{u,v} = softmax_v(Q_u K_v^T / sqrt(d_k) + M_{u,v}), where M is
the topology mask of "The Topology-Aware 2D Causal Mask".  Following
"Depth-First Flattening and KV Cache Reuse", the tree tokens' keys and values
sit in the same KV cache right after the request's prefix, at logical
positions [P, P + n).  Reading of the pages: every node also attends to all P
prefix positions (the verified context all candidates share), q-head h reads
KV head floor(h / G) with G = Hq / Hkv, and Q/K arrive already rotated.

Everything is widened to float64 exactly; the score vector is formed in full
(no tiling, no online softmax).
"""
from __future__ import annotations

import numpy as np

from . import BAD_KV
from .tree import topology_mask, validate


def logical_kv(k_cache, v_cache, table_row, length: int, g: int, block_size: int):
    """Contiguous K [length][D] and V [length][D] (float64) of one request and
    KV head, rebuilt through the block table.  Key and value blocks are both
    token-major, [Hkv][bs][D] (tree tokens append their rows to the cache)."""
    pos = np.arange(length)
    blk = np.asarray(table_row)[pos // block_size]
    slot = pos % block_size
    K = np.asarray(k_cache[blk, g, slot, :], dtype=np.float64)
    V = np.asarray(v_cache[blk, g, slot, :], dtype=np.float64)
    return K, V


def kv_status(table_row, P: int, n: int, block_size: int, num_blocks: int) -> int:
    """BAD_KV when positions [0, P + n) do not fit the request's block table or
    name a block outside the pool."""
    if P < 0:
        return BAD_KV
    length = P + n
    nblk = (length + block_size - 1) // block_size
    if nblk > len(table_row):
        return BAD_KV
    ids = np.asarray(table_row[:nblk])
    if np.any(ids < 0) or np.any(ids >= num_blocks):
        return BAD_KV
    return 0


def tree_attention_request(q_b, K_by_head, V_by_head, P: int, parent, n: int, sm_scale: float,
                           n_q_heads: int, n_kv_heads: int, rows=None) -> np.ndarray:
    """Outputs [n][Hq][D] (float64) of one request.

    q_b: [>=n][Hq][D]; K_by_head[g], V_by_head[g]: [P + n][D].
    rows: optional list of (u, h) pairs to compute; others are left NaN.
    """
    G = n_q_heads // n_kv_heads
    D = q_b.shape[-1]
    M = topology_mask(parent, n)
    out = np.full((n, n_q_heads, D), np.nan)
    want = None if rows is None else set((int(u), int(h)) for u, h in rows)
    for h in range(n_q_heads):
        g = h // G
        K, V = K_by_head[g], V_by_head[g]
        for u in range(n):
            if want is not None and (u, h) not in want:
                continue
            qv = np.asarray(q_b[u, h], dtype=np.float64)
            s = (K @ qv) * sm_scale            # every key: prefix then tree positions
            s[P:P + n] += M[u]                 # tree part: ancestors and self only
            s = s - s.max()
            w = np.exp(s)
            alpha = w / w.sum()
            out[u, h] = alpha @ V
    return out


def tree_attention(wl_q, k_cache, v_cache, block_table, prefix_len, n_nodes, parent, *,
                   n_q_heads: int, n_kv_heads: int, block_size: int, num_blocks: int,
                   n_max: int, sm_scale: float, requests=None, rows=None):
    """Batched oracle.  Returns (out, status): out[b] is [n_b][Hq][D] float64
    (None for a malformed request), status[b] the request's flags.

    requests: optional subset of request indices; rows: optional dict
    b -> list of (u, h) to compute (for sampled checks at full size).
    """
    B = len(prefix_len)
    outs = [None] * B
    status = np.zeros(B, dtype=np.int32)
    todo = range(B) if requests is None else requests
    for b in todo:
        n = int(n_nodes[b])
        st = validate(parent[b], n, n_max)
        if st == 0:
            st = kv_status(block_table[b], int(prefix_len[b]), n, block_size, num_blocks)
        status[b] = st
        if st:
            continue
        P = int(prefix_len[b])
        Ks, Vs = [], []
        for g in range(n_kv_heads):
            K, V = logical_kv(k_cache, v_cache, block_table[b], P + n, g, block_size)
            Ks.append(K)
            Vs.append(V)
        r = None if rows is None else rows.get(b, [])
        outs[b] = tree_attention_request(wl_q[b], Ks, Vs, P, parent[b], n, sm_scale,
                                         n_q_heads, n_kv_heads, rows=r)
    return outs, status
