"""CPU pin of the attention parity check's sensitivity to the tree mask.

At full size (prefix 2048 and 32768) one wrong ancestor bit among thousands of
prefix keys moves an N(0, 1) row by about 1 %, inside the 2e-2 tolerance.  The
GPU parity tests therefore add a workload whose queries make the tree keys
dominate each row's softmax (workloads.dominate_tree_keys).  Here the oracle's
own output for a parent array with one edge moved is shown to fail the check
on that workload, while the correct output rounded to bf16 (what the GPU
returns at best) passes it.
"""
import numpy as np
import pytest

from attn_check import TOL, passes, row_errors
from oracle.attention import tree_attention
from oracle.tree import validate
from tree_verification_amd.workloads import dominate_tree_keys, make_workload, round_to_bf16


def subtree(parent, n, c):
    out = [c]
    for i in range(c + 1, n):
        if parent[i] in out:
            out.append(i)
    return out


def depth_of(parent, u):
    d = 0
    while u > 0:
        u = int(parent[u])
        d += 1
    return d


def oracle_rows(wl, parent, rows):
    out, st = tree_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.prefix_len, wl.n_nodes,
                             parent, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                             block_size=wl.block_size, num_blocks=wl.num_blocks, n_max=wl.n_max,
                             sm_scale=wl.sm_scale, requests=[0], rows={0: rows})
    assert st[0] == 0
    return np.stack([out[0][u, h] for u, h in rows])


@pytest.mark.parametrize("name,prefix", [("llama8b", None), ("llama70b_share", 32768)])
@pytest.mark.parametrize("move", ["to_root", "deeper"])
def test_check_rejects_one_moved_edge(name, prefix, move):
    wl = make_workload(name, seed=77, with_logits=False, batch=1, prefix=prefix)
    dominate_tree_keys(wl, seed=78)
    n = int(wl.n_nodes[0])
    par = wl.parent[0]
    rng = np.random.default_rng(79)
    # a node at depth >= 2 (moving it to the root drops ancestors), or a node
    # whose new parent is deeper than its old one (adds ancestors)
    if move == "to_root":
        cands = [c for c in range(2, n) if depth_of(par, c) >= 2]
        c = int(rng.choice(cands))
        newp = 0
    else:
        cands = [(c, p) for c in range(2, n) for p in range(1, c)
                 if p != par[c] and c not in subtree(par, n, p) and depth_of(par, p) >= depth_of(par, c)]
        c, newp = cands[int(rng.integers(len(cands)))]
    moved = wl.parent.copy()
    moved[0, c] = newp
    assert validate(moved[0], n, wl.n_max) == 0
    heads = rng.choice(wl.n_q_heads, size=4, replace=False)
    rows = [(u, int(h)) for u in subtree(par, n, c) for h in heads]
    ref = oracle_rows(wl, wl.parent, rows)
    wrong = oracle_rows(wl, moved, rows)
    tol = TOL[wl.dtype]
    # the correct rows rounded to bf16 pass; every affected row of the moved
    # parent array fails the check
    assert passes(round_to_bf16(ref.astype(np.float32)), ref, tol)
    row, elem = row_errors(wrong, ref)
    fails = (row > tol) | (elem > tol)
    assert fails.all(), (float(row.min()), float(elem.min()))
