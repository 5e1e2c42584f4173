"""Pins of the oracle's tree attention (CPU only).

The oracle is compared with torch's scaled_dot_product_attention (float64, CPU)
on special cases where tree attention reduces to a textbook form: a chain tree
is causal attention over prefix + chain, a one-node tree is plain decode
attention, and any tree equals SDPA under the ancestor relation computed by
transitive closure (an algorithm independent of the oracle's parent walk).
"""
import numpy as np
import pytest
import torch

from oracle import BAD_KV
from oracle.attention import tree_attention
from tree_verification_amd.workloads import random_tree


def closure(parent, n):
    R = np.eye(n, dtype=bool)
    for c in range(1, n):
        R[c, parent[c]] = True
    for k in range(n):
        R = R | (R[:, [k]] & R[[k], :])
    return R


def scatter_paged(rng, Kl, Vl, block_size, shuffle=True, spare=3):
    """Lay logical per-request sequences Kl[b] / Vl[b] ([Hkv][L_b][D]) into a paged
    pool: K and V blocks [Hkv][bs][D]; returns caches + table."""
    B = len(Kl)
    Hkv, _, D = Kl[0].shape
    need = [(k.shape[1] + block_size - 1) // block_size for k in Kl]
    nb = sum(need) + spare
    ids = rng.permutation(nb) if shuffle else np.arange(nb)
    kc = rng.standard_normal((nb, Hkv, block_size, D))
    vc = rng.standard_normal((nb, Hkv, block_size, D))
    table = np.full((B, max(need)), -1, dtype=np.int64)
    off = 0
    for b in range(B):
        table[b, :need[b]] = ids[off:off + need[b]]
        off += need[b]
        for pos in range(Kl[b].shape[1]):
            blk, slot = table[b, pos // block_size], pos % block_size
            kc[blk, :, slot, :] = Kl[b][:, pos, :]
            vc[blk, :, slot, :] = Vl[b][:, pos, :]
    return kc, vc, table, nb


def sdpa_rows(q, K, V, allowed, scale, G):
    """q [n][Hq][D]; K/V [Hkv][L][D]; allowed [n][L] bool -> [n][Hq][D]."""
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]          # 1,Hq,n,D
    kt = torch.from_numpy(K).repeat_interleave(G, dim=0)[None]                        # 1,Hq,L,D
    vt = torch.from_numpy(V).repeat_interleave(G, dim=0)[None]
    m = torch.from_numpy(allowed)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o[0].numpy().transpose(1, 0, 2)


def run_case(rng, parents, prefixes, Hq, Hkv, D, bs=16, shuffle=True):
    B = len(parents)
    ns = [len(p) for p in parents]
    n_max = max(ns)
    q = rng.standard_normal((B, n_max, Hq, D))
    Kl = [rng.standard_normal((Hkv, P + n, D)) for P, n in zip(prefixes, ns)]
    Vl = [rng.standard_normal((Hkv, P + n, D)) for P, n in zip(prefixes, ns)]
    kc, vc, table, nb = scatter_paged(rng, Kl, Vl, bs, shuffle)
    parent = np.full((B, n_max), -1)
    for b in range(B):
        parent[b, :ns[b]] = parents[b]
    scale = 1.0 / np.sqrt(D)
    outs, st = tree_attention(q, kc, vc, table, np.array(prefixes), np.array(ns), parent,
                              n_q_heads=Hq, n_kv_heads=Hkv, block_size=bs, num_blocks=nb,
                              n_max=n_max, sm_scale=scale)
    assert np.all(st == 0)
    G = Hq // Hkv
    for b in range(B):
        P, n = prefixes[b], ns[b]
        allowed = np.zeros((n, P + n), dtype=bool)
        allowed[:, :P] = True
        allowed[:, P:] = closure(parents[b], n)
        ref = sdpa_rows(q[b, :n], Kl[b], Vl[b], allowed, scale, G)
        np.testing.assert_allclose(outs[b], ref, rtol=0, atol=1e-12)
    return outs


def test_chain_is_causal_attention():
    rng = np.random.default_rng(1)
    n, P, Hq, Hkv, D = 6, 37, 4, 2, 16
    chain = np.arange(-1, n - 1)
    outs = run_case(rng, [chain], [P], Hq, Hkv, D)
    # independently: causal mask by position (query at P+i sees keys <= P+i)
    assert outs[0].shape == (n, Hq, D)


def test_chain_equals_positional_causal_mask():
    rng = np.random.default_rng(2)
    n, P, Hq, Hkv, D = 5, 20, 2, 1, 8
    q = rng.standard_normal((1, n, Hq, D))
    K = rng.standard_normal((Hkv, P + n, D))
    V = rng.standard_normal((Hkv, P + n, D))
    kc, vc, table, nb = scatter_paged(rng, [K], [V], 16)
    outs, st = tree_attention(q, kc, vc, table, np.array([P]), np.array([n]),
                              np.arange(-1, n - 1)[None], n_q_heads=Hq, n_kv_heads=Hkv,
                              block_size=16, num_blocks=nb, n_max=n, sm_scale=0.3)
    pos = np.arange(P + n)
    allowed = pos[None, :] <= (P + np.arange(n))[:, None]
    ref = sdpa_rows(q[0], K, V, allowed, 0.3, Hq // Hkv)
    np.testing.assert_allclose(outs[0], ref, rtol=0, atol=1e-12)


def test_single_node_is_decode_attention():
    rng = np.random.default_rng(3)
    P, Hq, Hkv, D = 50, 8, 2, 32
    q = rng.standard_normal((1, 1, Hq, D))
    K = rng.standard_normal((Hkv, P + 1, D))
    V = rng.standard_normal((Hkv, P + 1, D))
    kc, vc, table, nb = scatter_paged(rng, [K], [V], 16)
    outs, _ = tree_attention(q, kc, vc, table, np.array([P]), np.array([1]), np.array([[-1]]),
                             n_q_heads=Hq, n_kv_heads=Hkv, block_size=16, num_blocks=nb,
                             n_max=1, sm_scale=1 / np.sqrt(D))
    ref = sdpa_rows(q[0], K, V, np.ones((1, P + 1), dtype=bool), 1 / np.sqrt(D), Hq // Hkv)
    np.testing.assert_allclose(outs[0], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kind", ["capped", "recursive", "star", "chain"])
def test_random_trees_batched_gqa(kind):
    rng = np.random.default_rng(4)
    parents = [random_tree(rng, n, kind, 3, 4) for n in (1, 5, 9, 13)]
    prefixes = [0, 17, 32, 5]
    run_case(rng, parents, prefixes, Hq=6, Hkv=3, D=16)


def test_zero_prefix_pure_tree():
    rng = np.random.default_rng(5)
    parents = [random_tree(rng, 12, "recursive")]
    run_case(rng, parents, [0], Hq=2, Hkv=2, D=8, bs=4)


def test_layout_invariance_identity_vs_shuffled():
    rng = np.random.default_rng(6)
    parents = [random_tree(rng, 7, "capped", 2, 3), random_tree(rng, 4, "chain")]
    a = run_case(np.random.default_rng(9), parents, [30, 3], 4, 2, 8, shuffle=True)
    b = run_case(np.random.default_rng(9), parents, [30, 3], 4, 2, 8, shuffle=False)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_relabel_invariance():
    """Renumbering nodes in another topological order permutes outputs identically."""
    rng = np.random.default_rng(7)
    n, P, Hq, Hkv, D = 9, 11, 2, 1, 8
    parent = random_tree(rng, n, "recursive")
    # another topological order: breadth-first
    order = [0]
    i = 0
    while i < len(order):
        order += [c for c in range(n) if parent[c] == order[i]]
        i += 1
    order = np.array(order)                 # order[new] = old
    new_of = np.empty(n, dtype=int)
    new_of[order] = np.arange(n)
    parent2 = np.array([-1] + [new_of[parent[order[k]]] for k in range(1, n)])
    q = rng.standard_normal((1, n, Hq, D))
    K = rng.standard_normal((Hkv, P + n, D))
    V = rng.standard_normal((Hkv, P + n, D))
    K2, V2 = K.copy(), V.copy()
    K2[:, P:] = K[:, P + order]
    V2[:, P:] = V[:, P + order]
    q2 = q[:, order]
    outs = []
    for qq, KK, VV, pp in ((q, K, V, parent), (q2, K2, V2, parent2)):
        kc, vc, table, nb = scatter_paged(np.random.default_rng(0), [KK], [VV], 4)
        o, _ = tree_attention(qq, kc, vc, table, np.array([P]), np.array([n]), pp[None],
                              n_q_heads=Hq, n_kv_heads=Hkv, block_size=4, num_blocks=nb,
                              n_max=n, sm_scale=0.5)
        outs.append(o[0])
    np.testing.assert_allclose(outs[1], outs[0][order], rtol=0, atol=1e-13)


def test_bad_block_table_flags():
    rng = np.random.default_rng(8)
    K = rng.standard_normal((1, 20, 4))
    V = rng.standard_normal((1, 20, 4))
    kc, vc, table, nb = scatter_paged(rng, [K], [V], 8, spare=0)
    table[0, 1] = nb  # out of pool
    _, st = tree_attention(rng.standard_normal((1, 2, 1, 4)), kc, vc, table, np.array([18]),
                           np.array([2]), np.array([[-1, 0]]), n_q_heads=1, n_kv_heads=1,
                           block_size=8, num_blocks=nb, n_max=2, sm_scale=0.5)
    assert st[0] == BAD_KV


def test_kv_status_cases():
    """The request-level KV checks, case by case against hand-worked answers:
    positions [0, P + n) need ceil((P + n) / bs) table entries, each naming a
    block inside the pool; a negative prefix is malformed."""
    from oracle.attention import kv_status
    row = np.array([3, 0, 5, -1, -1])          # three mapped blocks, two unused entries
    bs, nb = 8, 6
    assert kv_status(row, 0, 1, bs, nb) == 0             # one position: block 3
    assert kv_status(row, 20, 4, bs, nb) == 0            # 24 positions: exactly 3 blocks
    assert kv_status(row, 20, 5, bs, nb) == BAD_KV       # 25 positions: entry 3 is -1
    assert kv_status(row, -1, 2, bs, nb) == BAD_KV       # negative prefix
    assert kv_status(row, 39, 1, bs, nb) == BAD_KV       # 40 positions: 5 entries, two unmapped
    assert kv_status(row, 40, 1, bs, nb) == BAD_KV       # past the table (6 entries needed)
    assert kv_status(np.array([3, 6]), 9, 1, bs, nb) == BAD_KV   # block 6 outside a 6-block pool
    assert kv_status(np.array([3, 6]), 7, 1, bs, nb) == 0        # only block 3 is used
