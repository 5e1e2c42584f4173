"""Pins of the oracle's accepted-path KV compaction (CPU only)."""
import itertools

import numpy as np
import pytest

from oracle import BAD_PATH
from oracle.attention import logical_kv, tree_attention
from oracle.kv import kv_compact


def paged_pool(rng, Hkv, D, lengths, bs, shuffle=True):
    need = [(L + bs - 1) // bs for L in lengths]
    nb = sum(need) + 2
    ids = rng.permutation(nb) if shuffle else np.arange(nb)
    kc = rng.standard_normal((nb, Hkv, bs, D))
    vc = rng.standard_normal((nb, Hkv, bs, D))
    table = np.full((len(lengths), max(need)), -1, dtype=np.int64)
    off = 0
    for b, k in enumerate(need):
        table[b, :k] = ids[off:off + k]
        off += k
    return kc, vc, table, nb


def root_paths(parent, n):
    """Every root path [0, c1, ..., cL] (parent[c_{j+1}] = c_j)."""
    out = [[0]]
    frontier = [[0]]
    while frontier:
        nxt = []
        for p in frontier:
            for c in range(n):
                if parent[c] == p[-1]:
                    nxt.append(p + [c])
        out += nxt
        frontier = nxt
    return out


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_all_paths_of_all_small_trees(n):
    rng = np.random.default_rng(10 + n)
    Hkv, D, bs = 2, 3, 4
    for tail in itertools.product(*[range(i) for i in range(1, n)]):
        parent = np.array((-1,) + tail)
        P = int(rng.integers(0, 9))
        kc, vc, table, nb = paged_pool(rng, Hkv, D, [P + n], bs)
        before = [logical_kv(kc, vc, table[0], P + n, g, bs) for g in range(Hkv)]
        for path in root_paths(parent, n):
            L1 = len(path)
            prow = np.full(n, -7)
            prow[:L1] = path
            k2, v2, src, new_len, st = kv_compact(kc, vc, table, np.array([P]), prow[None],
                                                  np.array([L1]), block_size=bs, num_blocks=nb, n_max=n)
            assert st[0] == 0 and new_len[0] == P + L1
            assert list(src[0, :L1]) == [P + c for c in path] and np.all(src[0, L1:] == -1)
            for g in range(Hkv):
                K, V = logical_kv(k2, v2, table[0], P + L1, g, bs)
                K0, V0 = before[g]
                sel = list(range(P)) + [P + c for c in path]
                np.testing.assert_array_equal(K, K0[sel])
                np.testing.assert_array_equal(V, V0[sel])
            # blocks outside the request's slots [P, P + n) are untouched
            mask = np.ones(nb, dtype=bool)
            mask[table[0][table[0] >= 0]] = False
            np.testing.assert_array_equal(k2[mask], kc[mask])


def test_compacted_causal_attention_equals_tree_attention():
    """After compaction the path is an ordinary causal sequence: the last path
    node's attention over [0, P + L + 1) equals its tree-attention output."""
    rng = np.random.default_rng(42)
    Hq, Hkv, D, bs, n, P = 4, 2, 8, 4, 9, 13
    parent = np.array([-1, 0, 1, 1, 0, 4, 5, 3, 2])
    kc, vc, table, nb = paged_pool(rng, Hkv, D, [P + n], bs)
    q = rng.standard_normal((1, n, Hq, D))
    tree_out, _ = tree_attention(q, kc, vc, table, np.array([P]), np.array([n]), parent[None],
                                 n_q_heads=Hq, n_kv_heads=Hkv, block_size=bs, num_blocks=nb,
                                 n_max=n, sm_scale=0.35)
    for path in root_paths(parent, n):
        L1 = len(path)
        prow = np.full(n, -1)
        prow[:L1] = path
        k2, v2, _, new_len, _ = kv_compact(kc, vc, table, np.array([P]), prow[None], np.array([L1]),
                                           block_size=bs, num_blocks=nb, n_max=n)
        last = path[-1]
        for h in range(Hq):
            K, V = logical_kv(k2, v2, table[0], int(new_len[0]), h // (Hq // Hkv), bs)
            s = K @ q[0, last, h] * 0.35
            w = np.exp(s - s.max())
            o = (w / w.sum()) @ V
            np.testing.assert_allclose(o, tree_out[0][last, h], rtol=0, atol=1e-12)


def test_zero_length_and_bad_paths_are_no_ops():
    rng = np.random.default_rng(5)
    kc, vc, table, nb = paged_pool(rng, 1, 2, [10, 10, 10], 4)
    path = np.array([[0, 1, 2], [0, 2, 1], [1, 2, 0]])
    plen = np.array([0, 3, 2])
    k2, v2, src, new_len, st = kv_compact(kc, vc, table, np.array([5, 5, 5]), path, plen,
                                          block_size=4, num_blocks=nb, n_max=3)
    assert list(st) == [0, BAD_PATH, BAD_PATH]
    assert list(new_len) == [5, 5, 5]
    assert np.all(src == -1)
    np.testing.assert_array_equal(k2, kc)
    np.testing.assert_array_equal(v2, vc)
