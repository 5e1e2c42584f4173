"""Pins of the oracle's speculative-block pool (CPU only).

The pool is pinned by conservation (every block id is, at every moment, either
mapped by exactly one table slot or on the free stack exactly once), by the
closed-form block counts ceil(positions / block), by positions below the kept
length never changing block, by the stack's last-in-first-out order, and by a
hand-worked exhaustion example.
"""
import numpy as np
import pytest

from oracle import BAD_KV, POOL_EXHAUSTED
from oracle.pool import alloc_tree_blocks, release_blocks


def ceil_div(a, b):
    return -(-a // b)


def check_conservation(table, nblk, free, free_count, num_blocks):
    seen = []
    for b in range(table.shape[0]):
        seen += [int(x) for x in table[b, :nblk[b]]]
        assert (table[b, nblk[b]:] == -1).all()
    seen += [int(x) for x in free[:free_count]]
    assert sorted(seen) == list(range(num_blocks))


@pytest.mark.parametrize("seed", range(15))
def test_serving_loop_conserves_blocks(seed):
    rng = np.random.default_rng(seed)
    B, bs, max_blocks = int(rng.integers(1, 9)), int(rng.choice([1, 4, 16])), 24
    num_blocks = B * max_blocks
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    nblk = np.zeros(B, dtype=np.int32)
    free = rng.permutation(num_blocks).astype(np.int32)
    count = num_blocks
    P = rng.integers(0, 5 * bs, size=B).astype(np.int32)
    for step in range(12):
        n = rng.integers(1, 3 * bs + 2, size=B).astype(np.int32)
        old = table.copy()
        t2, nb2, f2, c2, spec, st = alloc_tree_blocks(table, nblk, P, n, free, count, block_size=bs,
                                                      num_blocks=num_blocks)
        check_conservation(t2, nb2, f2, c2, num_blocks)
        for b in range(B):
            need = ceil_div(int(P[b] + n[b]), bs)
            if need > max_blocks:                      # the table cannot hold the tree
                assert st[b] == BAD_KV and nb2[b] == nblk[b] and spec[b] == -1
                continue
            assert st[b] == 0                          # the pool holds every table's worth
            assert nb2[b] == max(nblk[b], need)
            assert spec[b] == nblk[b]
            assert (t2[b, :nblk[b]] == old[b, :nblk[b]]).all()   # existing blocks untouched
        assert count - c2 == int((nb2 - nblk).sum())                  # one stack segment
        table, nblk, free, count = t2, nb2, f2, c2
        # verification keeps prefix + some accepted path; the rest is released
        new_len = np.minimum(P + rng.integers(1, n + 1), nblk * bs).astype(np.int32)
        new_len = np.maximum(new_len, np.minimum(P, nblk * bs))
        old = table.copy()
        t3, nb3, f3, c3, st3 = release_blocks(table, nblk, new_len, free, count, block_size=bs,
                                              num_blocks=num_blocks)
        assert (st3 == 0).all()
        check_conservation(t3, nb3, f3, c3, num_blocks)
        for b in range(B):
            keep = ceil_div(int(new_len[b]), bs)
            assert nb3[b] == keep
            assert (t3[b, :keep] == old[b, :keep]).all()               # kept positions keep their blocks
        assert c3 - count == int((nblk - nb3).sum())
        table, nblk, free, count, P = t3, nb3, f3, c3, new_len


def test_release_then_alloc_is_last_in_first_out():
    bs, num_blocks = 4, 10
    table = np.array([[3, 7, 1, 8, -1, -1]], dtype=np.int32)
    free = np.array([0, 2, 4, 5, 6, 9, -1, -1, -1, -1], dtype=np.int32)
    t, nb, f, c, st = release_blocks(table, np.array([4]), np.array([5]), free, 6, block_size=bs,
                                     num_blocks=num_blocks)
    assert st[0] == 0 and list(t[0]) == [3, 7, -1, -1, -1, -1] and nb[0] == 2
    assert list(f[:c]) == [0, 2, 4, 5, 6, 9, 1, 8]
    t, nb, f, c, spec, st = alloc_tree_blocks(t, nb, np.array([5]), np.array([9]), f, c, block_size=bs,
                                              num_blocks=num_blocks)
    assert st[0] == 0 and spec[0] == 2 and list(t[0]) == [3, 7, 8, 1, -1, -1] and c == 6


def test_exhaustion_and_bad_requests():
    bs, num_blocks = 2, 8
    B = 5
    table = np.full((B, 4), -1, dtype=np.int32)
    free = np.arange(num_blocks, dtype=np.int32)
    P = np.array([0, 0, 2, 0, -1], dtype=np.int32)
    n = np.array([3, 4, 0, 1, 1], dtype=np.int32)
    nblk = np.array([0, 0, 1, 0, 0], dtype=np.int32)
    table[2, 0] = 7
    free = np.arange(7, dtype=np.int32)
    t, nb, f, c, spec, st = alloc_tree_blocks(table, nblk, P, n, free, 3, block_size=bs, num_blocks=num_blocks)
    # request 0 takes 2 of the 3 free blocks; request 1 needs 2 more: exhausted;
    # request 2 needs none; request 3 needs 1 but comes after a failure; request 4 is malformed
    assert list(st) == [0, POOL_EXHAUSTED, 0, POOL_EXHAUSTED, BAD_KV]
    assert list(t[0, :2]) == [2, 1] and c == 1 and list(spec) == [0, -1, 1, -1, -1]
    t, nb, f, c, spec, st = alloc_tree_blocks(table, nblk, P, n, free, 9, block_size=bs, num_blocks=num_blocks)
    assert (st == BAD_KV).all()
    # a release that would overfill the stack
    t, nb, f, c, st = release_blocks(np.array([[0, 1], [2, 3]], dtype=np.int32), np.array([2, 2]),
                                     np.array([0, 2]), np.zeros(4, dtype=np.int32), 3, block_size=1,
                                     num_blocks=4)
    assert list(st) == [POOL_EXHAUSTED, 0] and c == 3   # the second request moves nothing
    t, nb, f, c, st = release_blocks(np.array([[0, 1]], dtype=np.int32), np.array([2]), np.array([3]),
                                     np.zeros(4, dtype=np.int32), 0, block_size=1, num_blocks=4)
    assert st[0] == BAD_KV                  # new_len beyond the mapped blocks
