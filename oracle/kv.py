"""Accepted-path KV compaction oracle (test infrastructure only).

[guide] "Depth-First Flattening and KV Cache Reuse": the tree tokens append
their keys and values to the active cache; after verification only the
winning path is kept and the rest is dropped by moving the sequence-length
pointer.  That is copy-free only when the winning path is the leftmost
depth-first path; in general the accepted nodes' K/V must be gathered to the
slots right after the prefix: slot P + j <- slot P + path[j] for
j = 0..L (path[0] = 0 is the root), and the new length is P + L + 1.  The
final emitted token has no K/V yet (the next round computes it).
"""
from __future__ import annotations

import numpy as np

from . import BAD_KV, BAD_PATH


def path_status(path_row, path_len: int, n_max: int, P: int, table_row, block_size: int,
                num_blocks: int) -> int:
    if path_len < 0 or path_len > n_max:
        return BAD_PATH
    if path_len == 0:
        return 0
    if int(path_row[0]) != 0:
        return BAD_PATH
    for j in range(1, path_len):
        if not (int(path_row[j - 1]) < int(path_row[j]) < n_max):
            return BAD_PATH
    if P < 0:
        return BAD_KV
    last = P + int(path_row[path_len - 1])
    nblk = last // block_size + 1
    if nblk > len(table_row):
        return BAD_KV
    ids = np.asarray(table_row[:nblk])
    if np.any(ids < 0) or np.any(ids >= num_blocks):
        return BAD_KV
    return 0


def kv_compact(k_cache, v_cache, block_table, prefix_len, path, path_len, *, block_size: int,
               num_blocks: int, n_max: int):
    """Returns (k_new, v_new, src_pos, new_len, status) without touching the inputs.

    K and V blocks are both token-major, [Hkv][bs][D].  A request whose
    path_len is 0 (verification failed) or whose path is malformed is left
    unchanged: new_len = prefix_len and src_pos = -1.
    """
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    B = len(prefix_len)
    src_pos = np.full((B, n_max), -1, dtype=np.int32)
    new_len = np.array(prefix_len, dtype=np.int32, copy=True)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        P = int(prefix_len[b])
        L1 = int(path_len[b])
        st = path_status(path[b], L1, n_max, P, block_table[b], block_size, num_blocks)
        status[b] = st
        if st or L1 == 0:
            continue
        srcs = [P + int(path[b][j]) for j in range(L1)]

        def loc(pos):
            return int(block_table[b][pos // block_size]), pos % block_size

        # read every source first, then write: a later source may sit in an
        # earlier destination slot
        k_src = [k[loc(s)[0], :, loc(s)[1], :].copy() for s in srcs]
        v_src = [v[loc(s)[0], :, loc(s)[1], :].copy() for s in srcs]
        for j in range(L1):
            blk, slot = loc(P + j)
            k[blk, :, slot, :] = k_src[j]
            v[blk, :, slot, :] = v_src[j]
            src_pos[b, j] = srcs[j]
        new_len[b] = P + L1
    return k, v, src_pos, new_len, status
