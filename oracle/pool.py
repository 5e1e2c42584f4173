"""Paged speculative-block pool (test infrastructure only).

[guide] "PagedKV Allocation with Zero-Copy Pruning": the tree's KV goes into
blocks taken from the paged pool and marked speculative; once verification
has chosen the winning path, the blocks of the unselected branches go back to
the free pool in one metadata update.

Readings (the page gives no data structure; the design notes list these):
  - The free pool is a stack: free_ids[0 .. free_count) with the top at
    free_count - 1.  Allocation pops from the top, release pushes on top.
  - A request's table maps n_blocks blocks.  Allocation extends it to the
    ceil((prefix_len + n_nodes) / block) blocks that hold its prefix and its
    tree; the added blocks (from index n_blocks on) are the speculative ones.
  - Release keeps the ceil(new_len / block) blocks that hold the first new_len
    positions (new_len = prefix + accepted path after compaction) and returns
    every later block of the table.
  - Requests are served in batch order; pops and pushes of one call are one
    contiguous segment of the stack, so free_count changes once per call.  A
    request that the pool cannot serve (not enough free blocks, or a release
    that would overfill the stack) gets POOL_EXHAUSTED, and so does every later
    request that needs blocks moved.
"""
from __future__ import annotations

import numpy as np

from . import BAD_KV, POOL_EXHAUSTED


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def alloc_tree_blocks(block_table, n_blocks, prefix_len, n_nodes, free_ids, free_count: int, *,
                      block_size: int, num_blocks: int):
    """Returns (block_table, n_blocks, free_ids, free_count, spec_from, status), all new
    arrays; spec_from[b] is the first speculative table index (-1 when the request
    failed)."""
    table = np.array(block_table, dtype=np.int32, copy=True)
    nblk = np.array(n_blocks, dtype=np.int32, copy=True)
    free = np.array(free_ids, dtype=np.int32, copy=True)
    B, max_blocks = table.shape
    spec_from = np.full(B, -1, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    if not 0 <= free_count <= num_blocks:
        status[:] = BAD_KV
        return table, nblk, free, free_count, spec_from, status
    taken = 0          # blocks promised to earlier requests (served or not)
    served = 0         # blocks actually popped
    for b in range(B):
        P, n, nb = int(prefix_len[b]), int(n_nodes[b]), int(nblk[b])
        if P < 0 or n < 0 or not 0 <= nb <= max_blocks:
            status[b] = BAD_KV
            continue
        need = _ceil_div(P + n, block_size)
        if need > max_blocks:
            status[b] = BAD_KV
            continue
        extra = max(0, need - nb)
        taken += extra
        if extra > 0 and taken > free_count:
            status[b] = POOL_EXHAUSTED
            continue
        for j in range(extra):             # pop one block at a time from the top
            top = free_count - served - 1
            table[b, nb + j] = free[top]
            served += 1
        nblk[b] = nb + extra
        spec_from[b] = nb
    return table, nblk, free, free_count - served, spec_from, status


def release_blocks(block_table, n_blocks, new_len, free_ids, free_count: int, *, block_size: int,
                   num_blocks: int):
    """Returns (block_table, n_blocks, free_ids, free_count, status), all new arrays."""
    table = np.array(block_table, dtype=np.int32, copy=True)
    nblk = np.array(n_blocks, dtype=np.int32, copy=True)
    free = np.array(free_ids, dtype=np.int32, copy=True)
    B, max_blocks = table.shape
    status = np.zeros(B, dtype=np.int32)
    if not 0 <= free_count <= num_blocks:
        status[:] = BAD_KV
        return table, nblk, free, free_count, status
    promised = 0
    pushed = 0
    for b in range(B):
        L, nb = int(new_len[b]), int(nblk[b])
        if L < 0 or not 0 <= nb <= max_blocks:
            status[b] = BAD_KV
            continue
        keep = _ceil_div(L, block_size)
        if keep > nb:
            status[b] = BAD_KV
            continue
        ids = [int(x) for x in table[b, keep:nb]]
        if any(x < 0 or x >= num_blocks for x in ids):
            status[b] = BAD_KV
            continue
        promised += len(ids)
        if ids and free_count + promised > num_blocks:
            status[b] = POOL_EXHAUSTED
            continue
        for j, x in enumerate(ids):        # push in table order
            free[free_count + pushed] = x
            pushed += 1
            table[b, keep + j] = -1
        nblk[b] = keep
    return table, nblk, free, free_count + pushed, status
