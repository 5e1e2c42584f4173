"""GPU parity of the speculative-block pool: tables, block counts, the free stack,
its count, spec_from and status bit-exact against the oracle, call after call."""
import numpy as np
import pytest
import torch

from oracle import BAD_KV, POOL_EXHAUSTED
from oracle.pool import alloc_tree_blocks, release_blocks
from tree_verification_amd import binding as tv

pytestmark = pytest.mark.gpu


class DevPool:
    def __init__(self, table, nblk, free, count):
        self.table = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).cuda()
        self.nblk = torch.from_numpy(np.ascontiguousarray(nblk, dtype=np.int32)).cuda()
        self.free = torch.from_numpy(np.ascontiguousarray(free, dtype=np.int32)).cuda()
        self.count = torch.tensor([count], dtype=torch.int32).cuda()

    def host(self):
        torch.cuda.synchronize()
        return (self.table.cpu().numpy(), self.nblk.cpu().numpy(), self.free.cpu().numpy(),
                int(self.count.cpu().item()))


def i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def alloc_both(dp, ref, P, n, bs, num_blocks):
    spec, st = tv.kv_alloc_tree_blocks(dp.table, dp.nblk, i32(P), i32(n), dp.free, dp.count, block_size=bs)
    t, nb, f, c, rspec, rst = alloc_tree_blocks(*ref[:2], P, n, ref[2], ref[3], block_size=bs,
                                                num_blocks=num_blocks)
    gt = dp.host()
    assert np.array_equal(st.cpu().numpy(), rst)
    assert np.array_equal(spec.cpu().numpy(), rspec)
    assert np.array_equal(gt[0], t) and np.array_equal(gt[1], nb)
    assert np.array_equal(gt[2], f) and gt[3] == c
    return (t, nb, f, c), rst


def release_both(dp, ref, new_len, bs, num_blocks):
    st = tv.kv_release_blocks(dp.table, dp.nblk, i32(new_len), dp.free, dp.count, block_size=bs)
    t, nb, f, c, rst = release_blocks(*ref[:2], new_len, ref[2], ref[3], block_size=bs, num_blocks=num_blocks)
    gt = dp.host()
    assert np.array_equal(st.cpu().numpy(), rst)
    assert np.array_equal(gt[0], t) and np.array_equal(gt[1], nb)
    assert np.array_equal(gt[2], f) and gt[3] == c
    return (t, nb, f, c), rst


@pytest.mark.parametrize("B,bs,max_blocks,spare,seed", [
    (1, 16, 8, 0, 1),
    (16, 16, 520, 64, 2),     # ragged-like: prefixes up to 8192 tokens in 16-token blocks
    (300, 4, 12, 0, 3),       # two passes of the batch
    (64, 1, 20, -200, 4),     # a pool smaller than the batch's needs: exhaustion
])
def test_serving_loop_matches_oracle(B, bs, max_blocks, spare, seed):
    print(f"case pool B={B} bs={bs} max_blocks={max_blocks} spare={spare}", flush=True)
    rng = np.random.default_rng(seed)
    num_blocks = max(1, B * max_blocks // 2 + spare)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    nblk = np.zeros(B, dtype=np.int32)
    free = rng.permutation(num_blocks).astype(np.int32)
    ref = (table, nblk, free, num_blocks)
    dp = DevPool(*ref)
    P = rng.integers(0, max_blocks * bs // 2, size=B).astype(np.int32)
    for step in range(6):
        n = rng.integers(1, 2 * bs + 3, size=B).astype(np.int32)
        ref, st = alloc_both(dp, ref, P, n, bs, num_blocks)
        nblk = ref[1]
        ok = st == 0
        new_len = np.where(ok, np.minimum(P + rng.integers(1, n + 1), nblk * bs), P).astype(np.int32)
        new_len = np.minimum(new_len, nblk * bs)
        ref, st2 = release_both(dp, ref, new_len, bs, num_blocks)
        assert (st2 == 0).all()
        P = new_len
    if spare < 0:
        assert (st == POOL_EXHAUSTED).any()


def test_pool_errors_match_oracle():
    bs, num_blocks, B, max_blocks = 2, 8, 6, 4
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    table[2, 0] = 7
    table[5, :2] = [6, 9]            # a bad id to release
    nblk = np.array([0, 0, 1, 0, 0, 2], dtype=np.int32)
    free = np.concatenate([np.arange(6), [-1, -1]]).astype(np.int32)
    ref = (table, nblk, free, 3)
    dp = DevPool(*ref)
    P = np.array([0, 0, 2, 0, -1, 2], dtype=np.int32)
    n = np.array([3, 4, 0, 1, 1, 0], dtype=np.int32)
    ref, st = alloc_both(dp, ref, P, n, bs, num_blocks)
    assert list(st) == [0, POOL_EXHAUSTED, 0, POOL_EXHAUSTED, BAD_KV, 0]
    ref, st = release_both(dp, ref, np.array([1, 0, 2, 0, 0, 0], dtype=np.int32), bs, num_blocks)
    assert st[5] == BAD_KV and st[0] == 0
    # a free count outside the pool fails every request and changes nothing
    dp.count.fill_(99)
    ref = ref[:3] + (99,)
    ref, st = alloc_both(dp, ref, P, n, bs, num_blocks)
    assert (st == BAD_KV).all()
