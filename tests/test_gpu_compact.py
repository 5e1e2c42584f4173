"""GPU parity of accepted-path KV compaction: caches, src_pos and new_len bit-exact."""
import numpy as np
import pytest
import torch

from devdata import DevWorkload
from oracle.kv import kv_compact
from tree_verification_amd import binding as tv
from tree_verification_amd.workloads import make_workload

pytestmark = pytest.mark.gpu


def random_root_paths(wl, rng):
    path = np.full((wl.batch, wl.n_max), -1, dtype=np.int32)
    plen = np.zeros(wl.batch, dtype=np.int32)
    for b in range(wl.batch):
        n = int(wl.n_nodes[b])
        p = [0]
        while True:
            kids = [c for c in range(n) if wl.parent[b, c] == p[-1]]
            if not kids or rng.random() < 0.15:
                break
            p.append(kids[int(rng.integers(len(kids)))])
        path[b, :len(p)] = p
        plen[b] = len(p)
    return path, plen


def run_case(wl, path, plen):
    d = DevWorkload(wl, logits=False)
    pt = torch.from_numpy(path).cuda()
    pl = torch.from_numpy(plen).cuda()
    src, new_len, st = tv.kv_compact_accepted(d.k, d.v, d.table, d.prefix_len, pt, pl)
    torch.cuda.synchronize()
    kref, vref, sref, nref, stref = kv_compact(wl.k_cache, wl.v_cache, wl.block_table, wl.prefix_len,
                                               path, plen, block_size=wl.block_size,
                                               num_blocks=wl.num_blocks, n_max=wl.n_max)
    assert np.array_equal(st.cpu().numpy(), stref)
    assert np.array_equal(src.cpu().numpy(), sref)
    assert np.array_equal(new_len.cpu().numpy(), nref)
    assert np.array_equal(d.k.float().cpu().numpy(), kref)
    assert np.array_equal(d.v.float().cpu().numpy(), vref)


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("llama8b", dict(prefix=2048)),
    ("ragged", dict(batch=8, prefix=(30, 900))),
    ("chain", dict(batch=32, prefix=100)),
    ("llama70b_share", dict(batch=2, prefix=77)),
    ("llama8b", dict(prefix=5, n_nodes=128, tree="chain")),     # paths longer than one staging batch
])
def test_compact_random_paths(name, kw):
    wl = make_workload(name, seed=13, with_logits=False, **kw)
    path, plen = random_root_paths(wl, np.random.default_rng(3))
    if kw.get("tree") == "chain":
        plen[:] = wl.n_nodes
        path[0, :wl.n_max] = np.arange(wl.n_max)
    run_case(wl, path, plen)


def test_compact_adversarial_paths():
    """Paths that shift every slot by one, skip the first child, and the leftmost
    (copy-free) path, plus zero-length and malformed paths."""
    wl = make_workload("llama8b", seed=17, with_logits=False, batch=6, prefix=(31, 33), n_nodes=20,
                       tree="chain")
    path = np.full((6, wl.n_max), -1, dtype=np.int32)
    plen = np.zeros(6, dtype=np.int32)
    path[0, :5] = [0, 1, 2, 3, 4]            # leftmost: nothing moves
    plen[0] = 5
    wl.parent[1, :20] = [-1] + [0] * 19      # star: path [0, 7] moves one slot
    path[1, :2] = [0, 7]
    plen[1] = 2
    path[2, :4] = [0, 2, 3, 4]               # reads P+3 which is written by a later step
    plen[2] = 4
    plen[3] = 0                              # verification failed: untouched
    path[4, :3] = [0, 5, 3]                  # not increasing: rejected
    plen[4] = 3
    path[5, :2] = [1, 2]                     # does not start at the root
    plen[5] = 2
    run_case(wl, path, plen)


def test_compact_fp32_block_sizes():
    from tree_verification_amd import workloads as W
    for bs in (16, 64):
        W.CONFIGS["_k"] = dict(W.CONFIGS["tiny"], block_size=bs, paged=True, n_kv_heads=2, n_q_heads=2)
        W.CONFIG_ORDER.append("_k")
        try:
            wl = make_workload("_k", seed=bs, with_logits=False, batch=5, prefix=(10, 200), n_nodes=12)
        finally:
            W.CONFIG_ORDER.remove("_k")
            del W.CONFIGS["_k"]
        path, plen = random_root_paths(wl, np.random.default_rng(bs))
        run_case(wl, path, plen)
