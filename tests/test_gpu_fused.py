"""GPU parity of the verify-and-compact call (tree_verify_stochastic_compact).

Each case runs the two separate calls (tree_verify_stochastic, then
kv_compact_accepted of its path) on one copy of the caches and the fused call on
another: every output must be bit-identical, the caches included.  The fused
results are also checked against the oracle directly: the path and tokens per
request (inside the 1e-6 decision band when they differ) and the caches,
src_pos and new_len of the oracle's compaction of the GPU's path."""
from types import SimpleNamespace

import numpy as np
import pytest

from devdata import DevWorkload, i32
from oracle.kv import kv_compact
from oracle.verify import divergence_in_band, verify_stochastic
from tree_verification_amd import binding as tv
from tree_verification_amd.workloads import make_workload

pytestmark = pytest.mark.gpu

_CACHE = {}


def _workload(name):
    """Each workload is generated once per module (the batched ones take seconds)."""
    if name not in _CACHE:
        _CACHE[name] = make_workload(name)
    return _CACHE[name]


def _both(d, table=None, prefix_len=None, parent=None):
    table = d.table if table is None else table
    prefix_len = d.prefix_len if prefix_len is None else prefix_len
    parent = d.parent if parent is None else parent
    k1, v1, k2, v2 = d.k.clone(), d.v.clone(), d.k.clone(), d.v.clone()
    p, l, t, s = tv.tree_verify_stochastic(d.target, d.draft, d.tokens, parent, d.n_nodes, d.u_accept, d.u_sample)
    src, nl, kst = tv.kv_compact_accepted(k1, v1, table, prefix_len, p, l)
    sep = [x.cpu().numpy() for x in (p, l, t, s, src, nl, kst, k1.float(), v1.float())]
    res = tv.tree_verify_stochastic_compact(d.target, d.draft, d.tokens, parent, d.n_nodes, d.u_accept, d.u_sample,
                                            k2, v2, table, prefix_len)
    fused = [x.cpu().numpy() for x in res] + [k2.float().cpu().numpy(), v2.float().cpu().numpy()]
    return sep, fused


NAMES = ["path", "path_len", "out_tokens", "status", "src_pos", "new_len", "kv_status", "k_cache", "v_cache"]


def _same(sep, fused, wl):
    for name, a, b in zip(NAMES, sep, fused):
        if name == "path" or name == "out_tokens":   # entries past path_len are not outputs
            L = sep[1]
            for r in range(wl.batch):
                assert np.array_equal(a[r, :L[r]], b[r, :L[r]]), (name, r)
        else:
            assert np.array_equal(a, b), name


@pytest.mark.parametrize("name", ["tiny", "llama8b", "ragged", "chain", "llama70b_share"])
def test_fused_equals_separate_calls(name):
    wl = _workload(name)
    print(f"case fused {name}: B={wl.batch} n_max={wl.n_max} V={wl.vocab}", flush=True)
    d = DevWorkload(wl)
    sep, fused = _both(d)
    assert not sep[3].any() and not sep[6].any()
    _same(sep, fused, wl)


@pytest.mark.parametrize("name", ["tiny", "llama8b"])
def test_fused_against_the_oracle(name):
    wl = _workload(name)
    print(f"case fused-oracle {name}", flush=True)
    d = DevWorkload(wl)
    res = tv.tree_verify_stochastic_compact(d.target, d.draft, d.tokens, d.parent, d.n_nodes, d.u_accept,
                                            d.u_sample, d.k, d.v, d.table, d.prefix_len)
    gp, gl, gt, gs, src, nl, kst = (x.cpu().numpy() for x in res)
    assert not gs.any() and not kst.any()
    banded = 0
    for b in range(wl.batch):
        sl = slice(b, b + 1)
        paths, outs, traces, st = verify_stochastic(wl.target_logits[sl], wl.draft_logits[sl], wl.tokens[sl],
                                                    wl.parent[sl], wl.n_nodes[sl], wl.u_accept[sl],
                                                    wl.u_sample[sl], wl.n_max)
        L = int(gl[b])
        if list(gp[b, :L]) != paths[0] or list(gt[b, :L]) != outs[0]:
            assert divergence_in_band(traces[0], paths[0], outs[0], gp[b, :L], gt[b, :L]), b
            banded += 1
    assert banded <= 1
    path = np.full((wl.batch, wl.n_max), -1, dtype=np.int32)
    for b in range(wl.batch):
        path[b, :gl[b]] = gp[b, :gl[b]]
    kref, vref, sref, nref, stref = kv_compact(wl.k_cache, wl.v_cache, wl.block_table, wl.prefix_len, path, gl,
                                               block_size=wl.block_size, num_blocks=wl.num_blocks, n_max=wl.n_max)
    assert np.array_equal(kst, stref) and np.array_equal(src, sref) and np.array_equal(nl, nref)
    assert np.array_equal(d.k.float().cpu().numpy(), kref)
    assert np.array_equal(d.v.float().cpu().numpy(), vref)


@pytest.mark.parametrize("batch", [4, 8])
def test_fused_failed_requests(batch):
    """Requests that fail verification (n_nodes out of range, a malformed parent
    array, a non-finite target logit, a token outside the vocabulary) get path_len
    0, so their caches stay and new_len = prefix_len; a request whose block table
    names a block outside the pool fails compaction (kv_status BAD_KV).  The
    fused call and the two separate calls agree on every output."""
    wl = make_workload("llama8b", seed=71, vocab=2003, n_nodes=10, batch=batch)
    print(f"case fused failed requests ({batch} requests, vocabulary 2003)", flush=True)
    want = [0] * batch
    kv_want = [0] * batch
    if batch == 4:
        wl.n_nodes[1] = wl.n_max + 1
        wl.parent[2, 4] = 4
        want[1], want[2] = tv.REQ_BAD_NNODES, tv.REQ_BAD_PARENT
        bad_kv = 3
    else:
        wl.n_nodes[1] = 0
        wl.n_nodes[2] = wl.n_max + 1
        wl.parent[3, 4] = 4
        wl.target_logits[4, 3, 17] = np.nan
        wl.tokens[6, 1] = wl.vocab
        want[1:7] = [tv.REQ_BAD_NNODES, tv.REQ_BAD_NNODES, tv.REQ_BAD_PARENT, tv.REQ_NONFINITE, 0,
                     tv.REQ_BAD_TOKEN]
        bad_kv = 7
    table = wl.block_table.copy()
    table[bad_kv, 0] = wl.num_blocks + 7       # outside the pool
    kv_want[bad_kv] = tv.REQ_BAD_KV
    d = DevWorkload(wl)
    sep, fused = _both(d, table=i32(table, "cuda:0"))
    assert list(sep[3]) == want and list(sep[6]) == kv_want
    assert all(sep[1][b] == 0 for b in range(batch) if want[b])
    _same(sep, fused, wl)


def test_fused_repeated_calls_and_smaller_batch():
    """Repeated calls reuse the workspace's exchange slots and result words (each
    call leaves them cleared): a second call, and calls on the first 5 and then
    the first 3 requests, give the separate calls' results."""
    wl = _workload("ragged")
    print("case fused repeated calls (ragged, then its first 5 and 3 requests)", flush=True)
    d = DevWorkload(wl)
    for _ in range(2):
        sep, fused = _both(d)
        _same(sep, fused, wl)
    for nb in (5, 3):
        d.target, d.draft = d.target[:nb].contiguous(), d.draft[:nb].contiguous()
        for f in ("tokens", "parent", "u_accept", "u_sample", "table", "n_nodes", "prefix_len"):
            setattr(d, f, getattr(d, f)[:nb].contiguous())
        sep, fused = _both(d)
        _same(sep, fused, SimpleNamespace(batch=nb))


@pytest.mark.parametrize("bs", [16, 64])
def test_fused_fp32_paged_block_sizes(bs):
    """float32 caches, paged block tables (blocks scattered over the pool), two KV
    heads, block sizes 16 and 64, short and long prefixes: the fused kernel
    (3 requests) against the separate calls."""
    from tree_verification_amd import workloads as W
    W.CONFIGS["_f"] = dict(W.CONFIGS["tiny"], block_size=bs, paged=True, n_kv_heads=2, n_q_heads=2)
    W.CONFIG_ORDER.append("_f")
    try:
        wl = make_workload("_f", seed=100 + bs, batch=3, prefix=(10, 200), n_nodes=12)
    finally:
        W.CONFIG_ORDER.remove("_f")
        del W.CONFIGS["_f"]
    print(f"case fused fp32 paged block_size={bs}", flush=True)
    d = DevWorkload(wl)
    sep, fused = _both(d)
    assert not sep[3].any() and not sep[6].any()
    assert (sep[1] > 1).any()            # some request moves K/V
    _same(sep, fused, wl)


def test_fused_unaligned_caches():
    """Caches that start 2 bytes past an 8-byte boundary: the fused call then
    compacts with single-element moves in the compaction's own kernel; every
    output still equals the separate calls'."""
    import torch
    wl = make_workload("tiny", seed=321, batch=2)
    print("case fused unaligned caches", flush=True)
    d = DevWorkload(wl)

    def shifted(x):
        buf = torch.empty(x.numel() + 1, dtype=x.dtype, device=x.device)
        y = buf[1:].view(x.shape)
        y.copy_(x)
        assert y.data_ptr() % 8 != 0
        return y

    k1, v1, k2, v2 = d.k.clone(), d.v.clone(), shifted(d.k), shifted(d.v)
    p, l, t, s = tv.tree_verify_stochastic(d.target, d.draft, d.tokens, d.parent, d.n_nodes, d.u_accept, d.u_sample)
    src, nl, kst = tv.kv_compact_accepted(k1, v1, d.table, d.prefix_len, p, l)
    sep = [x.cpu().numpy() for x in (p, l, t, s, src, nl, kst, k1.float(), v1.float())]
    res = tv.tree_verify_stochastic_compact(d.target, d.draft, d.tokens, d.parent, d.n_nodes, d.u_accept,
                                            d.u_sample, k2, v2, d.table, d.prefix_len)
    fused = [x.cpu().numpy() for x in res] + [k2.float().cpu().numpy(), v2.float().cpu().numpy()]
    assert not sep[3].any() and not sep[6].any()
    assert (sep[1] > 1).any()            # some request moves K/V
    _same(sep, fused, wl)
