"""tree_verify_greedy_noalloc: the greedy verifier on the library's static
per-device scratch, for callers that cannot allocate.  Through the C ABI, two
calls in a row (the second with a smaller input, so it runs over what the first
left in the scratch) must equal tree_verify_greedy on a caller workspace bit for
bit, and the oracle's result too."""
import numpy as np
import pytest
import torch

from devdata import DevWorkload
from oracle.verify import verify_greedy
from tree_verification_amd import binding as tv
from tree_verification_amd.workloads import make_workload

pytestmark = pytest.mark.gpu


def _plant(wl, rng):
    # some children carry their parent's argmax, so paths run deeper than one node
    for b in range(wl.batch):
        for c in range(1, int(wl.n_nodes[b])):
            if rng.random() < 0.6:
                wl.tokens[b, c] = int(np.argmax(wl.target_logits[b, wl.parent[b, c]]))


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_workspace_entry_point(order):
    cases = [make_workload("ragged", seed=61, batch=6, prefix=(1, 2)),
             make_workload("llama8b", seed=62, vocab=30011, n_nodes=20, batch=3)]
    rng = np.random.default_rng(63)
    for i, wl in enumerate(cases):
        _plant(wl, rng)
        d = DevWorkload(wl)
        print(f"case noalloc call {i}: B={wl.batch} n_max={wl.n_max} V={wl.vocab}", flush=True)
        ref = tv.tree_verify_greedy(d.target, d.tokens, d.parent, d.n_nodes)
        got = tv.tree_verify_greedy_noalloc(d.target, d.tokens, d.parent, d.n_nodes)
        torch.cuda.synchronize()
        ref = [x.cpu().numpy() for x in ref]
        got = [x.cpu().numpy() for x in got]
        p0, l0, t0, s0 = ref
        p1, l1, t1, s1 = got
        assert np.array_equal(s0, s1) and not s1.any()
        assert np.array_equal(l0, l1)
        paths, outs, st = verify_greedy(wl.target_logits, wl.tokens, wl.parent, wl.n_nodes, wl.n_max)
        assert np.array_equal(s1, st)
        for b in range(wl.batch):
            L = int(l1[b])
            assert list(p1[b, :L]) == list(p0[b, :L]) == paths[b], b
            assert list(t1[b, :L]) == list(t0[b, :L]) == outs[b], b


def test_noalloc_nonfinite_after_clean_call():
    """A clean call, then one whose rows hold a NaN and an inf: the flags come
    from this call's rows only (nothing from the previous call's scratch)."""
    wl = make_workload("llama8b", seed=64, vocab=20000, n_nodes=16, batch=4)
    d = DevWorkload(wl)
    _, _, _, s = tv.tree_verify_greedy_noalloc(d.target, d.tokens, d.parent, d.n_nodes)
    torch.cuda.synchronize()
    assert not s.cpu().numpy().any()
    wl.target_logits[1, 3, 777] = np.nan
    wl.target_logits[2, 0, 19999] = np.inf
    d = DevWorkload(wl)
    _, _, _, s = tv.tree_verify_greedy_noalloc(d.target, d.tokens, d.parent, d.n_nodes)
    _, _, _, s_ref = tv.tree_verify_greedy(d.target, d.tokens, d.parent, d.n_nodes)
    torch.cuda.synchronize()
    assert list(s.cpu().numpy()) == list(s_ref.cpu().numpy()) == [0, tv.REQ_NONFINITE, tv.REQ_NONFINITE, 0]
