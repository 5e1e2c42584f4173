"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (the whole batch in one call of each entry point): stochastic
and greedy verification of every request against the oracle (bit-exact paths
and tokens; stochastic requests may differ only inside the 1e-6 decision band),
then KV compaction of the GPU's accepted paths (caches, src_pos and new_len
bit-exact).  Full-size attention is covered on sampled rows in
test_gpu_attention.py."""
import numpy as np
import pytest
import torch

from devdata import DevWorkload
from oracle.kv import kv_compact
from oracle.verify import divergence_in_band, linear_greedy, linear_speculative, verify_greedy, verify_stochastic
from tree_verification_amd import binding as tv
from tree_verification_amd.workloads import make_workload

pytestmark = pytest.mark.gpu

FULL = ["llama8b", "ragged", "chain", "llama70b_share"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_verify_and_compact(name):
    wl = make_workload(name)
    print(f"case full-size {name}: B={wl.batch} n_max={wl.n_max} nodes={int(wl.n_nodes.sum())} V={wl.vocab}",
          flush=True)
    d = DevWorkload(wl)

    p, l, t, s = tv.tree_verify_stochastic(d.target, d.draft, d.tokens, d.parent, d.n_nodes, d.u_accept,
                                           d.u_sample)
    gp, gl, gs = p.cpu().numpy(), l.cpu().numpy(), s.cpu().numpy()
    gt = t.cpu().numpy()
    assert not gs.any()
    banded = 0
    band_ids = set()
    for b in range(wl.batch):
        sl = slice(b, b + 1)
        paths, outs, traces, st = verify_stochastic(wl.target_logits[sl], wl.draft_logits[sl], wl.tokens[sl],
                                                    wl.parent[sl], wl.n_nodes[sl], wl.u_accept[sl],
                                                    wl.u_sample[sl], wl.n_max)
        assert st[0] == 0
        L = int(gl[b])
        if list(gp[b, :L]) != paths[0] or list(gt[b, :L]) != outs[0]:
            assert divergence_in_band(traces[0], paths[0], outs[0], gp[b, :L], gt[b, :L]), (b, list(gp[b, :L]), paths[0])
            banded += 1
            band_ids.add(b)
    print(f"  stochastic: {wl.batch} requests, {banded} inside the decision band", flush=True)
    assert banded <= 1

    gp2, gl2, gt2, gs2 = (x.cpu().numpy() for x in tv.tree_verify_greedy(d.target, d.tokens, d.parent, d.n_nodes))
    rp, ro, rs = verify_greedy(wl.target_logits, wl.tokens, wl.parent, wl.n_nodes, wl.n_max)
    assert np.array_equal(gs2, rs)
    for b in range(wl.batch):
        L = int(gl2[b])
        assert list(gp2[b, :L]) == rp[b] and list(gt2[b, :L]) == ro[b], b
    print("  greedy: every request bit-exact", flush=True)

    if name == "chain":
        # a chain tree is linear speculative decoding on the same uniforms
        def softmax(z):
            e = np.exp(z.astype(np.float64) - float(z.max()))
            return e / e.sum()
        for b in range(wl.batch):
            n = int(wl.n_nodes[b])
            pr = [softmax(wl.target_logits[b, i]) for i in range(n)]
            qr = [softmax(wl.draft_logits[b, i]) for i in range(n - 1)]
            lin = linear_speculative(pr, qr, wl.tokens[b, 1:n], wl.u_accept[b, 1:n], wl.u_sample[b, :n])
            L = int(gl[b])
            assert b in band_ids or list(gt[b, :L]) == lin, b
            assert list(gt2[b, :int(gl2[b])]) == linear_greedy(wl.target_logits[b, :n], wl.tokens[b, 1:n]), b
        print("  chain: every request equals linear speculative decoding (stochastic and greedy)", flush=True)

    # compaction of the accepted paths the GPU chose
    path = np.full((wl.batch, wl.n_max), -1, dtype=np.int32)
    for b in range(wl.batch):
        path[b, :gl[b]] = gp[b, :gl[b]]
    src, new_len, cst = tv.kv_compact_accepted(d.k, d.v, d.table, d.prefix_len, torch.from_numpy(path).cuda(),
                                               l)
    torch.cuda.synchronize()
    kref, vref, sref, nref, stref = kv_compact(wl.k_cache, wl.v_cache, wl.block_table, wl.prefix_len, path, gl,
                                               block_size=wl.block_size, num_blocks=wl.num_blocks, n_max=wl.n_max)
    assert np.array_equal(cst.cpu().numpy(), stref) and not stref.any()
    assert np.array_equal(src.cpu().numpy(), sref)
    assert np.array_equal(new_len.cpu().numpy(), nref)
    assert np.array_equal(d.k.float().cpu().numpy(), kref)
    assert np.array_equal(d.v.float().cpu().numpy(), vref)
    print("  compaction: caches, src_pos and new_len bit-exact", flush=True)
