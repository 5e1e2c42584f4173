"""The step (tree attention, stochastic verification, KV compaction; as three calls
and as attention plus the verify-and-compact call) captured as a HIP graph and
replayed: every replay, with eager calls and synchronisations between
the replays, gives exactly the eager results (the verifiers' workspaces and the
attention workspace are reused across replays, so this also checks that every call
leaves them as the next one expects)."""
import numpy as np
import pytest
import torch

from devdata import DevWorkload
from tree_verification_amd import binding as tv
from tree_verification_amd.workloads import make_workload

pytestmark = pytest.mark.gpu


def outputs(dw, k, v):
    B, n_max = dw.tokens.shape
    dev = dw.q.device
    o = dict(out=torch.empty_like(dw.q), ast=torch.empty(B, dtype=torch.int32, device=dev),
             path=torch.empty((B, n_max), dtype=torch.int32, device=dev),
             plen=torch.empty(B, dtype=torch.int32, device=dev),
             otok=torch.empty((B, n_max), dtype=torch.int32, device=dev),
             vst=torch.empty(B, dtype=torch.int32, device=dev),
             src=torch.empty((B, n_max), dtype=torch.int32, device=dev),
             nlen=torch.empty(B, dtype=torch.int32, device=dev),
             cst=torch.empty(B, dtype=torch.int32, device=dev), k=k, v=v)
    reset(o)
    return o


def reset(o):
    """Known contents in every output (entries a call leaves unwritten compare equal)."""
    for key, t in o.items():
        if key not in ("k", "v"):
            t.fill_(0 if key == "out" else -7)


def step(dw, o, fused):
    tv.tree_attn_forward(dw.q, o["k"], o["v"], dw.table, dw.prefix_len, dw.n_nodes, dw.parent, out=o["out"],
                         status=o["ast"])
    if fused:
        tv.tree_verify_stochastic_compact(dw.target, dw.draft, dw.tokens, dw.parent, dw.n_nodes, dw.u_accept,
                                          dw.u_sample, o["k"], o["v"], dw.table, dw.prefix_len, path=o["path"],
                                          path_len=o["plen"], out_tokens=o["otok"], status=o["vst"],
                                          src_pos=o["src"], new_len=o["nlen"], kv_status=o["cst"])
        return
    tv.tree_verify_stochastic(dw.target, dw.draft, dw.tokens, dw.parent, dw.n_nodes, dw.u_accept, dw.u_sample,
                              path=o["path"], path_len=o["plen"], out_tokens=o["otok"], status=o["vst"])
    tv.kv_compact_accepted(o["k"], o["v"], dw.table, dw.prefix_len, o["path"], o["plen"], src_pos=o["src"],
                           new_len=o["nlen"], status=o["cst"])


def snapshot(o):
    return {key: t.clone() for key, t in o.items()}


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name", ["tiny", "llama8b"])
def test_step_graph_replays_match_eager(name, fused):
    wl = make_workload(name)
    dw = DevWorkload(wl)
    k0, v0 = dw.k.clone(), dw.v.clone()
    # eager reference on its own cache copy
    ref = outputs(dw, k0.clone(), v0.clone())
    step(dw, ref, fused)
    torch.cuda.synchronize()
    ref = snapshot(ref)
    assert int(ref["ast"].abs().sum()) == 0 and int(ref["vst"].abs().sum()) == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g_out = outputs(dw, k0.clone(), v0.clone())
    with torch.cuda.stream(side):
        step(dw, g_out, fused)   # eager warm-up: the side stream's workspaces
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step(dw, g_out, fused)
    torch.cuda.synchronize()

    other = outputs(dw, k0.clone(), v0.clone())
    for rep in range(4):
        # the graph's caches back to the pristine prefix + tree (compaction moved slots)
        g_out["k"].copy_(k0)
        g_out["v"].copy_(v0)
        reset(g_out)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key, t in ref.items():
            assert torch.equal(g_out[key], t), (name, rep, key)
        # eager work between the replays, on the default stream and its workspaces
        other["k"].copy_(k0)
        other["v"].copy_(v0)
        reset(other)
        step(dw, other, fused)
        torch.cuda.synchronize()
        for key, t in ref.items():
            assert torch.equal(other[key], t), (name, rep, "eager", key)
