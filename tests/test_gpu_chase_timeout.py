"""An expired chase wait, forced from the host (TV_CHASE_SPIN_LIMIT, read once
per process, so the case runs in a child process): with a negative limit the
verifiers' path-chasing workgroups give up without polling, every request gets
TV_REQ_TIMEOUT, and the workspace is invalidated because node results may
still land in it; the next call on the same workspace reports
TV_REQ_BAD_WORKSPACE, and tree_verify_workspace_init makes it usable again;
verify-and-compact then moves no K/V and keeps every request's length.
Every workgroup still ends normally (the node and argmax workgroups finish
their own work).  The limit 0 polls once and must leave results either
complete or flagged.  Tree attention on a grid resident at once (its tiles'
key splits wait for each other before merging) and the tree expansion (each
request's workgroup waits for its rows' chunk results) follow the same
contract."""
import os
import subprocess
import sys
import textwrap

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = textwrap.dedent("""
    import sys
    sys.path.insert(0, {root!r})
    sys.path.insert(0, {tests!r})
    import ctypes
    import torch
    from devdata import DevWorkload
    from tree_verification_amd import binding as tv
    from tree_verification_amd.binding import VerifyDesc, load_library
    from tree_verification_amd.workloads import make_workload

    wl = make_workload("llama8b", seed=61, vocab=30011, n_nodes=20, batch=3)
    d = DevWorkload(wl)
    lib = load_library()
    desc = VerifyDesc()
    desc.batch, desc.n_max, desc.vocab, desc.temperature = wl.batch, wl.n_max, wl.vocab, 1.0
    need = lib.tree_verify_workspace_size(ctypes.byref(desc))
    for name in ("stochastic", "greedy", "compact"):
        ws = tv.init_verify_workspace(torch.zeros(need, dtype=torch.uint8, device="cuda:0"))
        k0, v0 = d.k.clone(), d.v.clone()
        for step in ("first", "again", "prepared"):
            if step == "prepared":
                tv.init_verify_workspace(ws)
            if name == "stochastic":
                p, l, t, s = tv.tree_verify_stochastic(d.target, d.draft, d.tokens, d.parent, d.n_nodes,
                                                       d.u_accept, d.u_sample, ws=ws)
            elif name == "greedy":
                p, l, t, s = tv.tree_verify_greedy(d.target, d.tokens, d.parent, d.n_nodes, ws=ws)
            else:
                p, l, t, s, src, nl, kst = tv.tree_verify_stochastic_compact(
                    d.target, d.draft, d.tokens, d.parent, d.n_nodes, d.u_accept, d.u_sample,
                    d.k, d.v, d.table, d.prefix_len, ws=ws)
            torch.cuda.synchronize()
            print(name.upper(), step, s.tolist(), l.tolist(), flush=True)
            if name == "compact":
                # a request without a path moves nothing and keeps its length
                same = bool(torch.equal(d.k, k0) and torch.equal(d.v, v0))
                print("COMPACTKV", step, [int(same)], (nl - d.prefix_len).tolist(), flush=True)

    # tree attention on a grid that is resident at once: the splits of a tile
    # wait for each other before merging
    wa = make_workload("llama8b", seed=62, with_logits=False, n_nodes=20, prefix=1500)
    da = DevWorkload(wa, logits=False)
    aneed = lib.tree_attn_workspace_size(ctypes.byref(tv.attn_desc(da.q, da.k, da.table)))
    aws = tv.init_verify_workspace(torch.zeros(aneed, dtype=torch.uint8, device="cuda:0"))
    for step in ("first", "again", "prepared"):
        if step == "prepared":
            tv.init_verify_workspace(aws)
        o, s = tv.tree_attn_forward(da.q, da.k, da.v, da.table, da.prefix_len, da.n_nodes, da.parent, ws=aws)
        torch.cuda.synchronize()
        print("ATTN", step, s.tolist(), [1], flush=True)

    # tree expansion: each request's workgroup waits for its rows' chunk results
    import numpy as np
    from tree_verification_amd.workloads import make_expand_rows
    eB, eF, eV, ek, en = 3, 2, 30011, 2, 32
    erows = torch.from_numpy(make_expand_rows(eB, eF, eV, 63)).cuda()
    efr = torch.zeros((eB, eF), dtype=torch.int32, device="cuda:0")
    enf = torch.full((eB,), eF, dtype=torch.int32, device="cuda:0")
    edesc = tv.ExpandDesc()
    edesc.batch, edesc.f_max, edesc.vocab, edesc.n_max, edesc.k = eB, eF, eV, en, ek
    eneed = lib.tree_expand_workspace_size(ctypes.byref(edesc))
    ews = tv.init_verify_workspace(torch.zeros(eneed, dtype=torch.uint8, device="cuda:0"))
    for step in ("first", "again", "prepared"):
        if step == "prepared":
            tv.init_verify_workspace(ews)
        etok = torch.zeros((eB, en), dtype=torch.int32, device="cuda:0")
        epar = torch.full((eB, en), -1, dtype=torch.int32, device="cuda:0")
        enn = torch.ones(eB, dtype=torch.int32, device="cuda:0")
        nf, nn, s = tv.tree_expand_topk(erows, efr, enf, etok, epar, enn, ek, ws=ews)
        torch.cuda.synchronize()
        print("EXPAND", step, s.tolist(), nn.tolist(), flush=True)
""")


def run_child(limit):
    env = dict(os.environ)
    env["TV_CHASE_SPIN_LIMIT"] = str(limit)
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    print("child TV_CHASE_SPIN_LIMIT", limit, flush=True)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    out = {}
    for ln in r.stdout.splitlines():
        name, step, rest = ln.split(" ", 2)
        st, ln_ = rest.split("] [")
        out[(name, step)] = (eval(st + "]"), eval("[" + ln_))
    return out


def test_expired_chase_invalidates_the_workspace():
    from tree_verification_amd import binding as tv
    out = run_child(-1)
    for step in ("first", "again", "prepared"):   # verify-and-compact: nothing moved, lengths kept
        same, dlen = out[("COMPACTKV", step)]
        assert same == [1] and dlen == [0] * 3, (step, same, dlen)
    for name in ("STOCHASTIC", "GREEDY", "COMPACT"):
        st, ln = out[(name, "first")]
        assert st == [tv.REQ_TIMEOUT] * 3 and ln == [0] * 3, (name, st)
        st, ln = out[(name, "again")]
        assert st == [tv.REQ_BAD_WORKSPACE] * 3 and ln == [0] * 3, (name, st)
        st, ln = out[(name, "prepared")]   # prepared again: the wait expires again, nothing else
        assert st == [tv.REQ_TIMEOUT] * 3, (name, st)
    # attention's split merge: the same contract for its workspace.  A split
    # that gives up at once invalidates the header while other splits of the
    # same call may still be in their prologue, so the forced call's request
    # reports TIMEOUT, BAD_WORKSPACE or both; never success.
    failed = (tv.REQ_TIMEOUT, tv.REQ_BAD_WORKSPACE, tv.REQ_TIMEOUT | tv.REQ_BAD_WORKSPACE)
    assert out[("ATTN", "first")][0][0] in failed, out[("ATTN", "first")]
    assert out[("ATTN", "again")][0] == [tv.REQ_BAD_WORKSPACE]
    assert out[("ATTN", "prepared")][0][0] in failed, out[("ATTN", "prepared")]
    # expansion: a request workgroup that gives up invalidates the header, which
    # another request of the same call may read first (then it reports
    # BAD_WORKSPACE and waits for nothing); at least one reports TIMEOUT
    for step in ("first", "prepared"):
        st, nn = out[("EXPAND", step)]
        assert all(s in (tv.REQ_TIMEOUT, tv.REQ_BAD_WORKSPACE) for s in st), (step, st)
        assert tv.REQ_TIMEOUT in st and nn == [0] * 3, (step, st, nn)
    assert out[("EXPAND", "again")] == ([tv.REQ_BAD_WORKSPACE] * 3, [0] * 3)


def test_one_polling_round_completes_or_flags():
    from tree_verification_amd import binding as tv
    out = run_child(0)
    for name in ("STOCHASTIC", "GREEDY", "COMPACT"):
        st, ln = out[(name, "first")]
        for s, L in zip(st, ln):
            assert (s == 0 and L >= 1) or (s == tv.REQ_TIMEOUT and L == 0), (name, st, ln)
        if all(s == 0 for s in st):   # nothing expired: the workspace stays usable
            st2, _ = out[(name, "again")]
            assert all(s in (0, tv.REQ_TIMEOUT) for s in st2), (name, st2)
        else:
            st2, _ = out[(name, "again")]
            assert st2 == [tv.REQ_BAD_WORKSPACE] * 3, (name, st2)
    st, _ = out[("ATTN", "first")]
    assert st in ([0], [tv.REQ_TIMEOUT], [tv.REQ_BAD_WORKSPACE], [tv.REQ_TIMEOUT | tv.REQ_BAD_WORKSPACE]), st
    st2, _ = out[("ATTN", "again")]
    assert st2 in (([0], [tv.REQ_TIMEOUT]) if st == [0] else ([tv.REQ_BAD_WORKSPACE],)), (st, st2)
    st, nn = out[("EXPAND", "first")]
    for s, n in zip(st, nn):
        assert (s == 0 and n == 4) or (s in (tv.REQ_TIMEOUT, tv.REQ_BAD_WORKSPACE) and n == 0), (st, nn)
    st2, _ = out[("EXPAND", "again")]
    if all(s == 0 for s in st):
        assert all(s in (0, tv.REQ_TIMEOUT, tv.REQ_BAD_WORKSPACE) for s in st2), st2
    else:
        assert st2 == [tv.REQ_BAD_WORKSPACE] * 3, st2
