"""TV_DEBUG=1 and TV_TRACE=1 (read once per process, so each case runs in a
child process): with TV_DEBUG the entry points print each malformed request on
stderr before launching and leave the per-request status flags and the outputs
exactly as without it; TV_TRACE changes no result."""
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
    import torch
    from devdata import DevWorkload
    from tree_verification_amd import binding as tv
    from tree_verification_amd.workloads import make_workload

    wl = make_workload("tiny", batch=4)
    dw = DevWorkload(wl)
    par = dw.parent.clone()
    par[1, 2] = 5            # request 1: a parent that is not an earlier node
    pre = dw.prefix_len.clone()
    pre[0] = 1 << 20         # request 0: a prefix that leaves its block table
    out, ast = tv.tree_attn_forward(dw.q, dw.k, dw.v, dw.table, pre, dw.n_nodes, par)
    path, plen, otok, vst = tv.tree_verify_greedy(dw.target, dw.tokens, par, dw.n_nodes)
    torch.cuda.synchronize()
    print("ATTN", ast.tolist())
    print("VERIFY", vst.tolist(), plen.tolist())
    ok = [b for b in range(ast.shape[0]) if b not in (0, 1)]
    print("OUTSUM", float(out[ok].float().abs().sum()))
""")


def run_child(env_extra):
    env = dict(os.environ)
    env.pop("TV_DEBUG", None)
    env.pop("TV_TRACE", None)
    env.update(env_extra)
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    print("child", env_extra, flush=True)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    return r


def result_lines(stdout):
    return [ln for ln in stdout.splitlines() if ln.split(" ", 1)[0] in ("ATTN", "VERIFY", "OUTSUM")]


def test_debug_reports_malformed_requests_and_changes_no_result():
    plain = run_child({})
    debug = run_child({"TV_DEBUG": "1"})
    trace = run_child({"TV_TRACE": "1"})
    assert "[tv debug]" not in plain.stderr
    err = debug.stderr
    assert "[tv debug] tree_attn_forward: request 1: parent[2] = 5" in err, err
    assert "[tv debug] tree_verify_greedy: request 1: parent[2] = 5" in err, err
    assert "[tv debug] tree_attn_forward: request 0: prefix" in err, err
    # exactly the malformed requests are named
    named = {ln.split("request ")[1].split(":")[0] for ln in err.splitlines() if ln.startswith("[tv debug]")}
    assert named == {"0", "1"}, err
    lines = result_lines(plain.stdout)
    assert len(lines) == 3
    assert result_lines(debug.stdout) == lines
    assert result_lines(trace.stdout) == lines
    ast = eval(lines[0].split(" ", 1)[1])
    assert ast[0] != 0 and ast[1] != 0 and all(s == 0 for s in ast[2:]), ast
