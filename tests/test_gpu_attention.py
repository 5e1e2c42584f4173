"""GPU parity of tree attention against the float64 oracle.

Tolerance (the attention output is a convex combination of value rows): per
(request, node, q-head) row, ||o - o_ref|| / ||o_ref|| <= 2e-2 for bf16 inputs
and 1e-5 for fp32 inputs, and element-wise |o - o_ref| <= tol * max |o_ref row|
(tests/attn_check.py).  Full-size cases also run on inputs whose tree keys
dominate the softmax, where one wrong ancestor bit fails the check
(tests/test_attn_check.py pins that on the CPU).
"""
import ctypes

import numpy as np
import pytest
import torch

from attn_check import TOL, worst_errors
from devdata import DevWorkload, out_to_np
from oracle.attention import tree_attention
from tree_verification_amd import binding as tv
from tree_verification_amd.workloads import dominate_tree_keys, make_workload

pytestmark = pytest.mark.gpu


def run_gpu(wl, **kw):
    d = DevWorkload(wl, logits=False)
    out, st = tv.tree_attn_forward(d.q, d.k, d.v, d.table, d.prefix_len, d.n_nodes, d.parent, **kw)
    torch.cuda.synchronize()
    return out_to_np(out), st.cpu().numpy(), d, out


def oracle(wl, requests=None, rows=None):
    return tree_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.prefix_len, wl.n_nodes,
                          wl.parent, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                          block_size=wl.block_size, num_blocks=wl.num_blocks, n_max=wl.n_max,
                          sm_scale=wl.sm_scale, requests=requests, rows=rows)


def check_all_rows(wl, out, status):
    ref, rst = oracle(wl)
    assert np.array_equal(status, rst)
    worst = (0.0, 0.0)
    for b in range(wl.batch):
        if rst[b]:
            continue
        n = int(wl.n_nodes[b])
        e = worst_errors(out[b, :n], ref[b])
        worst = (max(worst[0], e[0]), max(worst[1], e[1]))
    assert max(worst) <= TOL[wl.dtype], worst
    return worst


SMALL = [
    ("tiny", {}),
    ("llama8b", dict(prefix=300)),                                  # 4 row tiles x 3 key splits
    ("llama8b", dict(prefix=(0, 0), n_nodes=64)),                   # no prefix: pure tree attention
    ("ragged", dict(batch=4, prefix=(100, 700))),                   # paged, shuffled, ragged
    ("chain", dict(batch=16, prefix=257)),                          # R = 12..32: one partly filled row tile
    ("llama70b_share", dict(batch=1, prefix=500)),                  # 16 row tiles, N = 128
    ("llama8b", dict(prefix=333, n_nodes=1)),                       # single node: decode attention
    ("llama8b", dict(prefix=95, n_nodes=37, tree="star")),          # star tree, ragged row tile
    ("llama8b", dict(prefix=40, n_nodes=128, tree="chain")),        # maximum depth
    ("chain", dict(batch=5, prefix=17, n_nodes=(1, 3))),            # R = 4..12: mostly padding rows
    ("llama8b", dict(prefix=2000, n_nodes=3)),                      # 12 rows in a 64-row tile, many key splits
    ("ragged", dict(batch=6, prefix=(50, 3000), n_nodes=2)),        # 8-row tiles, balanced plan
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[f"{n}-{i}" for i, (n, _) in enumerate(SMALL)])
def test_attention_small(name, kw):
    wl = make_workload(name, seed=11, with_logits=False, **kw)
    print(f"case {name} {kw} B={wl.batch} Nmax={wl.n_max}", flush=True)
    out, st, _, _ = run_gpu(wl)
    check_all_rows(wl, out, st)


@pytest.mark.parametrize("dtype_cfg", ["tiny", "llama8b"])
@pytest.mark.parametrize("bs", [32, 64, 128])
def test_attention_block_sizes(dtype_cfg, bs):
    from tree_verification_amd import workloads as W
    cfg = dict(W.CONFIGS[dtype_cfg])
    W.CONFIGS["_bs"] = dict(cfg, block_size=bs, paged=True)
    W.CONFIG_ORDER.append("_bs")
    try:
        wl = make_workload("_bs", seed=5, with_logits=False, prefix=(150, 420),
                           n_nodes=20 if dtype_cfg == "llama8b" else 8, batch=3)
    finally:
        W.CONFIG_ORDER.remove("_bs")
        del W.CONFIGS["_bs"]
    out, st, _, _ = run_gpu(wl)
    check_all_rows(wl, out, st)


def custom(dtype, Hq, Hkv, D, n, P, B=2, seed=3, kind="capped"):
    from tree_verification_amd import workloads as W
    W.CONFIGS["_c"] = dict(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, dtype=dtype,
                           prefix=P, n_nodes=n, tree=kind, width=3, depth=6, vocab=50,
                           target_sd=1.0, draft_noise_sd=1.0, block_size=16, paged=True)
    W.CONFIG_ORDER.append("_c")
    try:
        return make_workload("_c", seed=seed, with_logits=False)
    finally:
        W.CONFIG_ORDER.remove("_c")
        del W.CONFIGS["_c"]


@pytest.mark.parametrize("dtype,Hq,Hkv,D,n,P,B", [
    ("bf16", 8, 2, 64, 30, (10, 300), 2),   # head_dim 64 on MFMA
    ("bf16", 4, 4, 64, 10, (0, 64), 2),     # G = 1, R < 16: one MFMA wave, padding rows
    ("f32", 8, 2, 128, 24, (50, 200), 2),   # fp32, R = 96: VALU over 6 row tiles
    ("f32", 2, 1, 64, 100, (1, 33), 2),     # fp32, deep tree, short prefix
    ("bf16", 16, 2, 128, 128, (3, 3), 2),   # R = 1024 with a 3-token prefix
    ("bf16", 16, 2, 64, 64, (10, 300), 8),  # head_dim 64 with 128-row tiles (16 pairs x 4 tiles)
])
def test_attention_shapes(dtype, Hq, Hkv, D, n, P, B):
    wl = custom(dtype, Hq, Hkv, D, n, P, B=B)
    print(f"case shapes {dtype} Hq={Hq} Hkv={Hkv} D={D} n={n} P={P} B={B}", flush=True)
    out, st, _, _ = run_gpu(wl)
    check_all_rows(wl, out, st)


FULL = ["tiny", "llama8b", "ragged", "chain", "llama70b_share"]


def check_sampled(wl, out, rows):
    ref, _ = oracle(wl, requests=sorted(rows), rows=rows)
    got = np.stack([out[b, u, h] for b, lst in rows.items() for u, h in lst])
    want = np.stack([ref[b][u, h] for b, lst in rows.items() for u, h in lst])
    worst = worst_errors(got, want)
    assert max(worst) <= TOL[wl.dtype], worst
    return worst


@pytest.mark.parametrize("name", FULL)
def test_attention_full_size_sampled(name):
    """Configurations at full size (the benchmark's launch shape); 64 sampled rows."""
    wl = make_workload(name, with_logits=False)
    print(f"case full {name} B={wl.batch} Nmax={wl.n_max} P={wl.prefix_len[:4]}", flush=True)
    out, st, _, _ = run_gpu(wl)
    assert np.all(st == 0)
    rng = np.random.default_rng(99)
    rows = {}
    for _ in range(64):
        b = int(rng.integers(wl.batch))
        u = int(rng.integers(int(wl.n_nodes[b])))
        h = int(rng.integers(wl.n_q_heads))
        rows.setdefault(b, []).append((u, h))
    check_sampled(wl, out, rows)


@pytest.mark.parametrize("name", ["llama8b", "llama70b_share"])
def test_attention_full_size_tree_dominant(name):
    """Full size (prefix 2048 / 32768) with the tree keys dominating every row's
    softmax: a single wrong ancestor bit would fail the check.  Rows: every
    node of the first request at four q-heads, plus every head of four nodes."""
    wl = make_workload(name, with_logits=False)
    dominate_tree_keys(wl, seed=5)
    print(f"case full tree-dominant {name} B={wl.batch} Nmax={wl.n_max}", flush=True)
    out, st, _, _ = run_gpu(wl)
    assert np.all(st == 0)
    rng = np.random.default_rng(6)
    n = int(wl.n_nodes[0])
    heads = rng.choice(wl.n_q_heads, size=4, replace=False)
    rows = {0: [(u, int(h)) for u in range(n) for h in heads]}
    for u in rng.choice(n, size=4, replace=False):
        rows[0] += [(int(u), h) for h in range(wl.n_q_heads) if h not in heads]
    check_sampled(wl, out, rows)


def test_attention_deterministic_and_workspace_reuse():
    wl = make_workload("llama8b", seed=2, with_logits=False, prefix=700)
    d = DevWorkload(wl, logits=False)
    a, _ = tv.tree_attn_forward(d.q, d.k, d.v, d.table, d.prefix_len, d.n_nodes, d.parent)
    b_, _ = tv.tree_attn_forward(d.q, d.k, d.v, d.table, d.prefix_len, d.n_nodes, d.parent)
    torch.cuda.synchronize()
    assert torch.equal(a, b_)


def test_attention_status_flags():
    wl = make_workload("llama8b", seed=4, with_logits=False, batch=5, prefix=(40, 90), n_nodes=12)
    wl.n_nodes[1] = 0                       # bad node count
    wl.parent[2, 5] = 7                     # parent after child
    wl.block_table[3, 1] = wl.num_blocks    # block outside the pool
    wl.prefix_len[4] = wl.max_blocks * wl.block_size   # positions past the table
    out, st, _, _ = run_gpu(wl)
    ref, rst = oracle(wl)
    assert list(st) == list(rst) == [0, tv.REQ_BAD_NNODES, tv.REQ_BAD_PARENT, tv.REQ_BAD_KV, tv.REQ_BAD_KV]
    n = int(wl.n_nodes[0])
    assert max(worst_errors(out[0, :n], ref[0])) <= TOL["bf16"]


def test_padding_rows_untouched():
    wl = make_workload("chain", seed=8, with_logits=False, batch=6, prefix=64)
    d = DevWorkload(wl, logits=False)
    out = torch.full_like(d.q, 7.0)
    tv.tree_attn_forward(d.q, d.k, d.v, d.table, d.prefix_len, d.n_nodes, d.parent, out=out)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    for b in range(wl.batch):
        assert np.all(o[b, int(wl.n_nodes[b]):] == 7.0)


def widen_table(wl, max_blocks):
    """The same workload with a block table of max_blocks entries per request
    (entries past the request's blocks are -1): a table sized for a longer
    context than the requests use."""
    t = np.full((wl.batch, max_blocks), -1, dtype=np.int32)
    t[:, :wl.max_blocks] = wl.block_table
    wl.block_table = t
    wl.max_blocks = max_blocks
    return wl


@pytest.mark.parametrize("name,kw", [("llama8b", dict(prefix=2048)), ("ragged", dict(batch=5, prefix=(200, 3000)))])
def test_attention_oversized_block_table(name, kw):
    """A table sized for 32K tokens of context gives the same output, bit for
    bit, as the exact-fit table: the split plan follows the requests' lengths."""
    wl = make_workload(name, seed=21, with_logits=False, **kw)
    print(f"case oversized table {name} {kw}", flush=True)
    out0, st0, _, _ = run_gpu(wl)
    widen_table(wl, 32768 // wl.block_size + 3)
    out1, st1, _, _ = run_gpu(wl)
    assert np.array_equal(st0, st1) and not st1.any()
    assert np.array_equal(out0, out1)
    check_all_rows(wl, out1, st1)


@pytest.mark.parametrize("scale,n_nodes", [(1e5, 40), (1e-6, 40), (1e5, 3), (1e-6, 3)])
def test_attention_split_partials_extreme_values(scale, n_nodes):
    """Values of magnitude 1e5 and 1e-6 through the split-K partials (fp16 with
    a per-row power-of-two scale), for a 40-node tree and a 3-node one (12 rows
    of a 64-row tile): the same tolerance as unit-scale values."""
    from tree_verification_amd.workloads import round_to_bf16
    wl = make_workload("llama8b", seed=23, with_logits=False, prefix=1500, n_nodes=n_nodes)
    wl.v_cache = round_to_bf16(wl.v_cache * np.float32(scale))
    print(f"case partial scale {scale}", flush=True)
    out, st, _, _ = run_gpu(wl)
    worst = check_all_rows(wl, out, st)
    print(f"  worst (row, element) error {worst}", flush=True)


def test_attention_ragged_balanced_plan_many_lengths():
    """A batch planned as a whole: lengths from 1 to ~6000 keys, some requests
    malformed (they get no split and their status), ragged row tiles."""
    wl = make_workload("ragged", seed=27, with_logits=False, batch=12, prefix=(0, 6000), n_nodes=32)
    wl.n_nodes[3] = 5
    wl.n_nodes[7] = 0                         # malformed: no split planned for it
    wl.prefix_len[9] = wl.max_blocks * wl.block_size   # past its table
    print("case balanced plan", flush=True)
    out, st, _, _ = run_gpu(wl)
    ref, rst = oracle(wl)
    assert list(st) == list(rst)
    assert st[7] == tv.REQ_BAD_NNODES and st[9] == tv.REQ_BAD_KV
    for b in range(wl.batch):
        if rst[b]:
            continue
        n = int(wl.n_nodes[b])
        assert max(worst_errors(out[b, :n], ref[b])) <= TOL["bf16"], b


def test_attention_uniform_plan_bad_sizes():
    """One request (uniform plan): malformed sizes are reported by its first workgroup."""
    wl = make_workload("llama8b", seed=29, with_logits=False, prefix=100, n_nodes=10)
    wl.n_nodes[0] = wl.n_max + 1
    _, st, _, _ = run_gpu(wl)
    assert st[0] == tv.REQ_BAD_NNODES


def test_attention_unprepared_workspace_is_reported():
    """A call whose tiles are split over keys merges them through counters in
    the workspace.  A workspace that was never prepared is detected from its
    header: the request gets TV_REQ_BAD_WORKSPACE and no counter is touched.
    Once prepared, repeated calls give identical outputs (every call leaves the
    counters at zero), including a smaller call in between."""
    wl = make_workload("llama8b", seed=31, with_logits=False, prefix=900)
    d = DevWorkload(wl, logits=False)
    wl2 = make_workload("llama8b", seed=32, with_logits=False, prefix=400, n_nodes=20)
    d2 = DevWorkload(wl2, logits=False)
    lib = tv.load_library()
    needs = [lib.tree_attn_workspace_size(ctypes.byref(tv.attn_desc(x.q, x.k, x.table))) for x in (d, d2)]
    assert min(needs) > 0
    ws = torch.zeros(max(needs), dtype=torch.uint8, device="cuda:0")
    _, st = tv.tree_attn_forward(d.q, d.k, d.v, d.table, d.prefix_len, d.n_nodes, d.parent, ws=ws)
    torch.cuda.synchronize()
    assert list(st.cpu().numpy()) == [tv.REQ_BAD_WORKSPACE]
    tv.init_verify_workspace(ws)
    a, st = tv.tree_attn_forward(d.q, d.k, d.v, d.table, d.prefix_len, d.n_nodes, d.parent, ws=ws)
    torch.cuda.synchronize()
    assert not st.cpu().numpy().any()
    check_all_rows(wl, out_to_np(a), st.cpu().numpy())
    # a shorter request through the same workspace, then the first one again
    o2, st2 = tv.tree_attn_forward(d2.q, d2.k, d2.v, d2.table, d2.prefix_len, d2.n_nodes, d2.parent, ws=ws)
    torch.cuda.synchronize()
    check_all_rows(wl2, out_to_np(o2), st2.cpu().numpy())
    for _ in range(3):
        b_, st = tv.tree_attn_forward(d.q, d.k, d.v, d.table, d.prefix_len, d.n_nodes, d.parent, ws=ws)
        torch.cuda.synchronize()
        assert not st.cpu().numpy().any()
        assert torch.equal(a, b_)
