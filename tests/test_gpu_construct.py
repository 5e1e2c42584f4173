"""GPU parity of token-tree construction: merge of candidates and top-k expansion.

Integer outputs (tokens, parents, node counts, node maps, frontiers, status) must
match the oracle exactly.  Expansion decisions compare float32 logits exactly on
both sides, so there is no tolerance.
"""
import numpy as np
import pytest
import torch

from oracle import NONFINITE, TREE_OVERFLOW
from oracle.construct import expand_level, expand_tree, merge_candidates
from tree_verification_amd import binding as tv
from tree_verification_amd.workloads import make_candidates, make_expand_rows

pytestmark = pytest.mark.gpu

BAD_LEN = 256
BAD_NNODES = 2


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def check_merge(toks, lens, root, n_max):
    B, M, L = toks.shape
    print(f"case merge B={B} M={M} L={L} n_max={n_max}", flush=True)
    t, p, n, no, st = [x.cpu().numpy() for x in tv.tree_merge_candidates(dev(toks), dev(lens), dev(root), n_max)]
    for b in range(B):
        if lens[b].min() < 0 or lens[b].max() > L:
            assert st[b] == BAD_LEN and n[b] == 0
            continue
        cands = [list(toks[b, i, :lens[b, i]]) for i in range(M)]
        rt, rp, rn, rno, rst = merge_candidates(int(root[b]), cands, n_max)
        assert st[b] == rst, b
        assert n[b] == rn, b
        if rst:
            continue
        assert list(t[b, :rn]) == rt, b
        assert list(p[b, :rn]) == rp, b
        for i in range(M):
            want = rno[i] + [-1] * (L - len(rno[i]))
            assert list(no[b, i]) == want, (b, i)
    return n


@pytest.mark.parametrize("B,M,L,vocab,share,seed", [
    (1, 3, 4, 5, 0.7, 1),        # small vocabulary: much sharing
    (8, 8, 8, 50, 0.7, 2),
    (64, 4, 8, 32000, 0.7, 3),   # a batch of four draft models' 8-token guesses
    (16, 17, 31, 3, 0.9, 4),     # ragged sizes, heavy sharing
    (4, 64, 32, 1000, 0.95, 5),  # maximum candidate count and length
    (32, 5, 6, 2, 0.0, 6),       # binary vocabulary without copying
])
def test_merge_matches_oracle(B, M, L, vocab, share, seed):
    toks, lens, root = make_candidates(B, M, L, vocab, seed, share)
    n = check_merge(toks, lens, root, 1024)
    assert n.max() > 1


def test_merge_edges():
    # empty candidates, all identical, a single candidate
    toks = np.zeros((3, 4, 5), dtype=np.int32)
    lens = np.zeros((3, 4), dtype=np.int32)
    toks[1, :, :] = [7, 8, 9, 10, 11]
    lens[1, :] = 5
    toks[2, 0, :3] = [1, 2, 3]
    lens[2, 0] = 3
    root = np.array([5, 6, 7], dtype=np.int32)
    n = check_merge(toks, lens, root, 16)
    assert list(n) == [1, 6, 4]
    # overflow at exactly n_max + 1 nodes, and a tree that fills n_max exactly
    toks, lens, root = make_candidates(8, 6, 6, 1000, 11, share=0.0, min_len=6)
    check_merge(toks, lens, root, 36)    # 1 + 36 nodes needed
    check_merge(toks, lens, root, 37)
    # out-of-range lengths flag only their request
    lens2 = lens.copy()
    lens2[3, 2] = 7
    lens2[5, 0] = -1
    check_merge(toks, lens2, root, 64)


def run_expand(rows, frontier, nfr, tokens, parent, n_nodes, k):
    d = [dev(x) for x in (rows, frontier, nfr, tokens, parent, n_nodes)]
    nf, nn, st = tv.tree_expand_topk(*d, k)
    torch.cuda.synchronize()
    return (d[3].cpu().numpy(), d[4].cpu().numpy(), d[5].cpu().numpy(), nf.cpu().numpy(), nn.cpu().numpy(),
            st.cpu().numpy())


def check_expand(rows, frontier, nfr, tokens, parent, n_nodes, k):
    B, F, V = rows.shape
    n_max = tokens.shape[1]
    print(f"case expand B={B} F={F} V={V} k={k} n_max={n_max}", flush=True)
    t, p, n, nf, nn, st = run_expand(rows, frontier, nfr, tokens, parent, n_nodes, k)
    for b in range(B):
        n0 = int(n_nodes[b])
        fr = [int(x) for x in frontier[b, :max(0, min(int(nfr[b]), F))]]
        if not 1 <= n0 <= n_max:
            assert st[b] == BAD_NNODES and nn[b] == 0
            continue
        if not 0 <= nfr[b] <= F or any(u < 0 or u >= n0 for u in fr):
            assert st[b] == BAD_LEN and nn[b] == 0
            continue
        rt, rp, rn, rfr, rst = expand_level(list(tokens[b]), list(parent[b]), n0, fr,
                                            [rows[b, f] for f in range(len(fr))], k, n_max)
        assert st[b] == rst, b
        assert n[b] == rn, b
        assert nn[b] == len(rfr), b
        assert list(t[b, :rn]) == rt, b
        assert list(p[b, :rn]) == rp, b
        assert list(nf[b, :len(rfr)]) == rfr, b
    return st


def fresh_trees(B, n_max, n0, seed):
    rng = np.random.default_rng(seed)
    tokens = np.zeros((B, n_max), dtype=np.int32)
    parent = np.full((B, n_max), -1, dtype=np.int32)
    for b in range(B):
        for u in range(1, n0):
            parent[b, u] = int(rng.integers(u))
        tokens[b, :n0] = rng.integers(0, 1000, size=n0)
    return tokens, parent, np.full(B, n0, dtype=np.int32)


@pytest.mark.parametrize("B,F,V,k,ties,seed", [
    (1, 1, 1000, 3, False, 1),
    (4, 3, 1000, 2, True, 2),          # many equal logits
    (2, 6, 128256, 2, False, 3),       # a Llama-3 vocabulary, 16 chunks
    (8, 4, 128256, 16, True, 4),       # largest k, ties
    (3, 5, 32003, 4, False, 5),        # vocabulary not a multiple of 4, ragged last chunk
    (5, 2, 8192, 8, False, 6),         # exactly one chunk
    (2, 2, 16, 16, True, 7),           # k = V
])
def test_expand_matches_oracle(B, F, V, k, ties, seed):
    rows = make_expand_rows(B, F, V, seed, ties=ties)
    tokens, parent, n_nodes = fresh_trees(B, 256, 5, seed)
    rng = np.random.default_rng(seed + 100)
    frontier = rng.integers(0, 5, size=(B, F)).astype(np.int32)
    nfr = rng.integers(0, F + 1, size=B).astype(np.int32)
    nfr[0] = F
    st = check_expand(rows, frontier, nfr, tokens, parent, n_nodes, k)
    assert (st == 0).all()


def test_expand_errors():
    B, F, V, k = 6, 3, 2000, 4
    rows = make_expand_rows(B, F, V, 9)
    tokens, parent, n_nodes = fresh_trees(B, 20, 8, 9)
    frontier = np.tile(np.arange(F, dtype=np.int32), (B, 1))
    nfr = np.full(B, F, dtype=np.int32)
    rows[1, 2, 77] = np.nan            # non-finite in a read row
    rows[2, 2, 1999] = np.inf          # non-finite in an unread row (n_frontier = 2)
    nfr[2] = 2
    frontier[3, 1] = 8                 # frontier id not yet a node
    n_nodes[4] = 0                     # bad node count
    nfr[5] = 4                         # more frontier rows than F
    st = check_expand(rows, frontier, nfr, tokens, parent, n_nodes, k)
    assert st[1] == NONFINITE and st[2] == 0 and st[3] == BAD_LEN and st[4] == BAD_NNODES
    assert st[5] == BAD_LEN and st[0] == 0
    # overflow: 8 + 3 * 4 = 20 fits exactly, one more row does not
    st = check_expand(rows[:1], frontier[:1], nfr[:1], tokens[:1], parent[:1], n_nodes[:1], 4)
    assert st[0] == 0
    tokens2, parent2, n2 = fresh_trees(1, 20, 9, 3)
    st = check_expand(rows[:1], frontier[:1], nfr[:1], tokens2, parent2, n2, 4)
    assert st[0] == TREE_OVERFLOW
    # The failed requests' chunk results were drained: the same workspace (one
    # per descriptor) serves a clean call of the same shape with new rows.
    rows3 = make_expand_rows(B, F, V, 10)
    tokens3, parent3, n3 = fresh_trees(B, 20, 8, 10)
    frontier3 = np.tile(np.arange(F, dtype=np.int32), (B, 1))
    st = check_expand(rows3, frontier3, np.full(B, F, dtype=np.int32), tokens3, parent3, n3, k)
    assert (st == 0).all()


def test_expand_unprepared_workspace_is_reported():
    from tree_verification_amd.binding import ExpandDesc, load_library
    import ctypes
    B, F, V, k = 2, 2, 9000, 3
    rows = make_expand_rows(B, F, V, 11)
    tokens, parent, n_nodes = fresh_trees(B, 32, 4, 11)
    frontier = np.zeros((B, F), dtype=np.int32)
    nfr = np.full(B, F, dtype=np.int32)
    d = ExpandDesc()
    d.batch, d.f_max, d.vocab, d.n_max, d.k = B, F, V, 32, k
    need = load_library().tree_expand_workspace_size(ctypes.byref(d))
    raw = torch.zeros(need, dtype=torch.uint8, device="cuda:0")   # zero, but no header
    args = [dev(x) for x in (rows, frontier, nfr, tokens, parent, n_nodes)]
    nf, nn, st = tv.tree_expand_topk(*args, k, ws=raw)
    torch.cuda.synchronize()
    assert st.tolist() == [tv.REQ_BAD_WORKSPACE] * B and nn.tolist() == [0] * B
    assert args[5].tolist() == [4] * B   # nothing appended
    tv.init_verify_workspace(raw)
    nf, nn, st = tv.tree_expand_topk(*args, k, ws=raw)
    torch.cuda.synchronize()
    assert st.tolist() == [0] * B and nn.tolist() == [F * k] * B


def test_expansion_schedule_on_gpu():
    """A whole tree, schedule <3, 2, 1, 1>, one call per level, against the oracle's
    level-by-level construction with the same draft rows."""
    B, V = 4, 50000
    schedule = [3, 2, 1, 1]
    table = {}
    rng = np.random.default_rng(21)

    def draft_row(b):
        def f(tokens, parent, u):
            path = []
            v = u
            while v > 0:
                path.append(tokens[v])
                v = parent[v]
            key = (b, tuple(path))
            if key not in table:
                table[key] = (rng.standard_normal(V) * 3.0).astype(np.float32)
            return table[key]
        return f

    want = [expand_tree(100 + b, schedule, draft_row(b), 64) for b in range(B)]
    tokens = np.zeros((B, 64), dtype=np.int32)
    parent = np.full((B, 64), -1, dtype=np.int32)
    tokens[:, 0] = 100 + np.arange(B)
    d_tok, d_par = dev(tokens), dev(parent)
    d_n = dev(np.ones(B, dtype=np.int32))
    frontier = np.zeros((B, 1), dtype=np.int32)
    nfr = np.ones(B, dtype=np.int32)
    for k in schedule:
        F = frontier.shape[1]
        t_host, p_host = d_tok.cpu().numpy(), d_par.cpu().numpy()
        rows = np.zeros((B, F, V), dtype=np.float32)
        for b in range(B):
            for f in range(int(nfr[b])):
                rows[b, f] = draft_row(b)(list(t_host[b]), list(p_host[b]), int(frontier[b, f]))
        nf, nn, st = tv.tree_expand_topk(dev(rows), dev(frontier), dev(nfr), d_tok, d_par, d_n, k)
        assert (st.cpu().numpy() == 0).all()
        frontier, nfr = nf.cpu().numpy(), nn.cpu().numpy()
    t, p, n = d_tok.cpu().numpy(), d_par.cpu().numpy(), d_n.cpu().numpy()
    for b in range(B):
        rt, rp, rn, rst = want[b]
        assert rst == 0 and n[b] == rn == 22
        assert list(t[b, :rn]) == rt and list(p[b, :rn]) == rp
