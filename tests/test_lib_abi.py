"""The C library loads, exports every function include/tree_verify.h declares, and
rejects malformed descriptors on the host (no GPU needed: these calls return before
any HIP call)."""
import ctypes
import os
import re

import pytest

from tree_verification_amd import binding as tv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tree_verify.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tv.LIB_PATH):
        from tree_verification_amd import build
        build.build()
    return tv.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    names = re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\([^;{}]*\)\s*;", src)
    return sorted(set(names))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("tree_attn_forward", "tree_verify_greedy", "tree_verify_stochastic", "kv_compact_accepted"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert names
    for n in names:
        assert hasattr(lib, n), n
    # and the binding's signature table covers them
    assert set(names) <= set(tv._SIGS)


def test_status_strings(lib):
    assert lib.tv_status_string(0) == b"TV_OK"
    assert lib.tv_status_string(-1) == b"TV_ERR_INVALID_ARG"
    assert lib.tv_status_string(-2) == b"TV_ERR_UNSUPPORTED"
    assert lib.tv_status_string(-3) == b"TV_ERR_WORKSPACE"
    assert lib.tv_status_string(-4) == b"TV_ERR_HIP"


def good_attn_desc():
    d = tv.AttnDesc()
    d.batch, d.n_max, d.n_q_heads, d.n_kv_heads = 1, 8, 4, 2
    d.head_dim, d.block_size, d.max_blocks_per_seq, d.num_blocks = 64, 16, 4, 4
    d.dtype, d.sm_scale = tv.TV_BF16, 0.0
    return d


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 96, -2), ("n_max", 0, -2), ("n_max", 129, -2), ("block_size", 24, -2),
    ("dtype", 7, -2), ("n_kv_heads", 3, -1), ("batch", -1, -1), ("num_blocks", 0, -1),
])
def test_attention_rejects_bad_descriptors(lib, field, value, code):
    d = good_attn_desc()
    setattr(d, field, value)
    rc = lib.tree_attn_forward(ctypes.byref(d), *([None] * 10), 0, None)
    assert rc == code


def test_null_descriptors(lib):
    assert lib.tree_attn_forward(None, *([None] * 10), 0, None) == -1
    assert lib.tree_verify_greedy(None, *([None] * 9), 0, None) == -1
    assert lib.tree_verify_stochastic(None, *([None] * 12), 0, None) == -1
    assert lib.kv_compact_accepted(None, *([None] * 10)) == -1
    assert lib.tree_verify_stochastic_compact(None, None, *([None] * 19), 0, None) == -1
    assert lib.tree_attn_workspace_size(None) == 0
    assert lib.tree_verify_workspace_size(None) == 0


def test_empty_batch_is_a_no_op(lib):
    d = good_attn_desc()
    d.batch = 0
    assert lib.tree_attn_forward(ctypes.byref(d), *([None] * 10), 0, None) == 0
    assert lib.kv_compact_accepted(ctypes.byref(d), *([None] * 10)) == 0
    v = tv.VerifyDesc()
    v.batch, v.n_max, v.vocab, v.temperature = 0, 4, 10, 1.0
    assert lib.tree_verify_greedy(ctypes.byref(v), *([None] * 9), 0, None) == 0


@pytest.mark.parametrize("field,value,code", [
    ("vocab", 0, -1), ("n_max", 200, -2), ("temperature", 0.0, -1), ("temperature", -1.0, -1),
])
def test_verify_rejects_bad_descriptors(lib, field, value, code):
    v = tv.VerifyDesc()
    v.batch, v.n_max, v.vocab, v.temperature = 2, 4, 10, 1.0
    setattr(v, field, value)
    assert lib.tree_verify_greedy(ctypes.byref(v), *([None] * 9), 0, None) == code
    assert lib.tree_verify_stochastic(ctypes.byref(v), *([None] * 12), 0, None) == code


def test_missing_pointers_rejected(lib):
    d = good_attn_desc()
    assert lib.tree_attn_forward(ctypes.byref(d), *([None] * 10), 0, None) == -1
    v = tv.VerifyDesc()
    v.batch, v.n_max, v.vocab, v.temperature = 2, 4, 10, 1.0
    assert lib.tree_verify_greedy(ctypes.byref(v), *([None] * 9), 0, None) == -1


def _fused(lib, v, d, ptr=None, ws_bytes=0):
    return lib.tree_verify_stochastic_compact(ctypes.byref(v) if v is not None else None,
                                              ctypes.byref(d) if d is not None else None,
                                              *([ptr] * 19), ws_bytes, None)


def test_fused_verify_compact_rejections(lib):
    """The verify-and-compact call checks both descriptors, their agreement and its
    pointers before any launch (nothing is dereferenced on these paths)."""
    v = tv.VerifyDesc()
    v.batch, v.n_max, v.vocab, v.temperature = 2, 4, 10, 1.0
    d = good_attn_desc()
    d.batch, d.n_max = 2, 4
    assert _fused(lib, None, d) == -1
    assert _fused(lib, v, None) == -1
    bad = good_attn_desc()
    bad.batch, bad.n_max, bad.head_dim = 2, 4, 96
    assert _fused(lib, v, bad) == -2                   # compaction descriptor unsupported
    v.temperature = 0.0
    assert _fused(lib, v, d) == -1                     # verification descriptor invalid
    v.temperature = 1.0
    d.batch = 3
    assert _fused(lib, v, d) == -1                     # batches differ
    d.batch, d.n_max = 2, 8
    assert _fused(lib, v, d) == -1                     # n_max differs
    d.n_max = 4
    assert _fused(lib, v, d) == -1                     # null pointers
    v.batch = d.batch = 0
    assert _fused(lib, v, d) == 0                      # empty batch: no-op
    v.batch = d.batch = 2
    dummy = ctypes.c_void_p(4096)   # never dereferenced: the workspace check fails first
    assert _fused(lib, v, d, dummy, 0) == -3


def test_stochastic_vocabulary_limit(lib):
    v = tv.VerifyDesc()
    v.batch, v.n_max, v.vocab, v.temperature = 1, 4, 64 * 8192 + 1, 1.0
    dummy = ctypes.c_void_p(4096)   # never dereferenced: the call fails before any launch
    assert lib.tree_verify_stochastic(ctypes.byref(v), *([dummy] * 12), 0, None) == -2


def test_construction_descriptors_rejected(lib):
    m = tv.MergeDesc()
    m.batch, m.n_cand, m.max_len, m.n_max = 1, 65, 4, 16
    assert lib.tree_merge_candidates(ctypes.byref(m), *([None] * 9)) == -2   # over 64 candidates
    m.n_cand = 0
    assert lib.tree_merge_candidates(ctypes.byref(m), *([None] * 9)) == -1
    m.n_cand, m.max_len = 4, 33
    assert lib.tree_merge_candidates(ctypes.byref(m), *([None] * 9)) == -2
    m.max_len, m.n_max = 4, 1025
    assert lib.tree_merge_candidates(ctypes.byref(m), *([None] * 9)) == -2
    m.n_max, m.batch = 16, 0
    assert lib.tree_merge_candidates(ctypes.byref(m), *([None] * 9)) == 0    # nothing to do
    m.batch = 1
    assert lib.tree_merge_candidates(ctypes.byref(m), *([None] * 9)) == -1   # missing pointers
    assert lib.tree_merge_candidates(None, *([None] * 9)) == -1

    e = tv.ExpandDesc()
    e.batch, e.f_max, e.vocab, e.n_max, e.k = 1, 2, 100, 64, 17
    assert lib.tree_expand_workspace_size(ctypes.byref(e)) == 0
    assert lib.tree_expand_topk(ctypes.byref(e), *([None] * 10), 0, None) == -2
    e.k = 0
    assert lib.tree_expand_topk(ctypes.byref(e), *([None] * 10), 0, None) == -1
    e.vocab, e.k = 10, 11                                                      # k > V
    assert lib.tree_expand_topk(ctypes.byref(e), *([None] * 10), 0, None) == -1
    e.vocab, e.k = 200000, 16                                                  # 25 chunks x 16 keys
    assert lib.tree_expand_topk(ctypes.byref(e), *([None] * 10), 0, None) == -2
    e.vocab, e.k = 128256, 4
    need = lib.tree_expand_workspace_size(ctypes.byref(e))
    assert need >= 2 * 16 * 4 * 8
    assert lib.tree_expand_topk(ctypes.byref(e), *([None] * 10), 0, None) == -1
    dummy = ctypes.c_void_p(4096)   # never dereferenced: these calls fail before any launch
    odd = ctypes.c_void_p(4100)
    assert lib.tree_expand_topk(ctypes.byref(e), odd, *([dummy] * 9), need, None) == -1
    assert lib.tree_expand_topk(ctypes.byref(e), *([dummy] * 10), need - 1, None) == -3
    assert need >= 256 + 2 * 16 * 4 * 8                                        # header, then the key slots
    assert lib.tree_expand_topk(ctypes.byref(e), *([dummy] * 9), ctypes.c_void_p(4096 + 64), need, None) == -1


def test_binding_arity_matches_header():
    """Each ctypes signature takes exactly the parameters the header declares."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    for name, params in re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\(([^;{}]*)\)\s*;", src):
        n = 0 if params.strip() in ("", "void") else params.count(",") + 1
        assert len(tv._SIGS[name][1]) == n, name


def test_pool_descriptors_rejected(lib):
    d = good_attn_desc()
    assert lib.kv_alloc_tree_blocks(ctypes.byref(d), *([None] * 9)) == -1     # missing pointers
    assert lib.kv_release_blocks(ctypes.byref(d), *([None] * 7)) == -1
    d.block_size = 0
    assert lib.kv_alloc_tree_blocks(ctypes.byref(d), *([None] * 9)) == -1
    d.block_size, d.num_blocks = 16, 0
    assert lib.kv_release_blocks(ctypes.byref(d), *([None] * 7)) == -1
    d.num_blocks, d.batch = 4, 0
    assert lib.kv_alloc_tree_blocks(ctypes.byref(d), *([None] * 9)) == 0      # nothing to do
    assert lib.kv_release_blocks(None, *([None] * 7)) == -1


def test_budget_rejects_bad_descriptors(lib):
    d = tv.BudgetDesc()
    d.batch, d.n_max = 2, 129
    assert lib.tree_expected_accept_length(ctypes.byref(d), *([None] * 7)) == -2
    d.n_max = 0
    assert lib.tree_expected_accept_length(ctypes.byref(d), *([None] * 7)) == -2
    d.batch, d.n_max = -1, 8
    assert lib.tree_expected_accept_length(ctypes.byref(d), *([None] * 7)) == -1
    d.batch = 2
    assert lib.tree_expected_accept_length(ctypes.byref(d), *([None] * 7)) == -1   # null arrays
    d.batch = 0
    assert lib.tree_expected_accept_length(ctypes.byref(d), *([None] * 7)) == 0    # nothing to do
    assert lib.tree_expected_accept_length(None, *([None] * 7)) == -1
    assert lib.tree_budget_select(-1, 3, None, None, None) == -1
    assert lib.tree_budget_select(2, 3, None, None, None) == -1


def test_budget_select_is_the_oracle_lookup(lib):
    """tree_budget_select is host code: compared with the oracle's goodput table."""
    import numpy as np
    from oracle.budget import select_budget
    rng = np.random.default_rng(77)
    for _ in range(200):
        S, I = int(rng.integers(1, 9)), int(rng.integers(1, 6))
        al = 1.0 + rng.random(S) * 4
        itl = rng.random((I, S)) * 10
        # special entries: non-positive, infinite and NaN latencies, exact ties
        for _ in range(int(rng.integers(0, 4))):
            itl[rng.integers(I), rng.integers(S)] = rng.choice([0.0, -1.0, np.inf, np.nan])
        if S > 1 and rng.random() < 0.3:
            al[1], itl[:, 1] = 2 * al[0], 2 * itl[:, 0]
        assert tv.tree_budget_select(al, itl) == select_budget(al, itl)


def test_greedy_noalloc_rejects_oversized_scratch(lib):
    """The static scratch holds tree_verify_greedy_noalloc_max_scratch() bytes; a
    descriptor needing more is refused on the host with TV_ERR_WORKSPACE before
    any HIP call (the pointers are never touched)."""
    cap = lib.tree_verify_greedy_noalloc_max_scratch()
    assert cap == 4 << 20
    d = tv.VerifyDesc()
    # 12 bytes per (node, 8192-logit chunk): 8 x 128 nodes x 512 chunks = 6 MiB
    d.batch, d.n_max, d.vocab, d.temperature = 8, 128, 512 * 8192, 1.0
    fake = [ctypes.c_void_p(4096 * (i + 1)) for i in range(8)]
    rc = lib.tree_verify_greedy_noalloc(ctypes.byref(d), *fake, None)
    assert rc == -3
    d.batch = 0
    assert lib.tree_verify_greedy_noalloc(ctypes.byref(d), *fake, None) == 0


def test_workspace_init_argument_checks(lib):
    assert lib.tree_verify_workspace_init(None, 4096, None) == -3
    assert lib.tree_verify_workspace_init(ctypes.c_void_p(4096), 255, None) == -3
    assert lib.tree_verify_workspace_init(ctypes.c_void_p(4096 + 16), 4096, None) == -1
