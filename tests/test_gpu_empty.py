"""Every entry point called through the binding with an empty batch: the call
succeeds, launches nothing that touches memory, and returns empty outputs."""
import pytest
import torch

from tree_verification_amd import binding as tv

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def z(shape, dtype=torch.int32):
    return torch.zeros(shape, dtype=dtype, device=DEV)


def test_empty_batch_every_entry_point():
    n_max, Hq, Hkv, D, bs, nblk, V = 8, 4, 2, 64, 16, 4, 1000
    q = z((0, n_max, Hq, D), torch.bfloat16)
    k = torch.randn((nblk, Hkv, bs, D), device=DEV).to(torch.bfloat16)
    v = torch.randn((nblk, Hkv, bs, D), device=DEV).to(torch.bfloat16)
    table, pre, nn, par = z((0, 3)), z((0,)), z((0,)), z((0, n_max))
    out, st = tv.tree_attn_forward(q, k, v, table, pre, nn, par)
    assert out.shape == (0, n_max, Hq, D) and st.shape == (0,)

    logits = z((0, n_max, V), torch.float32)
    tok, u = z((0, n_max)), z((0, n_max), torch.float32)
    for res in (tv.tree_verify_greedy(logits, tok, par, nn),
                tv.tree_verify_stochastic(logits, logits, tok, par, nn, u, u)):
        assert [tuple(x.shape) for x in res] == [(0, n_max), (0,), (0, n_max), (0,)]

    src, new_len, cst = tv.kv_compact_accepted(k, v, table, pre, z((0, n_max)), z((0,)))
    assert src.shape == (0, n_max) and new_len.shape == (0,)
    res = tv.tree_verify_stochastic_compact(logits, logits, tok, par, nn, u, u, k, v, table, pre)
    assert [tuple(x.shape) for x in res] == [(0, n_max), (0,), (0, n_max), (0,), (0, n_max), (0,), (0,)]

    merged = tv.tree_merge_candidates(z((0, 3, 5)), z((0, 3)), z((0,)), n_max)
    assert merged[2].shape == (0,)
    nf, nnew, est = tv.tree_expand_topk(z((0, 2, V), torch.float32), z((0, 2)), z((0,)), z((0, n_max)),
                                        z((0, n_max)), z((0,)), 2)
    assert nf.shape == (0, 4) and nnew.shape == (0,)

    free, count = torch.arange(nblk, dtype=torch.int32, device=DEV), torch.tensor([nblk], dtype=torch.int32,
                                                                                  device=DEV)
    spec, ast = tv.kv_alloc_tree_blocks(z((0, 3)), z((0,)), z((0,)), z((0,)), free, count, block_size=bs)
    rst = tv.kv_release_blocks(z((0, 3)), z((0,)), z((0,)), free, count, block_size=bs)
    assert spec.shape == (0,) and rst.shape == (0,)

    reach, al, bst = tv.tree_expected_accept_length(z((0, n_max)), z((0,)), z((0, n_max), torch.float64))
    assert reach.shape == (0, n_max) and al.shape == (0,)
    torch.cuda.synchronize()
    assert int(count.item()) == nblk and torch.equal(free, torch.arange(nblk, dtype=torch.int32, device=DEV))
