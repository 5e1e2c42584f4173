"""Statistical checks of the GPU stochastic verifier on 10^6 seeded trials.

* chi-square: an order-1 Markov target on the guide's mask-figure tree shape;
  the first two emitted tokens (taken from a second round when the first round
  emits only one) must follow P[start] x P;
* the first 20 000 trials also match the oracle request by request (outside
  the 1e-6 decision band);
* chains with p = (a, 1 - a) and q = (1, 0): the mean number of emitted tokens
  per round is the chapter's E[T] = (1 - a^(g+1)) / (1 - a), and the share of
  rounds accepting at least k drafts is the guide's a^k.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from markov_trials import SHAPE, chi_square_pvalue, draw_round, markov_tables, softmax_rows
from oracle.verify import divergence_in_band, verify_stochastic_request
from tree_verification_amd import binding as tv

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
BATCH = 200_000


def gpu_rounds(tok, tl, dl, ua, us, parent):
    """Run the trials through tree_verify_stochastic in batches; returns
    (path_len, out_tokens, status, paths) on the host."""
    T, n = tok.shape
    plen = np.empty(T, dtype=np.int32)
    paths = np.empty((T, n), dtype=np.int32)
    outs = np.empty((T, n), dtype=np.int32)
    st = np.empty(T, dtype=np.int32)
    par = np.broadcast_to(parent, (min(T, BATCH), n))
    for s in range(0, T, BATCH):
        e = min(T, s + BATCH)
        f = lambda a: torch.from_numpy(np.ascontiguousarray(a[s:e])).to(DEV)
        nn = torch.full((e - s,), n, dtype=torch.int32, device=DEV)
        pt = torch.from_numpy(np.ascontiguousarray(par[: e - s])).to(DEV)
        pa, pl, ot, ss = tv.tree_verify_stochastic(f(tl), f(dl), f(tok), pt, nn, f(ua), f(us))
        torch.cuda.synchronize()
        paths[s:e] = pa.cpu().numpy()
        plen[s:e] = pl.cpu().numpy()
        outs[s:e] = ot.cpu().numpy()
        st[s:e] = ss.cpu().numpy()
    return plen, outs, st, paths


def test_two_token_chi_square_million_trials():
    V, T, start = 4, 1_000_000, 1
    LT, LQ = markov_tables(700, V)
    rng = np.random.default_rng(702)
    n = len(SHAPE)
    tok, tl, dl, ua, us = draw_round(rng, LT, LQ, np.full(T, start))
    print("round 1", flush=True)
    plen, outs, st, gpaths = gpu_rounds(tok, tl, dl, ua, us, SHAPE)
    assert not st.any()
    x1 = outs[:, 0].astype(np.int64)
    x2 = np.where(plen > 1, outs[:, 1], -1).astype(np.int64)

    # the first trials match the oracle request by request
    mism = 0
    for t in range(20_000):
        path, out, trace = verify_stochastic_request(tl[t], dl[t], tok[t], SHAPE, n, ua[t], us[t])
        L = int(plen[t])
        if list(gpaths[t, :L]) != path or list(outs[t, :L]) != out:
            assert divergence_in_band(trace, path, out, gpaths[t, :L], outs[t, :L]), (t, list(outs[t, :L]), out)
            mism += 1
    assert mism <= 2

    need = np.nonzero(x2 < 0)[0]
    tok2, tl2, dl2, ua2, us2 = draw_round(rng, LT, LQ, x1[need])
    print("round 2", len(need), flush=True)
    plen2, outs2, st2, _ = gpu_rounds(tok2, tl2, dl2, ua2, us2, SHAPE)
    assert not st2.any()
    x2[need] = outs2[:, 0]
    counts = np.zeros((V, V))
    np.add.at(counts, (x1, x2), 1)
    Pt = softmax_rows(LT)
    expected = np.outer(Pt[start], np.ones(V)) * Pt * T
    chi2, pval = chi_square_pvalue(counts, expected)
    assert pval > 1e-3, (chi2, pval, counts.tolist())


@pytest.mark.parametrize("row", range(4))
def test_expected_tokens_per_round_on_chains(golden_dir, row):
    g = json.load(open(os.path.join(golden_dir, "expected_tokens.json")))
    r = g["expected_tokens_per_round"][row]
    a, gamma, T = r["alpha"], r["gamma"], 200_000
    n = gamma + 1
    lt = np.array([math.log(a), math.log(1.0 - a)], dtype=np.float32)
    ld = np.array([0.0, -1e4], dtype=np.float32)          # q = (1, 0): every draft proposes token 0
    tl = np.broadcast_to(lt, (T, n, 2)).copy()
    dl = np.broadcast_to(ld, (T, n, 2)).copy()
    tok = np.zeros((T, n), dtype=np.int32)
    rng = np.random.default_rng(800 + row)
    ua = rng.random((T, n), dtype=np.float32)
    us = rng.random((T, n), dtype=np.float32)
    parent = np.arange(-1, n - 1, dtype=np.int32)
    plen, _, st, _ = gpu_rounds(tok, tl, dl, ua, us, parent)
    assert not st.any()
    se = plen.std(ddof=1) / math.sqrt(T)
    assert abs(plen.mean() - r["E_T"]) < 5 * se + 1e-4, (r, plen.mean(), se)
    if row == 0:
        K = plen - 1
        for k in range(1, gamma + 1):
            frac = float(np.mean(K >= k))
            s = math.sqrt(frac * (1 - frac) / T)
            assert abs(frac - a ** k) < 5 * s + 1e-4, (k, frac, a ** k)
