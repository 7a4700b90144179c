"""GPU exact-mass selector against the fp64 oracle: exact page scores (the
log-sum-exp of q.k/sqrt(128) over each full page's real keys) and the
selection that the unchanged select pass makes from them. Bars as for the
summary scores: <= 1e-3 abs on scores; selected sets identical except keys
within 1e-4 of the k-th."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import SCORE_TOL, host, say, selection_ok

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def locks():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_page_selection_amd as m
    m.lib()
    return m


CASES = [
    dict(config=1),
    dict(config=2, ctx=16 * 700, batch=2, seq_lens=[16 * 700, 16 * 333 + 5]),
    dict(config=2, ctx=16 * 400, n_kv_heads=16, n_q_heads=32),   # G = 2
    dict(config=2, ctx=16 * 400, n_kv_heads=4, n_q_heads=32),    # G = 8
    dict(config=5, ctx=16 * 1200, budget=512),                   # G = 16
    dict(config=3, ctx=16 * 900, batch=2),                       # planted carrier
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()
                                                                if k != "seq_lens"))
def test_exact_scores_and_selection(locks, case):
    w = workloads.make(device=DEV, seed=31, **case)
    pt_d = w.page_table.clone()
    if w.max_pages > 40:
        pt_d[0, 17] = -1                  # an absent page
        w.page_table = pt_d
    dims = locks.make_dims(w.q, w.k_cache, w.page_table)
    ws = locks.new_workspace(dims, w.budget, DEV)
    scores = torch.full((w.batch, w.n_q_heads, w.max_pages), float("nan"), device=DEV)
    locks.exact_score_pages(w.q, w.k_cache, w.page_table, w.seq_lens, w.budget, ws,
                            page_scores=scores)
    sel = torch.empty(w.batch, w.n_kv_heads, w.k_pages, dtype=torch.int32, device=DEV)
    locks.select_pages(w.q, w.k_cache, w.page_table, w.seq_lens, w.budget, sel, ws,
                       page_scores=scores)
    torch.cuda.synchronize()
    q, pt, sl = host(w)
    ref = oracle.exact_scores(q, workloads.bf16_bits(w.k_cache), pt, sl)
    g = scores.cpu().numpy()
    valid = np.isfinite(ref)
    # pages j < n_b that are absent get exactly -inf; entries j >= n_b are
    # never written (they keep the NaN fill)
    n_b = np.minimum(sl // 16, w.max_pages)
    inside = np.broadcast_to(np.arange(w.max_pages)[None, None, :] < n_b[:, None, None], g.shape)
    assert np.all(g[~valid & inside] == -np.inf)
    assert np.all(np.isnan(g[~inside]))
    err = float(np.abs(g[valid] - ref[valid]).max())
    keys = oracle.group_keys(ref, w.n_kv_heads)
    o_sel = oracle.select(keys, w.k_pages)
    swaps = selection_ok(sel.cpu().numpy(), o_sel, keys, w.k_pages, np.isfinite(keys).sum(-1))
    say(f"  exact {w.recipe}: score err {err:.2e}, near-tie swaps {swaps}")
    assert err <= SCORE_TOL
