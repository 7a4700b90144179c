"""Variant summary formats (precision / rank ablation) on the GPU against the
fp64 oracle: the variant scorer on oracle-built records (scores within
1e-3), and the variant builder against oracle records (reconstruction error
within 1.05x the oracle's plus 1e-3 of the page energy; page scores within
5e-2 on pages whose oracle eigengap at the format's rank is >= 1.5)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import SCORE_TOL, host, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
FORMATS = [(r, vb) for r in (4, 8, 16) for vb in (2, 4, 16)]


@pytest.fixture(scope="module")
def locks():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_page_selection_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def small():
    return workloads.make(2, device=DEV, ctx=16 * 300, batch=2, seed=41,
                          seq_lens=[16 * 300, 16 * 211 + 7])


@pytest.mark.parametrize("fmt", FORMATS, ids=lambda f: f"r{f[0]}-v{f[1]}")
def test_variant_scores_on_oracle_records(locks, small, fmt):
    r, vb = fmt
    w = small
    q, pt, sl = host(w)
    kb = workloads.bf16_bits(w.k_cache)
    summ = oracle.build_summaries_variant(kb, pt, sl, r, vb)
    ws = locks.new_workspace(locks.make_dims(w.q, w.k_cache, w.page_table), w.budget, DEV)
    scores = torch.full((w.batch, w.n_q_heads, w.max_pages), float("nan"), device=DEV)
    locks.score_pages_variant(w.q, torch.from_numpy(summ).to(DEV), w.k_cache, w.page_table,
                              w.seq_lens, w.budget, r, vb, ws, page_scores=scores)
    torch.cuda.synchronize()
    ref = oracle.scores_variant(q, summ, pt, sl, w.n_kv_heads, r, vb)
    valid = np.isfinite(ref)
    err = float(np.abs(scores.cpu().numpy()[valid] - ref[valid]).max())
    say(f"  variant r{r} v{vb} scores: max err {err:.2e}")
    assert err <= SCORE_TOL


@pytest.mark.parametrize("fmt", [(8, 4), (16, 16), (4, 2)], ids=lambda f: f"r{f[0]}-v{f[1]}")
def test_variant_scores_at_group_16(locks, fmt):
    r, vb = fmt
    w = workloads.make(5, device=DEV, ctx=16 * 400, budget=512, seed=43)
    q, pt, sl = host(w)
    summ = oracle.build_summaries_variant(workloads.bf16_bits(w.k_cache), pt, sl, r, vb)
    ws = locks.new_workspace(locks.make_dims(w.q, w.k_cache, w.page_table), w.budget, DEV)
    scores = torch.empty(w.batch, w.n_q_heads, w.max_pages, device=DEV)
    locks.score_pages_variant(w.q, torch.from_numpy(summ).to(DEV), w.k_cache, w.page_table,
                              w.seq_lens, w.budget, r, vb, ws, page_scores=scores)
    torch.cuda.synchronize()
    ref = oracle.scores_variant(q, summ, pt, sl, w.n_kv_heads, r, vb)
    assert float(np.abs(scores.cpu().numpy() - ref).max()) <= SCORE_TOL


@pytest.mark.parametrize("fmt", FORMATS, ids=lambda f: f"r{f[0]}-v{f[1]}")
def test_variant_build_against_oracle_records(locks, small, fmt):
    r, vb = fmt
    w = small
    g = locks.build_summaries_variant(w.k_cache, w.page_table, w.seq_lens, r, vb)
    torch.cuda.synchronize()
    g = g.cpu().numpy()
    pt = w.page_table.cpu().numpy()
    kb = workloads.bf16_bits(w.k_cache)
    rng = np.random.default_rng(r * 100 + vb)
    items = [(b, j, h) for b in range(w.batch) for j in range(int(w.seq_lens[b]) // 16)
             for h in range(w.n_kv_heads)]
    rec_bad = score_bad = gap = 0
    for i in rng.choice(len(items), size=300, replace=False):
        b, j, h = items[i]
        blk = pt[b, j]
        keys = oracle.bf16_bits_to_f64(kb[blk, h])
        D = keys - keys.mean(0)
        lam = np.linalg.eigvalsh(D @ D.T)[::-1]
        o = oracle.unpack_record_variant(oracle.build_record_variant(kb[blk, h], r, vb), r, vb)
        gg = oracle.unpack_record_variant(g[blk, h], r, vb)
        errs = [np.linalg.norm(D - C @ V.T) for _, V, C in (o, gg)]
        rec_bad += errs[1] > 1.05 * errs[0] + 1e-3 * np.linalg.norm(D)
        if r >= 15 or lam[r] <= 1e-9 * lam[0] or lam[r - 1] / lam[r] >= 1.5:
            gap += 1
            for _ in range(2):
                qq = rng.standard_normal(128)
                if abs(oracle.page_score_f64(qq, *o) - oracle.page_score_f64(qq, *gg)) > 5e-2:
                    score_bad += 1
    say(f"  variant build r{r} v{vb}: recon bad {rec_bad}, gap pages {gap}, score bad {score_bad}")
    assert rec_bad == 0 and score_bad == 0
