"""The shared-basis comparison on the GPU (Proposition 1: blog post, "Why
shared-basis sparse attention is structurally broken"; technical summary,
section 3): records built on the GPU under one fixed shared projection per
(sequence, KV head) against the oracle's, their scores through the variant
scorer against the oracle's, and the blind direction itself on planted
pages: a carrier whose in-page structure lies in the null space of the
shared basis is dropped by the shared-basis selector and kept by LOCKS's
page-local summaries and by the exact selector."""
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


def f16_ulp(x):
    """One unit in the last place of fp16 at |x| (normal range; subnormal step below)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -14)))
    return 2.0 ** (e - 10)


def retained(sel, carrier, n_full, Hkv):
    """Fraction of (sequence, KV head) that keep their carrier, over the
    sequences whose carrier lies among their full pages."""
    return float(np.mean([carrier[b] in sel[b, h] for b in range(len(carrier))
                          for h in range(Hkv) if carrier[b] < n_full[b]]))


@pytest.mark.parametrize("hkv", [8, 2], ids=["G4", "G16"])
def test_shared_basis_records_scores_and_blind_direction(locks, hkv):
    w = workloads.make(2, device=DEV, ctx=16 * 2000, batch=2, budget=512, n_kv_heads=hkv,
                       n_q_heads=32, keys="shared", seed=5,
                       seq_lens=[16 * 2000, 16 * 1500 + 9])
    say(f"shared-basis comparison: {w.recipe}")
    q, pt, sl = host(w)
    kb = workloads.bf16_bits(w.k_cache)
    B, Hq, Hkv, N, k = w.batch, w.n_q_heads, w.n_kv_heads, w.max_pages, w.k_pages
    basis = w.shared_basis.contiguous()
    g_rec = locks.build_summaries_shared(w.k_cache, w.page_table, w.seq_lens, basis)
    torch.cuda.synchronize()
    o_rec = oracle.build_summaries_shared(kb, pt, sl, basis.double().cpu().numpy())
    g_np = g_rec.cpu().numpy()
    # records: V = fp16(W) bit for bit; mu and C within one fp16 step of the
    # oracle's (fp32 sums on the GPU, fp64 in the oracle, then one rounding)
    worst = 0.0
    for b in range(B):
        for j in range(0, int(sl[b]) // 16, 37):
            for h in range(Hkv):
                gm, gV, gC = oracle.unpack_record_variant(g_np[pt[b, j], h], 8, 16)
                om, oV, oC = oracle.unpack_record_variant(o_rec[pt[b, j], h], 8, 16)
                assert np.array_equal(gV, oV)
                for x, y in ((gm, om), (gC, oC)):
                    d = np.abs(x - y) / f16_ulp(y)
                    worst = max(worst, float(d.max()))
    assert worst <= 1.0 + 1e-9, f"records differ by {worst} fp16 steps"
    # scores of the GPU records: the variant scorer against the oracle's
    dims = locks.make_dims(w.q, w.k_cache, w.page_table)
    ws = locks.new_workspace(dims, w.budget, DEV)
    ps = torch.full((B, Hq, N), float("nan"), device=DEV)
    sh_sel = torch.empty(B, Hkv, k, dtype=torch.int32, device=DEV)
    locks.score_pages_variant(w.q, g_rec, w.k_cache, w.page_table, w.seq_lens, w.budget, 8, 16,
                              ws, page_scores=ps)
    locks.select_pages(w.q, w.k_cache, w.page_table, w.seq_lens, w.budget, sh_sel, ws, page_scores=ps)
    torch.cuda.synchronize()
    o_sc = oracle.scores_variant(q, g_np, pt, sl, Hkv, 8, 16)
    valid = np.isfinite(o_sc)
    err = float(np.abs(ps.cpu().numpy()[valid] - o_sc[valid]).max())
    assert err <= SCORE_TOL, f"shared-basis score error {err}"
    o_keys = oracle.group_keys(o_sc, Hkv)
    swaps = selection_ok(sh_sel.cpu().numpy(), oracle.select(o_keys, k), o_keys, k,
                         np.isfinite(o_keys).sum(-1))
    # the blind direction: exact and LOCKS keep every carrier, the shared basis none
    summ = locks.build_summaries(w.k_cache, w.page_table, w.seq_lens)
    _, lk_sel = locks.decode_step(w.q, summ, w.k_cache, w.v_cache, w.page_table, w.seq_lens,
                                  w.budget)
    ex_sel = torch.empty_like(sh_sel)
    locks.exact_score_pages(w.q, w.k_cache, w.page_table, w.seq_lens, w.budget, ws)
    locks.select_pages(w.q, w.k_cache, w.page_table, w.seq_lens, w.budget, ex_sel, ws)
    torch.cuda.synchronize()
    car = w.carrier.cpu().numpy()
    assert np.any(car < sl // 16), "premise: some carrier lies among the full pages"
    r_ex, r_lk, r_sh = (retained(s.cpu().numpy(), car, sl // 16, Hkv) for s in (ex_sel, lk_sel, sh_sel))
    say(f"  records within {worst:.2f} fp16 steps, score err {err:.2e}, near-tie swaps {swaps}; "
        f"carrier retained: exact {r_ex:.2f}, LOCKS {r_lk:.2f}, shared basis {r_sh:.2f}")
    assert r_ex == 1.0 and r_lk == 1.0 and r_sh == 0.0
