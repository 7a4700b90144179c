"""Helpers shared by the GPU parity tests: run the HIP path and the fp64 oracle
on the same bits and compare them to the bars the decode path is held to:
  page scores within 1e-3 absolute; selected page sets identical except pages
  whose oracle key lies within 1e-4 of the k-th key; attention output within
  2e-2 max-abs with cosine >= 0.999, against the oracle run on the GPU's set.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads

SCORE_TOL = 1e-3
TIE_TOL = 1e-4
OUT_TOL = 2e-2
COS_MIN = 0.999


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(w: workloads.Workload):
    return (w.q.cpu().numpy(), w.page_table.cpu().numpy(), w.seq_lens.cpu().numpy())


def compact_cache(w: workloads.Workload, sel: np.ndarray):
    """Host bits of only the blocks the selection (and each sequence's tail
    page) touches, with a page table remapped onto them (unlisted pages become
    absent). Keeps full-size parity
    cheap: the oracle reads the same bytes the GPU read."""
    pt = w.page_table.cpu().numpy()
    sl = w.seq_lens.cpu().numpy()
    B, Hkv, k = sel.shape
    N = pt.shape[1]
    blocks = set()
    for b in range(B):
        ids = sel[b].reshape(-1)
        ids = ids[(ids >= 0) & (ids < N)]
        blocks.update(pt[b, np.unique(ids)].tolist())
        n = min(int(sl[b]) // 16, N)
        if n < N and sl[b] > 16 * n:  # the tail page is attended too
            blocks.add(int(pt[b, n]))
    blocks = sorted(b for b in blocks if 0 <= b < w.num_blocks)
    remap = -np.ones(w.num_blocks, dtype=np.int64)
    remap[blocks] = np.arange(len(blocks))
    idx = torch.tensor(blocks if blocks else [0], dtype=torch.long, device=w.k_cache.device)
    kb = workloads.bf16_bits(w.k_cache.index_select(0, idx))
    vb = workloads.bf16_bits(w.v_cache.index_select(0, idx))
    new_pt = np.where(pt >= 0, remap[np.clip(pt, 0, w.num_blocks - 1)], -1).astype(np.int32)
    return kb, vb, new_pt


def selection_ok(g_sel: np.ndarray, o_sel: np.ndarray, o_keys: np.ndarray, k: int,
                 n_valid: np.ndarray):
    """Checks the GPU selection against the oracle's; returns #near-tie swaps."""
    B, Hkv, _ = g_sel.shape
    swaps = 0
    for b in range(B):
        for h in range(Hkv):
            g = g_sel[b, h]
            m = int(min(k, n_valid[b, h]))
            assert np.all(g[m:] == -1), "unused slots must be -1"
            gv = g[:m]
            assert np.all(np.diff(gv) > 0), "selected ids must be strictly ascending"
            keys = o_keys[b, h]
            assert np.all(np.isfinite(keys[gv])), "selected an absent page"
            if m == 0:
                continue
            kth = np.sort(keys[np.isfinite(keys)])[::-1][m - 1]
            diff = set(gv.tolist()) ^ set(o_sel[b, h, :m].tolist())
            for j in diff:
                assert abs(keys[j] - kth) <= TIE_TOL, (
                    f"(b={b}, kvh={h}) page {j} key {keys[j]:.6f} vs k-th {kth:.6f}")
            swaps += len(diff) // 2
    return swaps


def out_ok(g: np.ndarray, ref: np.ndarray):
    g = g.astype(np.float64)
    err = float(np.abs(g - ref).max()) if g.size else 0.0
    num = float((g * ref).sum())
    den = float(np.sqrt((g * g).sum() * (ref * ref).sum()))
    cos = num / den if den > 0 else 1.0
    assert err <= OUT_TOL, f"output max-abs error {err}"
    assert cos >= COS_MIN, f"output cosine {cos}"
    return err, cos


def decode_and_check(w: workloads.Workload, summ: torch.Tensor, budget: int | None = None,
                     full_oracle_attention: bool = True):
    """GPU decode step vs the oracle on the same packed summaries."""
    import kv_page_selection_amd as locks
    budget = budget or w.budget
    k = budget // 16
    dev = w.q.device
    scores = torch.full((w.batch, w.n_q_heads, w.max_pages), float("nan"), device=dev)
    out, sel = locks.decode_step(w.q, summ, w.k_cache, w.v_cache, w.page_table, w.seq_lens,
                                 budget, page_scores=scores)
    torch.cuda.synchronize()
    q, pt, sl = host(w)
    sm = summ.cpu().numpy()
    o_sc = oracle.scores(q, sm, pt, sl, w.n_kv_heads)
    valid = np.isfinite(o_sc)
    g_sc = scores.cpu().numpy()
    s_err = float(np.abs(g_sc[valid] - o_sc[valid]).max()) if valid.any() else 0.0
    assert s_err <= SCORE_TOL, f"page score error {s_err}"
    o_keys = oracle.group_keys(o_sc, w.n_kv_heads)
    o_sel = oracle.select(o_keys, k)
    g_sel = sel.cpu().numpy()
    n_valid = np.isfinite(o_keys).sum(-1)
    swaps = selection_ok(g_sel, o_sel, o_keys, k, n_valid)
    if full_oracle_attention:
        kb, vb = workloads.bf16_bits(w.k_cache), workloads.bf16_bits(w.v_cache)
        ref = oracle.attention(q, kb, vb, pt, sl, g_sel)
    else:
        kb, vb, cpt = compact_cache(w, g_sel)
        ref = oracle.attention(q, kb, vb, cpt, sl, g_sel)
    err, cos = out_ok(out.cpu().numpy(), ref)
    say(f"  {w.recipe} budget={budget}: score err {s_err:.2e}, near-tie swaps {swaps}, "
        f"out max-abs {err:.2e}, cos {cos:.7f}")
    return dict(score_err=s_err, swaps=swaps, out_err=err, cos=cos, out=out, sel=sel,
                scores=scores, o_keys=o_keys)


def plant_cutoff_tie(w: workloads.Workload, summ_host: np.ndarray, dup: int, seed: int = 0):
    """Maps `dup` low-scoring logical pages of sequence 0 onto the physical
    block of one page near the k-th place of (sequence 0, KV head 0), so that
    dup + 1 pages share one record and their group keys are bit-identical. The
    records are indexed by block, so no rebuild is needed. The page is chosen
    so that the tied pages straddle the k-th place after the remap (the extra
    copies move every head's total mass, hence every key). Returns the new
    host page table and the tied logical pages."""
    q, pt0, sl = host(w)
    k = w.k_pages
    n = int(sl[0]) // 16
    keys = oracle.group_keys(oracle.scores(q, summ_host, pt0, sl, w.n_kv_heads), w.n_kv_heads)
    order = np.lexsort((np.arange(n), -keys[0, 0, :n]))
    rng = np.random.default_rng(seed)
    victims = np.sort(rng.choice(order[n // 2:], size=dup, replace=False))  # far below the cut-off
    for r in sorted(range(max(0, k - 4 * dup), min(n // 2, k + dup)), key=lambda r: abs(r - k)):
        j0 = int(order[r])
        pt = pt0.copy()
        pt[0, victims] = pt[0, j0]
        kk = oracle.group_keys(oracle.scores(q, summ_host, pt, sl, w.n_kv_heads),
                               w.n_kv_heads)[0, 0]
        above = int((kk > kk[j0]).sum())
        near = (np.abs(kk - kk[j0]) <= 2 * TIE_TOL) & (kk != kk[j0])
        if above < k < above + dup + 1 and not near.any():
            return pt, np.sort(np.append(victims, j0))
    raise AssertionError("no page near the cut-off gives a straddling tie")


def cutoff_tie_premise(o_keys: np.ndarray, tied: np.ndarray, k: int):
    """The tied pages straddle the k-th place of (sequence 0, KV head 0) and
    no other key there lies within the near-tie band of theirs, so both sides
    must keep exactly the same ids there: those above, then the lowest tied
    ids. Returns the count above the tie."""
    kk = o_keys[0, 0]
    tie = kk[tied[0]]
    assert np.all(kk[tied] == tie), "tied pages must have bit-identical oracle keys"
    above = int((kk > tie).sum())
    assert above < k < above + len(tied), f"tie does not straddle the cut-off ({above}, {len(tied)})"
    near = (np.abs(kk - tie) <= 2 * TIE_TOL) & (kk != tie)
    assert not near.any(), "another key lies in the near-tie band of the planted tie"
    return above
