"""A decode step in which some pages have just filled (blog post, "How LOCKS
works": a page's summary is built once, when its 16th token lands; technical
summary, section 2 mechanism 4: the whole step in one graph, the summary
build off the decode critical path).

locks_decode_step_fill attends a just-filled page in full, never reads its
summary, and builds that summary in workgroups of its own scoring launch.
Checked: the step matches the oracle's reading of a just-filled page; the
records it builds are the bytes the whole-cache build writes (stale bytes in
their place before the step do not matter); the step captured in a graph
replays bit for bit like the eager call; and the next step scores the new
pages from the records the step built."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import SCORE_TOL, compact_cache, decode_and_check, host, out_ok, say, selection_ok

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def locks():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_page_selection_amd as m
    m.lib()
    return m


def check_fill_step(w, summ, filled, out, sel, ps):
    """GPU fill step against the oracle's composition on the same records."""
    q, pt, sl = host(w)
    sm = summ.cpu().numpy()
    kb, vb = workloads.bf16_bits(w.k_cache), workloads.bf16_bits(w.v_cache)
    fl = filled.cpu().numpy()
    o_out, o_sel, o_sc, o_keys = oracle.decode_step_fill(q, sm, kb, vb, pt, sl, w.budget, fl)
    g_sc = ps.cpu().numpy()
    valid = np.isfinite(o_sc)
    s_err = float(np.abs(g_sc[valid] - o_sc[valid]).max()) if valid.any() else 0.0
    assert s_err <= SCORE_TOL, f"page score error {s_err}"
    n_full = np.minimum(sl // 16, w.max_pages)
    held = (fl != 0) & (n_full > 0) & (sl == 16 * n_full)
    for b in np.nonzero(held)[0]:  # a just-filled page is never scored
        assert np.all(np.isnan(g_sc[b, :, n_full[b] - 1])), "the new page was scored"
    g_sel = sel.cpu().numpy()
    swaps = selection_ok(g_sel, o_sel, o_keys, w.k_pages, np.isfinite(o_keys).sum(-1))
    extra = np.where(held, n_full - 1, -1).astype(np.int32)
    listed = np.concatenate([g_sel, np.repeat(extra[:, None, None], w.n_kv_heads, axis=1)], axis=2)
    err, cos = out_ok(out.cpu().numpy(), oracle.attention(q, kb, vb, pt, sl, listed))
    say(f"  fill step: score err {s_err:.2e}, near-tie swaps {swaps}, out max-abs {err:.2e}, cos {cos:.7f}")


@pytest.mark.parametrize("config,hkv", [(2, 8), (2, 32), (2, 4), (5, 2)], ids=["G4", "G1", "G8", "G16"])
def test_fill_step_builds_the_new_pages_inside_the_step(locks, config, hkv):
    say(f"step with page fills, config {config}, {hkv} KV heads")
    lens = [16 * 600, 16 * 411 + 7, 16 * 350, 16 * 200, 16 * 90]
    w = workloads.make(config, device=DEV, ctx=16 * 601, batch=5, budget=512, n_kv_heads=hkv,
                       n_q_heads=32, seq_lens=lens, seed=61)
    pt = w.page_table.cpu().numpy()
    # sequences 0, 2 and 4 just filled their last page; 1 is mid-page (its
    # mark is ignored); 3's last page filled in an earlier step
    filled = torch.tensor([1, 1, 1, 0, 1], dtype=torch.int32, device=DEV)
    new = torch.tensor([pt[0, 599], pt[2, 349], pt[4, 89]], dtype=torch.long, device=DEV)
    summ = locks.build_summaries(w.k_cache, w.page_table, w.seq_lens)
    fresh = summ.clone()  # the whole-cache build's records

    def stale():  # the new pages' records are not built yet: garbage in their place
        summ[new] = 0xA5

    dims = locks.make_dims(w.q, w.k_cache, w.page_table)
    ws = locks.new_workspace(dims, w.budget, DEV)

    def buffers():
        return (torch.empty_like(w.q),
                torch.empty(w.batch, w.n_kv_heads, w.k_pages, dtype=torch.int32, device=DEV),
                torch.full((w.batch, w.n_q_heads, w.max_pages), float("nan"), device=DEV))

    stale()
    e_out, e_sel, e_ps = buffers()
    locks.decode_step(w.q, summ, w.k_cache, w.v_cache, w.page_table, w.seq_lens, w.budget,
                      out=e_out, selected=e_sel, page_scores=e_ps, workspace=ws, filled=filled)
    torch.cuda.synchronize()
    assert torch.equal(summ, fresh), "the step's records differ from the whole-cache build's"
    check_fill_step(w, summ, filled, e_out, e_sel, e_ps)

    # the step captured in a graph, replayed with stale records each time
    out, sel, ps = buffers()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        locks.decode_step(w.q, summ, w.k_cache, w.v_cache, w.page_table, w.seq_lens, w.budget,
                          out=out, selected=sel, page_scores=ps, workspace=ws, filled=filled)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        locks.decode_step(w.q, summ, w.k_cache, w.v_cache, w.page_table, w.seq_lens, w.budget,
                          out=out, selected=sel, page_scores=ps, workspace=ws, filled=filled)
    for rep in range(3):
        stale()
        out.zero_()
        sel.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, e_out) and torch.equal(sel, e_sel), f"replay {rep} differs from eager"
        assert torch.equal(summ, fresh), f"replay {rep}: records differ from the whole-cache build"
        _ = (w.q * 2).sum().item()  # eager work between replays

    # the next step (one more token each): the new pages are scored from the
    # records the step built
    w.seq_lens = w.seq_lens + 1
    decode_and_check(w, summ)


@pytest.mark.parametrize("config,budget", [(4, 2048), (5, 512)], ids=["1M-G4", "1M-G16"])
def test_full_size_fill_step(locks, config, budget):
    """The step with a page fill at the full 1M-token layers, in the launch
    configuration the benchmark times for its step with page fills: the
    records the scoring launch builds for the just-filled page are the
    whole-cache build's bytes; the other pages' scores, the selection and the
    output (over the selected pages plus the new one, only those K/V blocks
    copied to the host) match the oracle's reading of a just-filled page."""
    say(f"full-size step with a page fill, config {config}, budget {budget}")
    w = workloads.make(config, device=DEV, budget=budget)
    q, pt, sl = host(w)
    n = int(sl[0]) // 16
    assert sl[0] == 16 * n and n == w.max_pages, "premise: the last page is full"
    summ = locks.build_summaries(w.k_cache, w.page_table, w.seq_lens)
    fresh = summ.clone()
    summ[int(pt[0, n - 1])] = 0xA5  # not built yet: garbage in its place
    filled = torch.ones(1, dtype=torch.int32, device=DEV)
    scores = torch.full((1, w.n_q_heads, w.max_pages), float("nan"), device=DEV)
    out, sel = locks.decode_step(w.q, summ, w.k_cache, w.v_cache, w.page_table, w.seq_lens, budget,
                                 page_scores=scores, filled=filled)
    torch.cuda.synchronize()
    assert torch.equal(summ, fresh), "the step's records differ from the whole-cache build's"
    del fresh
    sm = summ.cpu().numpy()
    o_sc = oracle.scores(q, sm, pt, sl - 16, w.n_kv_heads)  # the new page is not scored
    g_sc = scores.cpu().numpy()
    assert np.all(np.isnan(g_sc[0, :, n - 1])), "the new page was scored"
    valid = np.isfinite(o_sc)
    s_err = float(np.abs(g_sc[valid] - o_sc[valid]).max()) if valid.any() else 0.0
    assert s_err <= SCORE_TOL, f"page score error {s_err}"
    o_keys = oracle.group_keys(o_sc, w.n_kv_heads)
    k = budget // 16
    g_sel = sel.cpu().numpy()
    swaps = selection_ok(g_sel, oracle.select(o_keys, k), o_keys, k, np.isfinite(o_keys).sum(-1))
    listed = np.concatenate([g_sel, np.full((1, w.n_kv_heads, 1), n - 1, dtype=np.int32)], axis=2)
    kb, vb, cpt = compact_cache(w, listed)
    err, cos = out_ok(out.cpu().numpy(), oracle.attention(q, kb, vb, cpt, sl, listed))
    say(f"  score err {s_err:.2e}, near-tie swaps {swaps}, out max-abs {err:.2e}, cos {cos:.7f}")
