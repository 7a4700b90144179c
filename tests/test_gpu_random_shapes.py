"""GPU parity on seeded random shapes: the whole decode step through the C ABI
against the fp64 oracle, with the bars of every other parity test (page scores
<= 1e-3 abs; selected sets identical except keys within 1e-4 of the k-th;
output <= 2e-2 max-abs, cosine >= 0.999).

Each case draws a batch, a KV head count, a GQA group size, the page-table
width, every sequence's length (empty sequences, sequences holding only a
partly filled page and ragged lengths included), a few absent page-table
entries (-1 or past the cache) in some draws, and a budget from 1 to 512
pages, so it meets combinations the fixed cases leave out: grids on either
side of the launch-shape switches (one or two waves' worth of scoring
workgroups, ranking inside or outside the attention launch, 1024- to
4096-page select chunks, tile or range bounds). Sizes keep the oracle within
seconds per case. The first 20 draws also run as steps in which some
sequences' last page has just filled (built inside the scoring launch),
through the attention entry points on caller-given lists and dense, and
through the summary build."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import decode_and_check, host, out_ok, say
from test_gpu_build import compare_builds
from test_gpu_fill import check_fill_step

pytestmark = pytest.mark.gpu

DEV = "cuda"
SEEDS = list(range(7001, 7041))


@pytest.fixture(scope="module")
def locks():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_page_selection_amd as m
    m.lib()
    return m


def draw(seed: int) -> dict:
    """One seeded shape: at most 64 query heads and 4 x 2500 pages."""
    rng = np.random.default_rng(seed)
    group = int(rng.choice([1, 2, 4, 8, 16]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    while group * hkv > 64:
        hkv //= 2
    batch = int(rng.integers(1, 5))
    pages = int(rng.integers(1, 2501))  # page-table width
    lens = []
    for _ in range(batch):
        u = rng.random()
        if u < 0.1:
            lens.append(0)                                    # empty
        elif u < 0.2:
            lens.append(int(rng.integers(1, 16)))             # a partly filled page only
        elif u < 0.5:
            lens.append(16 * pages)                           # every page full
        else:
            lens.append(int(rng.integers(1, 16 * pages + 1)))  # ragged
    k = int(rng.choice([1, 2, 7, 32, 128, 129, 256, 300, 512]))
    absent = []  # (sequence, page, entry): entry -1 or past the cache's blocks
    if rng.random() < 0.4:
        for _ in range(int(rng.integers(1, 6))):
            b = int(rng.integers(0, batch))
            if lens[b] >= 16:
                absent.append((b, int(rng.integers(0, lens[b] // 16)), int(rng.choice([-1, 1 << 20]))))
    return dict(batch=batch, n_kv_heads=hkv, n_q_heads=group * hkv, ctx=16 * pages, seq_lens=lens,
                budget=16 * k, seed=seed), absent


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shape_matches_the_oracle(locks, seed):
    case, absent = draw(seed)
    say(f"random shape {case} absent {absent}")
    w = workloads.make(2, device=DEV, **case)
    if absent:
        pt = w.page_table.clone()
        for b, j, e in absent:
            pt[b, j] = e
        w.page_table = pt
    summ = locks.build_summaries(w.k_cache, w.page_table, w.seq_lens)
    r = decode_and_check(w, summ, full_oracle_attention=False)
    sel = r["sel"].cpu().numpy()
    k = case["budget"] // 16
    for b, n in enumerate(case["seq_lens"]):
        full = n // 16
        gone = {j for bb, j, _ in absent if bb == b}
        n_keep = min(k, full - len(gone))
        kept = sel[b][:, :n_keep]
        assert np.all(kept >= 0) and np.all(kept < full), f"sequence {b}: a kept id outside its full pages"
        assert not gone & set(kept.ravel().tolist()), f"sequence {b}: an absent page was kept"
        assert np.all(sel[b][:, n_keep:] == -1), f"sequence {b}: entries past the kept pages are not -1"
        assert np.all(np.diff(kept, axis=-1) > 0), f"sequence {b}: kept ids not ascending"
    del w, summ
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seed", SEEDS[:20])
def test_random_shape_fill_step_matches_the_oracle(locks, seed):
    """The same shapes (no absent entries) as steps with page fills: each
    sequence is marked filled with probability 0.6; a marked sequence whose
    length is a whole number of pages has just filled its last page, whose
    record holds garbage before the step and the whole-cache build's bytes
    after it."""
    case, _ = draw(seed)
    rng = np.random.default_rng(seed + 1)
    marks = [int(rng.random() < 0.6) for _ in range(case["batch"])]
    say(f"random shape fill step {case} filled {marks}")
    w = workloads.make(2, device=DEV, **case)
    pt = w.page_table.cpu().numpy()
    summ = locks.build_summaries(w.k_cache, w.page_table, w.seq_lens)
    fresh = summ.clone()
    for b, n in enumerate(case["seq_lens"]):
        if marks[b] and n > 0 and n % 16 == 0:
            summ[int(pt[b, n // 16 - 1])] = 0xA5  # not built yet
    filled = torch.tensor(marks, dtype=torch.int32, device=DEV)
    ps = torch.full((w.batch, w.n_q_heads, w.max_pages), float("nan"), device=DEV)
    out, sel = locks.decode_step(w.q, summ, w.k_cache, w.v_cache, w.page_table, w.seq_lens, w.budget,
                                 page_scores=ps, filled=filled)
    torch.cuda.synchronize()
    assert torch.equal(summ, fresh), "the step's records differ from the whole-cache build's"
    check_fill_step(w, summ, filled, out, sel, ps)
    del w, summ, fresh
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seed", SEEDS[:20])
def test_random_shape_attention_on_caller_lists_and_dense(locks, seed):
    """The attention entry points on the same shapes (absent entries
    included): sparse attention over a caller-given list per (sequence, KV
    head) of distinct ids in shuffled order with -1 and out-of-range entries
    mixed in (both skipped), and dense attention over every page; both against
    the oracle's attention over the same lists, plus each sequence's tail."""
    case, absent = draw(seed)
    rng = np.random.default_rng(seed + 2)
    say(f"random shape attention {case} absent {absent}")
    w = workloads.make(2, device=DEV, **case)
    if absent:
        pt = w.page_table.clone()
        for b, j, e in absent:
            pt[b, j] = e
        w.page_table = pt
    B, hkv, k = w.batch, w.n_kv_heads, w.k_pages
    sel = np.full((B, hkv, k), -1, dtype=np.int32)
    for b, n in enumerate(case["seq_lens"]):
        full = n // 16
        for h in range(hkv):
            ids = rng.permutation(full)[: max(0, k - 2)] if full else np.zeros(0, dtype=np.int64)
            junk = [-1, full + int(rng.integers(0, 4)), -5][: k - len(ids)]
            row = np.concatenate([ids, np.array(junk, dtype=np.int64)])
            sel[b, h, : len(row)] = rng.permutation(row)
    q, pt, sl = host(w)
    kb, vb = workloads.bf16_bits(w.k_cache), workloads.bf16_bits(w.v_cache)
    ws = locks.new_workspace(locks.make_dims(w.q, w.k_cache, w.page_table), case["budget"], DEV)
    out = torch.full_like(w.q, float("nan"))
    locks.sparse_attention(w.q, w.k_cache, w.v_cache, w.page_table, w.seq_lens, case["budget"],
                           torch.from_numpy(sel).to(DEV), out, ws)
    dense = locks.dense_attention(w.q, w.k_cache, w.v_cache, w.page_table, w.seq_lens)
    torch.cuda.synchronize()
    e_s, c_s = out_ok(out.cpu().numpy(), oracle.attention(q, kb, vb, pt, sl, sel))
    e_d, c_d = out_ok(dense.cpu().numpy(), oracle.attention(q, kb, vb, pt, sl))
    say(f"  sparse max-abs {e_s:.2e} cos {c_s:.7f}; dense max-abs {e_d:.2e} cos {c_d:.7f}")
    del w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seed", SEEDS[:20])
def test_random_shape_build_writes_exactly_the_full_pages(locks, seed):
    """The summary build on the same shapes (absent entries included) writes
    the record of every block that a full page of some sequence maps to, and
    no other (tail pages, pages past a sequence's length, absent entries and
    unreferenced blocks keep their bytes); sampled records meet the oracle
    bars of the build tests."""
    case, absent = draw(seed)
    say(f"random shape build {case} absent {absent}")
    w = workloads.make(2, device=DEV, **case)
    if absent:
        pt = w.page_table.clone()
        for b, j, e in absent:
            pt[b, j] = e
        w.page_table = pt
    summ = torch.full((w.num_blocks, w.n_kv_heads, locks.summary_record_bytes()), 0xAB, dtype=torch.uint8,
                      device=DEV)
    locks.build_summaries(w.k_cache, w.page_table, w.seq_lens, summaries=summ)
    torch.cuda.synchronize()
    pt = w.page_table.cpu().numpy()
    built = {int(pt[b, j]) for b, n in enumerate(case["seq_lens"]) for j in range(n // 16)
             if 0 <= pt[b, j] < w.num_blocks}
    untouched = np.all(summ.cpu().numpy().reshape(w.num_blocks, -1) == 0xAB, axis=1)
    for blk in range(w.num_blocks):
        assert untouched[blk] != (blk in built), f"block {blk}: built {blk in built}, untouched {untouched[blk]}"
    if built:
        compare_builds(w, summ, n_sample=300, seed=seed)
    del w, summ
    torch.cuda.empty_cache()
