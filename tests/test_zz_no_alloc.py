"""The no-allocation decode step (locks_decode_step_noalloc), for callers that
cannot allocate: same kernels as locks_decode_step, its workspace the
library's per-GPU scratch. Checked through the C ABI against the existing
entry point on two calls in a row, the second on a smaller input; both must
agree bit for bit (selected ids, output, page scores)."""
import ctypes

import pytest
import torch

import workloads
from parity import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def locks():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_page_selection_amd as m
    m.lib()
    return m


def both(locks, w):
    k = w.k_pages
    outs = []
    for noalloc in (False, True):
        out = torch.full_like(w.q, float("nan"))
        sel = torch.full((w.batch, w.n_kv_heads, k), -7, dtype=torch.int32, device=DEV)
        ps = torch.full((w.batch, w.n_q_heads, w.max_pages), float("nan"), device=DEV)
        summ = w.summ
        if noalloc:
            locks.decode_step_noalloc(w.q, summ, w.k_cache, w.v_cache, w.page_table, w.seq_lens,
                                      w.budget, out, sel, page_scores=ps)
        else:
            locks.decode_step(w.q, summ, w.k_cache, w.v_cache, w.page_table, w.seq_lens,
                              w.budget, out=out, selected=sel, page_scores=ps)
        torch.cuda.synchronize()
        outs.append((out, sel, ps))
    return outs


def test_noalloc_matches_decode_step_on_two_calls(locks):
    cases = [dict(config=3, ctx=16 * 3000, batch=3, budget=2048, seed=91,
                  seq_lens=[16 * 3000, 16 * 2111 + 5, 16 * 900]),
             dict(config=2, ctx=16 * 700, batch=1, budget=512, seed=92)]  # smaller, second
    for case in cases:
        say(f"no-alloc step {case}")
        w = workloads.make(device=DEV, **case)
        w.summ = locks.build_summaries(w.k_cache, w.page_table, w.seq_lens)
        (o_ref, s_ref, p_ref), (o, s, p) = both(locks, w)
        assert torch.equal(s, s_ref), "selected ids differ"
        assert torch.equal(o, o_ref), "outputs differ"
        n_b = (w.seq_lens // 16).clamp(max=w.max_pages)
        for b in range(w.batch):  # entries j < n_b are written, the same bits
            n = int(n_b[b])
            assert torch.equal(p[b, :, :n], p_ref[b, :, :n])
        assert bool(torch.isfinite(o).all())


def test_noalloc_refuses_dims_beyond_its_scratch(locks):
    """A workload whose workspace exceeds the scratch is refused on the host
    with LOCKS_ERR_WORKSPACE and a message; nothing is enqueued."""
    lib = locks.lib()
    d = locks.Dims(64, 32, 8, 128, 16, 8, 65536, 64 * 65536)
    need = locks.workspace_bytes(d, 2048)
    assert need > locks.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 20)
    st = lib.locks_decode_step_noalloc(ctypes.byref(d), fake, fake, fake, fake, fake, fake, 2048,
                                       fake, fake, None, None)
    assert st == locks.ERR_WORKSPACE and b"scratch" in lib.locks_last_error()
