"""C ABI checks that need no GPU: the library loads, exports every entry point
include/locks.h declares, and rejects bad arguments on the host before
anything is enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "locks.h")


@pytest.fixture(scope="module")
def L():
    import kv_page_selection_amd as m
    if not os.path.exists(m.LIB_PATH):
        from kv_page_selection_amd import _build
        _build.build()
    return m


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(locks_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for name in ("locks_build_summaries", "locks_build_blocks", "locks_decode_step",
                 "locks_score_pages",
                 "locks_select_pages", "locks_sparse_attention", "locks_dense_attention",
                 "locks_workspace_bytes", "locks_summary_record_bytes", "locks_last_error"):
        assert name in syms


def test_library_exports_every_declared_symbol(L):
    lib = L.lib()
    missing = [s for s in declared_symbols() if not hasattr(lib, s)]
    assert not missing, f"not exported: {missing}"


def dims(L, **kw):
    d = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, page_size=16, rank=8,
             max_pages_per_seq=65536, num_blocks=65536)
    d.update(kw)
    return L.Dims(*[d[k] for k, _ in L.Dims._fields_])


def test_record_size(L):
    assert L.summary_record_bytes() == 784


def test_variant_record_sizes_match_the_oracle_layout(L):
    """Host-side: the library's variant record sizes equal those of the
    independently written oracle layout; unsupported formats are refused."""
    import oracle
    for r in (4, 8, 16):
        for vb in (2, 4, 16):
            assert L.variant_record_bytes(r, vb) == oracle.variant_record_bytes(r, vb)
    for bad in ((8, 8), (2, 4), (32, 16)):
        with pytest.raises(L.LocksError) as e:
            L.variant_record_bytes(*bad)
        assert e.value.status == L.ERR_UNSUPPORTED


def test_workspace_sizing_and_validation(L):
    n = L.workspace_bytes(dims(L), 2048)
    assert n > 32 * 65536 * 4  # holds at least the per-head page scores
    assert L.workspace_bytes(dims(L), 512) < n
    with pytest.raises(L.LocksError) as e:
        L.workspace_bytes(dims(L), 2040)  # not a multiple of 16
    assert e.value.status == L.ERR_INVALID_ARG
    for bad in (dict(head_dim=64), dict(page_size=32), dict(rank=4), dict(n_q_heads=24)):
        with pytest.raises(L.LocksError) as e:
            L.workspace_bytes(dims(L, **bad), 512)
        assert e.value.status == L.ERR_UNSUPPORTED, bad
    for bad in (dict(batch=2, n_kv_heads=40000, n_q_heads=40000),
                dict(batch=1, n_kv_heads=40000, n_q_heads=640000),  # launch-grid limits
                dict(n_kv_heads=8, n_q_heads=32, num_blocks=11_000_000)):  # 32-bit record offsets
        with pytest.raises(L.LocksError) as e:
            L.workspace_bytes(dims(L, **bad), 512)
        assert e.value.status == L.ERR_UNSUPPORTED, bad
    with pytest.raises(L.LocksError) as e:
        L.workspace_bytes(dims(L, n_q_heads=30), 512)
    assert e.value.status == L.ERR_INVALID_ARG
    with pytest.raises(L.LocksError) as e:
        L.workspace_bytes(dims(L, batch=0), 512)
    assert e.value.status == L.ERR_INVALID_ARG


def test_entry_points_reject_null_and_small_workspace_on_host(L):
    lib = L.lib()
    d = dims(L)
    P = ctypes.c_void_p
    fake = P(1 << 20)  # aligned, never dereferenced: validation fails first
    st = lib.locks_decode_step(ctypes.byref(d), None, fake, fake, fake, fake, fake, 2048, fake,
                               fake, None, fake, 16, None)
    assert st == L.ERR_INVALID_ARG and b"q is NULL" in lib.locks_last_error()
    st = lib.locks_decode_step(ctypes.byref(d), fake, fake, fake, fake, fake, fake, 2048, fake,
                               fake, None, fake, 16, None)
    assert st == L.ERR_WORKSPACE and b"too small" in lib.locks_last_error()
    st = lib.locks_decode_step(ctypes.byref(d), fake, P((1 << 20) + 4), fake, fake, fake, fake,
                               2048, fake, fake, None, fake, 1 << 40, None)
    assert st == L.ERR_INVALID_ARG and b"aligned" in lib.locks_last_error()
    st = lib.locks_build_summaries(ctypes.byref(d), None, fake, fake, fake, None)
    assert st == L.ERR_INVALID_ARG
    # block-list build: n < 0 refused, n == 0 enqueues nothing, NULL list refused
    st = lib.locks_build_blocks(ctypes.byref(d), fake, fake, -1, fake, None)
    assert st == L.ERR_INVALID_ARG and b"n_blocks" in lib.locks_last_error()
    assert lib.locks_build_blocks(ctypes.byref(d), fake, None, 0, fake, None) == L.OK
    st = lib.locks_build_blocks(ctypes.byref(d), fake, None, 4, fake, None)
    assert st == L.ERR_INVALID_ARG and b"blocks is NULL" in lib.locks_last_error()
    st = lib.locks_dense_attention(None, fake, fake, fake, fake, fake, fake, fake, 1 << 40, None)
    assert st == L.ERR_INVALID_ARG and b"dims is NULL" in lib.locks_last_error()


def test_binding_refuses_cpu_tensors(L):
    import torch
    q = torch.zeros(1, 4, 128)
    kc = torch.zeros(8, 1, 16, 128, dtype=torch.bfloat16)
    pt = torch.zeros(1, 8, dtype=torch.int32)
    sl = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError):
        L.dense_attention(q, kc, kc, pt, sl)


def _valid_cpu_args(torch, B=2, Hq=8, Hkv=2, N=6, nb=16, budget=32):
    """Well-formed tensors for every binding call, on the CPU (so each call
    fails only at its device check, after every shape and dtype check)."""
    k = budget // 16
    return dict(
        q=torch.zeros(B, Hq, 128), kc=torch.zeros(nb, Hkv, 16, 128, dtype=torch.bfloat16),
        vc=torch.zeros(nb, Hkv, 16, 128, dtype=torch.bfloat16),
        pt=torch.zeros(B, N, dtype=torch.int32), sl=torch.zeros(B, dtype=torch.int32),
        summ=torch.zeros(nb, Hkv, 784, dtype=torch.uint8),
        out=torch.zeros(B, Hq, 128), sel=torch.zeros(B, Hkv, k, dtype=torch.int32),
        ps=torch.zeros(B, Hq, N), ws=torch.zeros(4096, dtype=torch.uint8), budget=budget)


def _calls(L, a):
    """Every binding entry point over the argument dict a."""
    return {
        "decode_step": lambda: L.decode_step(a["q"], a["summ"], a["kc"], a["vc"], a["pt"], a["sl"],
                                             a["budget"], out=a["out"], selected=a["sel"],
                                             page_scores=a["ps"], workspace=a["ws"]),
        "score_pages": lambda: L.score_pages(a["q"], a["summ"], a["kc"], a["pt"], a["sl"],
                                             a["budget"], a["ws"], page_scores=a["ps"]),
        "exact_score_pages": lambda: L.exact_score_pages(a["q"], a["kc"], a["pt"], a["sl"],
                                                         a["budget"], a["ws"], page_scores=a["ps"]),
        "select_pages": lambda: L.select_pages(a["q"], a["kc"], a["pt"], a["sl"], a["budget"],
                                               a["sel"], a["ws"], page_scores=a["ps"]),
        "sparse_attention": lambda: L.sparse_attention(a["q"], a["kc"], a["vc"], a["pt"], a["sl"],
                                                       a["budget"], a["sel"], a["out"], a["ws"]),
        "dense_attention": lambda: L.dense_attention(a["q"], a["kc"], a["vc"], a["pt"], a["sl"],
                                                     out=a["out"], workspace=a["ws"]),
        "build_summaries": lambda: L.build_summaries(a["kc"], a["pt"], a["sl"], summaries=a["summ"]),
        "build_blocks": lambda: L.build_blocks(a["kc"], a["sl"], a["summ"]),
    }


def test_binding_validates_shapes_dtypes_and_devices_before_any_call(L):
    """Every argument's dtype and shape is checked before the C call (the C ABI
    cannot see the size behind a device pointer): an undersized or mistyped
    tensor raises ValueError naming it; well-formed CPU tensors raise at the
    device check."""
    import torch
    good = _valid_cpu_args(torch)
    for name, call in _calls(L, good).items():
        with pytest.raises(ValueError, match="cuda device"):
            call()
    bad = {  # argument -> wrong replacement, with the calls that take it
        "q": [torch.zeros(2, 8, 64), torch.zeros(3, 8, 128), torch.zeros(2, 7, 128),
              torch.zeros(2, 8, 128, dtype=torch.float64)],
        "kc": [torch.zeros(16, 2, 16, 64, dtype=torch.bfloat16), torch.zeros(16, 2, 16, 128)],
        "vc": [torch.zeros(16, 1, 16, 128, dtype=torch.bfloat16), torch.zeros(16, 2, 16, 128)],
        "pt": [torch.zeros(2, 6, dtype=torch.int64), torch.zeros(12, dtype=torch.int32)],
        "sl": [torch.zeros(1, dtype=torch.int32), torch.zeros(2, dtype=torch.int64)],
        "summ": [torch.zeros(16, 2, 776, dtype=torch.uint8), torch.zeros(15, 2, 784, dtype=torch.uint8),
                 torch.zeros(16, 2, 784, dtype=torch.int8)],
        "out": [torch.zeros(2, 8, 127), torch.zeros(2, 8, 128, dtype=torch.float16)],
        "sel": [torch.zeros(2, 2, 1, dtype=torch.int32), torch.zeros(2, 2, 2, dtype=torch.int64)],
        "ps": [torch.zeros(2, 8, 5), torch.zeros(2, 8, 6, dtype=torch.float64)],
        "ws": [torch.zeros(4096, dtype=torch.int32), torch.zeros(64, 64, dtype=torch.uint8)],
        "budget": [24, 0],
    }
    uses = {"decode_step": "q summ kc vc pt sl out sel ps ws budget",
            "score_pages": "q summ kc pt sl ps ws budget",
            "exact_score_pages": "q kc pt sl ps ws budget",
            "select_pages": "q kc pt sl sel ps ws budget",
            "sparse_attention": "q kc vc pt sl sel out ws budget",
            "dense_attention": "q kc vc pt sl out ws",
            "build_summaries": "kc pt sl summ",
            "build_blocks": "kc summ"}
    for fn, args in uses.items():
        for arg in args.split():
            for wrong in bad[arg]:
                a = dict(good)
                a[arg] = wrong
                with pytest.raises(ValueError) as e:
                    _calls(L, a)[fn]()
                assert "cuda device" not in str(e.value), (fn, arg, str(e.value))
    # non-contiguous and mixed-device tensors
    a = dict(good)
    a["q"] = torch.zeros(2, 128, 8).transpose(1, 2)
    with pytest.raises(ValueError, match="contiguous"):
        _calls(L, a)["decode_step"]()
    a = dict(good)
    a["out"] = torch.zeros(2, 8, 128, device="meta")
    with pytest.raises(ValueError, match="one device"):
        _calls(L, a)["decode_step"]()


def test_noalloc_step_refuses_workloads_beyond_its_scratch_on_host(L):
    """locks_decode_step_noalloc checks the workspace its dims need against the
    library's scratch before anything else touches the GPU."""
    lib = L.lib()
    d = dims(L, batch=64, num_blocks=64 * 65536)
    assert L.workspace_bytes(d, 2048) > L.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 20)
    st = lib.locks_decode_step_noalloc(ctypes.byref(d), fake, fake, fake, fake, fake, fake, 2048,
                                       fake, fake, None, None)
    assert st == L.ERR_WORKSPACE and b"scratch" in lib.locks_last_error()
