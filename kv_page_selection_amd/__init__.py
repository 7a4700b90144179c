"""Python binding of liblocks.so, the MI355X LOCKS decode path.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in include/locks.h. PyTorch provides device memory and the current
stream. There is no CPU fallback: if the library is not built, importing the
functions works but every call raises.

The names mirror the C entry points: build_summaries, decode_step,
score_pages, select_pages, sparse_attention, dense_attention,
workspace_bytes, summary_record_bytes.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblocks.so")

HEAD_DIM = 128
PAGE_SIZE = 16
RANK = 8

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
NOALLOC_SCRATCH_BYTES = 64 << 20  # LOCKS_NOALLOC_SCRATCH_BYTES


class Dims(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "page_size", "rank",
        "max_pages_per_seq", "num_blocks")]


class LocksError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"LOCKS status {status}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded liblocks.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                "g.build()'` (hipcc, gfx950). There is no fallback path.")
        L = ctypes.CDLL(LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        D = ctypes.POINTER(Dims)
        L.locks_summary_record_bytes.argtypes = []
        L.locks_summary_record_bytes.restype = S
        L.locks_last_error.argtypes = []
        L.locks_last_error.restype = ctypes.c_char_p
        L.locks_workspace_bytes.argtypes = [D, I, ctypes.POINTER(S)]
        L.locks_build_summaries.argtypes = [D, P, P, P, P, P]
        L.locks_build_blocks.argtypes = [D, P, P, I, P, P]
        L.locks_decode_step.argtypes = [D, P, P, P, P, P, P, I, P, P, P, P, S, P]
        L.locks_decode_step_noalloc.argtypes = [D, P, P, P, P, P, P, I, P, P, P, P]
        L.locks_decode_step_fill.argtypes = [D, P, P, P, P, P, P, P, I, P, P, P, P, S, P]
        L.locks_score_pages.argtypes = [D, P, P, P, P, I, P, P, S, P]
        L.locks_exact_score_pages.argtypes = [D, P, P, P, P, I, P, P, S, P]
        L.locks_variant_record_bytes.argtypes = [I, I, ctypes.POINTER(S)]
        L.locks_build_summaries_variant.argtypes = [D, P, P, P, I, I, P, P]
        L.locks_score_pages_variant.argtypes = [D, P, P, P, P, I, I, I, P, P, S, P]
        L.locks_build_summaries_shared.argtypes = [D, P, P, P, P, P, P]
        L.locks_select_pages.argtypes = [D, P, P, I, P, P, P, S, P]
        L.locks_sparse_attention.argtypes = [D, P, P, P, P, P, I, P, P, P, S, P]
        L.locks_dense_attention.argtypes = [D, P, P, P, P, P, P, P, S, P]
        for name in ("locks_workspace_bytes", "locks_build_summaries", "locks_build_blocks",
                     "locks_decode_step", "locks_decode_step_noalloc", "locks_decode_step_fill",
                     "locks_score_pages", "locks_exact_score_pages", "locks_select_pages",
                     "locks_variant_record_bytes", "locks_build_summaries_variant",
                     "locks_score_pages_variant", "locks_build_summaries_shared",
                     "locks_sparse_attention",
                     "locks_dense_attention"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != OK:
        raise LocksError(status, lib().locks_last_error().decode())


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("LOCKS tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_dims(q_or_batch, k_cache: torch.Tensor, page_table: torch.Tensor,
              n_q_heads: int | None = None) -> Dims:
    """Dims from tensors: q [B, Hq, 128] (or a batch size plus n_q_heads),
    k_cache [num_blocks, Hkv, 16, 128], page_table [B, max_pages]."""
    if isinstance(q_or_batch, torch.Tensor):
        B, Hq = int(q_or_batch.shape[0]), int(q_or_batch.shape[1])
    else:
        B, Hq = int(q_or_batch), int(n_q_heads)
    return Dims(B, Hq, int(k_cache.shape[1]), HEAD_DIM, PAGE_SIZE, RANK,
                int(page_table.shape[1]), int(k_cache.shape[0]))


def summary_record_bytes() -> int:
    return int(lib().locks_summary_record_bytes())


def workspace_bytes(dims: Dims, budget_tokens: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().locks_workspace_bytes(ctypes.byref(dims), int(budget_tokens), ctypes.byref(n)))
    return int(n.value)


def new_workspace(dims: Dims, budget_tokens: int, device) -> torch.Tensor:
    """A workspace of the size the C ABI asks for (zero-filled for tidiness)."""
    return torch.zeros(workspace_bytes(dims, budget_tokens), dtype=torch.uint8, device=device)


def _tensor(t, name: str, dtype: torch.dtype, shape) -> None:
    """Raises ValueError unless t is a contiguous tensor of this dtype and shape
    (None in `shape` accepts any extent there)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != len(shape) or any(w is not None and int(g) != w for g, w in zip(t.shape, shape)):
        want = "[" + ", ".join("*" if w is None else str(w) for w in shape) + "]"
        raise ValueError(f"{name} must have shape {want}, got {list(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _devices(named: dict) -> torch.device:
    """Every tensor on one cuda device (the C ABI takes device pointers only)."""
    devs = {n: t.device for n, t in named.items() if t is not None}
    dev = next(iter(devs.values()))
    for n, d in devs.items():
        if d != dev:
            raise ValueError(f"all LOCKS tensors must be on one device: {n} is on {d}, not {dev}")
    if dev.type != "cuda":
        raise ValueError("LOCKS runs on the GPU only; tensors must be on a cuda device")
    return dev


def _check_common(q, k_cache, page_table, seq_lens):
    """Shapes shared by every call: k_cache bf16 [num_blocks, Hkv, 16, 128],
    page_table int32 [B, max_pages], seq_lens int32 [B] and (when given) q f32
    [B, Hq, 128] with Hq a multiple of Hkv. Returns (B, Hq, Hkv, max_pages,
    num_blocks); Hq is None without q."""
    _tensor(k_cache, "k_cache", torch.bfloat16, (None, None, PAGE_SIZE, HEAD_DIM))
    _tensor(page_table, "page_table", torch.int32, (None, None))
    B, N = int(page_table.shape[0]), int(page_table.shape[1])
    nb, hkv = int(k_cache.shape[0]), int(k_cache.shape[1])
    _tensor(seq_lens, "seq_lens", torch.int32, (B,))
    hq = None
    if q is not None:
        _tensor(q, "q", torch.float32, (B, None, HEAD_DIM))
        hq = int(q.shape[1])
        if hkv == 0 or hq % hkv != 0:
            raise ValueError(f"q's {hq} heads must be a multiple of the caches' {hkv} KV heads")
    return B, hq, hkv, N, nb


def _pages(budget_tokens: int) -> int:
    if int(budget_tokens) < PAGE_SIZE or int(budget_tokens) % PAGE_SIZE != 0:
        raise ValueError("budget_tokens must be a positive multiple of 16")
    return int(budget_tokens) // PAGE_SIZE


def _workspace(workspace) -> None:
    _tensor(workspace, "workspace", torch.uint8, (None,))


def build_summaries(k_cache: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                    summaries: torch.Tensor | None = None, n_q_heads: int = 1) -> torch.Tensor:
    """Summary records [num_blocks, Hkv, 784] (uint8) of every full page."""
    B, _, hkv, N, nb = _check_common(None, k_cache, page_table, seq_lens)
    if summaries is not None:
        _tensor(summaries, "summaries", torch.uint8, (nb, hkv, summary_record_bytes()))
    dev = _devices(dict(k_cache=k_cache, page_table=page_table, seq_lens=seq_lens,
                        summaries=summaries))
    dims = Dims(B, hkv, hkv, HEAD_DIM, PAGE_SIZE, RANK, N, nb)
    if summaries is None:
        summaries = torch.zeros(nb, hkv, summary_record_bytes(), dtype=torch.uint8, device=dev)
    _check(lib().locks_build_summaries(ctypes.byref(dims), _ptr(k_cache), _ptr(page_table),
                                       _ptr(seq_lens), _ptr(summaries), _stream(dev)))
    return summaries


def build_blocks(k_cache: torch.Tensor, blocks: torch.Tensor, summaries: torch.Tensor) -> torch.Tensor:
    """Rebuilds, in place, the records of the listed physical blocks (every KV
    head): the pages that just filled. blocks: int32 [n] on the device;
    entries outside [0, num_blocks) are skipped."""
    _tensor(k_cache, "k_cache", torch.bfloat16, (None, None, PAGE_SIZE, HEAD_DIM))
    nb, hkv = int(k_cache.shape[0]), int(k_cache.shape[1])
    _tensor(blocks, "blocks", torch.int32, (None,))
    _tensor(summaries, "summaries", torch.uint8, (nb, hkv, summary_record_bytes()))
    dev = _devices(dict(k_cache=k_cache, blocks=blocks, summaries=summaries))
    dims = Dims(1, hkv, hkv, HEAD_DIM, PAGE_SIZE, RANK, 1, nb)
    _check(lib().locks_build_blocks(ctypes.byref(dims), _ptr(k_cache), _ptr(blocks),
                                    blocks.numel(), _ptr(summaries), _stream(dev)))
    return summaries


def decode_step(q, summaries, k_cache, v_cache, page_table, seq_lens, budget_tokens: int,
                out=None, selected=None, page_scores=None, workspace=None, filled=None):
    """One LOCKS decode step. Returns (out [B,Hq,128] f32, selected [B,Hkv,k] i32).
    filled (int32 [B], optional): nonzero where the sequence's last page filled
    in this step; that page is attended in full and not scored, and the step
    builds its summary records into `summaries` (locks_decode_step_fill)."""
    B, hq, hkv, N, nb = _check_common(q, k_cache, page_table, seq_lens)
    k = _pages(budget_tokens)
    _tensor(summaries, "summaries", torch.uint8, (nb, hkv, summary_record_bytes()))
    _tensor(v_cache, "v_cache", torch.bfloat16, tuple(k_cache.shape))
    if out is not None:
        _tensor(out, "out", torch.float32, (B, hq, HEAD_DIM))
    if selected is not None:
        _tensor(selected, "selected", torch.int32, (B, hkv, k))
    if page_scores is not None:
        _tensor(page_scores, "page_scores", torch.float32, (B, hq, N))
    if workspace is not None:
        _workspace(workspace)
    if filled is not None:
        _tensor(filled, "filled", torch.int32, (B,))
    dev = _devices(dict(q=q, summaries=summaries, k_cache=k_cache, v_cache=v_cache,
                        page_table=page_table, seq_lens=seq_lens, out=out, selected=selected,
                        page_scores=page_scores, workspace=workspace, filled=filled))
    dims = make_dims(q, k_cache, page_table)
    if out is None:
        out = torch.empty_like(q)
    if selected is None:
        selected = torch.empty(B, hkv, k, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = new_workspace(dims, budget_tokens, dev)
    if filled is None:
        _check(lib().locks_decode_step(
            ctypes.byref(dims), _ptr(q), _ptr(summaries), _ptr(k_cache), _ptr(v_cache),
            _ptr(page_table), _ptr(seq_lens), int(budget_tokens), _ptr(out), _ptr(selected),
            _ptr(page_scores), _ptr(workspace), workspace.numel(), _stream(dev)))
    else:
        _check(lib().locks_decode_step_fill(
            ctypes.byref(dims), _ptr(q), _ptr(summaries), _ptr(k_cache), _ptr(v_cache),
            _ptr(page_table), _ptr(seq_lens), _ptr(filled), int(budget_tokens), _ptr(out),
            _ptr(selected), _ptr(page_scores), _ptr(workspace), workspace.numel(), _stream(dev)))
    return out, selected


def decode_step_noalloc(q, summaries, k_cache, v_cache, page_table, seq_lens, budget_tokens: int,
                        out, selected, page_scores=None):
    """decode_step for callers that cannot allocate: the workspace is the
    library's own per-GPU scratch (NOALLOC_SCRATCH_BYTES); out and selected are
    the caller's. Calls that overlap on one GPU race on that scratch."""
    B, hq, hkv, N, nb = _check_common(q, k_cache, page_table, seq_lens)
    k = _pages(budget_tokens)
    _tensor(summaries, "summaries", torch.uint8, (nb, hkv, summary_record_bytes()))
    _tensor(v_cache, "v_cache", torch.bfloat16, tuple(k_cache.shape))
    _tensor(out, "out", torch.float32, (B, hq, HEAD_DIM))
    _tensor(selected, "selected", torch.int32, (B, hkv, k))
    if page_scores is not None:
        _tensor(page_scores, "page_scores", torch.float32, (B, hq, N))
    dev = _devices(dict(q=q, summaries=summaries, k_cache=k_cache, v_cache=v_cache,
                        page_table=page_table, seq_lens=seq_lens, out=out, selected=selected,
                        page_scores=page_scores))
    dims = make_dims(q, k_cache, page_table)
    _check(lib().locks_decode_step_noalloc(
        ctypes.byref(dims), _ptr(q), _ptr(summaries), _ptr(k_cache), _ptr(v_cache),
        _ptr(page_table), _ptr(seq_lens), int(budget_tokens), _ptr(out), _ptr(selected),
        _ptr(page_scores), _stream(dev)))
    return out, selected


def score_pages(q, summaries, k_cache, page_table, seq_lens, budget_tokens: int, workspace,
                page_scores=None):
    """Phase 1 (k_cache only supplies the dims)."""
    B, hq, hkv, N, nb = _check_common(q, k_cache, page_table, seq_lens)
    _pages(budget_tokens)
    _tensor(summaries, "summaries", torch.uint8, (nb, hkv, summary_record_bytes()))
    _workspace(workspace)
    if page_scores is not None:
        _tensor(page_scores, "page_scores", torch.float32, (B, hq, N))
    dev = _devices(dict(q=q, summaries=summaries, k_cache=k_cache, page_table=page_table,
                        seq_lens=seq_lens, workspace=workspace, page_scores=page_scores))
    dims = make_dims(q, k_cache, page_table)
    _check(lib().locks_score_pages(ctypes.byref(dims), _ptr(q), _ptr(summaries), _ptr(page_table),
                                   _ptr(seq_lens), int(budget_tokens), _ptr(page_scores),
                                   _ptr(workspace), workspace.numel(), _stream(dev)))


def exact_score_pages(q, k_cache, page_table, seq_lens, budget_tokens: int, workspace,
                      page_scores=None):
    """Reference phase 1: exact page masses from the keys (then select_pages
    selects by exact mass)."""
    B, hq, hkv, N, nb = _check_common(q, k_cache, page_table, seq_lens)
    _pages(budget_tokens)
    _workspace(workspace)
    if page_scores is not None:
        _tensor(page_scores, "page_scores", torch.float32, (B, hq, N))
    dev = _devices(dict(q=q, k_cache=k_cache, page_table=page_table, seq_lens=seq_lens,
                        workspace=workspace, page_scores=page_scores))
    dims = make_dims(q, k_cache, page_table)
    _check(lib().locks_exact_score_pages(ctypes.byref(dims), _ptr(q), _ptr(k_cache),
                                         _ptr(page_table), _ptr(seq_lens), int(budget_tokens),
                                         _ptr(page_scores), _ptr(workspace), workspace.numel(),
                                         _stream(dev)))


def variant_record_bytes(rank: int, v_bits: int) -> int:
    """Bytes per record of the (rank, V bits) variant format."""
    n = ctypes.c_size_t(0)
    _check(lib().locks_variant_record_bytes(rank, v_bits, ctypes.byref(n)))
    return n.value


def build_summaries_variant(k_cache, page_table, seq_lens, rank: int, v_bits: int,
                            summaries=None):
    """Variant records [num_blocks, Hkv, variant_record_bytes] of every full page."""
    B, _, hkv, N, nb = _check_common(None, k_cache, page_table, seq_lens)
    nbytes = variant_record_bytes(rank, v_bits)
    if summaries is not None:
        _tensor(summaries, "summaries", torch.uint8, (nb, hkv, nbytes))
    dev = _devices(dict(k_cache=k_cache, page_table=page_table, seq_lens=seq_lens,
                        summaries=summaries))
    dims = Dims(B, hkv, hkv, HEAD_DIM, PAGE_SIZE, RANK, N, nb)
    if summaries is None:
        summaries = torch.zeros(nb, hkv, nbytes, dtype=torch.uint8, device=dev)
    _check(lib().locks_build_summaries_variant(ctypes.byref(dims), _ptr(k_cache), _ptr(page_table),
                                               _ptr(seq_lens), rank, v_bits, _ptr(summaries),
                                               _stream(dev)))
    return summaries


def build_summaries_shared(k_cache, page_table, seq_lens, basis, summaries=None):
    """Shared-basis comparison records [num_blocks, Hkv, variant_record_bytes(8, 16)]
    of every full page under basis [B, Hkv, 128, 8] (f32): mu, C = (K - mu) W,
    V = W as fp16 values; score them with score_pages_variant(rank=8, v_bits=16)."""
    B, _, hkv, N, nb = _check_common(None, k_cache, page_table, seq_lens)
    _tensor(basis, "basis", torch.float32, (B, hkv, HEAD_DIM, RANK))
    nbytes = variant_record_bytes(RANK, 16)
    if summaries is not None:
        _tensor(summaries, "summaries", torch.uint8, (nb, hkv, nbytes))
    dev = _devices(dict(k_cache=k_cache, page_table=page_table, seq_lens=seq_lens, basis=basis,
                        summaries=summaries))
    dims = Dims(B, hkv, hkv, HEAD_DIM, PAGE_SIZE, RANK, N, nb)
    if summaries is None:
        summaries = torch.zeros(nb, hkv, nbytes, dtype=torch.uint8, device=dev)
    _check(lib().locks_build_summaries_shared(ctypes.byref(dims), _ptr(k_cache), _ptr(page_table),
                                              _ptr(seq_lens), _ptr(basis), _ptr(summaries),
                                              _stream(dev)))
    return summaries


def score_pages_variant(q, summaries, k_cache, page_table, seq_lens, budget_tokens: int, rank: int,
                        v_bits: int, workspace, page_scores=None):
    """Phase 1 from variant records (then select_pages / sparse_attention as usual)."""
    B, hq, hkv, N, nb = _check_common(q, k_cache, page_table, seq_lens)
    _pages(budget_tokens)
    _tensor(summaries, "summaries", torch.uint8, (nb, hkv, variant_record_bytes(rank, v_bits)))
    _workspace(workspace)
    if page_scores is not None:
        _tensor(page_scores, "page_scores", torch.float32, (B, hq, N))
    dev = _devices(dict(q=q, summaries=summaries, k_cache=k_cache, page_table=page_table,
                        seq_lens=seq_lens, workspace=workspace, page_scores=page_scores))
    dims = make_dims(q, k_cache, page_table)
    _check(lib().locks_score_pages_variant(ctypes.byref(dims), _ptr(q), _ptr(summaries),
                                           _ptr(page_table), _ptr(seq_lens), int(budget_tokens),
                                           rank, v_bits, _ptr(page_scores), _ptr(workspace),
                                           workspace.numel(), _stream(dev)))


def select_pages(q, k_cache, page_table, seq_lens, budget_tokens: int, selected, workspace,
                 page_scores=None):
    """Phase 2 (q and k_cache only supply the dims)."""
    B, hq, hkv, N, nb = _check_common(q, k_cache, page_table, seq_lens)
    k = _pages(budget_tokens)
    _tensor(selected, "selected", torch.int32, (B, hkv, k))
    _workspace(workspace)
    if page_scores is not None:
        _tensor(page_scores, "page_scores", torch.float32, (B, hq, N))
    dev = _devices(dict(q=q, k_cache=k_cache, page_table=page_table, seq_lens=seq_lens,
                        selected=selected, workspace=workspace, page_scores=page_scores))
    dims = make_dims(q, k_cache, page_table)
    _check(lib().locks_select_pages(ctypes.byref(dims), _ptr(page_table), _ptr(seq_lens),
                                    int(budget_tokens), _ptr(selected), _ptr(page_scores),
                                    _ptr(workspace), workspace.numel(), _stream(dev)))


def sparse_attention(q, k_cache, v_cache, page_table, seq_lens, budget_tokens: int, selected,
                     out, workspace):
    """Phase 3: attention over the pages listed in `selected` [B, Hkv, budget/16]."""
    B, hq, hkv, N, nb = _check_common(q, k_cache, page_table, seq_lens)
    k = _pages(budget_tokens)
    _tensor(v_cache, "v_cache", torch.bfloat16, tuple(k_cache.shape))
    _tensor(selected, "selected", torch.int32, (B, hkv, k))
    _tensor(out, "out", torch.float32, (B, hq, HEAD_DIM))
    _workspace(workspace)
    dev = _devices(dict(q=q, k_cache=k_cache, v_cache=v_cache, page_table=page_table,
                        seq_lens=seq_lens, selected=selected, out=out, workspace=workspace))
    dims = make_dims(q, k_cache, page_table)
    _check(lib().locks_sparse_attention(
        ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        _ptr(seq_lens), int(budget_tokens), _ptr(selected), _ptr(out), _ptr(workspace),
        workspace.numel(), _stream(dev)))


def dense_attention(q, k_cache, v_cache, page_table, seq_lens, out=None, workspace=None):
    """Dense decode attention over every full page (the comparator)."""
    B, hq, hkv, N, nb = _check_common(q, k_cache, page_table, seq_lens)
    _tensor(v_cache, "v_cache", torch.bfloat16, tuple(k_cache.shape))
    if out is not None:
        _tensor(out, "out", torch.float32, (B, hq, HEAD_DIM))
    if workspace is not None:
        _workspace(workspace)
    dev = _devices(dict(q=q, k_cache=k_cache, v_cache=v_cache, page_table=page_table,
                        seq_lens=seq_lens, out=out, workspace=workspace))
    dims = make_dims(q, k_cache, page_table)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = new_workspace(dims, PAGE_SIZE, dev)
    _check(lib().locks_dense_attention(
        ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        _ptr(seq_lens), _ptr(out), _ptr(workspace), workspace.numel(), _stream(dev)))
    return out
