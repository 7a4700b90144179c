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
        L.locks_score_pages.argtypes = [D, P, P, P, P, I, P, P, S, P]
        L.locks_exact_score_pages.argtypes = [D, P, P, P, P, I, P, P, S, P]
        L.locks_variant_record_bytes.argtypes = [I, I, ctypes.POINTER(S)]
        L.locks_build_summaries_variant.argtypes = [D, P, P, P, I, I, P, P]
        L.locks_score_pages_variant.argtypes = [D, P, P, P, P, I, I, I, P, P, S, P]
        L.locks_select_pages.argtypes = [D, P, P, I, P, P, P, S, P]
        L.locks_sparse_attention.argtypes = [D, P, P, P, P, P, I, P, P, P, S, P]
        L.locks_dense_attention.argtypes = [D, P, P, P, P, P, P, P, S, P]
        for name in ("locks_workspace_bytes", "locks_build_summaries", "locks_build_blocks",
                     "locks_decode_step",
                     "locks_score_pages", "locks_exact_score_pages", "locks_select_pages",
                     "locks_variant_record_bytes", "locks_build_summaries_variant",
                     "locks_score_pages_variant",
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


def _check_common(q, k_cache, page_table, seq_lens):
    if q is not None and (q.dtype != torch.float32 or q.dim() != 3 or q.shape[2] != HEAD_DIM):
        raise ValueError("q must be float32 [B, Hq, 128]")
    if k_cache.dtype != torch.bfloat16 or k_cache.dim() != 4 or tuple(k_cache.shape[2:]) != (16, 128):
        raise ValueError("caches must be bfloat16 [num_blocks, Hkv, 16, 128]")
    if page_table.dtype != torch.int32 or page_table.dim() != 2:
        raise ValueError("page_table must be int32 [B, max_pages]")
    if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1:
        raise ValueError("seq_lens must be int32 [B]")
    dev = k_cache.device
    for t in (q, page_table, seq_lens):
        if t is not None and t.device != dev:
            raise ValueError("all LOCKS tensors must be on the same device")
    if dev.type != "cuda":
        raise ValueError("LOCKS runs on the GPU only; tensors must be on a cuda device")


def build_summaries(k_cache: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                    summaries: torch.Tensor | None = None, n_q_heads: int = 1) -> torch.Tensor:
    """Summary records [num_blocks, Hkv, 784] (uint8) of every full page."""
    _check_common(None, k_cache, page_table, seq_lens)
    dims = make_dims(page_table.shape[0], k_cache, page_table, n_q_heads=k_cache.shape[1])
    if summaries is None:
        summaries = torch.zeros(k_cache.shape[0], k_cache.shape[1], summary_record_bytes(),
                                dtype=torch.uint8, device=k_cache.device)
    _check(lib().locks_build_summaries(ctypes.byref(dims), _ptr(k_cache), _ptr(page_table),
                                       _ptr(seq_lens), _ptr(summaries), _stream(k_cache.device)))
    return summaries


def build_blocks(k_cache: torch.Tensor, blocks: torch.Tensor, summaries: torch.Tensor) -> torch.Tensor:
    """Rebuilds, in place, the records of the listed physical blocks (every KV
    head): the pages that just filled. blocks: int32 [n] on the device;
    entries outside [0, num_blocks) are skipped."""
    _check_common(None, k_cache, torch.zeros(1, 1, dtype=torch.int32, device=k_cache.device),
                  torch.zeros(1, dtype=torch.int32, device=k_cache.device))
    if blocks.dtype != torch.int32 or blocks.dim() != 1 or blocks.device != k_cache.device:
        raise ValueError("blocks must be int32 [n] on the caches' device")
    if summaries.dtype != torch.uint8 or tuple(summaries.shape) != (
            k_cache.shape[0], k_cache.shape[1], summary_record_bytes()):
        raise ValueError("summaries must be uint8 [num_blocks, Hkv, 784]")
    blocks = blocks.contiguous()
    dims = Dims(1, k_cache.shape[1], k_cache.shape[1], HEAD_DIM, 16, 8, 1, k_cache.shape[0])
    _check(lib().locks_build_blocks(ctypes.byref(dims), _ptr(k_cache), _ptr(blocks),
                                    blocks.numel(), _ptr(summaries), _stream(k_cache.device)))
    return summaries


def decode_step(q, summaries, k_cache, v_cache, page_table, seq_lens, budget_tokens: int,
                out=None, selected=None, page_scores=None, workspace=None):
    """One LOCKS decode step. Returns (out [B,Hq,128] f32, selected [B,Hkv,k] i32)."""
    _check_common(q, k_cache, page_table, seq_lens)
    dims = make_dims(q, k_cache, page_table)
    dev = q.device
    k = budget_tokens // PAGE_SIZE
    if out is None:
        out = torch.empty_like(q)
    if selected is None:
        selected = torch.empty(dims.batch, dims.n_kv_heads, k, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = new_workspace(dims, budget_tokens, dev)
    _check(lib().locks_decode_step(
        ctypes.byref(dims), _ptr(q), _ptr(summaries), _ptr(k_cache), _ptr(v_cache),
        _ptr(page_table), _ptr(seq_lens), int(budget_tokens), _ptr(out), _ptr(selected),
        _ptr(page_scores), _ptr(workspace), workspace.numel(), _stream(dev)))
    return out, selected


def score_pages(q, summaries, k_cache, page_table, seq_lens, budget_tokens: int, workspace,
                page_scores=None):
    """Phase 1 (k_cache only supplies the dims)."""
    _check_common(q, k_cache, page_table, seq_lens)
    dims = make_dims(q, k_cache, page_table)
    _check(lib().locks_score_pages(ctypes.byref(dims), _ptr(q), _ptr(summaries), _ptr(page_table),
                                   _ptr(seq_lens), int(budget_tokens), _ptr(page_scores),
                                   _ptr(workspace), workspace.numel(), _stream(q.device)))


def exact_score_pages(q, k_cache, page_table, seq_lens, budget_tokens: int, workspace,
                      page_scores=None):
    """Reference phase 1: exact page masses from the keys (then select_pages
    selects by exact mass)."""
    _check_common(q, k_cache, page_table, seq_lens)
    dims = make_dims(q, k_cache, page_table)
    _check(lib().locks_exact_score_pages(ctypes.byref(dims), _ptr(q), _ptr(k_cache),
                                         _ptr(page_table), _ptr(seq_lens), int(budget_tokens),
                                         _ptr(page_scores), _ptr(workspace), workspace.numel(),
                                         _stream(q.device)))


def variant_record_bytes(rank: int, v_bits: int) -> int:
    """Bytes per record of the (rank, V bits) variant format."""
    n = ctypes.c_size_t(0)
    _check(lib().locks_variant_record_bytes(rank, v_bits, ctypes.byref(n)))
    return n.value


def build_summaries_variant(k_cache, page_table, seq_lens, rank: int, v_bits: int,
                            summaries=None):
    """Variant records [num_blocks, Hkv, variant_record_bytes] of every full page."""
    _check_common(None, k_cache, page_table, seq_lens)
    dims = make_dims(page_table.shape[0], k_cache, page_table, n_q_heads=k_cache.shape[1])
    if summaries is None:
        summaries = torch.zeros(k_cache.shape[0], k_cache.shape[1],
                                variant_record_bytes(rank, v_bits), dtype=torch.uint8,
                                device=k_cache.device)
    _check(lib().locks_build_summaries_variant(ctypes.byref(dims), _ptr(k_cache), _ptr(page_table),
                                               _ptr(seq_lens), rank, v_bits, _ptr(summaries),
                                               _stream(k_cache.device)))
    return summaries


def score_pages_variant(q, summaries, k_cache, page_table, seq_lens, budget_tokens: int, rank: int,
                        v_bits: int, workspace, page_scores=None):
    """Phase 1 from variant records (then select_pages / sparse_attention as usual)."""
    _check_common(q, k_cache, page_table, seq_lens)
    dims = make_dims(q, k_cache, page_table)
    _check(lib().locks_score_pages_variant(ctypes.byref(dims), _ptr(q), _ptr(summaries),
                                           _ptr(page_table), _ptr(seq_lens), int(budget_tokens),
                                           rank, v_bits, _ptr(page_scores), _ptr(workspace),
                                           workspace.numel(), _stream(q.device)))


def select_pages(q, k_cache, page_table, seq_lens, budget_tokens: int, selected, workspace,
                 page_scores=None):
    """Phase 2 (q and k_cache only supply the dims)."""
    _check_common(q, k_cache, page_table, seq_lens)
    dims = make_dims(q, k_cache, page_table)
    _check(lib().locks_select_pages(ctypes.byref(dims), _ptr(page_table), _ptr(seq_lens),
                                    int(budget_tokens), _ptr(selected), _ptr(page_scores),
                                    _ptr(workspace), workspace.numel(), _stream(q.device)))


def sparse_attention(q, k_cache, v_cache, page_table, seq_lens, budget_tokens: int, selected,
                     out, workspace):
    """Phase 3: attention over the pages listed in `selected` [B, Hkv, budget/16]."""
    _check_common(q, k_cache, page_table, seq_lens)
    dims = make_dims(q, k_cache, page_table)
    _check(lib().locks_sparse_attention(
        ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        _ptr(seq_lens), int(budget_tokens), _ptr(selected), _ptr(out), _ptr(workspace),
        workspace.numel(), _stream(q.device)))


def dense_attention(q, k_cache, v_cache, page_table, seq_lens, out=None, workspace=None):
    """Dense decode attention over every full page (the comparator)."""
    _check_common(q, k_cache, page_table, seq_lens)
    dims = make_dims(q, k_cache, page_table)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = new_workspace(dims, PAGE_SIZE, q.device)
    _check(lib().locks_dense_attention(
        ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        _ptr(seq_lens), _ptr(out), _ptr(workspace), workspace.numel(), _stream(q.device)))
    return out
