"""fp64 CPU oracle of the LOCKS decode path — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
import this package. It wraps ``locks_oracle.c`` (plain C, double precision)
with ctypes and numpy arrays; it never touches the GPU library, and the GPU
library never touches it.

Sources, cited by title and section:
  (A) "LOCKS: per-page SVD cuts KV-cache reads 10x at 1M context" — "How LOCKS
      works" (summary contents, page-score equation), "Code" (build, scoring,
      top-k and attention steps).
  (B) "LOCKS – 효율적인 롱 컨텍스트 디코딩을 위한 페이지 로컬 압축 키 요약"
      (gist.science, paper 2607.24555) — section 2, mechanisms 1-3.

Parity pins for every function are in ``tests/test_oracle_pins.py``. The
quantised path is pinned in pieces (the quantiser against numpy's fp16
rounding, the record layout against a record packed with numpy, the
unquantised score against the exact page LSE) and end to end from the record
on: the decode step's scores equal scipy's log-sum-exp over the keys a record
reconstructs (decoded there independently), and its selection is the stable
top-k of group keys formed there from them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "locks_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblocks_oracle.so")

PAGE = 16
DIM = 128
RANK = 8
RECORD_BYTES = 784


def build(force: bool = True) -> str:
    """Compile locks_oracle.c with gcc (-O2, OpenMP). Returns the .so path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=gnu11", "-Wall",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_double.restype = ctypes.c_double
        L.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_double.restype = ctypes.c_double
        L.oracle_double_to_f16.argtypes = [ctypes.c_double]
        L.oracle_double_to_f16.restype = ctypes.c_uint16
        L.oracle_jacobi_eigh.argtypes = [I, P, P, P]
        L.oracle_jacobi_eigh.restype = I
        L.oracle_page_summary_f64.argtypes = [P, I, P, P, P, P]
        L.oracle_page_summary_f64.restype = None
        L.oracle_build_record.argtypes = [P, P, P, P, P, P]
        L.oracle_build_record.restype = None
        L.oracle_unpack_record.argtypes = [P, P, P, P]
        L.oracle_unpack_record.restype = None
        L.oracle_build_summaries.argtypes = [I, I, I, I, P, P, P, P]
        L.oracle_build_summaries.restype = None
        L.oracle_page_score_f64.argtypes = [P, P, P, P, I]
        L.oracle_page_score_f64.restype = ctypes.c_double
        L.oracle_exact_page_lse.argtypes = [P, P]
        L.oracle_exact_page_lse.restype = ctypes.c_double
        L.oracle_scores.argtypes = [I, I, I, I, I, P, P, P, P, P]
        L.oracle_scores.restype = None
        L.oracle_group_keys.argtypes = [I, I, I, I, P, P]
        L.oracle_group_keys.restype = None
        L.oracle_select.argtypes = [I, I, I, P, I, P]
        L.oracle_select.restype = None
        L.oracle_attention.argtypes = [I, I, I, I, I, P, P, P, P, P, P, I, P]
        L.oracle_attention.restype = None
        L.oracle_decode_step.argtypes = [I, I, I, I, I, P, P, P, P, P, P, I, P, P, P, P]
        L.oracle_decode_step.restype = None
        L.oracle_exact_scores.argtypes = [I, I, I, I, I, P, P, P, P, P]
        L.oracle_exact_scores.restype = None
        L.oracle_variant_record_bytes.argtypes = [I, I]
        L.oracle_variant_record_bytes.restype = ctypes.c_size_t
        L.oracle_build_record_variant.argtypes = [P, I, I, P]
        L.oracle_build_record_variant.restype = None
        L.oracle_unpack_record_variant.argtypes = [P, I, I, P, P, P]
        L.oracle_unpack_record_variant.restype = None
        L.oracle_build_summaries_variant.argtypes = [I, I, I, I, P, P, P, I, I, P]
        L.oracle_build_summaries_variant.restype = None
        L.oracle_scores_variant.argtypes = [I, I, I, I, I, P, P, I, I, P, P, P]
        L.oracle_scores_variant.restype = None
        L.oracle_build_record_shared.argtypes = [P, P, I, P]
        L.oracle_build_record_shared.restype = None
        L.oracle_build_summaries_shared.argtypes = [I, I, I, I, P, P, P, P, I, P]
        L.oracle_build_summaries_shared.restype = None
        L.oracle_shared_basis.argtypes = [I, I, I, I, P, P, P, I, P]
        L.oracle_shared_basis.restype = None
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = I
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _as(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


# ---------------------------------------------------------------- formats

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16/int16) -> float64, exactly."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f16_bits_to_f64(h: int) -> float:
    return float(lib().oracle_f16_to_double(int(h) & 0xFFFF))


def f64_to_f16_bits(x: float) -> int:
    return int(lib().oracle_double_to_f16(float(x)))


# ---------------------------------------------------------------- build

def jacobi_eigh(a: np.ndarray):
    """Cyclic Jacobi on a symmetric matrix: (eigenvalues, eigenvectors as columns, sweeps)."""
    a = _as(a, np.float64).copy()
    n = a.shape[0]
    w = np.zeros(n)
    u = np.zeros((n, n))
    sweeps = lib().oracle_jacobi_eigh(n, _ptr(a), _ptr(w), _ptr(u))
    return w, u, sweeps


def page_summary_f64(keys: np.ndarray, rank: int = RANK):
    """Unquantised rank-r summary of one page (keys: 16x128 float64).

    Returns mu[128], V[128, r], C[16, r], lam[16] (descending)."""
    keys = _as(keys, np.float64)
    assert keys.shape == (PAGE, DIM) and 1 <= rank <= 16
    mu = np.zeros(DIM)
    V = np.zeros((DIM, rank))
    C = np.zeros((PAGE, rank))
    lam = np.zeros(PAGE)
    lib().oracle_page_summary_f64(_ptr(keys), rank, _ptr(mu), _ptr(V), _ptr(C), _ptr(lam))
    return mu, V, C, lam


def build_record(keys_bf16: np.ndarray):
    """Quantised 784-byte record of one page from its 16x128 bf16 bits.

    Returns (record uint8[784], lam[16], mu, V, C unquantised)."""
    kb = _as(keys_bf16, np.uint16)
    assert kb.shape == (PAGE, DIM)
    rec = np.zeros(RECORD_BYTES, dtype=np.uint8)
    lam = np.zeros(PAGE)
    mu = np.zeros(DIM)
    V = np.zeros((DIM, RANK))
    C = np.zeros((PAGE, RANK))
    lib().oracle_build_record(_ptr(kb), _ptr(rec), _ptr(lam), _ptr(mu), _ptr(V), _ptr(C))
    return rec, lam, mu, V, C


def unpack_record(rec: np.ndarray):
    """Dequantised (mu[128], V[128, 8], C[16, 8]) of one record."""
    rec = _as(rec, np.uint8)
    assert rec.shape == (RECORD_BYTES,)
    mu = np.zeros(DIM)
    V = np.zeros((DIM, RANK))
    C = np.zeros((PAGE, RANK))
    lib().oracle_unpack_record(_ptr(rec), _ptr(mu), _ptr(V), _ptr(C))
    return mu, V, C


def build_summaries(k_cache_bits: np.ndarray, page_table: np.ndarray, seq_lens: np.ndarray,
                    summaries: np.ndarray | None = None) -> np.ndarray:
    """Records for every full page. k_cache_bits: uint16 [num_blocks, Hkv, 16, 128]."""
    kc = _as(k_cache_bits, np.uint16)
    nb, hkv = kc.shape[0], kc.shape[1]
    pt = _as(page_table, np.int32)
    sl = _as(seq_lens, np.int32)
    if summaries is None:
        summaries = np.zeros((nb, hkv, RECORD_BYTES), dtype=np.uint8)
    lib().oracle_build_summaries(pt.shape[0], hkv, pt.shape[1], nb, _ptr(kc), _ptr(pt),
                                 _ptr(sl), _ptr(summaries))
    return summaries


def build_blocks(k_cache_bits: np.ndarray, blocks, summaries: np.ndarray) -> np.ndarray:
    """The records of the listed physical blocks (every KV head) rebuilt in a
    copy of `summaries`, as when those pages fill (A "How LOCKS works": a
    page's summary is built once, when its 16th token lands). Entries < 0 or
    >= num_blocks are skipped; the other records are left as they were."""
    kc = _as(k_cache_bits, np.uint16)
    out = np.array(summaries, dtype=np.uint8, copy=True)
    for blk in np.asarray(blocks, dtype=np.int64).ravel():
        if 0 <= blk < kc.shape[0]:
            for h in range(kc.shape[1]):
                out[blk, h] = build_record(kc[blk, h])[0]
    return out


# ------------------------------------------ variant formats (precision / rank ablation)

VARIANT_RANKS = (4, 8, 16)
VARIANT_VBITS = (2, 4, 16)


def variant_record_bytes(rank: int, vbits: int) -> int:
    """Bytes per record of the (rank, V bits) variant format."""
    assert rank in VARIANT_RANKS and vbits in VARIANT_VBITS
    return int(lib().oracle_variant_record_bytes(rank, vbits))


def build_record_variant(keys_bf16: np.ndarray, rank: int, vbits: int) -> np.ndarray:
    """Variant record of one page from its 16x128 bf16 bits (the same
    unquantised summary as build_record, stored at rank `rank` with V in
    `vbits` bits: 2 or 4 = integer codes, 16 = fp16; mu and C int8 or fp16)."""
    kb = _as(keys_bf16, np.uint16)
    assert kb.shape == (PAGE, DIM)
    rec = np.zeros(variant_record_bytes(rank, vbits), dtype=np.uint8)
    lib().oracle_build_record_variant(_ptr(kb), rank, vbits, _ptr(rec))
    return rec


def unpack_record_variant(rec: np.ndarray, rank: int, vbits: int):
    """Decoded (mu[128], V[128, rank], C[16, rank]) of one variant record."""
    rec = _as(rec, np.uint8)
    assert rec.shape == (variant_record_bytes(rank, vbits),)
    mu, V, C = np.zeros(DIM), np.zeros((DIM, rank)), np.zeros((PAGE, rank))
    lib().oracle_unpack_record_variant(_ptr(rec), rank, vbits, _ptr(mu), _ptr(V), _ptr(C))
    return mu, V, C


def build_summaries_variant(k_cache_bits, page_table, seq_lens, rank: int, vbits: int,
                            summaries: np.ndarray | None = None) -> np.ndarray:
    """Variant records [num_blocks, Hkv, variant_record_bytes] of every full page."""
    kc = _as(k_cache_bits, np.uint16)
    nb, hkv = kc.shape[0], kc.shape[1]
    pt = _as(page_table, np.int32)
    if summaries is None:
        summaries = np.zeros((nb, hkv, variant_record_bytes(rank, vbits)), dtype=np.uint8)
    lib().oracle_build_summaries_variant(pt.shape[0], hkv, pt.shape[1], nb, _ptr(kc), _ptr(pt),
                                         _ptr(_as(seq_lens, np.int32)), rank, vbits,
                                         _ptr(summaries))
    return summaries


def scores_variant(q, summaries, page_table, seq_lens, num_kv_heads: int, rank: int,
                   vbits: int) -> np.ndarray:
    """s_hat[b, h, j] from variant records (-inf for absent pages and j >= n_b)."""
    q = _as(q, np.float32)
    B, Hq, _ = q.shape
    pt = _as(page_table, np.int32)
    sm = _as(summaries, np.uint8)
    out = np.zeros((B, Hq, pt.shape[1]))
    lib().oracle_scores_variant(B, Hq, num_kv_heads, pt.shape[1], sm.shape[0], _ptr(q), _ptr(sm),
                                rank, vbits, _ptr(pt), _ptr(_as(seq_lens, np.int32)), _ptr(out))
    return out


# ------------------ shared-basis comparison (Proposition 1: blind directions)

def build_record_shared(keys_bf16: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Record of one page under a fixed shared basis W [128, r]: mu = the keys'
    mean, C = (K - mu) W, V = W, in the variant layout with fp16 values
    (rank r, v_bits 16), so that scores_variant scores it (A "Why shared-basis
    sparse attention is structurally broken"; B section 3, Proposition 1)."""
    kb = _as(keys_bf16, np.uint16)
    W = _as(W, np.float64)
    r = W.shape[1]
    assert kb.shape == (PAGE, DIM) and W.shape == (DIM, r)
    rec = np.zeros(variant_record_bytes(r, 16), dtype=np.uint8)
    lib().oracle_build_record_shared(_ptr(kb), _ptr(W), r, _ptr(rec))
    return rec


def build_summaries_shared(k_cache_bits, page_table, seq_lens, basis,
                           summaries: np.ndarray | None = None) -> np.ndarray:
    """Shared-basis records of every full page; basis [B, Hkv, 128, r] holds
    each (sequence, KV head)'s fixed projection."""
    kc = _as(k_cache_bits, np.uint16)
    nb, hkv = kc.shape[0], kc.shape[1]
    pt = _as(page_table, np.int32)
    basis = _as(basis, np.float64)
    r = basis.shape[-1]
    if summaries is None:
        summaries = np.zeros((nb, hkv, variant_record_bytes(r, 16)), dtype=np.uint8)
    lib().oracle_build_summaries_shared(pt.shape[0], hkv, pt.shape[1], nb, _ptr(kc), _ptr(pt),
                                        _ptr(_as(seq_lens, np.int32)), _ptr(basis), r,
                                        _ptr(summaries))
    return summaries


def shared_basis(k_cache_bits, page_table, seq_lens, rank: int = RANK) -> np.ndarray:
    """[B, Hkv, 128, rank]: per (sequence, KV head), the top eigenvectors of the
    pooled within-page deviation scatter over the sequence's full pages (the
    one projection a sequence-level selector shares across pages)."""
    kc = _as(k_cache_bits, np.uint16)
    nb, hkv = kc.shape[0], kc.shape[1]
    pt = _as(page_table, np.int32)
    out = np.zeros((pt.shape[0], hkv, DIM, rank))
    lib().oracle_shared_basis(pt.shape[0], hkv, pt.shape[1], nb, _ptr(kc), _ptr(pt),
                              _ptr(_as(seq_lens, np.int32)), rank, _ptr(out))
    return out


# ---------------------------------------------------------------- decode

def page_score_f64(q: np.ndarray, mu: np.ndarray, V: np.ndarray, C: np.ndarray) -> float:
    """s_hat for one head and one page from (unquantised or dequantised) summaries."""
    q = _as(q, np.float64)
    V = _as(V, np.float64)
    C = _as(C, np.float64)
    r = V.shape[1]
    assert V.shape == (DIM, r) and C.shape == (PAGE, r)
    return float(lib().oracle_page_score_f64(_ptr(q), _ptr(_as(mu, np.float64)), _ptr(V),
                                             _ptr(C), r))


def exact_page_lse(q: np.ndarray, keys: np.ndarray) -> float:
    """log sum_i exp(q.k_i / sqrt(128)) over a page's real keys."""
    return float(lib().oracle_exact_page_lse(_ptr(_as(q, np.float64)),
                                             _ptr(_as(keys, np.float64))))


def exact_scores(q, k_cache_bits, page_table, seq_lens) -> np.ndarray:
    """Exact page scores log sum_i exp(q.k_i / sqrt(128)) over every full page's
    real keys (the exact-mass selector; -inf for absent pages and j >= n_b)."""
    q = _as(q, np.float32)
    B, Hq, _ = q.shape
    kc = _as(k_cache_bits, np.uint16)
    pt = _as(page_table, np.int32)
    out = np.zeros((B, Hq, pt.shape[1]))
    lib().oracle_exact_scores(B, Hq, kc.shape[1], pt.shape[1], kc.shape[0], _ptr(q), _ptr(kc),
                              _ptr(pt), _ptr(_as(seq_lens, np.int32)), _ptr(out))
    return out


def scores(q, summaries, page_table, seq_lens, num_kv_heads: int) -> np.ndarray:
    """s_hat[b, h, j] (float64; -inf for absent pages and j >= n_b)."""
    q = _as(q, np.float32)
    B, Hq, _ = q.shape
    pt = _as(page_table, np.int32)
    sm = _as(summaries, np.uint8)
    out = np.zeros((B, Hq, pt.shape[1]))
    lib().oracle_scores(B, Hq, num_kv_heads, pt.shape[1], sm.shape[0], _ptr(q), _ptr(sm),
                        _ptr(pt), _ptr(_as(seq_lens, np.int32)), _ptr(out))
    return out


def group_keys(scores_: np.ndarray, num_kv_heads: int) -> np.ndarray:
    s = _as(scores_, np.float64)
    B, Hq, N = s.shape
    out = np.zeros((B, num_kv_heads, N))
    lib().oracle_group_keys(B, Hq, num_kv_heads, N, _ptr(s), _ptr(out))
    return out


def select(keys: np.ndarray, k: int) -> np.ndarray:
    kk = _as(keys, np.float64)
    B, Hkv, N = kk.shape
    out = np.zeros((B, Hkv, k), dtype=np.int32)
    lib().oracle_select(B, Hkv, N, _ptr(kk), k, _ptr(out))
    return out


def attention(q, k_cache_bits, v_cache_bits, page_table, seq_lens, selected=None) -> np.ndarray:
    """Attention over the listed pages (selected[b, kvh, :]) or, with None, every full
    page, plus each sequence's tail (the seq_len % 16 tokens of its partly filled page)."""
    q = _as(q, np.float32)
    B, Hq, _ = q.shape
    kc = _as(k_cache_bits, np.uint16)
    vc = _as(v_cache_bits, np.uint16)
    pt = _as(page_table, np.int32)
    hkv = kc.shape[1]
    sel = None if selected is None else _as(selected, np.int32)
    k = 0 if sel is None else sel.shape[2]
    out = np.zeros((B, Hq, DIM))
    lib().oracle_attention(B, Hq, hkv, pt.shape[1], kc.shape[0], _ptr(q), _ptr(kc), _ptr(vc),
                           _ptr(pt), _ptr(_as(seq_lens, np.int32)), _ptr(sel), k, _ptr(out))
    return out


def decode_step(q, summaries, k_cache_bits, v_cache_bits, page_table, seq_lens,
                budget_tokens: int):
    """Whole step: returns (out[B,Hq,128], selected[B,Hkv,k], scores, keys)."""
    q = _as(q, np.float32)
    B, Hq, _ = q.shape
    kc = _as(k_cache_bits, np.uint16)
    vc = _as(v_cache_bits, np.uint16)
    pt = _as(page_table, np.int32)
    sm = _as(summaries, np.uint8)
    hkv = kc.shape[1]
    N = pt.shape[1]
    k = budget_tokens // PAGE
    out = np.zeros((B, Hq, DIM))
    sel = np.zeros((B, hkv, k), dtype=np.int32)
    sc = np.zeros((B, Hq, N))
    ky = np.zeros((B, hkv, N))
    lib().oracle_decode_step(B, Hq, hkv, N, kc.shape[0], _ptr(q), _ptr(sm), _ptr(kc), _ptr(vc),
                             _ptr(pt), _ptr(_as(seq_lens, np.int32)), budget_tokens, _ptr(out),
                             _ptr(sel), _ptr(sc), _ptr(ky))
    return out, sel, sc, ky


def decode_step_fill(q, summaries, k_cache_bits, v_cache_bits, page_table, seq_lens,
                     budget_tokens: int, filled):
    """Decode step in which the sequences marked by filled[b] != 0 (with a
    length that is a positive multiple of 16) have just filled their last
    page, page n_b - 1, whose summary is not built yet (A "How LOCKS works": a
    summary is built once, when its page fills; B mechanism 4: building stays
    off the decode critical path). Reading: that page is treated as the
    newest, summary-less page, like a partly filled tail: never scored or
    selected, all 16 of its tokens attended. Composed from the pinned steps:
    scores over the first n_b - 1 pages, group keys, top-k, then attention
    over the kept pages plus page n_b - 1. Returns (out, selected, scores,
    keys) as decode_step does."""
    q = _as(q, np.float32)
    pt = _as(page_table, np.int32)
    sl = _as(seq_lens, np.int32)
    filled = np.asarray(filled).ravel()
    B, N = pt.shape
    hkv = np.asarray(k_cache_bits).shape[1]
    n_full = np.minimum(np.maximum(sl // PAGE, 0), N)
    held = (filled != 0) & (n_full > 0) & (sl == PAGE * n_full)
    sl_scored = np.where(held, sl - PAGE, sl).astype(np.int32)
    sc = scores(q, summaries, pt, sl_scored, hkv)
    ky = group_keys(sc, hkv)
    k = budget_tokens // PAGE
    sel = select(ky, k)
    extra = np.where(held, n_full - 1, -1).astype(np.int32)
    listed = np.concatenate([sel, np.repeat(extra[:, None, None], hkv, axis=1)], axis=2)
    out = attention(q, k_cache_bits, v_cache_bits, pt, sl, listed)
    return out, sel, sc, ky
