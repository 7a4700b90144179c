"""Pins of the fp64 oracle against things other than itself.

Each test ties an oracle function to a closed form, a library routine
(LAPACK via numpy, torch's SDPA, scipy's logsumexp on real keys), an invariant
the mathematics fixes, or a brute force on tiny inputs. Sources:
(A) "LOCKS: per-page SVD cuts KV-cache reads 10x at 1M context", sections
"How LOCKS works" and "Code"; (B) the gist.science technical summary of paper
2607.24555, section 2 mechanisms 1-3 and section 3 (theory).
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

PAGE, DIM = 16, 128


def rng(seed):
    return np.random.default_rng(seed)


def exact_lse(q, keys):
    """Library form of the exact per-page log-sum-exp of q.k/sqrt(d)."""
    return float(logsumexp(keys @ q / math.sqrt(DIM)))


def planted_page(r, rank, noise=0.0, scale=1.0):
    mu = r.standard_normal(DIM) * scale
    basis, _ = np.linalg.qr(r.standard_normal((DIM, rank)))
    coef = r.standard_normal((PAGE, rank)) / np.arange(1, rank + 1)
    return mu + coef @ basis.T + noise * r.standard_normal((PAGE, DIM))


# ------------------------------------------------------------ number formats

def test_bf16_decode_matches_torch(orc):
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    ours = np.array([orc.lib().oracle_bf16_to_double(int(b)) for b in bits[finite][::7]])
    ref = torch.from_numpy(bits[finite][::7].view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(ours, ref)


def test_f16_decode_all_patterns_match_numpy(orc):
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    ours = np.array([orc.f16_bits_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_f16_encode_round_half_even_matches_numpy(orc):
    r = rng(1)
    xs = np.concatenate([
        r.standard_normal(4000) * 10.0 ** r.integers(-9, 5, 4000),
        np.array([0.0, 65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                  2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11]),
    ])
    for x in xs:
        for s in (1.0, -1.0):
            got = orc.f64_to_f16_bits(s * x)
            with np.errstate(over="ignore"):
                want = int(np.array([s * x]).astype(np.float16).view(np.uint16)[0])
            assert got == want, (s * x, hex(got), hex(want))


# ------------------------------------------------------------ eigensolver

@pytest.mark.parametrize("seed", range(6))
def test_jacobi_matches_lapack(orc, seed):
    r = rng(seed)
    d = r.standard_normal((PAGE, DIM)) * r.uniform(0.1, 3)
    a = d @ d.T
    w, u, sweeps = orc.jacobi_eigh(a)
    ref = np.linalg.eigvalsh(a)
    assert np.allclose(np.sort(w), ref, rtol=1e-11, atol=1e-11 * ref.max())
    assert np.allclose(u.T @ u, np.eye(PAGE), atol=1e-12)
    assert np.allclose(a @ u, u * w, atol=1e-10 * ref.max())
    assert sweeps < 30


def test_jacobi_diagonal_and_degenerate(orc):
    w, u, sweeps = orc.jacobi_eigh(np.diag(np.arange(16.0)))
    assert sweeps == 0 and np.array_equal(w, np.arange(16.0))
    w, u, _ = orc.jacobi_eigh(np.ones((16, 16)))  # rank one: eigenvalues {16, 0 x15}
    assert np.allclose(np.sort(w), [0.0] * 15 + [16.0], atol=1e-12)


# ------------------------------------------------------------ summary build

@pytest.mark.parametrize("seed", range(4))
def test_rank15_reconstruction_makes_scores_exact(orc, seed):
    """Centred 16-token deviations have rank <= 15, so an unquantised rank-15
    summary reproduces every key and the page score equals the exact LSE
    (A page-score equation; the centring makes the 16th direction null)."""
    r = rng(100 + seed)
    keys = r.standard_normal((PAGE, DIM)) * 1.5 + r.standard_normal(DIM)
    mu, V, C, lam = orc.page_summary_f64(keys, rank=15)
    assert np.allclose(mu[None, :] + C @ V.T, keys, atol=1e-11)
    for t in range(5):
        q = r.standard_normal(DIM) * (1 + t)
        assert abs(orc.page_score_f64(q, mu, V, C) - exact_lse(q, keys)) < 1e-11


def test_planted_rank8_page_scores_exact_at_rank8(orc):
    r = rng(7)
    for _ in range(5):
        keys = planted_page(r, 8)
        mu, V, C, lam = orc.page_summary_f64(keys, rank=8)
        assert np.abs(lam[8:]).max() < 1e-13 * lam[0]  # null up to fp64 rounding
        q = r.standard_normal(DIM)
        assert abs(orc.page_score_f64(q, mu, V, C) - exact_lse(q, keys)) < 1e-11


@pytest.mark.parametrize("rank", [1, 2, 4, 8, 12])
def test_eckart_young_tail_energy(orc, rank):
    """The page-local basis is residual-optimal: ||D - C V^T||_F^2 equals the
    sum of the discarded squared singular values of D (B section 3, theory;
    Eckart-Young), checked against LAPACK's SVD."""
    r = rng(rank)
    keys = planted_page(r, 10, noise=0.1)
    mu, V, C, lam = orc.page_summary_f64(keys, rank=rank)
    D = keys - keys.mean(0)
    sv = np.linalg.svd(D, compute_uv=False)
    assert np.allclose(mu, keys.mean(0), atol=1e-14)
    assert np.allclose(lam, np.concatenate([sv ** 2, np.zeros(PAGE - len(sv))]), atol=1e-10)
    resid = np.sum((D - C @ V.T) ** 2)
    assert abs(resid - np.sum(sv[rank:] ** 2)) < 1e-9 * np.sum(sv ** 2)
    assert np.allclose(V.T @ V, np.eye(rank), atol=1e-12)     # orthonormal basis
    assert np.allclose(C, D @ V, atol=1e-12)                 # coefficients = projections
    for k in range(rank):                                     # sign convention
        dm = int(np.argmax(np.abs(V[:, k])))
        assert V[dm, k] > 0


def test_constant_page_has_zero_basis_and_closed_form_score(orc):
    r = rng(3)
    row = r.standard_normal(DIM)
    keys = np.tile(row, (PAGE, 1))
    mu, V, C, lam = orc.page_summary_f64(keys, rank=8)
    assert np.all(V == 0) and np.all(C == 0) and np.allclose(lam, 0)
    q = r.standard_normal(DIM)
    # all 16 logits equal: LSE = logit + ln 16
    assert abs(orc.page_score_f64(q, mu, V, C) - (q @ row / math.sqrt(DIM) + math.log(16))) < 1e-12


# ------------------------------------------------------------ quantised record

def bf16_round(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16), t.double().numpy()


def test_record_quantiser_bounds_and_pack_roundtrip(orc):
    r = rng(11)
    for _ in range(20):
        bits, keys = bf16_round(planted_page(r, 8, noise=0.05, scale=r.uniform(0.1, 4)))
        rec, lam, mu, V, C = orc.build_record(bits)
        mu_h, V_h, C_h = orc.unpack_record(rec)
        scales = [orc.f16_bits_to_f64(int(rec[768 + 2 * i]) | (int(rec[769 + 2 * i]) << 8))
                  for i in range(3)]
        for x, xh, s, qmax in ((mu, mu_h, scales[0], 127), (V, V_h, scales[1], 7),
                               (C, C_h, scales[2], 127)):
            amax = np.abs(x).max()
            # scale is the fp16 rounding of absmax/qmax (numpy's float16 as the library check)
            assert s == float(np.float16(amax / qmax))
            codes = xh / s
            assert np.array_equal(codes, np.round(codes))       # integer codes
            assert np.abs(codes).max() == qmax                    # absmax maps to +-qmax
            assert np.all(np.abs(x - xh) <= s / 2 * (1 + 1e-12))  # half-step error bound
        assert np.all(rec[776:] == 0) and rec[774] == 0 and rec[775] == 0


def test_record_format_matches_documented_layout(orc):
    """Byte-level check of the documented record layout with a record built
    here independently (numpy bit packing), decoded by the oracle."""
    r = rng(5)
    vc = r.integers(-7, 8, size=(DIM, 8))
    mc = r.integers(-127, 128, size=DIM)
    cc = r.integers(-127, 128, size=(PAGE, 8))
    s = np.array([0.03125, 0.25, 0.0078125], dtype=np.float16)
    rec = np.zeros(784, dtype=np.uint8)
    nib = (vc & 0xF).astype(np.uint8)                  # [d][k] two's complement nibbles
    for k in range(8):
        col = nib[:, k].reshape(16, 2, 4)              # [word][half][byte]
        rec[k * 64:(k + 1) * 64] = (col[:, 0, :] | (col[:, 1, :] << 4)).reshape(-1)
    rec[512:640] = mc.astype(np.int8).view(np.uint8)
    rec[640:768] = cc.reshape(-1).astype(np.int8).view(np.uint8)
    rec[768:774] = s.view(np.uint8)
    mu, V, C = orc.unpack_record(rec)
    assert np.array_equal(mu, mc * float(s[0]))
    assert np.array_equal(V, vc * float(s[1]))
    assert np.array_equal(C, cc * float(s[2]))


def test_build_blocks_rebuilds_only_the_listed_blocks(orc):
    """Building the records of a block list (pages that just filled) gives each
    listed block's records as the whole-cache build does and leaves the rest."""
    r = rng(35)
    B, Hkv, N = 2, 2, 4
    kb, kd, vb, vd, pt = small_cache(r, B, Hkv, N, extra=2)
    lens = np.full(B, N * PAGE, dtype=np.int32)
    full = orc.build_summaries(kb, pt, lens)
    stale = np.full_like(full, 0xAB)
    blocks = np.array([pt[1, 2], -1, pt[0, 0], kb.shape[0], pt[1, 2]], dtype=np.int32)
    got = orc.build_blocks(kb, blocks, stale)
    for blk in range(kb.shape[0]):
        want = full[blk] if blk in (pt[1, 2], pt[0, 0]) else stale[blk]
        assert np.array_equal(got[blk], want), blk


# ------------------------------------------------------------ variant formats

def decode_variant_numpy(rec, r, vb):
    """Independent decoder of the documented variant layout (V [d][k] then mu
    then C [16][r], little-endian bit fields, then fp16 scales)."""
    mb = 16 if vb == 16 else 8
    nv, nm, nc = DIM * r * vb // 8, DIM * mb // 8, PAGE * r * mb // 8
    bits = np.unpackbits(rec, bitorder="little").astype(np.int64)

    def field(off, n, b):
        return (bits[off * 8: off * 8 + n * b].reshape(n, b) << np.arange(b)).sum(1)

    sc = rec[nv + nm + nc: nv + nm + nc + 6].view(np.float16).astype(np.float64)

    def values(v, b, scale):
        if b == 16:
            return v.astype(np.uint16).view(np.float16).astype(np.float64), None
        c = np.where(v >= 2 ** (b - 1), v - 2 ** b, v)
        return scale * c, c

    V, vc = values(field(0, DIM * r, vb), vb, sc[1])
    mu, mc = values(field(nv, DIM, mb), mb, sc[0])
    C, cc = values(field(nv + nm, PAGE * r, mb), mb, sc[2])
    assert np.all(rec[nv + nm + nc + 6:] == 0)  # fourth scale slot and padding
    return mu, V.reshape(DIM, r), C.reshape(PAGE, r), (mc, vc, cc), sc


@pytest.mark.parametrize("r", [4, 8, 16])
@pytest.mark.parametrize("vb", [2, 4, 16])
def test_variant_records_decode_independently_and_quantise_correctly(orc, r, vb):
    rr = rng(300 + 10 * r + vb)
    keys = planted_page(rr, 8, noise=0.05)
    kb, kd = bf16_round(keys)
    rec = orc.build_record_variant(kb, r, vb)
    mu, V, C, codes, sc = decode_variant_numpy(rec, r, vb)
    mu_o, V_o, C_o = orc.unpack_record_variant(rec, r, vb)
    assert np.array_equal(mu, mu_o) and np.array_equal(V, V_o) and np.array_equal(C, C_o)
    mu_u, V_u, C_u, _ = orc.page_summary_f64(kd, rank=r)
    if vb == 16:  # stored values are numpy's fp16 rounding of the unquantised summary
        for got, want in ((mu, mu_u), (V, V_u), (C, C_u)):
            assert np.array_equal(got, want.astype(np.float16).astype(np.float64))
        assert np.all(sc[:3] == 1.0)
    else:
        qv = 2 ** (vb - 1) - 1
        for (c, q, x, s) in ((codes[1], qv, V_u, sc[1]), (codes[0], 127, mu_u, sc[0]),
                             (codes[2], 127, C_u, sc[2])):
            assert s == np.float16(np.abs(x).max() / q)
            assert np.abs(c).max() <= q
            inside = np.abs(x.ravel()) <= s * q
            assert np.all(np.abs(x.ravel()[inside] - s * c[inside]) <= s / 2 * (1 + 1e-9))
        if vb == 2:
            assert set(np.unique(codes[1])) <= {-1, 0, 1}


def test_variant_int4_rank8_holds_the_shipped_values(orc):
    """Same quantiser, another byte layout: the int4 rank-8 variant decodes to
    exactly the values of the shipped 784-byte record."""
    rr = rng(321)
    for _ in range(3):
        kb, _ = bf16_round(planted_page(rr, 8, noise=0.05))
        a = orc.unpack_record(orc.build_record(kb)[0])
        b = orc.unpack_record_variant(orc.build_record_variant(kb, 8, 4), 8, 4)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


def test_variant_fp16_rank16_scores_track_the_exact_page_lse(orc):
    """Rank 16 spans every centred page (rank <= 15), so an fp16-stored rank-16
    summary scores within fp16 rounding of the exact LSE on the real keys."""
    rr = rng(331)
    for _ in range(4):
        kb, kd = bf16_round(rr.standard_normal((PAGE, DIM)))
        mu, V, C = orc.unpack_record_variant(orc.build_record_variant(kb, 16, 16), 16, 16)
        for _ in range(3):
            q = rr.standard_normal(DIM)
            assert abs(orc.page_score_f64(q, mu, V, C) - exact_lse(q, kd)) < 2e-2


def test_summary_payload_is_about_ten_percent(orc):
    """(A "How LOCKS works"; B mechanism 1): the summary is about 10% of the
    page's KV bytes. Payload 776 B vs 16 tokens x 128 x bf16 x (K+V)."""
    payload = 128 * 8 // 2 + 128 + 16 * 8 + 6
    assert payload == 774
    assert 0.09 < (payload + 2) / (PAGE * DIM * 2 * 2) < 0.105
    assert 784 / (PAGE * DIM * 2 * 2) < 0.1


# ------------------------------------------------------------ group keys + top-k

def test_exact_scores_match_scipy_logsumexp_on_real_keys(orc):
    """The exact-mass selector's page scores: scipy's logsumexp over each full
    page's real keys; absent pages and pages past the full ones are -inf."""
    r = rng(29)
    B, Hq, Hkv, N = 2, 4, 2, 6
    kb, kd, vb, vd, pt = small_cache(r, B, Hkv, N)
    q = r.standard_normal((B, Hq, DIM)).astype(np.float32)
    lens = np.array([N * PAGE, 3 * PAGE + 9], dtype=np.int32)
    pt[0, 2] = -1
    got = orc.exact_scores(q, kb, pt, lens)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            for j in range(N):
                if j >= lens[b] // PAGE or pt[b, j] < 0:
                    assert got[b, h, j] == -np.inf
                else:
                    ref = exact_lse(q[b, h].astype(np.float64), kd[pt[b, j], h // G])
                    assert abs(got[b, h, j] - ref) < 1e-12


def test_group_keys_are_log_mean_shares(orc):
    r = rng(21)
    B, Hkv, G, N = 2, 3, 4, 37
    s = r.standard_normal((B, Hkv * G, N)) * 3
    keys = orc.group_keys(s, Hkv)
    # shares of each head sum to one, so the group-mean share sums to one too
    assert np.allclose(np.exp(keys).sum(-1), 1.0, atol=1e-12)
    # per-head constant offsets cancel (normalisation by each head's total)
    s2 = s + r.standard_normal((B, Hkv * G, 1)) * 5
    assert np.allclose(orc.group_keys(s2, Hkv), keys, atol=1e-12)
    # permuting heads inside a group changes nothing
    perm = np.concatenate([kv * G + r.permutation(G) for kv in range(Hkv)])
    assert np.allclose(orc.group_keys(s[:, perm], Hkv), keys, atol=1e-12)
    # a group of identical heads reduces to a single head (G = 1 case)
    same = np.repeat(s[:, ::G][:, :, None, :], G, axis=2).reshape(B, Hkv * G, N)
    assert np.allclose(orc.group_keys(same, Hkv), orc.group_keys(s[:, ::G], Hkv), atol=1e-12)
    # G = 1: the key is the score minus a per-row constant -> same order as the score
    k1 = orc.group_keys(s[:, :Hkv], Hkv)
    d = k1 - s[:, :Hkv]
    assert np.allclose(d, d[..., :1], atol=1e-12)


def test_group_keys_average_shares_not_scores(orc):
    """Two heads, two pages: head 0 puts almost all mass on page 0, head 1
    splits evenly. Mean share: page 0 = (1 + .5)/2 = .75."""
    s = np.log(np.array([[[1 - 1e-9, 1e-9], [0.5, 0.5]]]))
    keys = orc.group_keys(s, 1)
    assert np.allclose(np.exp(keys[0, 0]), [0.75 - 5e-10, 0.25 + 5e-10], atol=1e-12)


def test_select_matches_stable_full_sort(orc):
    r = rng(31)
    for trial in range(30):
        N = int(r.integers(1, 60))
        k = int(r.integers(1, 70))
        keys = np.round(r.standard_normal((2, 3, N)), 1)     # many exact ties
        keys[r.random(keys.shape) < 0.1] = -np.inf            # absent pages
        sel = orc.select(keys, k)
        for b in range(2):
            for h in range(3):
                kk = keys[b, h]
                order = np.lexsort((np.arange(N), -kk))        # key desc, then id asc
                order = [j for j in order if np.isfinite(kk[j])][:k]
                want = sorted(order) + [-1] * (k - len(order))
                assert list(sel[b, h]) == want


# ------------------------------------------------------------ attention

def sdpa_ref(q, keys, vals):
    """torch SDPA in float64 on the CPU (library routine)."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None, :], torch.from_numpy(keys)[None, None],
        torch.from_numpy(vals)[None, None])
    return out[0, 0, 0].numpy()


def small_cache(r, B, Hkv, N, extra=3):
    nb = B * N + extra
    kb, kd = bf16_round(r.standard_normal((nb, Hkv, PAGE, DIM)))
    vb, vd = bf16_round(r.standard_normal((nb, Hkv, PAGE, DIM)))
    pt = r.permutation(nb)[: B * N].reshape(B, N).astype(np.int32)
    return kb, kd, vb, vd, pt


def test_dense_attention_matches_sdpa(orc):
    r = rng(41)
    B, Hq, Hkv, N = 2, 4, 2, 5
    kb, kd, vb, vd, pt = small_cache(r, B, Hkv, N)
    q = r.standard_normal((B, Hq, DIM)).astype(np.float32)
    lens = np.array([N * PAGE, 3 * PAGE + 7], dtype=np.int32)  # second: 7-token tail
    out = orc.attention(q, kb, vb, pt, lens)
    G = Hq // Hkv
    for b in range(B):
        # every token of the sequence, i.e. its full pages and then its tail
        flat = lambda x: x[pt[b], h // G].reshape(-1, DIM)[: lens[b]]
        for h in range(Hq):
            ref = sdpa_ref(q[b, h].astype(np.float64), flat(kd), flat(vd))
            assert np.allclose(out[b, h], ref, atol=1e-12)


def test_sparse_attention_matches_sdpa_on_gathered_tokens(orc):
    r = rng(43)
    B, Hq, Hkv, N, k = 1, 2, 1, 9, 4
    kb, kd, vb, vd, pt = small_cache(r, B, Hkv, N)
    q = r.standard_normal((B, Hq, DIM)).astype(np.float32)
    lens = np.array([N * PAGE], dtype=np.int32)
    sel = np.array([[[1, 4, 7, -1]]], dtype=np.int32)
    out = orc.attention(q, kb, vb, pt, lens, sel)
    blks = pt[0, [1, 4, 7]]
    for h in range(Hq):
        ref = sdpa_ref(q[0, h].astype(np.float64), kd[blks, 0].reshape(-1, DIM),
                       vd[blks, 0].reshape(-1, DIM))
        assert np.allclose(out[0, h], ref, atol=1e-12)
    empty = orc.attention(q, kb, vb, pt, lens, np.full((1, 1, 4), -1, dtype=np.int32))
    assert np.all(empty == 0)


def test_sparse_attention_adds_the_tail_and_never_reads_past_it(orc):
    """The partly filled page has no summary (summaries are built when a page
    fills) and is always attended: the selected pages' tokens plus the tail's,
    nothing after seq_len (planted NaNs there must not reach the output)."""
    r = rng(45)
    B, Hq, Hkv, N = 2, 4, 2, 9
    kb, kd, vb, vd, pt = small_cache(r, B, Hkv, N)
    q = r.standard_normal((B, Hq, DIM)).astype(np.float32)
    lens = np.array([5 * PAGE + 11, 1 * PAGE + 1], dtype=np.int32)
    for b in range(B):  # NaN keys and values after each sequence's last token
        n, t = lens[b] // PAGE, lens[b] % PAGE
        kb[pt[b, n], :, t:] = 0x7FC0
        vb[pt[b, n], :, t:] = 0x7FC0
        kb[pt[b, n + 1:], :] = 0x7FC0
        vb[pt[b, n + 1:], :] = 0x7FC0
    sel = np.array([[[0, 3, 4]] * Hkv, [[0, -1, -1]] * Hkv], dtype=np.int32)
    out = orc.attention(q, kb, vb, pt, lens, sel)
    G = Hq // Hkv
    for b in range(B):
        n, t = lens[b] // PAGE, lens[b] % PAGE
        for h in range(Hq):
            pages = [j for j in sel[b, h // G] if 0 <= j < n]
            keys = np.concatenate([kd[pt[b, pages], h // G].reshape(-1, DIM),
                                   kd[pt[b, n], h // G, :t]])
            vals = np.concatenate([vd[pt[b, pages], h // G].reshape(-1, DIM),
                                   vd[pt[b, n], h // G, :t]])
            ref = sdpa_ref(q[b, h].astype(np.float64), keys, vals)
            assert np.all(np.isfinite(out[b, h]))
            assert np.allclose(out[b, h], ref, atol=1e-12)


def test_tail_only_sequence_attends_its_tokens(orc):
    """A sequence shorter than one page: no page can be selected; the output
    is the softmax over its few tokens (one token: exactly that value row)."""
    r = rng(47)
    kb, kd, vb, vd, pt = small_cache(r, 1, 1, 3)
    q = r.standard_normal((1, 2, DIM)).astype(np.float32)
    one = orc.attention(q, kb, vb, pt, np.array([1], dtype=np.int32),
                        np.full((1, 1, 2), -1, dtype=np.int32))
    assert np.array_equal(one[0, 0], vd[pt[0, 0], 0, 0]) and np.array_equal(one[0, 1], vd[pt[0, 0], 0, 0])
    five = orc.attention(q, kb, vb, pt, np.array([5], dtype=np.int32))
    for h in range(2):
        ref = sdpa_ref(q[0, h].astype(np.float64), kd[pt[0, 0], 0, :5], vd[pt[0, 0], 0, :5])
        assert np.allclose(five[0, h], ref, atol=1e-12)


# ------------------------------------------------------------ whole step

def oracle_inputs(r, B, Hq, Hkv, N, structured=True):
    nb = B * N + 2
    keys = np.stack([np.stack([planted_page(r, 8, noise=0.05) if structured
                               else r.standard_normal((PAGE, DIM))
                               for _ in range(Hkv)]) for _ in range(nb)])
    kb, kd = bf16_round(keys)
    vb, vd = bf16_round(r.standard_normal((nb, Hkv, PAGE, DIM)))
    pt = r.permutation(nb)[: B * N].reshape(B, N).astype(np.int32)
    q = r.standard_normal((B, Hq, DIM)).astype(np.float32)
    return kb, kd, vb, vd, pt, q


def test_full_budget_reproduces_dense_attention(orc):
    """budget = whole sequence -> every page kept -> exactly dense attention
    (A "Code": the sparse output against the full-KV output)."""
    r = rng(51)
    B, Hq, Hkv, N = 2, 8, 2, 6
    kb, kd, vb, vd, pt, q = oracle_inputs(r, B, Hq, Hkv, N)
    lens = np.full(B, N * PAGE, dtype=np.int32)
    summ = orc.build_summaries(kb, pt, lens)
    out, sel, sc, ky = orc.decode_step(q, summ, kb, vb, pt, lens, N * PAGE)
    assert np.array_equal(sel, np.tile(np.arange(N, dtype=np.int32), (B, Hkv, 1)))
    dense = orc.attention(q, kb, vb, pt, lens)
    assert np.allclose(out, dense, atol=1e-13)


def test_scores_from_records_match_unpacked_formula_and_selection_order(orc):
    r = rng(61)
    B, Hq, Hkv, N = 1, 4, 2, 20
    kb, kd, vb, vd, pt, q = oracle_inputs(r, B, Hq, Hkv, N)
    lens = np.array([N * PAGE - 5], dtype=np.int32)      # last page partial -> ignored
    summ = orc.build_summaries(kb, pt, lens)
    out, sel, sc, ky = orc.decode_step(q, summ, kb, vb, pt, lens, 5 * PAGE)
    n = N - 1
    assert np.all(np.isneginf(sc[..., n:])) and np.all(np.isfinite(sc[..., :n]))
    G = Hq // Hkv
    for h in range(Hq):
        for j in range(n):
            mu, V, C = orc.unpack_record(summ[pt[0, j], h // G])
            assert sc[0, h, j] == orc.page_score_f64(q[0, h].astype(np.float64), mu, V, C)
    for kvh in range(Hkv):
        order = np.lexsort((np.arange(n), -ky[0, kvh, :n]))[:5]
        assert list(sel[0, kvh]) == sorted(order)


def np_decode_record(rec):
    """Decoder of the documented record layout written here with numpy bit
    operations; it shares nothing with the oracle's unpacking."""
    rec = np.asarray(rec, dtype=np.uint8)
    s = rec[768:774].copy().view(np.float16).astype(np.float64)  # s_mu, s_V, s_C
    w = rec[:512].reshape(8, 16, 4).astype(np.int64)             # [k][word][byte]
    nib = np.stack([w & 0xF, w >> 4], axis=2)                    # [k][word][half][byte]
    nib = np.where(nib > 7, nib - 16, nib)                       # 4-bit two's complement
    V = nib.reshape(8, DIM).T * s[1]                             # d = 8 word + 4 half + byte
    mu = rec[512:640].view(np.int8).astype(np.float64) * s[0]
    C = rec[640:768].view(np.int8).astype(np.float64).reshape(PAGE, 8) * s[2]
    return mu, V, C


def test_quantised_scores_and_selection_match_reconstructed_keys(orc):
    """End to end on quantised records (A "How LOCKS works": the score is the
    log-sum-exp of the page's reconstructed logits; B mechanism 3: the group
    key averages each head's mass share): every page score of the oracle's
    decode step equals scipy's log-sum-exp over the 16 keys the record
    reconstructs, mu + V c_i, with the record decoded here independently; and
    its selection is the stable top-k of group keys formed here from those
    scores. This ties the quantised composition (build -> record -> score ->
    key -> top-k) to the definition rather than to the oracle's factored form
    q.mu + (V^T q).c_i."""
    r = rng(71)
    B, Hq, Hkv, N, k = 2, 8, 2, 24, 6
    kb, kd, vb, vd, pt, q = oracle_inputs(r, B, Hq, Hkv, N)
    lens = np.array([N * PAGE, N * PAGE - 21], dtype=np.int32)  # the second ends in a tail
    summ = orc.build_summaries(kb, pt, lens)
    out, sel, sc, ky = orc.decode_step(q, summ, kb, vb, pt, lens, k * PAGE)
    G = Hq // Hkv
    for b in range(B):
        n = int(lens[b]) // PAGE
        ref = np.empty((Hq, n))
        for h in range(Hq):
            qh = q[b, h].astype(np.float64)
            for j in range(n):
                mu, V, C = np_decode_record(summ[pt[b, j], h // G])
                ref[h, j] = exact_lse(qh, mu + C @ V.T)
        assert np.allclose(sc[b, :, :n], ref, rtol=0, atol=1e-9)
        for kvh in range(Hkv):
            s = ref[kvh * G:(kvh + 1) * G]
            share = np.exp(s - logsumexp(s, axis=1, keepdims=True))  # per head, sums to 1
            key = np.log(share.mean(axis=0))
            top = np.lexsort((np.arange(n), -key))[:k]
            assert list(sel[b, kvh]) == sorted(top.tolist())


@pytest.mark.parametrize("rank", [2, 4, 8])
def test_theorem1_mass_retention_bound(orc, rank):
    """(A "How LOCKS works", Theorem 1; B section 3 retention guarantees.)
    Reading: eta = max over tokens of |q.(k - k_hat)|/sqrt(d) for the
    unquantised rank-r reconstruction k_hat. Each page score is then within eta
    of the exact page LSE, so the exact mass of the pages chosen by the
    estimated score is at least e^(-4 eta) (indeed e^(-2 eta)) times the exact
    mass of the best k pages."""
    r = rng(70 + rank)
    N, k = 64, 8
    pages = [planted_page(r, 10, noise=0.05) for _ in range(N)]
    q = r.standard_normal(DIM)
    est, exact, eta = [], [], 0.0
    for keys in pages:
        mu, V, C, lam = orc.page_summary_f64(keys, rank=rank)
        est.append(orc.page_score_f64(q, mu, V, C))
        exact.append(exact_lse(q, keys))
        khat = mu[None, :] + C @ V.T
        eta = max(eta, float(np.max(np.abs((keys - khat) @ q)) / math.sqrt(DIM)))
    est, exact = np.array(est), np.array(exact)
    chosen = orc.select(est[None, None, :], k)[0, 0]
    best = np.argsort(-exact)[:k]
    mass = lambda idx: np.exp(exact[idx]).sum()
    assert mass(chosen) >= math.exp(-2 * eta) * mass(best) * (1 - 1e-12)
    assert mass(chosen) >= math.exp(-4 * eta) * mass(best)


# ------------------------------------------ variant drivers over a paged cache

def bf16_f64(bits):
    """bf16 bit patterns -> float64 via torch (exact)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.double().numpy()


def variant_cache(r):
    """A tiny paged cache: 2 sequences, 2 KV heads (G = 2), a permuted page
    table with one absent page (block id -1) and one block id past the cache,
    a ragged tail in the second sequence, and unreferenced blocks."""
    B, Hq, Hkv, N = 2, 4, 2, 7
    nb = B * N + 3
    keys = np.stack([np.stack([planted_page(r, 8, noise=0.05) for _ in range(Hkv)])
                     for _ in range(nb)])
    kb, _ = bf16_round(keys)
    pt = r.permutation(nb)[: B * N].reshape(B, N).astype(np.int32)
    pt[0, 2] = -1          # absent page inside n_b
    pt[1, 4] = nb + 5      # block id outside [0, num_blocks): absent as well
    lens = np.array([N * PAGE, 5 * PAGE + 9], dtype=np.int32)  # 7 and 5 full pages
    q = r.standard_normal((B, Hq, DIM)).astype(np.float32)
    return kb, pt, lens, q, Hkv


@pytest.mark.parametrize("r", [4, 8, 16])
@pytest.mark.parametrize("vb", [2, 4, 16])
def test_variant_build_driver_places_records_through_the_page_table(orc, r, vb):
    """(A "Caveats": the int4 / int2 / unquantised summaries compared; B
    mechanism 1: one record per page, built from that page's keys.) Every full
    present page (b, j) gets, at [page_table[b][j], kvh], the record of its own
    key tile, decoded here by the independent numpy decoder; absent pages, the
    tail page and unreferenced blocks leave the output untouched."""
    rr = rng(400 + 10 * r + vb)
    kb, pt, lens, _, Hkv = variant_cache(rr)
    nb = kb.shape[0]
    nbytes = orc.variant_record_bytes(r, vb)
    fill = np.full((nb, Hkv, nbytes), 0xA5, dtype=np.uint8)
    got = orc.build_summaries_variant(kb, pt, lens, r, vb, summaries=fill.copy())
    written = set()
    for b in range(pt.shape[0]):
        for j in range(int(lens[b]) // PAGE):
            blk = int(pt[b, j])
            if 0 <= blk < nb:
                written.add(blk)
    for blk in range(nb):
        for h in range(Hkv):
            if blk not in written:
                assert np.all(got[blk, h] == 0xA5), (blk, h)
                continue
            mu, V, C, _, _ = decode_variant_numpy(got[blk, h], r, vb)
            ref = decode_variant_numpy(orc.build_record_variant(kb[blk, h], r, vb), r, vb)
            assert np.array_equal(mu, ref[0]) and np.array_equal(V, ref[1]) and np.array_equal(C, ref[2])
            if vb == 16:
                # fp16 storage: the record holds this tile's rank-r summary, so
                # its residual is the tile's SVD tail energy (Eckart-Young),
                # up to fp16 rounding
                keys = bf16_f64(kb[blk, h])
                dev = keys - keys.mean(0)
                sv = np.linalg.svd(dev, compute_uv=False)
                tail = math.sqrt(float((sv[r:] ** 2).sum()))
                res = np.linalg.norm(mu[None, :] + C @ V.T - keys)
                assert abs(res - tail) <= 1e-3 * np.linalg.norm(keys), (blk, h, res, tail)


@pytest.mark.parametrize("r", [4, 8, 16])
@pytest.mark.parametrize("vb", [2, 4, 16])
def test_variant_score_driver_is_the_lse_of_reconstructed_keys(orc, r, vb):
    """(A "How LOCKS works": a page's score is the log-sum-exp of its
    reconstructed in-page logits; B mechanism 2.) Every score the variant
    driver writes equals scipy's log-sum-exp over the 16 keys mu + V c_i that
    the record at [page_table[b][j], h / G] reconstructs (independent decoder);
    absent pages, the tail page and pages past n_b score -inf."""
    rr = rng(500 + 10 * r + vb)
    kb, pt, lens, q, Hkv = variant_cache(rr)
    summ = orc.build_summaries_variant(kb, pt, lens, r, vb)
    sc = orc.scores_variant(q, summ, pt, lens, Hkv, r, vb)
    B, Hq, N = sc.shape
    G = Hq // Hkv
    nb = kb.shape[0]
    for b in range(B):
        n = int(lens[b]) // PAGE
        for h in range(Hq):
            for j in range(N):
                blk = int(pt[b, j])
                if j >= n or not (0 <= blk < nb):
                    assert sc[b, h, j] == -np.inf, (b, h, j)
                    continue
                mu, V, C, _, _ = decode_variant_numpy(summ[blk, h // G], r, vb)
                want = exact_lse(q[b, h].astype(np.float64), mu[None, :] + C @ V.T)
                assert abs(sc[b, h, j] - want) <= 1e-9, (b, h, j, sc[b, h, j], want)


# ------------------------------------------ step with a page that just filled

def test_fill_step_attends_the_new_page_in_full_and_never_scores_it(orc):
    """(A "How LOCKS works": a page's summary is built once, when it fills; B
    mechanism 4: off the decode critical path.) Reading: in the step where a
    sequence's last page fills, that page has no summary yet and is attended
    like a tail. Pins: its score is -inf and it is never selected; an unmarked
    sequence gets exactly the plain step; at a full budget the output is
    torch's SDPA over every token of the sequence; and at a small budget it is
    SDPA over the kept pages plus all 16 tokens of the new page."""
    r = rng(81)
    B, Hq, Hkv, N, k = 3, 4, 2, 12, 3
    kb, kd, vb, vd, pt, q = oracle_inputs(r, B, Hq, Hkv, N)
    lens = np.array([N * PAGE, 9 * PAGE, 7 * PAGE + 5], dtype=np.int32)
    fill = np.array([1, 0, 1], dtype=np.int32)  # the third: length not a multiple of 16
    summ = orc.build_summaries(kb, pt, lens)
    out, sel, sc, ky = orc.decode_step_fill(q, summ, kb, vb, pt, lens, k * PAGE, fill)
    ref = orc.decode_step(q, summ, kb, vb, pt, lens, k * PAGE)
    for b in (1, 2):  # unmarked, and marked but mid-page: the plain step
        assert np.array_equal(sel[b], ref[1][b]) and np.array_equal(out[b], ref[0][b])
    assert np.all(np.isneginf(sc[0, :, N - 1])) and np.all(np.isfinite(sc[0, :, : N - 1]))
    assert not np.any(sel[0] == N - 1)
    G = Hq // Hkv
    for h in range(Hq):  # kept pages plus the whole new page, through SDPA
        pages = sorted(sel[0, h // G].tolist()) + [N - 1]
        want = sdpa_ref(q[0, h].astype(np.float64), kd[pt[0, pages], h // G].reshape(-1, DIM),
                        vd[pt[0, pages], h // G].reshape(-1, DIM))
        assert np.allclose(out[0, h], want, atol=1e-12)
    full, fsel, _, _ = orc.decode_step_fill(q, summ, kb, vb, pt, lens, N * PAGE, fill)
    assert list(fsel[0, 0, : N - 1]) == list(range(N - 1)) and np.all(fsel[0, :, N - 1:] == -1)
    for h in range(Hq):
        keys = kd[pt[0], h // G].reshape(-1, DIM)
        vals = vd[pt[0], h // G].reshape(-1, DIM)
        assert np.allclose(full[0, h], sdpa_ref(q[0, h].astype(np.float64), keys, vals), atol=1e-12)


# ------------------ shared-basis comparison (Proposition 1: blind directions)

def test_shared_basis_is_the_top_eigenspace_of_pooled_page_deviations(orc):
    """(B section 3: a shared basis built from the sequence.) The oracle's
    shared basis equals numpy's eigh of the pooled within-page deviation
    scatter, column by column (sign rule: largest-|.| entry positive)."""
    r = rng(91)
    B, Hkv, N = 2, 2, 12
    kb, kd, vb, vd, pt, q = oracle_inputs(r, B, 2 * Hkv, Hkv, N, structured=False)
    lens = np.array([N * PAGE, 9 * PAGE + 3], dtype=np.int32)
    pt[1, 4] = -1  # an absent page is left out
    W = orc.shared_basis(kb, pt, lens, rank=8)
    for b in range(B):
        for h in range(Hkv):
            n = int(lens[b]) // PAGE
            tiles = [kd[pt[b, j], h] for j in range(n) if pt[b, j] >= 0]
            S = sum((t - t.mean(0)).T @ (t - t.mean(0)) for t in tiles)
            lam, U = np.linalg.eigh(S)
            top = U[:, ::-1][:, :8]
            top = top * np.sign(top[np.abs(top).argmax(0), np.arange(8)])
            assert np.allclose(W[b, h], top, atol=1e-8), (b, h)


def test_shared_record_holds_mean_and_projected_deviations(orc):
    """A shared-basis record (variant layout, fp16 values) decodes, by the
    independent numpy decoder, to fp16(W), fp16(mean of the keys) and
    fp16((K - mu) W)."""
    r = rng(92)
    kb, kd = bf16_round(planted_page(r, 8, noise=0.05))
    W, _ = np.linalg.qr(r.standard_normal((DIM, 8)))
    rec = orc.build_record_shared(kb, W)
    mu, V, C, _, sc = decode_variant_numpy(rec, 8, 16)
    f16 = lambda x: x.astype(np.float16).astype(np.float64)
    assert np.array_equal(V, f16(W)) and np.array_equal(mu, f16(kd.mean(0)))
    assert np.array_equal(C, f16((kd - kd.mean(0)) @ W)) and np.all(sc[:3] == 1.0)


def test_shared_basis_is_blind_to_deviations_in_its_null_space(orc):
    """Proposition 1 (A "Why shared-basis sparse attention is structurally
    broken"; B section 3): a fixed shared projection cannot see page content
    in its null space. A page whose deviations lie there scores exactly
    q.mu/sqrt(d) + ln 16 from its shared record (the coefficients vanish),
    whatever those deviations are, while its exact LSE and its page-local
    LOCKS score (unquantised rank 8) see them; deviations inside span(W)
    are scored exactly by the shared record too."""
    r = rng(93)
    W, _ = np.linalg.qr(r.standard_normal((DIM, 8)))
    q = r.standard_normal(DIM)
    u = q - W @ (W.T @ q)
    u /= np.linalg.norm(u)
    mu = np.round(r.standard_normal(DIM) * 64) / 64  # exact in bf16 and fp16
    alpha = np.full(PAGE, -1.0)
    alpha[3] = 15.0
    keys = mu[None, :] + alpha[:, None] * u[None, :]
    kb, kd = bf16_round(keys)
    m, V, C = orc.unpack_record_variant(orc.build_record_shared(kb, W), 8, 16)
    blind = orc.page_score_f64(q, m, V, C)
    closed = float(q @ m) / math.sqrt(DIM) + math.log(PAGE)
    assert abs(blind - closed) < 1e-2, (blind, closed)  # C is fp16 of a ~0 projection
    exact = exact_lse(q, kd)
    mu_l, V_l, C_l, _ = orc.page_summary_f64(kd, rank=8)
    local = orc.page_score_f64(q, mu_l, V_l, C_l)
    assert abs(local - exact) < 1e-9 and exact - blind > 1.0
    # deviations inside span(W): the shared record reconstructs them
    keys_in = mu[None, :] + (r.standard_normal((PAGE, 8)) / np.arange(1, 9)) @ W.T
    kb2, kd2 = bf16_round(keys_in)
    m2, V2, C2 = orc.unpack_record_variant(orc.build_record_shared(kb2, W), 8, 16)
    assert abs(orc.page_score_f64(q, m2, V2, C2) - exact_lse(q, kd2)) < 2e-2


def test_shared_driver_places_records_with_each_sequence_basis(orc):
    """Every full present page (b, j) gets, at [page_table[b][j], kvh], the
    shared record of its own tile under basis[b][kvh]; other blocks untouched."""
    rr = rng(94)
    kb, pt, lens, q, Hkv = variant_cache(rr)
    B = pt.shape[0]
    basis = np.stack([np.stack([np.linalg.qr(rr.standard_normal((DIM, 8)))[0] for _ in range(Hkv)])
                      for _ in range(B)])
    nb = kb.shape[0]
    fill = np.full((nb, Hkv, orc.variant_record_bytes(8, 16)), 0x5A, dtype=np.uint8)
    got = orc.build_summaries_shared(kb, pt, lens, basis, summaries=fill.copy())
    seen = set()
    for b in range(B):
        for j in range(int(lens[b]) // PAGE):
            blk = int(pt[b, j])
            if 0 <= blk < nb:
                seen.add(blk)
                for h in range(Hkv):
                    assert np.array_equal(got[blk, h], orc.build_record_shared(kb[blk, h], basis[b, h]))
    for blk in set(range(nb)) - seen:
        assert np.all(got[blk] == 0x5A)
