"""Seeded generators: shapes, structure and statistics of the five workloads
(the structured-key recipe: centroid N(0, I), random orthonormal rank-8 page
basis, coefficients N(0, (1/k)^2), noise N(0, 0.05^2))."""
import json
import math
import os

import numpy as np
import torch

import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def test_orthonormal_rows():
    g = torch.Generator().manual_seed(0)
    b = workloads._orthonormal_rows(g, 64, "cpu")
    eye = torch.bmm(b, b.transpose(1, 2))
    assert torch.allclose(eye, torch.eye(8).expand(64, 8, 8), atol=1e-5)


def test_structured_key_statistics():
    g = torch.Generator().manual_seed(1)
    keys = workloads.structured_keys(g, 4000, "cpu").double()
    mu = keys.mean(1)                                    # page centroids
    assert abs(mu.mean().item()) < 0.02 and abs(mu.var().item() - 1.0) < 0.02
    dev = keys - mu[:, None, :]
    sv2 = torch.linalg.svdvals(dev) ** 2                  # [pages, 16]
    # total deviation energy: 15 dof x (sum_k 1/k^2 + 128 * 0.05^2)
    total = 15 * (sum(1.0 / k ** 2 for k in range(1, 9)) + 128 * 0.05 ** 2)
    assert abs(sv2.sum(1).mean().item() / total - 1) < 0.02
    # leading direction carries ~15 (coefficient std 1) plus a little noise
    assert abs(sv2[:, 0].mean().item() / 15.0 - 1) < 0.1
    assert sv2[:, 15].max().item() < 1e-20                 # centring removes one dof


def test_workload_layout_and_page_table():
    w = workloads.make(2, ctx=2048, seed=5, extra_blocks=3)
    assert w.q.shape == (1, 32, 128) and w.q.dtype == torch.float32
    assert w.k_cache.shape == (w.num_blocks, 8, 16, 128) and w.k_cache.dtype == torch.bfloat16
    pt = w.page_table
    assert pt.shape == (1, 128) and len(set(pt.flatten().tolist())) == 128
    assert int(pt.max()) < w.num_blocks
    w2 = workloads.make(2, ctx=2048, seed=5, extra_blocks=3)
    assert torch.equal(w.k_cache, w2.k_cache) and torch.equal(w.q, w2.q)


def test_carrier_centroid_points_along_group_query():
    w = workloads.make(3, ctx=1024, batch=2, seed=9)
    G = w.group
    for b in range(2):
        p = int(w.carrier[b])
        assert 0 <= p < w.max_pages
        for kvh in range(w.n_kv_heads):
            u = w.q[b, kvh * G:(kvh + 1) * G].mean(0)
            mu = w.k_cache[int(w.page_table[b, p]), kvh].float().mean(0)
            cos = torch.dot(u, mu) / (u.norm() * mu.norm())
            assert abs(cos.item() - 0.9) < 0.01


def test_sketch_constants_golden():
    g = json.load(open(os.path.join(HERE, "golden", "sketch_constants.json")))
    n_top = g["token_budget"] // g["page_size"]
    assert n_top == g["n_top_pages"]
    assert n_top * g["page_size"] == g["attended_tokens"]
    assert f"{100 * g['attended_tokens'] / g['seq_len']:.1f}" == g["attended_percent_printed"]
    p = workloads.PRESETS
    assert p[2]["budget"] == g["token_budget"]
    payload = g["d_head"] * g["rank"] // 2 + g["d_head"] + g["page_size"] * g["rank"] + 6
    page_kv = g["page_size"] * g["d_head"] * 2 * 2
    assert math.isclose(payload / page_kv, g["summary_fraction_of_page_kv_approx"], rel_tol=0.1)


def test_shared_keys_workload_premise():
    """The blind-direction workload: the planted common basis S is what a
    sequence-level PCA of the page deviations finds (the oracle's shared
    basis spans it, once the sequence has enough pages that S's weakest
    direction outweighs the one carrier's), and every carrier's deviations lie
    in S's null space."""
    import numpy as np
    import oracle
    w = workloads.make(2, ctx=16 * 2000, batch=2, budget=512, keys="shared", seed=5,
                       n_kv_heads=2, n_q_heads=8)
    q, pt, sl = w.q.numpy(), w.page_table.numpy(), w.seq_lens.numpy()
    kb = workloads.bf16_bits(w.k_cache)
    S = w.shared_basis.double().numpy()
    W = oracle.shared_basis(kb, pt, sl)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            cosines = np.linalg.svd(S[b, h].T @ W[b, h], compute_uv=False)
            assert cosines.min() > 0.99, (b, h, cosines.min())
            keys = w.k_cache[pt[b, w.carrier[b]], h].double().numpy()
            dev = keys - keys.mean(0)
            inside = np.linalg.norm(dev @ S[b, h]) / np.linalg.norm(dev)
            assert inside < 0.05, (b, h, inside)  # only the 0.05-std noise and bf16 rounding
