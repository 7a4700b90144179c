"""Seeded synthetic inputs for the LOCKS decode path (shared by tests and bench).

This module holds none of the method's arithmetic: it only draws random keys,
values and queries with the shapes and structure of the five workloads, lays
them out in a paged KV cache behind a random page table, and returns them.
Both the GPU path and the CPU oracle consume exactly the bits it produces.

Workloads (ctx = tokens per sequence, 16 tokens per page, head dim 128):
  1  one head, 4K ctx, iid N(0,1) K/V/q, budget 512 (32 pages)
  2  32 q / 8 kv heads (Llama-3.1-8B layer shape), 128K ctx, structured
     per-page low-rank keys, iid N(0,1) values, budget 2048
  3  as 2 at 256K ctx, batch 8, one planted carrier page per sequence whose
     centroid points along the group's mean query direction (cosine 0.9)
  4  as 2 at 1M ctx, budgets 512 and 2048
  5  32 q / 2 kv heads (GLM-4-9B layer shape), 1M ctx, budget 512
Structured keys of one page: k_i = mu + sum_k c_ik b_k + e_i with mu ~ N(0, I),
{b_k} a random orthonormal 8x128 basis drawn per page, c_ik ~ N(0, (1/k)^2) and
e_i ~ N(0, 0.05^2 I).
keys="shared" (the blind-direction workload of the shared-basis comparison):
every page of a (sequence, KV head) varies in one common orthonormal 8x128
basis S (returned as shared_basis, S^T per (sequence, KV head)); one planted
carrier page per sequence instead holds a centroid ~ N(0, I) plus, along the
unit vector u of the group's mean query with its component in span(S)
removed, one token at +spike and the other 15 at -spike/15 (so its deviations
lie in the null space of S).
"""
from __future__ import annotations

import dataclasses
import math

import torch

PAGE = 16
DIM = 128
RANK = 8


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    max_pages: int
    num_blocks: int
    budget: int
    q: torch.Tensor          # f32 [B, Hq, 128]
    k_cache: torch.Tensor    # bf16 [num_blocks, Hkv, 16, 128]
    v_cache: torch.Tensor    # bf16 [num_blocks, Hkv, 16, 128]
    page_table: torch.Tensor  # i32 [B, max_pages]
    seq_lens: torch.Tensor   # i32 [B]
    carrier: torch.Tensor | None = None  # i32 [B] logical page of the planted carrier
    shared_basis: torch.Tensor | None = None  # f32 [B, Hkv, 128, 8] (keys="shared")
    seed: int = 0
    recipe: str = ""

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def k_pages(self) -> int:
        return self.budget // PAGE


PRESETS = {
    1: dict(batch=1, n_q_heads=1, n_kv_heads=1, ctx=4096, budget=512, keys="iid"),
    2: dict(batch=1, n_q_heads=32, n_kv_heads=8, ctx=131072, budget=2048, keys="structured"),
    3: dict(batch=8, n_q_heads=32, n_kv_heads=8, ctx=262144, budget=2048, keys="structured",
            carrier=True),
    4: dict(batch=1, n_q_heads=32, n_kv_heads=8, ctx=1048576, budget=2048, keys="structured"),
    5: dict(batch=1, n_q_heads=32, n_kv_heads=2, ctx=1048576, budget=512, keys="structured"),
}


def _orthonormal_rows(gen: torch.Generator, n: int, device) -> torch.Tensor:
    """n random 8x128 matrices with orthonormal rows (Gram-Schmidt of Gaussians)."""
    g = torch.randn(n, RANK, DIM, generator=gen, device=device, dtype=torch.float32)
    rows = []
    for r in range(RANK):
        v = g[:, r, :]
        for _ in range(2):  # two passes keep the rows orthonormal to float32 rounding
            for u in rows:
                v = v - (v * u).sum(-1, keepdim=True) * u
        v = v / v.norm(dim=-1, keepdim=True)
        rows.append(v)
    return torch.stack(rows, dim=1)


def structured_keys(gen: torch.Generator, n_pages: int, device, noise_std: float = 0.05,
                    rank: int = RANK) -> torch.Tensor:
    """Keys [n_pages, 16, 128] f32: centroid + rank-8 page-local structure + noise."""
    mu = torch.randn(n_pages, DIM, generator=gen, device=device)
    basis = _orthonormal_rows(gen, n_pages, device)[:, :rank, :]
    sig = 1.0 / torch.arange(1, rank + 1, device=device, dtype=torch.float32)
    coef = torch.randn(n_pages, PAGE, rank, generator=gen, device=device) * sig
    noise = torch.randn(n_pages, PAGE, DIM, generator=gen, device=device) * noise_std
    return mu[:, None, :] + torch.bmm(coef, basis) + noise


def shared_subspace_keys(gen: torch.Generator, n_pages: int, S: torch.Tensor, device,
                         noise_std: float = 0.05) -> torch.Tensor:
    """Keys [n_pages, 16, 128] f32 whose in-page variation lies in the rows of S
    (8 x 128, orthonormal), common to all pages: centroid + coefficients in S +
    noise."""
    mu = torch.randn(n_pages, DIM, generator=gen, device=device)
    sig = 1.0 / torch.arange(1, RANK + 1, device=device, dtype=torch.float32)
    coef = torch.randn(n_pages, PAGE, RANK, generator=gen, device=device) * sig
    noise = torch.randn(n_pages, PAGE, DIM, generator=gen, device=device) * noise_std
    return mu[:, None, :] + coef @ S + noise


def make(config: int, device="cpu", ctx: int | None = None, batch: int | None = None,
         budget: int | None = None, seed: int | None = None, n_kv_heads: int | None = None,
         n_q_heads: int | None = None, keys: str | None = None,
         seq_lens: list[int] | None = None, extra_blocks: int = 0,
         chunk_pages: int = 8192, spike: float = 16.0) -> Workload:
    """Workload `config` (1..5) with optional overrides (smaller ctx for tests,
    ragged seq_lens, spare physical blocks). seq_lens entries may be shorter
    than ctx; ctx sets max_pages = ctx // 16."""
    p = dict(PRESETS[config])
    for name, val in (("ctx", ctx), ("batch", batch), ("budget", budget),
                      ("n_kv_heads", n_kv_heads), ("n_q_heads", n_q_heads), ("keys", keys)):
        if val is not None:
            p[name] = val
    B, Hq, Hkv = p["batch"], p["n_q_heads"], p["n_kv_heads"]
    N = p["ctx"] // PAGE
    seed = (1000 + config) if seed is None else seed
    device = torch.device(device)
    num_blocks = B * N + extra_blocks

    lens = torch.full((B,), N * PAGE, dtype=torch.int32) if seq_lens is None else \
        torch.tensor(seq_lens, dtype=torch.int32)
    assert lens.numel() == B

    # physical blocks: one seeded random permutation over all blocks
    gperm = torch.Generator(device="cpu").manual_seed(seed)
    perm = torch.randperm(num_blocks, generator=gperm)
    page_table = perm[: B * N].view(B, N).to(torch.int32)

    k_cache = torch.zeros(num_blocks, Hkv, PAGE, DIM, dtype=torch.bfloat16, device=device)
    v_cache = torch.zeros(num_blocks, Hkv, PAGE, DIM, dtype=torch.bfloat16, device=device)
    q = torch.empty(B, Hq, DIM, dtype=torch.float32, device=device)
    shared = p["keys"] == "shared"
    carrier = torch.full((B,), -1, dtype=torch.int32) if (p.get("carrier") or shared) else None
    shared_basis = torch.empty(B, Hkv, DIM, RANK, device=device) if shared else None
    G = Hq // Hkv
    pt_dev = page_table.to(device=device, dtype=torch.long)

    for b in range(B):
        gen = torch.Generator(device=device).manual_seed(seed * 100 + b)
        q[b] = torch.randn(Hq, DIM, generator=gen, device=device)
        cpage = None
        if carrier is not None:
            cpage = int(torch.randint(0, N, (1,), generator=gen, device=device).item())
            carrier[b] = cpage
        for kvh in range(Hkv):
            if shared:
                S = _orthonormal_rows(gen, 1, device)[0]  # 8 x 128
                shared_basis[b, kvh] = S.t()
            for j0 in range(0, N, chunk_pages):
                n = min(chunk_pages, N - j0)
                if p["keys"] == "iid":
                    kk = torch.randn(n, PAGE, DIM, generator=gen, device=device)
                elif shared:
                    kk = shared_subspace_keys(gen, n, S, device)
                else:
                    kk = structured_keys(gen, n, device)
                if shared and j0 <= cpage < j0 + n:
                    # planted carrier: deviations along u, the group's mean
                    # query with its span(S) component removed
                    u = q[b, kvh * G:(kvh + 1) * G].mean(0)
                    u = u - S.t() @ (S @ u)
                    u = u / u.norm()
                    alpha = torch.full((PAGE,), -spike / (PAGE - 1), device=device)
                    i0 = int(torch.randint(0, PAGE, (1,), generator=gen, device=device).item())
                    alpha[i0] = spike
                    mu_c = torch.randn(DIM, generator=gen, device=device)
                    noise = torch.randn(PAGE, DIM, generator=gen, device=device) * 0.05
                    kk[cpage - j0] = mu_c[None, :] + alpha[:, None] * u[None, :] + noise
                elif cpage is not None and j0 <= cpage < j0 + n:
                    # planted carrier: centroid along the group's mean-q direction
                    u = q[b, kvh * G:(kvh + 1) * G].mean(0)
                    u = u / u.norm()
                    w = torch.randn(DIM, generator=gen, device=device)
                    w = w - (w @ u) * u
                    w = w / w.norm()
                    page = kk[cpage - j0]
                    mu_old = page.mean(0)
                    mu_new = mu_old.norm() * (0.9 * u + math.sqrt(1 - 0.81) * w)
                    kk[cpage - j0] = page - mu_old + mu_new
                blocks = pt_dev[b, j0:j0 + n]
                k_cache[blocks, kvh] = kk.to(torch.bfloat16)
                v_cache[blocks, kvh] = torch.randn(n, PAGE, DIM, generator=gen,
                                                   device=device).to(torch.bfloat16)
    recipe = (f"config {config}: B={B} Hq={Hq} Hkv={Hkv} ctx={p['ctx']} budget={p['budget']} "
              f"keys={p['keys']} seed={seed}")
    return Workload(name=f"config{config}", batch=B, n_q_heads=Hq, n_kv_heads=Hkv,
                    max_pages=N, num_blocks=num_blocks, budget=p["budget"], q=q,
                    k_cache=k_cache, v_cache=v_cache, page_table=page_table.to(device),
                    seq_lens=lens.to(device), carrier=carrier, seed=seed, recipe=recipe,
                    shared_basis=shared_basis)


def bf16_bits(t: torch.Tensor):
    """Host numpy uint16 view of a bf16 tensor's bits (for the CPU oracle)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")
