"""Seeded synthetic inputs for the paged-attention and pool-write workloads.

This module only draws random numbers and lays out page tables.  It holds none
of the method's arithmetic (no attention, no normalisation, no rotation and no
pool addressing), so that the HIP path and the CPU oracle can both consume what
it returns without sharing any of the computation they are compared on.

Every draw goes through a ``torch.Generator`` seeded by the caller.  Floating
point values are drawn in fp32 and cast to bf16 with round-to-nearest-even
(torch's cast), so both sides see the same bf16 bits.

The workload shapes follow the serving geometry the pages describe: a local
(sliding-window) family at head_dim 256 with 16 query / 8 KV heads and a global
family at head_dim 512 with 16 query / 1 KV head, both over pools of 16-slot
pages (PR "feat(gemma4): paged KV serving across both attention families",
Description).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "normal_bf16",
    "uniform_lengths",
    "PageTable",
    "random_page_table",
    "lengths_to_indptr",
    "AttentionCase",
    "attention_case",
    "PrepCase",
    "prep_case",
    "decode_batch",
    "LOCAL",
    "GLOBAL",
]

# Head geometry of the two KV families (query heads, KV heads, head_dim).
LOCAL = dict(num_qo_heads=16, num_kv_heads=8, head_dim=256)
GLOBAL = dict(num_qo_heads=16, num_kv_heads=1, head_dim=512)


def generator(seed: int, device: str | torch.device = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_bf16(shape, std: float, gen: torch.Generator, mean: float = 0.0,
                device: str | torch.device = "cpu") -> torch.Tensor:
    """N(mean, std^2) drawn in fp32 on ``device`` and cast to bf16 (RNE)."""
    x = torch.randn(tuple(shape), generator=gen, dtype=torch.float32, device=device)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x.to(torch.bfloat16)


def uniform_lengths(n: int, lo: int, hi: int, gen: torch.Generator) -> list[int]:
    """n integers drawn uniformly from the closed range [lo, hi]."""
    return [int(v) for v in torch.randint(lo, hi + 1, (n,), generator=gen)]


def lengths_to_indptr(lengths) -> np.ndarray:
    out = np.zeros(len(lengths) + 1, dtype=np.int32)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out


@dataclass
class PageTable:
    """CSR page table: request b owns kv_page_indices[indptr[b]:indptr[b+1]]."""
    kv_page_indptr: np.ndarray      # int32 [batch+1]
    kv_page_indices: np.ndarray     # int32 [nnz]
    kv_last_page_len: np.ndarray    # int32 [batch], in [1, page_size]


def random_page_table(kv_lens, page_size: int, num_pages: int, gen: torch.Generator,
                      shared_perm: torch.Tensor | None = None) -> PageTable:
    """Give each request ceil(kv_len / page_size) distinct pages, taken as
    consecutive chunks of one random permutation of the pool, so tables are
    random and never overlap."""
    n_pages = [(int(n) + page_size - 1) // page_size for n in kv_lens]
    need = sum(n_pages)
    if need > num_pages:
        raise ValueError(f"pool of {num_pages} pages cannot hold {need}")
    perm = shared_perm if shared_perm is not None else torch.randperm(num_pages, generator=gen)
    indices = perm[:need].to(torch.int32).numpy().copy()
    last = np.array([int(n) - (c - 1) * page_size for n, c in zip(kv_lens, n_pages)],
                    dtype=np.int32)
    return PageTable(lengths_to_indptr(n_pages), indices, last)


def ring_page_table(kv_lens, ring_pages, page_size: int, num_pages: int,
                    gen: torch.Generator) -> PageTable:
    """Resident-window tables: request b holds min(ceil(kv_len_b / P), ring_pages[b])
    distinct random pages; when kv_len_b is larger the pages are a ring and
    the last-page length is that of position kv_len_b - 1."""
    n_pages = [min((int(n) + page_size - 1) // page_size, int(r)) for n, r in zip(kv_lens, ring_pages)]
    need = sum(n_pages)
    if need > num_pages:
        raise ValueError(f"pool of {num_pages} pages cannot hold {need}")
    perm = torch.randperm(num_pages, generator=gen)
    indices = perm[:need].to(torch.int32).numpy().copy()
    last = np.array([(int(n) - 1) % page_size + 1 for n in kv_lens], dtype=np.int32)
    return PageTable(lengths_to_indptr(n_pages), indices, last)


@dataclass
class AttentionCase:
    """One batch for a paged attention entry, all tensors on the CPU."""
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    num_layers: int
    layer: int
    qo_lens: list
    kv_lens: list
    qo_indptr: np.ndarray
    table: PageTable
    q: torch.Tensor                 # bf16 [sum(qo_lens), H_q, D]
    pool: torch.Tensor              # bf16, flat, every element drawn
    extra: dict = field(default_factory=dict)

    @property
    def pool_numel(self) -> int:
        return self.pool.numel()


def pool_numel(num_layers, num_pages, num_kv_heads, page_size, head_dim) -> int:
    """Element count of a whole-page pool holding a K and a V block per page."""
    return num_layers * num_pages * 2 * num_kv_heads * page_size * head_dim


def attention_case(seed: int, qo_lens, kv_lens, *, num_qo_heads: int, num_kv_heads: int,
                   head_dim: int, page_size: int = 16, num_pages: int | None = None,
                   num_layers: int = 1, layer: int = 0, std: float = 0.25,
                   fill_pool: bool = True) -> AttentionCase:
    """Q and the whole pool ~ N(0, std^2) in bf16, random non-overlapping page
    tables.  ``fill_pool=False`` leaves the pool zero (callers that fill it
    themselves, e.g. on the device)."""
    assert len(qo_lens) == len(kv_lens)
    gen = generator(seed)
    need = sum((int(n) + page_size - 1) // page_size for n in kv_lens)
    if num_pages is None:
        num_pages = need
    table = random_page_table(kv_lens, page_size, num_pages, gen)
    total_q = int(sum(qo_lens))
    q = normal_bf16((total_q, num_qo_heads, head_dim), std, gen)
    numel = pool_numel(num_layers, num_pages, num_kv_heads, page_size, head_dim)
    if fill_pool:
        pool = normal_bf16((numel,), std, gen)
    else:
        pool = torch.zeros(numel, dtype=torch.bfloat16)
    return AttentionCase(num_qo_heads, num_kv_heads, head_dim, page_size, num_pages,
                         num_layers, layer, list(map(int, qo_lens)), list(map(int, kv_lens)),
                         lengths_to_indptr(qo_lens), table, q, pool)


def decode_batch(head_dim: int, device, num_requests: int = 64, lo: int = 512,
                 hi: int = 8192, num_pages: int = 32768, seed: int = 5) -> AttentionCase:
    """One-token decode batch of a serving step: ``num_requests`` requests with
    KV lengths ~ U[lo, hi] (one query each), random page tables over a pool of
    ``num_pages`` 16-slot pages, Q and the whole pool ~ N(0, 0.25^2).  The
    pool is drawn directly on ``device`` (it is several GiB at head_dim 256);
    Q stays on the CPU like the other cases."""
    fam = LOCAL if head_dim == 256 else GLOBAL
    hkv = fam["num_kv_heads"]
    kv = uniform_lengths(num_requests, lo, hi, generator(seed))
    gen = generator(50 + head_dim)
    table = random_page_table(kv, 16, num_pages, gen)
    numel = pool_numel(1, num_pages, hkv, 16, head_dim)
    pool = normal_bf16((numel,), 0.25, generator(500 + head_dim, device), device=device)
    q = normal_bf16((num_requests, fam["num_qo_heads"], head_dim), 0.25, gen)
    return AttentionCase(fam["num_qo_heads"], hkv, head_dim, 16, num_pages, 1, 0,
                         [1] * num_requests, list(map(int, kv)),
                         lengths_to_indptr([1] * num_requests), table, q, pool)


@dataclass
class PrepCase:
    """Inputs of one pool-write prep call, all on the CPU."""
    head_dim: int
    num_qo_heads: int
    num_kv_heads: int
    page_size: int
    num_pages: int
    num_layers: int
    layer: int
    qo_lens: list
    kv_lens: list
    qo_indptr: np.ndarray
    table: PageTable
    q_in: torch.Tensor | None       # bf16 [T, H_q, D] (hd256 only)
    k_in: torch.Tensor              # bf16 [T, H_kv, D]
    v_in: torch.Tensor | None       # bf16 [T, H_kv, D] (hd256 only)
    q_norm_w: torch.Tensor | None   # bf16 [D]
    k_norm_w: torch.Tensor          # bf16 [D]
    rope_positions: int
    rope_theta: float
    eps: float


def prep_case(seed: int, qo_lens, start_pos, *, head_dim: int, num_kv_heads: int,
              num_qo_heads: int = 16, page_size: int = 16, num_pages: int | None = None,
              num_layers: int = 8, layer: int = 3, rope_positions: int = 16384,
              rope_theta: float = 10000.0, eps: float = 1e-6, with_q_v: bool = True,
              extra_pages: int = 0, with_q: bool = False) -> PrepCase:
    """Projections ~ N(0, 1) in bf16, norm weights 1 + N(0, 0.1^2) in bf16.

    Request b writes tokens at positions start_pos[b] .. start_pos[b]+qo_lens[b]-1,
    so its table covers kv_len = start_pos + qo_len keys."""
    gen = generator(seed)
    kv_lens = [int(s) + int(n) for s, n in zip(start_pos, qo_lens)]
    need = sum((n + page_size - 1) // page_size for n in kv_lens)
    if num_pages is None:
        num_pages = need + extra_pages
    table = random_page_table(kv_lens, page_size, num_pages, gen)
    t = int(sum(qo_lens))
    q_in = normal_bf16((t, num_qo_heads, head_dim), 1.0, gen) if with_q_v else None
    k_in = normal_bf16((t, num_kv_heads, head_dim), 1.0, gen)
    v_in = normal_bf16((t, num_kv_heads, head_dim), 1.0, gen) if with_q_v else None
    q_w = normal_bf16((head_dim,), 0.1, gen, mean=1.0) if with_q_v else None
    k_w = normal_bf16((head_dim,), 0.1, gen, mean=1.0)
    if with_q and not with_q_v:
        # queries without V (the global family), drawn after everything else so
        # the K-only cases keep their inputs
        q_in = normal_bf16((t, num_qo_heads, head_dim), 1.0, gen)
        q_w = normal_bf16((head_dim,), 0.1, gen, mean=1.0)
    return PrepCase(head_dim, num_qo_heads, num_kv_heads, page_size, num_pages, num_layers,
                    layer, list(map(int, qo_lens)), kv_lens, lengths_to_indptr(qo_lens), table,
                    q_in, k_in, v_in, q_w, k_w, rope_positions, rope_theta, eps)
