"""Pool geometry and page-table gather for the oracle (test infrastructure only).

Pool layout.  The pages say only that each layer's K and V sit in "blocks" at
"layout-derived pool offsets" and that the prep checks a "layer offset" and a
whole-page pool (issue "gemma4: serving prep needs pool-write forms -- hd256 QKV
in one pass, hd512 V alongside K", Proposed Plan and Acceptance Criteria).  The
reading taken here, a convention and therefore parity unpinned:

    per (layer, page): a K block [kv_head][slot][dim], then a V block
    [kv_head][dim][slot] (dim-major: keys contiguous for each dim),

a flat bf16 buffer of exactly L * N * 2 * H_kv * P * D elements, layers outer,
pages next.

Page table.  Attention finds each key through a page table: a list of page ids
per request plus the number of filled slots in its final page (PR
"feat(kernels): Rust wrapper for the hd256 windowed paged prefill",
Description).  Reading: CSR form, request b
owns ids[indptr[b]:indptr[b+1]] (at least one page) and its KV length is
(n_pages - 1) * page_size + last_page_len with 1 <= last_page_len <= page_size.
Logical key j of the request lives at page ids[j // P], slot j % P.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .bf16 import bf16_bits, bits_to_f64


@dataclass(frozen=True)
class PoolGeometry:
    num_layers: int
    num_pages: int
    num_kv_heads: int
    page_size: int
    head_dim: int

    @property
    def block(self) -> int:
        """Elements of one K (or V) block of one page."""
        return self.num_kv_heads * self.page_size * self.head_dim

    @property
    def numel(self) -> int:
        return self.num_layers * self.num_pages * 2 * self.block


def kv_blocks(pool, geom: PoolGeometry):
    """(K, V) views of a flat pool (uint16 bits, or any numpy array):
    K [L, N, H, P, D] and V [L, N, H, D, P]."""
    arr = bf16_bits(pool) if not isinstance(pool, np.ndarray) or pool.dtype == np.uint16 else pool
    if arr.size != geom.numel:
        raise ValueError(f"pool has {arr.size} elements, geometry needs {geom.numel}")
    g = geom
    pages = arr.reshape(g.num_layers, g.num_pages, 2, g.block)
    k = pages[:, :, 0, :].reshape(g.num_layers, g.num_pages, g.num_kv_heads, g.page_size,
                                  g.head_dim)
    v = pages[:, :, 1, :].reshape(g.num_layers, g.num_pages, g.num_kv_heads, g.head_dim,
                                  g.page_size)
    return k, v


def kv_lengths(kv_page_indptr, kv_last_page_len, page_size: int) -> np.ndarray:
    """kv_len[b] = (n_pages[b] - 1) * page_size + last_page_len[b]."""
    indptr = np.asarray(kv_page_indptr, dtype=np.int64)
    last = np.asarray(kv_last_page_len, dtype=np.int64)
    n = indptr[1:] - indptr[:-1]
    return (n - 1) * page_size + last


def resident_start(n_pages: int, kv_len: int, page_size: int) -> int:
    """First absolute position a request's pages still hold: 0 while they
    cover every position, else kv_len - n_pages * page_size (a resident
    window keeps only the last n_pages * page_size positions)."""
    return max(0, int(kv_len) - int(n_pages) * int(page_size))


def gather_kv(kblk: np.ndarray, vblk: np.ndarray, layer: int, page_ids, kv_len: int,
              page_size: int):
    """Logical K and V of one request, float64 [kv_len, H_kv, D] each.

    Key j is read from page page_ids[(j // page_size) % n_pages], slot
    j % page_size: the plain table while the pages cover all kv_len positions,
    the slot map of a resident window (a ring of the request's pages) once
    kv_len exceeds them.  Keys before ``resident_start`` are no longer held;
    their rows come back as zeros and callers must not use them."""
    page_ids = np.asarray(page_ids, dtype=np.int64)
    j = np.arange(kv_len, dtype=np.int64)
    page = page_ids[(j // page_size) % len(page_ids)]
    slot = j % page_size
    # advanced indices around a slice: the gathered key axis comes first
    k = bits_to_f64(kblk[layer, page, :, slot, :])     # [kv_len, H, D]
    v = bits_to_f64(vblk[layer, page, :, :, slot])     # [kv_len, H, D]
    gone = j < resident_start(len(page_ids), kv_len, page_size)
    k[gone] = 0.0
    v[gone] = 0.0
    return k, v
