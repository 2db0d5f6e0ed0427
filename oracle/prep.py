"""Pool-write prep oracle, float64 on the CPU (test infrastructure only).

Definitions followed (issue "gemma4: serving prep needs pool-write forms --
hd256 QKV in one pass, hd512 V alongside K", Description and Proposed Plan):

* hd256 (local layers, which have their own V projection): Q is normalised and
  rotated into a contiguous output; K is normalised and rotated, V is
  normalised without a weight and not rotated; K and V are written directly
  into the layer's pool pages.
* hd512 (global layers): K is normalised with its weight and rotated; V is
  the raw K normalised without a weight, reusing K's normalising denominator,
  and is not rotated.  The global family's Q takes the query rule of the hd256
  prep at head_dim 512 (the pages give that rule once, for Q, without tying it
  to a head_dim; reading taken here).
* Slot contract: token t of a request lands at position start_pos + t, page
  ids[(start_pos + t) // P], slot (start_pos + t) % P, in the given layer.

Readings where the pages are silent (conventions, parity unpinned except where
a library routine pins them, see below):

* RMSNorm: x * w / sqrt(mean(x^2) + eps) over the head dimension, the weight a
  direct multiplier (weights near 1), eps passed explicitly (1e-6 in the
  workloads).  Norm before rotation.  Pinned against torch's rms_norm.
* RoPE: rotate-half pairs (i, i + D/2), angle p * theta^(-2i/D) for i < D/2,
  applied to the full head.  Pinned against the rotate-half rotary embedding of
  the transformers library (LLaMA form) and by invariants (identity at p = 0,
  additivity in p, pair norms preserved, dot products depend on p - p' only).
* The oracle computes angles itself in float64; it never reads the cos/sin
  tables the GPU entries take.
"""
from __future__ import annotations

import numpy as np

from .bf16 import to_f64
from .layout import PoolGeometry, kv_blocks, kv_lengths


def inv_rms(x: np.ndarray, eps: float) -> np.ndarray:
    """1 / sqrt(mean(x^2) + eps) over the last axis (keepdims)."""
    return 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rms_norm_weighted(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    return x * inv_rms(x, eps) * w


def rope_rotate_half(y: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate pairs (i, i + D/2) of y[..., T, H, D] by pos[T] * theta^(-2i/D)."""
    d = y.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = float(theta) ** (-2.0 * i / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]   # [T, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = y[..., :half], y[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def token_positions(qo_indptr, kv_page_indptr, kv_last_page_len, page_size: int,
                    kv_len=None) -> np.ndarray:
    """Absolute position of every token: start_pos_b + t, start_pos_b = kv_len_b - qo_len_b
    (kv_len from the pages, or given for resident windows)."""
    qo_indptr = np.asarray(qo_indptr, dtype=np.int64)
    if kv_len is None:
        kv_len = kv_lengths(kv_page_indptr, kv_last_page_len, page_size)
    pos = np.empty(int(qo_indptr[-1]), dtype=np.int64)
    for b in range(len(qo_indptr) - 1):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        start = int(kv_len[b]) - (q1 - q0)
        pos[q0:q1] = start + np.arange(q1 - q0)
    return pos


def qkv_prep_hd256(q_in, k_in, v_in, q_norm_w, k_norm_w, pos, eps: float, theta: float):
    """Contiguous token-major outputs (q_out [T,Hq,D], k_rows [T,Hkv,D], v_rows [T,Hkv,D])."""
    q = to_f64(q_in)
    k = to_f64(k_in)
    v = to_f64(v_in)
    wq = to_f64(q_norm_w)
    wk = to_f64(k_norm_w)
    q_out = rope_rotate_half(rms_norm_weighted(q, wq, eps), pos, theta)
    k_rows = rope_rotate_half(rms_norm_weighted(k, wk, eps), pos, theta)
    v_rows = v * inv_rms(v, eps)
    return q_out, k_rows, v_rows


def kv_prep_hd512(k_in, k_norm_w, pos, eps: float, theta: float):
    """K and V rows [T, Hkv, D] from the raw K alone; both use the same inv_rms(k)."""
    k = to_f64(k_in)
    wk = to_f64(k_norm_w)
    inv = inv_rms(k, eps)
    k_rows = rope_rotate_half(k * inv * wk, pos, theta)
    v_rows = k * inv
    return k_rows, v_rows


def q_prep_hd512(q_in, q_norm_w, pos, eps: float, theta: float):
    """Global-family query rows [T, Hq, 512]: the query rule of the hd256 prep
    (weighted RMSNorm, then rotate-half RoPE at the token's position) at
    head_dim 512, written contiguously."""
    q = to_f64(q_in)
    wq = to_f64(q_norm_w)
    return rope_rotate_half(rms_norm_weighted(q, wq, eps), pos, theta)


def expected_pool_writes(geom: PoolGeometry, layer: int, qo_indptr, kv_page_indptr,
                         kv_page_indices, kv_last_page_len, kv_len=None):
    """For every token, the (page, slot) it is written to in ``layer``: position
    p in page ids[(p // P) mod n_pages] (the plain table, or a resident
    window's ring), slot p mod P."""
    pos = token_positions(qo_indptr, kv_page_indptr, kv_last_page_len, geom.page_size, kv_len)
    qo_indptr = np.asarray(qo_indptr, dtype=np.int64)
    kv_page_indptr = np.asarray(kv_page_indptr, dtype=np.int64)
    ids = np.asarray(kv_page_indices, dtype=np.int64)
    page = np.empty_like(pos)
    for b in range(len(qo_indptr) - 1):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        pages = ids[kv_page_indptr[b]:kv_page_indptr[b + 1]]
        page[q0:q1] = pages[(pos[q0:q1] // geom.page_size) % len(pages)]
    slot = pos % geom.page_size
    return page, slot


def apply_pool_writes(pool_f64: np.ndarray, geom: PoolGeometry, layer: int, page, slot,
                      k_rows, v_rows):
    """Write K/V rows into a flat float64 pool copy (layout of ``oracle.layout``),
    in place.  Returns a flat boolean mask of the elements written."""
    kb, vb = kv_blocks(pool_f64, geom)
    mask = np.zeros(pool_f64.shape, dtype=bool)
    mk, mv = kv_blocks(mask, geom)
    for t in range(len(page)):
        kb[layer, page[t], :, slot[t], :] = k_rows[t]
        vb[layer, page[t], :, :, slot[t]] = v_rows[t]
        mk[layer, page[t], :, slot[t], :] = True
        mv[layer, page[t], :, :, slot[t]] = True
    return mask
