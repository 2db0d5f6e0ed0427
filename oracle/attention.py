"""Paged attention oracle, float64 on the CPU (test infrastructure only).

Definition followed (PR "feat(kernels): Rust wrapper for the hd256 windowed
paged prefill", Description; PR "feat(gemma4): paged KV serving across both
attention families", Description):

  For request b with kv_len_b keys (from its page table) and qo_len_b queries,
  query i sits at absolute position p_i = kv_len_b - qo_len_b + i, i.e.
  start_pos + i: the queries are the last qo_len_b tokens of the KV (the prep
  writes slot start_pos + token before attention reads it).  Query head h reads
  KV head g = h // (H_q / H_kv) (contiguous GQA groups of H_q / H_kv query
  heads).  Key j is allowed for query i when

      0 <= p_i - j <= window_left      (window_left >= 0; inclusive distance)
      0 <= p_i - j                     (window_left == -1; full causal)

  so a query sees at most window_left + 1 keys and always sees itself.
  kv_len_b is the absolute KV length: from the pages by default, or given
  explicitly for a resident window, whose pages hold only the last
  n_pages * page_size positions as a ring (position p in page (p // P) mod
  n_pages; issue "gemma4: serving prep needs pool-write forms", Proposed
  Plan: past the window, slots and positions need a separate map).  A query
  that would see a key the ring no longer holds is an error.  With
  s_j = sm_scale * <q_i,h , K_j,g>, the output is sum_j softmax(s)_j V_j,g,
  softmax in base e over the allowed keys only.  sm_scale is whatever the caller
  passes (the model runs unscaled attention, sm_scale = 1).

Readings where the pages are silent: no logit soft-cap, no ALiBi, no sinks;
window_left < -1 is meaningless (the library rejects it; here it raises).
One matrix product per (request, head) is the only library step; masking and
softmax are written out.  Pinned by tests against a brute-force loop, torch's
scaled_dot_product_attention in float64, closed forms (window_left = 0,
sm_scale = 0, one-hot values), and the page-permutation, window-saturation,
GQA-replication and decode-equals-prefill-row invariants.
"""
from __future__ import annotations

import numpy as np

from .layout import PoolGeometry, kv_blocks, gather_kv, kv_lengths, resident_start
from .bf16 import to_f64


def allowed_keys(pos: np.ndarray, kv_len: int, window_left: int) -> np.ndarray:
    """Boolean [len(pos), kv_len]: key j allowed for the query at position pos[i]."""
    if window_left < -1:
        raise ValueError("window_left must be >= -1")
    j = np.arange(kv_len, dtype=np.int64)[None, :]
    dist = np.asarray(pos, dtype=np.int64)[:, None] - j
    ok = dist >= 0
    if window_left >= 0:
        ok &= dist <= window_left
    return ok


def attention_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, pos: np.ndarray,
                   sm_scale: float, window_left: int) -> np.ndarray:
    """Masked softmax attention for one head: q_rows [n, D], k/v [kv_len, D]."""
    s = float(sm_scale) * (q_rows @ k.T)
    ok = allowed_keys(pos, k.shape[0], window_left)
    s = np.where(ok, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    w = np.where(ok, np.exp(s), 0.0)
    w = w / w.sum(axis=1, keepdims=True)
    return w @ v


def paged_attention(q, pool, geom: PoolGeometry, layer: int, qo_indptr, kv_page_indptr,
                    kv_page_indices, kv_last_page_len, sm_scale: float, window_left: int,
                    requests=None, samples=None, kv_len=None) -> np.ndarray:
    """float64 output [sum(qo), H_q, D].

    q: bf16 tensor / uint16 bits / float array [sum(qo), H_q, D].
    pool: flat bf16 pool in the layout of ``oracle.layout``.
    requests: optional subset of request indices to compute (others stay NaN).
    samples: optional list of (token_index, head) pairs; only those rows are
        computed (others stay NaN).
    kv_len: optional absolute KV lengths (resident windows); default from the
        pages and last-page lengths.
    """
    qf = to_f64(q)
    n_tok, h_q, d = qf.shape
    h_kv = geom.num_kv_heads
    if h_kv <= 0 or h_q % h_kv != 0:
        raise ValueError("query heads must be a positive multiple of KV heads")
    group = h_q // h_kv
    if d != geom.head_dim:
        raise ValueError("head_dim mismatch")
    kblk, vblk = kv_blocks(pool, geom)
    qo_indptr = np.asarray(qo_indptr, dtype=np.int64)
    kv_page_indptr = np.asarray(kv_page_indptr, dtype=np.int64)
    kv_page_indices = np.asarray(kv_page_indices, dtype=np.int64)
    if kv_len is None:
        kv_len = kv_lengths(kv_page_indptr, kv_last_page_len, geom.page_size)
    kv_len = np.asarray(kv_len, dtype=np.int64)
    batch = len(qo_indptr) - 1
    out = np.full((n_tok, h_q, d), np.nan)

    want = None
    if samples is not None:
        want = {}
        for tok, h in samples:
            b = int(np.searchsorted(qo_indptr, tok, side="right") - 1)
            want.setdefault(b, []).append((int(tok), int(h)))
    todo = range(batch) if requests is None else requests
    if want is not None:
        todo = sorted(want)
    for b in todo:
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        qo_len = q1 - q0
        n_kv = int(kv_len[b])
        if qo_len < 1 or n_kv < qo_len:
            raise ValueError(f"request {b}: qo_len {qo_len}, kv_len {n_kv}")
        pages = kv_page_indices[kv_page_indptr[b]:kv_page_indptr[b + 1]]
        k, v = gather_kv(kblk, vblk, layer, pages, n_kv, geom.page_size)
        start = n_kv - qo_len
        first = resident_start(len(pages), n_kv, geom.page_size)
        if first > 0:
            seen = allowed_keys(start + np.arange(qo_len, dtype=np.int64), n_kv, window_left)
            if seen[:, :first].any():
                raise ValueError(f"request {b}: a query sees a key the ring no longer holds")
        if want is None:
            pos = start + np.arange(qo_len, dtype=np.int64)
            for h in range(h_q):
                g = h // group
                out[q0:q1, h, :] = attention_rows(qf[q0:q1, h, :], k[:, g, :], v[:, g, :],
                                                  pos, sm_scale, window_left)
        else:
            for tok, h in want[b]:
                g = h // group
                pos = np.array([start + (tok - q0)], dtype=np.int64)
                out[tok, h, :] = attention_rows(qf[tok:tok + 1, h, :], k[:, g, :], v[:, g, :],
                                                pos, sm_scale, window_left)[0]
    return out
