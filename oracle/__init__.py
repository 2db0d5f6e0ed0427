"""fp64 CPU oracle for paged sliding-window prefill and the fused pool-write prep.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The library
(``paged_sliding_window_page_amd``) never imports it, and this package imports
nothing from the library: the two share no kernels, headers, helpers, tables or
constants.  Inputs reach both sides from ``synth`` (random draws and page tables
only).

What it computes, from the three pages:

* PR "feat(kernels): Rust wrapper for the hd256 windowed paged prefill",
  Description: attention that reads K/V through a page table (page ids plus
  the last page's length), with an explicit ``sm_scale`` and a ``window_left``
  that is an inclusive distance.
* issue "gemma4: serving prep needs pool-write forms -- hd256 QKV in one pass,
  hd512 V alongside K", Description and Proposed Plan: the pool-write prep that
  RMS-normalises and rotates Q and K, weightless-normalises V, and writes K/V
  into the layer's pool pages at slot start_pos + token.
* PR "feat(gemma4): paged KV serving across both attention families",
  Description: the two families (local hd256 / 8 KV heads with a window, global
  hd512 / 1 KV head full attention) and decode as the prefill entry at one token.

Everything is float64 on the CPU and deliberately unblocked.  The module-level
docstrings of ``attention`` and ``prep`` state every reading taken where the
pages are silent, and which parts are pinned by tests and which are conventions
("parity unpinned (convention)": the pool layout, the RMSNorm weight form and
eps, and the RoPE pairing, whose frequency schedule and pairing are pinned only
against a library routine).
"""
from .bf16 import bf16_bits, bits_to_f64, to_f64, f64_to_bf16_bits
from .layout import PoolGeometry, kv_blocks, gather_kv, kv_lengths
from .attention import paged_attention, attention_rows, allowed_keys
from .prep import (inv_rms, rms_norm_weighted, rope_rotate_half, qkv_prep_hd256,
                   kv_prep_hd512, q_prep_hd512, token_positions, expected_pool_writes,
                   apply_pool_writes)

__all__ = [
    "bf16_bits", "bits_to_f64", "to_f64", "f64_to_bf16_bits",
    "PoolGeometry", "kv_blocks", "gather_kv", "kv_lengths",
    "paged_attention", "attention_rows", "allowed_keys",
    "inv_rms", "rms_norm_weighted", "rope_rotate_half", "qkv_prep_hd256",
    "kv_prep_hd512", "q_prep_hd512", "token_positions", "expected_pool_writes", "apply_pool_writes",
]
