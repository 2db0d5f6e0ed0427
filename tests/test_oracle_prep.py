"""Pins for the pool-write prep oracle (CPU only).

Library routines (torch rms_norm in float64; the rotate-half rotary embedding
of the transformers library), closed forms and invariants of the prep
definition (issue "gemma4: serving prep needs pool-write forms -- hd256 QKV in
one pass, hd512 V alongside K", Description and Proposed Plan).
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).normal(0.0, std, size=shape)


# ------------------------------------------------------------ RMSNorm ----

def test_rms_norm_matches_torch():
    x = _rand((7, 3, 256), 1)
    w = 1.0 + _rand((256,), 2, 0.1)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (256,), torch.from_numpy(w), eps=1e-6)
    np.testing.assert_allclose(oracle.rms_norm_weighted(x, w, 1e-6), ref.numpy(), rtol=1e-14,
                               atol=1e-14)


def test_weightless_norm_closed_form():
    """mean(y^2) = ms / (ms + eps) for y = x * inv_rms(x)."""
    x = _rand((5, 8, 512), 3, 0.01)
    eps = 1e-4
    y = x * oracle.inv_rms(x, eps)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), ms / (ms + eps), rtol=1e-13)


# --------------------------------------------------------------- RoPE ----

def _hf_rope(y, pos, theta):
    """Rotate-half rotary embedding from transformers (LLaMA form), float32 angles."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb
    t, h, d = y.shape
    cfg = LlamaConfig(hidden_size=d * h, num_attention_heads=h, head_dim=d, rope_theta=theta,
                      max_position_embeddings=max(int(pos.max()) + 1, 16))
    emb = LlamaRotaryEmbedding(cfg)
    x = torch.from_numpy(y).transpose(0, 1)[None]                 # [1, H, T, D]
    cos, sin = emb(x.float(), torch.from_numpy(pos)[None])
    out, _ = apply_rotary_pos_emb(x, x, cos.double(), sin.double())
    return out[0].transpose(0, 1).numpy()


@pytest.mark.parametrize("d", [256, 512])
def test_rope_matches_transformers_rotate_half(d):
    y = _rand((64, 2, d), 4)
    pos = np.arange(0, 1280, 20)
    got = oracle.rope_rotate_half(y, pos, 10000.0)
    ref = _hf_rope(y, pos, 10000.0)
    # transformers forms the angles in float32: |angle error| <= ~1280 * 2^-23
    np.testing.assert_allclose(got, ref, rtol=0, atol=2e-3)
    # and tightly at small positions, where float32 angles are nearly exact
    small = np.arange(0, 8)
    np.testing.assert_allclose(oracle.rope_rotate_half(y[:8], small, 10000.0),
                               _hf_rope(y[:8], small, 10000.0), rtol=0, atol=1e-5)


def test_rope_identity_at_zero_and_pair_norms():
    y = _rand((3, 4, 256), 5)
    np.testing.assert_array_equal(oracle.rope_rotate_half(y, np.zeros(3, np.int64), 1e4), y)
    r = oracle.rope_rotate_half(y, np.array([1, 500, 16383]), 1e4)
    n0 = y[..., :128] ** 2 + y[..., 128:] ** 2
    n1 = r[..., :128] ** 2 + r[..., 128:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)


def test_rope_additive_and_relative():
    y = _rand((1, 1, 512), 6)
    z = _rand((1, 1, 512), 7)
    p, r = 1234, 77
    once = oracle.rope_rotate_half(y, np.array([p + r]), 1e4)
    twice = oracle.rope_rotate_half(oracle.rope_rotate_half(y, np.array([p]), 1e4),
                                    np.array([r]), 1e4)
    np.testing.assert_allclose(once, twice, atol=1e-10)
    dots = []
    for base in (0, 100, 9000):
        a = oracle.rope_rotate_half(y, np.array([base + 37]), 1e4)
        b = oracle.rope_rotate_half(z, np.array([base]), 1e4)
        dots.append(float(np.sum(a * b)))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-10)


def test_rope_closed_form_small_case():
    """D = 4, x = (3, 0, 4, 0) normalised without weight or eps -> (1.2, 0, 1.6, 0);
    position 1 rotates pair (0, 2) by 1 rad and pair (1, 3) by 1e4^(-1/2) rad."""
    x = np.array([[[3.0, 0.0, 4.0, 0.0]]])
    y = x * oracle.inv_rms(x, 0.0)
    np.testing.assert_allclose(y, [[[1.2, 0.0, 1.6, 0.0]]], atol=1e-15)
    r = oracle.rope_rotate_half(y, np.array([1]), 10000.0)[0, 0]
    c, s = np.cos(1.0), np.sin(1.0)
    np.testing.assert_allclose(r, [1.2 * c - 1.6 * s, 0.0, 1.6 * c + 1.2 * s, 0.0], atol=1e-15)


# ------------------------------------------------------------ the preps ----

def test_hd256_prep_parts():
    case = synth.prep_case(9, [40], [0], head_dim=256, num_kv_heads=8)
    pos = np.arange(40)
    q_out, k_rows, v_rows = oracle.qkv_prep_hd256(case.q_in, case.k_in, case.v_in,
                                                  case.q_norm_w, case.k_norm_w, pos,
                                                  case.eps, case.rope_theta)
    # V: torch's weightless rms_norm of V itself (its own denominator)
    v = torch.from_numpy(oracle.to_f64(case.v_in))
    np.testing.assert_allclose(v_rows, torch.nn.functional.rms_norm(v, (256,), eps=1e-6).numpy(),
                               rtol=1e-13, atol=1e-13)
    # Q, K at position 0: plain weighted rms_norm (rotation is the identity)
    q = torch.from_numpy(oracle.to_f64(case.q_in))
    wq = torch.from_numpy(oracle.to_f64(case.q_norm_w))
    np.testing.assert_allclose(q_out[0], torch.nn.functional.rms_norm(q[0], (256,), wq, 1e-6).numpy(),
                               rtol=1e-13, atol=1e-13)
    # and the rotation is the transformers rotate-half form
    qn = oracle.rms_norm_weighted(oracle.to_f64(case.q_in), oracle.to_f64(case.q_norm_w), 1e-6)
    np.testing.assert_allclose(q_out, _hf_rope(qn, pos, 1e4), atol=1e-4)
    kn = oracle.rms_norm_weighted(oracle.to_f64(case.k_in), oracle.to_f64(case.k_norm_w), 1e-6)
    np.testing.assert_allclose(k_rows, _hf_rope(kn, pos, 1e4), atol=1e-4)


def test_hd512_v_is_weightless_norm_of_raw_k():
    case = synth.prep_case(10, [24], [100], head_dim=512, num_kv_heads=1, with_q_v=False)
    pos = 100 + np.arange(24)
    k_rows, v_rows = oracle.kv_prep_hd512(case.k_in, case.k_norm_w, pos, case.eps,
                                          case.rope_theta)
    k = torch.from_numpy(oracle.to_f64(case.k_in))
    np.testing.assert_allclose(v_rows, torch.nn.functional.rms_norm(k, (512,), eps=1e-6).numpy(),
                               rtol=1e-13, atol=1e-13)
    wk = oracle.to_f64(case.k_norm_w)
    np.testing.assert_allclose(k_rows, _hf_rope(v_rows * wk, pos, 1e4), atol=1e-4)


def test_hd512_query_prep():
    """Global-family Q: torch's weighted rms_norm at position 0 (rotation is the
    identity there), the transformers rotate-half rotation at head_dim 512
    elsewhere, and pair norms = those of the normalised rows."""
    case = synth.prep_case(11, [20], [300], head_dim=512, num_kv_heads=1, with_q_v=False,
                           with_q=True)
    pos = 300 + np.arange(20)
    q_out = oracle.q_prep_hd512(case.q_in, case.q_norm_w, pos, case.eps, case.rope_theta)
    assert q_out.shape == (20, 16, 512)
    q = torch.from_numpy(oracle.to_f64(case.q_in))
    wq = torch.from_numpy(oracle.to_f64(case.q_norm_w))
    qn = torch.nn.functional.rms_norm(q, (512,), wq, 1e-6).numpy()
    at0 = oracle.q_prep_hd512(case.q_in[:1], case.q_norm_w, np.array([0]), case.eps,
                              case.rope_theta)
    np.testing.assert_allclose(at0, qn[:1], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(q_out, _hf_rope(qn, pos, 1e4), atol=2e-3)
    np.testing.assert_allclose(q_out[..., :256] ** 2 + q_out[..., 256:] ** 2,
                               qn[..., :256] ** 2 + qn[..., 256:] ** 2, rtol=1e-11)


def test_hd512_unit_weight_position_zero_gives_k_equal_v():
    k = synth.normal_bf16((1, 1, 512), 1.0, synth.generator(3))
    w = torch.ones(512, dtype=torch.bfloat16)
    k_rows, v_rows = oracle.kv_prep_hd512(k, w, np.array([0]), 1e-6, 1e4)
    np.testing.assert_array_equal(k_rows, v_rows)


# ---------------------------------------------------------- placement ----

def test_scatter_then_gather_roundtrip():
    """Rows written at slot start_pos + t read back, through the page table, as
    keys start_pos .. start_pos + n - 1 of each request; nothing else is written."""
    case = synth.prep_case(12, [5, 33, 16], [11, 0, 48], head_dim=8, num_kv_heads=2,
                           num_layers=3, layer=1, extra_pages=4)
    g = oracle.PoolGeometry(case.num_layers, case.num_pages, 2, case.page_size, 8)
    t = case.table
    page, slot = oracle.expected_pool_writes(g, 1, case.qo_indptr, t.kv_page_indptr,
                                             t.kv_page_indices, t.kv_last_page_len)
    n = len(page)
    k_rows = np.arange(n * 2 * 8, dtype=np.float64).reshape(n, 2, 8) + 1.0
    v_rows = -k_rows
    pool = np.zeros(g.numel)
    mask = oracle.apply_pool_writes(pool, g, 1, page, slot, k_rows, v_rows)
    assert mask.sum() == n * 2 * 2 * 8 == np.count_nonzero(pool)
    per_layer = mask.reshape(3, -1)
    assert not per_layer[0].any() and not per_layer[2].any()
    # read back with flat indices: K block [H][P][D], V block [H][D][P]
    blk = 2 * 16 * 8
    d = np.arange(8)
    pos = oracle.token_positions(case.qo_indptr, t.kv_page_indptr, t.kv_last_page_len, 16)
    for b in range(3):
        q0, q1 = case.qo_indptr[b], case.qo_indptr[b + 1]
        ids = t.kv_page_indices[t.kv_page_indptr[b]:t.kv_page_indptr[b + 1]]
        for tok in range(q0, q1):
            p = pos[tok]
            assert p == [11, 0, 48][b] + tok - q0
            base = (1 * g.num_pages + ids[p // 16]) * 2 * blk
            for hh in range(2):
                np.testing.assert_array_equal(pool[base + (hh * 16 + p % 16) * 8 + d], k_rows[tok, hh])
                np.testing.assert_array_equal(pool[base + blk + (hh * 8 + d) * 16 + p % 16],
                                              v_rows[tok, hh])


def test_bf16_helpers():
    x = torch.tensor([1.0, -2.5, 3.140625, 0.0, 1e-3, 65504.0], dtype=torch.float32).to(torch.bfloat16)
    np.testing.assert_array_equal(oracle.to_f64(x), x.to(torch.float64).numpy())
    back = oracle.f64_to_bf16_bits(oracle.to_f64(x))
    np.testing.assert_array_equal(back, oracle.bf16_bits(x))
    # ties to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert oracle.f64_to_bf16_bits(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    assert oracle.f64_to_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82
