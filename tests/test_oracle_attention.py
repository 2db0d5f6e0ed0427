"""Pins for the attention oracle: things other than the oracle itself that fix
what windowed paged prefill must return (CPU only).

The pages print no worked numbers, so the pins are a hand-derived example
(tests/golden), a library routine (torch scaled_dot_product_attention in
float64), brute force on tiny inputs, closed forms and the invariants the
contract implies (PR "feat(kernels): Rust wrapper for the hd256 windowed paged
prefill", Description; PR "feat(gemma4): paged KV serving across both attention
families", Description).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _geom(case):
    return oracle.PoolGeometry(case.num_layers, case.num_pages, case.num_kv_heads,
                               case.page_size, case.head_dim)


def _run(case, sm_scale=1.0, window_left=-1, pool=None, table=None, samples=None):
    t = table or case.table
    return oracle.paged_attention(case.q, case.pool if pool is None else pool, _geom(case),
                                  case.layer, case.qo_indptr, t.kv_page_indptr,
                                  t.kv_page_indices, t.kv_last_page_len, sm_scale,
                                  window_left, samples=samples)


def _flat_k(g, layer, page, head, slot, d):
    """Flat index of a K element: per (layer, page) a K block [H][P][D] then a V block."""
    blk = g.num_kv_heads * g.page_size * g.head_dim
    return ((layer * g.num_pages + page) * 2) * blk + (head * g.page_size + slot) * g.head_dim + d


def _flat_v(g, layer, page, head, d, slot):
    """Flat index of a V element: the V block is dim-major, [H][D][P]."""
    blk = g.num_kv_heads * g.page_size * g.head_dim
    return ((layer * g.num_pages + page) * 2 + 1) * blk + (head * g.head_dim + d) * g.page_size + slot


def _logical_kv(case, pool=None):
    """K, V [kv_len, H, D] per request, read element by element through the page
    table with flat indices (independent of oracle.gather_kv / kv_blocks)."""
    g = _geom(case)
    bits = oracle.bf16_bits(case.pool if pool is None else pool).reshape(-1)
    d = np.arange(g.head_dim)
    out = []
    for b in range(len(case.kv_lens)):
        ids = case.table.kv_page_indices[case.table.kv_page_indptr[b]:case.table.kv_page_indptr[b + 1]]
        ks, vs = [], []
        for j in range(case.kv_lens[b]):
            page, slot = ids[j // case.page_size], j % case.page_size
            ks.append([oracle.bits_to_f64(bits[_flat_k(g, case.layer, page, hh, slot, d)])
                       for hh in range(g.num_kv_heads)])
            vs.append([oracle.bits_to_f64(bits[_flat_v(g, case.layer, page, hh, d, slot)])
                       for hh in range(g.num_kv_heads)])
        out.append((np.array(ks), np.array(vs)))
    return out


# ---------------------------------------------------------------- golden ----

@pytest.mark.parametrize("window", ["-1", "1", "0"])
def test_hand_derived_example(window):
    g = json.load(open(os.path.join(GOLDEN, "attention_tiny.json")))
    geo = oracle.PoolGeometry(**g["geometry"])
    pool = torch.tensor(g["pool"], dtype=torch.float32).to(torch.bfloat16)
    q = torch.tensor(g["q"], dtype=torch.float32).to(torch.bfloat16)
    o = oracle.paged_attention(q, pool, geo, 0, g["qo_indptr"], g["kv_page_indptr"],
                               g["kv_page_indices"], g["kv_last_page_len"], math.log(2.0),
                               int(window))
    np.testing.assert_allclose(o, np.array(g["expected"][window]), rtol=0, atol=1e-14)


# ------------------------------------------------------------ brute force ----

def _brute(q_rows, k, v, pos, scale, window_left):
    """Per-query loop in plain Python floats: pick keys by the inclusive
    distance rule, softmax with an explicit max, weighted sum of values."""
    out = np.zeros_like(q_rows)
    for i in range(q_rows.shape[0]):
        keys = [j for j in range(k.shape[0])
                if pos[i] - j >= 0 and (window_left < 0 or pos[i] - j <= window_left)]
        sc = [scale * sum(float(a) * float(b) for a, b in zip(q_rows[i], k[j])) for j in keys]
        mx = max(sc)
        e = [math.exp(s - mx) for s in sc]
        z = sum(e)
        for w, j in zip(e, keys):
            out[i] += (w / z) * v[j]
    return out


@pytest.mark.parametrize("group", [1, 2, 4])
@pytest.mark.parametrize("seq", [1, 2, 5, 8])
def test_brute_force_small(group, seq):
    h_kv = 2
    case = synth.attention_case(100 + seq * 10 + group, [seq, max(1, seq - 1)],
                                [seq, seq + 3], num_qo_heads=h_kv * group,
                                num_kv_heads=h_kv, head_dim=8, page_size=4, num_pages=9)
    logical = _logical_kv(case)
    q = oracle.to_f64(case.q)
    for wl in range(-1, 9):
        o = _run(case, sm_scale=0.7, window_left=wl)
        for b, (k, v) in enumerate(logical):
            q0, q1 = case.qo_indptr[b], case.qo_indptr[b + 1]
            pos = case.kv_lens[b] - (q1 - q0) + np.arange(q1 - q0)
            for h in range(h_kv * group):
                ref = _brute(q[q0:q1, h], k[:, h // group], v[:, h // group], pos, 0.7, wl)
                np.testing.assert_allclose(o[q0:q1, h], ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------- library SDPA ----

@pytest.mark.parametrize("wl", [-1, 0, 3, 16, 40])
def test_matches_torch_sdpa_fp64(wl):
    case = synth.attention_case(7, [33, 1, 20], [50, 17, 20], num_qo_heads=8, num_kv_heads=2,
                                head_dim=16, page_size=16, num_pages=12)
    o = _run(case, sm_scale=0.37, window_left=wl)
    logical = _logical_kv(case)
    q = oracle.to_f64(case.q)
    for b, (k, v) in enumerate(logical):
        q0, q1 = case.qo_indptr[b], case.qo_indptr[b + 1]
        n_q, n_kv = q1 - q0, case.kv_lens[b]
        pos = torch.arange(n_kv - n_q, n_kv)[:, None]
        j = torch.arange(n_kv)[None, :]
        mask = (pos - j >= 0) & ((pos - j <= wl) if wl >= 0 else torch.ones_like(j, dtype=torch.bool))
        qt = torch.from_numpy(q[q0:q1]).transpose(0, 1)            # [H, n_q, D]
        kt = torch.from_numpy(k).transpose(0, 1).repeat_interleave(4, dim=0)
        vt = torch.from_numpy(v).transpose(0, 1).repeat_interleave(4, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt.contiguous(), vt.contiguous(), attn_mask=mask, scale=0.37)
        np.testing.assert_allclose(o[q0:q1], ref.transpose(0, 1).numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------ closed forms ----

def test_window_zero_returns_own_value():
    case = synth.attention_case(3, [40], [70], num_qo_heads=4, num_kv_heads=2, head_dim=32,
                                page_size=16, num_pages=8)
    o = _run(case, sm_scale=1.0, window_left=0)
    (k, v), = _logical_kv(case)
    pos = 70 - 40 + np.arange(40)
    for h in range(4):
        np.testing.assert_array_equal(o[:, h], v[pos, h // 2])


@pytest.mark.parametrize("wl", [-1, 0, 1, 5, 15, 16, 17, 63])
def test_uniform_weights_reveal_inclusive_window(wl):
    """sm_scale = 0 makes every allowed key weigh the same; with one-hot values
    (V[j] = e_j) the output lists the attended keys: exactly the window_left + 1
    most recent positions (all earlier ones when window_left = -1)."""
    kv, qo, d = 64, 24, 64
    case = synth.attention_case(11, [qo], [kv], num_qo_heads=2, num_kv_heads=1, head_dim=d,
                                page_size=16, num_pages=4)
    g = _geom(case)
    bits = oracle.bf16_bits(case.pool).copy()
    ids = case.table.kv_page_indices
    one = np.uint16(0x3F80)   # bf16 1.0
    for j in range(kv):
        bits[_flat_v(g, 0, ids[j // 16], 0, np.arange(d), j % 16)] = 0
        bits[_flat_v(g, 0, ids[j // 16], 0, j, j % 16)] = one
    o = _run(case, sm_scale=0.0, window_left=wl, pool=bits)
    for i in range(qo):
        p = kv - qo + i
        lo = 0 if wl < 0 else max(0, p - wl)
        want = np.zeros(d)
        want[lo:p + 1] = 1.0 / (p + 1 - lo)
        for h in range(2):
            np.testing.assert_allclose(o[i, h], want, rtol=0, atol=1e-15)


def test_constant_values_give_constant_output():
    case = synth.attention_case(5, [30, 9], [45, 9], num_qo_heads=4, num_kv_heads=4,
                                head_dim=16, page_size=8, num_pages=9)
    g = _geom(case)
    bits = oracle.bf16_bits(case.pool).copy()
    bits.reshape(g.num_layers, g.num_pages, 2, -1)[:, :, 1] = np.uint16(0x3FC0)  # 1.5 in V
    o = _run(case, sm_scale=2.0, window_left=7, pool=bits)
    np.testing.assert_allclose(o, 1.5, rtol=0, atol=1e-14)


# -------------------------------------------------------------- invariants ----

def test_page_permutation_invariance():
    """Moving every page to another physical slot of the pool (and remapping the
    table) changes nothing: paging is pure addressing."""
    case = synth.attention_case(21, [37, 64, 5], [100, 64, 77], num_qo_heads=4,
                                num_kv_heads=2, head_dim=32, page_size=16, num_pages=40)
    base = _run(case, window_left=20)
    g = _geom(case)
    bits = oracle.bf16_bits(case.pool).reshape(g.num_layers, g.num_pages, -1)
    perm = np.random.default_rng(0).permutation(g.num_pages)
    moved = np.empty_like(bits)
    moved[:, perm] = bits                  # page p now lives at perm[p]
    t = case.table
    t2 = synth.PageTable(t.kv_page_indptr, perm[t.kv_page_indices].astype(np.int32),
                         t.kv_last_page_len)
    out = _run(case, window_left=20, pool=moved.reshape(-1), table=t2)
    np.testing.assert_array_equal(out, base)


def test_saturated_window_equals_full_causal():
    case = synth.attention_case(8, [50, 3], [90, 40], num_qo_heads=4, num_kv_heads=1,
                                head_dim=16, page_size=16, num_pages=10)
    full = _run(case, window_left=-1)
    for wl in (89, 90, 1000, 10 ** 6):
        np.testing.assert_array_equal(_run(case, window_left=wl), full)
    assert not np.array_equal(_run(case, window_left=88), full)


def test_gqa_replicated_heads():
    """Copying KV head g into heads g*group .. g*group+group-1 and running with
    one query head per KV head reproduces the grouped result (the group is the
    integer quotient H_q / H_kv, heads taken in contiguous blocks)."""
    group, h_kv = 4, 2
    case = synth.attention_case(31, [20], [45], num_qo_heads=group * h_kv, num_kv_heads=h_kv,
                                head_dim=16, page_size=16, num_pages=3)
    base = _run(case, sm_scale=0.8, window_left=9)
    g = _geom(case)
    kb, vb = oracle.kv_blocks(case.pool, g)
    kr = np.repeat(kb, group, axis=2).reshape(g.num_layers, g.num_pages, 1, -1)
    vr = np.repeat(vb, group, axis=2).reshape(g.num_layers, g.num_pages, 1, -1)
    rep = np.concatenate([kr, vr], axis=2)
    g2 = oracle.PoolGeometry(g.num_layers, g.num_pages, h_kv * group, g.page_size, g.head_dim)
    t = case.table
    out = oracle.paged_attention(case.q, rep.reshape(-1), g2, 0, case.qo_indptr,
                                 t.kv_page_indptr, t.kv_page_indices, t.kv_last_page_len,
                                 0.8, 9)
    np.testing.assert_array_equal(out, base)


@pytest.mark.parametrize("wl", [-1, 6])
def test_decode_equals_prefill_row(wl):
    """A one-token call whose KV ends at position p gives row p of the prefill
    over the same pages (decode runs through the prefill entry at one token)."""
    kv = 40
    case = synth.attention_case(41, [kv], [kv], num_qo_heads=2, num_kv_heads=1, head_dim=16,
                                page_size=8, num_pages=5)
    full = _run(case, sm_scale=1.0, window_left=wl)
    ids = case.table.kv_page_indices
    for p in (0, 7, 8, 9, 39):
        n_pages = p // 8 + 1
        t = synth.PageTable(np.array([0, n_pages], np.int32), ids[:n_pages].copy(),
                            np.array([p - (n_pages - 1) * 8 + 1], np.int32))
        q1 = case.q[p:p + 1]
        o = oracle.paged_attention(q1, case.pool, _geom(case), 0, np.array([0, 1], np.int32),
                                   t.kv_page_indptr, t.kv_page_indices, t.kv_last_page_len,
                                   1.0, wl)
        np.testing.assert_allclose(o[0], full[p], rtol=0, atol=1e-13)


def test_sampled_rows_match_full():
    case = synth.attention_case(55, [30, 12], [30, 50], num_qo_heads=4, num_kv_heads=2,
                                head_dim=16, page_size=16, num_pages=6)
    full = _run(case, window_left=10)
    samples = [(0, 0), (29, 3), (30, 1), (41, 2)]
    part = _run(case, window_left=10, samples=samples)
    for tok, h in samples:
        np.testing.assert_allclose(part[tok, h], full[tok, h], rtol=0, atol=1e-13)


def test_unused_pages_and_tail_slots_are_never_read():
    """NaN in pages outside the table and in slots past last_page_len leaves the
    output unchanged."""
    case = synth.attention_case(61, [20, 7], [37, 7], num_qo_heads=2, num_kv_heads=1,
                                head_dim=16, page_size=16, num_pages=8)
    base = _run(case, window_left=-1)
    g = _geom(case)
    bits = oracle.bf16_bits(case.pool).copy()
    used = set(case.table.kv_page_indices.tolist())
    by_page = bits.reshape(g.num_layers, g.num_pages, -1)
    for p in range(g.num_pages):
        if p not in used:
            by_page[:, p] = np.uint16(0x7FA5)
    t = case.table
    for b in range(2):
        last_page = t.kv_page_indices[t.kv_page_indptr[b + 1] - 1]
        for slot in range(t.kv_last_page_len[b], g.page_size):
            for hh in range(g.num_kv_heads):
                bits[_flat_k(g, 0, last_page, hh, slot, np.arange(g.head_dim))] = np.uint16(0x7FA5)
                bits[_flat_v(g, 0, last_page, hh, np.arange(g.head_dim), slot)] = np.uint16(0x7FA5)
    out = _run(case, window_left=-1, pool=bits)
    np.testing.assert_array_equal(out, base)


def test_rejects_bad_window():
    case = synth.attention_case(1, [2], [2], num_qo_heads=1, num_kv_heads=1, head_dim=4,
                                page_size=2, num_pages=1)
    with pytest.raises(ValueError):
        _run(case, window_left=-2)


# ------------------------------------------------------ resident windows ----

def _ring_fixture(seed, kv, qo, ring_pages, window_left, page_size=16, heads=(4, 2), d=32):
    """An unwrapped pool holding positions 0..kv-1 and a ring of ring_pages
    pages holding the last ring_pages * P of them, copied position by position
    with this test's own index formula (ring page (p // P) mod n, slot p mod P)."""
    rng = np.random.default_rng(seed)
    hq, hkv = heads
    n_full = (kv + page_size - 1) // page_size
    num_pages = n_full + ring_pages
    g = oracle.PoolGeometry(1, num_pages, hkv, page_size, d)
    bits = oracle.f64_to_bf16_bits(rng.normal(0, 0.5, g.numel))
    kb, vb = oracle.kv_blocks(bits, g)
    full_ids = np.arange(n_full)
    ring_ids = n_full + rng.permutation(ring_pages)
    first = kv - ring_pages * page_size
    for p in range(max(first, 0), kv):
        src, dst = full_ids[p // page_size], ring_ids[(p // page_size) % ring_pages]
        kb[0, dst, :, p % page_size, :] = kb[0, src, :, p % page_size, :]
        vb[0, dst, :, :, p % page_size] = vb[0, src, :, :, p % page_size]
    q = oracle.f64_to_bf16_bits(rng.normal(0, 0.5, (qo, hq, d)))
    return g, bits, q, full_ids, ring_ids


@pytest.mark.parametrize("kv,qo,ring,wl", [(300, 40, 10, 100), (300, 1, 8, 127), (1000, 17, 9, 120),
                                           (160, 20, 10, 140)])
def test_ring_attention_equals_the_unwrapped_cache(kv, qo, ring, wl):
    g, bits, q, full_ids, ring_ids = _ring_fixture(kv + qo, kv, qo, ring, wl)
    n_full = len(full_ids)
    full = oracle.paged_attention(q, bits, g, 0, [0, qo], [0, n_full], full_ids,
                                  [kv - (n_full - 1) * 16], 0.3, wl)
    wrapped = oracle.paged_attention(q, bits, g, 0, [0, qo], [0, ring], ring_ids,
                                     [(kv - 1) % 16 + 1], 0.3, wl, kv_len=[kv])
    np.testing.assert_allclose(wrapped, full, rtol=0, atol=1e-14)


def test_ring_refuses_a_key_it_no_longer_holds():
    g, bits, q, _, ring_ids = _ring_fixture(5, 300, 40, 10, 100)
    with pytest.raises(ValueError):      # window 121 + 40 queries need 161 > 160 slots
        oracle.paged_attention(q, bits, g, 0, [0, 40], [0, 10], ring_ids, [12], 1.0, 121,
                               kv_len=[300])
    with pytest.raises(ValueError):      # no window at all
        oracle.paged_attention(q, bits, g, 0, [0, 40], [0, 10], ring_ids, [12], 1.0, -1,
                               kv_len=[300])


def test_ring_placement_of_prep_writes():
    """Positions 290..309 of a 10-page ring land in ring page (p // 16) mod 10,
    slot p mod 16."""
    g = oracle.PoolGeometry(2, 40, 1, 16, 8)
    ids = np.array([7, 3, 31, 0, 12, 5, 9, 22, 18, 1])
    page, slot = oracle.expected_pool_writes(g, 1, [0, 20], [0, 10], ids, [(310 - 1) % 16 + 1],
                                             kv_len=[310])
    p = np.arange(290, 310)
    np.testing.assert_array_equal(page, ids[(p // 16) % 10])
    np.testing.assert_array_equal(slot, p % 16)
