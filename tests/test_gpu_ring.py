"""Resident windows (a ring of pages per request, §8(f) f1) on cuda:0.

Contract: once a request's absolute KV length exceeds its pages, the pages
hold only its last n_pages * page_size positions, position p in page
(p // P) mod n_pages, slot p mod P (issue "gemma4: serving prep needs
pool-write forms", Proposed Plan: once the window has wrapped, a position
and its cache slot differ and need their own map).  Masks and RoPE stay absolute.  Checked
against the fp64 oracle, whose ring map is pinned on the CPU against an
unwrapped copy of the same cache: windowed prefill and decode (both forms)
over wrapped and unwrapped requests in one batch, and the prep writing a
step through the ring (placement bit for bit) followed by attention over it.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import paged_sliding_window_page_amd as psw
from gpu_util import SENTINEL, check_close, say, to_np64

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _ring_case(seed, qo, kv, ring, num_pages=None, d=256, hkv=8):
    gen = synth.generator(seed)
    need = sum(min((k + 15) // 16, r) for k, r in zip(kv, ring))
    num_pages = num_pages or need + 3
    table = synth.ring_page_table(kv, ring, 16, num_pages, gen)
    q = synth.normal_bf16((sum(qo), 16, d), 0.25, gen)
    numel = synth.pool_numel(1, num_pages, hkv, 16, d)
    pool = synth.normal_bf16((numel,), 0.25, gen)
    g = oracle.PoolGeometry(1, num_pages, hkv, 16, d)
    return g, table, q, pool, synth.lengths_to_indptr(qo)


def _plan(g, table, qo_indptr, kv, hkv=8, d=256):
    return psw.Plan(qo_indptr, table.kv_page_indptr, table.kv_page_indices,
                    table.kv_last_page_len, num_qo_heads=16, num_kv_heads=hkv, head_dim=d,
                    page_size=16, num_pages=g.num_pages, kv_len=kv)


def _attend(g, table, qo_indptr, kv, q, pool, wl, mode=None, decode=False):
    plan = _plan(g, table, qo_indptr, kv)
    if mode is not None:
        plan.set_decode_mode(mode)
    pool_d = pool.to(DEV) if pool.device.type == "cpu" else pool
    pd = psw.pool_desc(pool_d, num_layers=1, num_pages=g.num_pages, page_size=16,
                       num_kv_heads=g.num_kv_heads, head_dim=g.head_dim)
    o = torch.full((q.shape[0], 16, g.head_dim), float("nan"), dtype=torch.bfloat16, device=DEV)
    if decode:
        psw.paged_decode_window_hd256(plan, pd, 0, q.to(DEV), 1.0, wl, o)
    else:
        psw.paged_prefill_window_hd256(plan, pd, 0, q.to(DEV), 1.0, wl, o)
    torch.cuda.synchronize()
    plan.close()
    return to_np64(o)


@pytest.mark.parametrize("wl,qo,kv,ring", [
    (1023, [100, 37, 1, 64], [3000, 500, 2000, 1200], [72, 40, 66, 75]),
    (255, [16, 33, 9], [4000, 290, 777], [18, 19, 17]),
    (127, [128, 5], [1000, 640], [16, 9]),
])
def test_ring_prefill_matches_oracle(wl, qo, kv, ring):
    g, table, q, pool, qi = _ring_case(7 + wl, qo, kv, ring)
    say(f"[gpu] ring prefill wl={wl} qo={qo} kv={kv} ring={ring}")
    gpu = _attend(g, table, qi, kv, q, pool, wl)
    ref = oracle.paged_attention(q, pool, g, 0, qi, table.kv_page_indptr, table.kv_page_indices,
                                 table.kv_last_page_len, 1.0, wl, kv_len=kv)
    check_close(gpu, ref, f"ring prefill wl={wl}")


@pytest.mark.parametrize("mode", [psw.DECODE_SPLIT, psw.DECODE_DIRECT, psw.DECODE_AUTO])
def test_ring_decode_matches_oracle(mode):
    kv = [5000, 1500, 1024, 700, 3333, 64]
    ring = [65, 64, 70, 100, 64, 4]
    qo = [1] * len(kv)
    g, table, q, pool, qi = _ring_case(21 + mode, qo, kv, ring)
    say(f"[gpu] ring decode mode={mode} kv={kv} ring={ring}")
    gpu = _attend(g, table, qi, kv, q, pool, 1023, mode=mode, decode=True)
    ref = oracle.paged_attention(q, pool, g, 0, qi, table.kv_page_indptr, table.kv_page_indices,
                                 table.kv_last_page_len, 1.0, 1023, kv_len=kv)
    check_close(gpu, ref, f"ring decode mode {mode}")


def test_ring_prep_then_attention():
    """A step of 50 tokens at positions 1950..1999 written through a 70-page
    ring (it overwrites positions 830..879), then windowed attention over it."""
    qo, kv, ring = [50, 20], [2000, 300], [70, 30]
    g, table, _, _, qi = _ring_case(31, qo, kv, ring, d=256)
    gen = synth.generator(32)
    q_in = synth.normal_bf16((70, 16, 256), 1.0, gen)
    k_in = synth.normal_bf16((70, 8, 256), 1.0, gen)
    v_in = synth.normal_bf16((70, 8, 256), 1.0, gen)
    wq = synth.normal_bf16((256,), 0.1, gen, mean=1.0)
    wk = synth.normal_bf16((256,), 0.1, gen, mean=1.0)
    # a pool with every slot holding a valid older value
    pool = synth.normal_bf16((g.numel,), 0.5, gen).to(DEV)
    before = pool.view(torch.int16).clone()
    c = torch.empty(4096, 128, dtype=torch.float32, device=DEV)
    s = torch.empty_like(c)
    psw.rope_tables(c, s, 4096, 256, 1e4)
    plan = _plan(g, table, qi, kv)
    pd = psw.pool_desc(pool, num_layers=1, num_pages=g.num_pages, page_size=16, num_kv_heads=8,
                       head_dim=256)
    q_out = torch.empty(70, 16, 256, dtype=torch.bfloat16, device=DEV)
    say("[gpu] ring prep + attention")
    psw.qkv_norm_rope_paged_prefill_hd256(plan, pd, 0, q_in.to(DEV), k_in.to(DEV), v_in.to(DEV),
                                          wq.to(DEV), wk.to(DEV), c, s, 1e-6, q_out)
    o = torch.full((70, 16, 256), float("nan"), dtype=torch.bfloat16, device=DEV)
    psw.paged_prefill_window_hd256(plan, pd, 0, q_out, 1.0, 1023, o)
    torch.cuda.synchronize()
    plan.device_errors()
    plan.close()
    pos = oracle.token_positions(qi, table.kv_page_indptr, table.kv_last_page_len, 16, kv)
    q_ref, k_ref, v_ref = oracle.qkv_prep_hd256(q_in, k_in, v_in, wq, wk, pos, 1e-6, 1e4)
    check_close(to_np64(q_out), q_ref, "ring prep Q")
    page, slot = oracle.expected_pool_writes(g, 0, qi, table.kv_page_indptr,
                                             table.kv_page_indices, table.kv_last_page_len, kv)
    b_bits = before.cpu().numpy().view(np.uint16)
    expect = oracle.bits_to_f64(b_bits)
    mask = oracle.apply_pool_writes(expect, g, 0, page, slot, k_ref, v_ref)
    after = pool.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(after[~mask], b_bits[~mask])
    say(f"  placement exact: {int(mask.sum())} elements written through the ring")
    check_close(oracle.bits_to_f64(after[mask]), expect[mask], "ring prep K/V")
    ref = oracle.paged_attention(q_out.cpu(), after, g, 0, qi, table.kv_page_indptr,
                                 table.kv_page_indices, table.kv_last_page_len, 1.0, 1023,
                                 kv_len=kv)
    check_close(to_np64(o), ref, "ring attention after prep")
