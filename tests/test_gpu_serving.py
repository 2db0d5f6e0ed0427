"""Both KV families served through two steps (prefill, then one decode token)
with page tables issued by the two-family accounting, on cuda:0.

Contract (PR "feat(gemma4): paged KV serving across both attention families",
Description): each family with its own pool, a request holding pages in both; each
step's prep writes the new tokens at their absolute positions through the
step's tables and attention reads the whole KV back; decode is the prefill
entry at one token; the frontier moves only after the step.  Checked per step
and family: the pool holds the oracle's prep rows at the oracle's placement
(bit for bit outside the written slots) and attention over that pool matches
the oracle.
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

PAGES = 48
LAYERS, LAYER = 2, 1
WINDOW = 127          # local window (inclusive distance), KV stays within 128 keys
FAM = {psw.KV_LOCAL: dict(d=256, hkv=8), psw.KV_GLOBAL: dict(d=512, hkv=1)}


def _tables(positions, d):
    c = torch.empty(positions, d // 2, dtype=torch.float32, device=DEV)
    s = torch.empty_like(c)
    psw.rope_tables(c, s, positions, d, 1e4)
    return c, s


def _geom(fam):
    return oracle.PoolGeometry(LAYERS, PAGES, FAM[fam]["hkv"], 16, FAM[fam]["d"])


def _inputs(tokens, seed):
    g = synth.generator(seed)
    x = {}
    x["q256"] = synth.normal_bf16((tokens, 16, 256), 1.0, g)
    x["k256"] = synth.normal_bf16((tokens, 8, 256), 1.0, g)
    x["v256"] = synth.normal_bf16((tokens, 8, 256), 1.0, g)
    x["q512"] = synth.normal_bf16((tokens, 16, 512), 1.0, g)
    x["k512"] = synth.normal_bf16((tokens, 1, 512), 1.0, g)
    return x


def test_two_families_prefill_then_decode():
    srv = psw.KvServer(PAGES, PAGES, window_left=WINDOW, rope_positions=256)
    reqs = [srv.request(), srv.request()]
    w = {k: synth.normal_bf16((d,), 0.1, synth.generator(900 + d), mean=1.0)
         for k, d in (("wq256", 256), ("wk256", 256), ("wq512", 512), ("wk512", 512))}
    w_dev = {k: v.to(DEV) for k, v in w.items()}
    tabs = {256: _tables(256, 256), 512: _tables(256, 512)}
    pools = {}
    for fam in FAM:
        g = _geom(fam)
        pools[fam] = torch.full((g.numel,), SENTINEL, dtype=torch.int16,
                                device=DEV).view(torch.bfloat16)
    for step, new in enumerate(([70, 101], [1, 1])):
        for r, n in zip(reqs, new):
            srv.admit(r, n)
        x = _inputs(sum(new), 910 + step)
        for fam, geo in FAM.items():
            d, hkv = geo["d"], geo["hkv"]
            g = _geom(fam)
            qo, kvp, idx, last, _ = srv.step_tables(reqs, fam)
            say(f"[gpu] serving step {step} family {d}: qo {np.diff(qo).tolist()} "
                f"pages {np.diff(kvp).tolist()}")
            plan = psw.Plan(qo, kvp, idx, last, num_qo_heads=16, num_kv_heads=hkv, head_dim=d,
                            page_size=16, num_pages=PAGES)
            pd = psw.pool_desc(pools[fam], num_layers=LAYERS, num_pages=PAGES, page_size=16,
                               num_kv_heads=hkv, head_dim=d)
            before = pools[fam].view(torch.int16).clone()
            c, s = tabs[d]
            q_out = torch.empty(sum(new), 16, d, dtype=torch.bfloat16, device=DEV)
            if d == 256:
                psw.qkv_norm_rope_paged_prefill_hd256(
                    plan, pd, LAYER, x["q256"].to(DEV), x["k256"].to(DEV), x["v256"].to(DEV),
                    w_dev["wq256"], w_dev["wk256"], c, s, 1e-6, q_out)
            else:
                psw.k_v_norm_rope_paged_prefill_hd512(plan, pd, LAYER, x["k512"].to(DEV),
                                                      w_dev["wk512"], c, s, 1e-6)
                psw.q_norm_rope_prefill_hd512(plan, x["q512"].to(DEV), w_dev["wq512"], c, s,
                                              1e-6, q_out)
            o = torch.full((sum(new), 16, d), float("nan"), dtype=torch.bfloat16, device=DEV)
            if d == 256:
                psw.paged_prefill_window_hd256(plan, pd, LAYER, q_out, 1.0, WINDOW, o)
            else:
                psw.paged_prefill_hd512(plan, pd, LAYER, q_out, 1.0, o)
            torch.cuda.synchronize()
            plan.device_errors()
            plan.close()
            # the pool: oracle rows at the oracle's placement, nothing else touched
            pos = oracle.token_positions(qo, kvp, last, 16)
            if d == 256:
                q_ref, k_ref, v_ref = oracle.qkv_prep_hd256(x["q256"], x["k256"], x["v256"],
                                                            w["wq256"], w["wk256"], pos, 1e-6, 1e4)
            else:
                k_ref, v_ref = oracle.kv_prep_hd512(x["k512"], w["wk512"], pos, 1e-6, 1e4)
                q_ref = oracle.q_prep_hd512(x["q512"], w["wq512"], pos, 1e-6, 1e4)
            check_close(to_np64(q_out), q_ref, f"step {step} Q hd{d}")
            page, slot = oracle.expected_pool_writes(g, LAYER, qo, kvp, idx, last)
            expect = oracle.bits_to_f64(before.cpu().numpy().view(np.uint16))
            mask = oracle.apply_pool_writes(expect, g, LAYER, page, slot, k_ref, v_ref)
            after = pools[fam].view(torch.int16).cpu().numpy().view(np.uint16)
            np.testing.assert_array_equal(after[~mask], before.cpu().numpy().view(np.uint16)[~mask])
            check_close(oracle.bits_to_f64(after[mask]), expect[mask], f"step {step} K/V hd{d}")
            # attention over the pool as written, from the queries as written
            ref = oracle.paged_attention(q_out.cpu(), after, g, LAYER, qo, kvp, idx, last, 1.0,
                                         WINDOW if d == 256 else -1)
            check_close(to_np64(o), ref, f"step {step} attention hd{d}")
        for r in reqs:
            srv.commit(r)
        assert [r.state().frontier for r in reqs] == [sum(n[i] for n in ([70, 101], [1, 1])[:step + 1]) for i in range(2)]
    for r in reqs:
        srv.release(r)
    assert srv.free_pages() == (PAGES, PAGES)
    srv.close()


def test_local_family_runs_past_its_window_through_a_ring():
    """The local family with a ring of 10 pages (160 slots) and window 127:
    a 100-token prefill, four 20-token steps (the KV runs to 180 and wraps),
    then two decode steps, each written by the prep through the step's tables
    and read back by windowed attention; every step against the oracle."""
    srv = psw.KvServer(64, 64, window_left=127, rope_positions=512, local_ring_pages=10)
    r = srv.request()
    wq = synth.normal_bf16((256,), 0.1, synth.generator(940), mean=1.0)
    wk = synth.normal_bf16((256,), 0.1, synth.generator(941), mean=1.0)
    c, s = _tables(512, 256)
    g = oracle.PoolGeometry(1, 64, 8, 16, 256)
    pool = torch.full((g.numel,), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    pd = psw.pool_desc(pool, num_layers=1, num_pages=64, page_size=16, num_kv_heads=8,
                       head_dim=256)
    for step, n in enumerate([100, 20, 20, 20, 20, 1, 1]):
        srv.admit(r, n)
        qo, kvp, idx, last, kvl = srv.step_tables([r], psw.KV_LOCAL)
        say(f"[gpu] ring serving step {step}: n={n} kv={int(kvl[0])} pages={int(kvp[-1])}")
        gen = synth.generator(950 + step)
        q_in = synth.normal_bf16((n, 16, 256), 1.0, gen)
        k_in = synth.normal_bf16((n, 8, 256), 1.0, gen)
        v_in = synth.normal_bf16((n, 8, 256), 1.0, gen)
        plan = psw.Plan(qo, kvp, idx, last, num_qo_heads=16, num_kv_heads=8, head_dim=256,
                        page_size=16, num_pages=64, kv_len=kvl)
        q_out = torch.empty(n, 16, 256, dtype=torch.bfloat16, device=DEV)
        psw.qkv_norm_rope_paged_prefill_hd256(plan, pd, 0, q_in.to(DEV), k_in.to(DEV),
                                              v_in.to(DEV), wq.to(DEV), wk.to(DEV), c, s, 1e-6,
                                              q_out)
        o = torch.full((n, 16, 256), float("nan"), dtype=torch.bfloat16, device=DEV)
        psw.paged_prefill_window_hd256(plan, pd, 0, q_out, 1.0, 127, o)
        torch.cuda.synchronize()
        plan.device_errors()
        plan.close()
        after = pool.view(torch.int16).cpu().numpy().view(np.uint16)
        ref = oracle.paged_attention(q_out.cpu(), after, g, 0, qo, kvp, idx, last, 1.0, 127,
                                     kv_len=kvl)
        check_close(to_np64(o), ref, f"ring serving step {step}")
        srv.commit(r)
    assert r.state().frontier == 182 and r.state().local_held == 10
    srv.release(r)
    srv.close()
