"""Two-family page accounting on the host (no GPU).

Contract (PR "feat(gemma4): paged KV serving across both attention families",
Description and Verification; its review thread on when the frontier may
move): each family has its own pool; a step needs the ceiling of its
post-step KV length over the page size, less the pages already held; both
families are reserved before anything is kept, and when one side cannot be
granted the other is handed back, leaving both pools as they were; every
bound (window, RoPE tables, matching frontiers) is checked before any state
changes; a request is only valid against its own server; the frontier moves
on commit and nowhere else.
"""
import math

import numpy as np
import pytest

import paged_sliding_window_page_amd as psw


def _code(fn):
    with pytest.raises(psw.PswError) as e:
        fn()
    return e.value.status


def _server(**kw):
    a = dict(local_pages=64, global_pages=64, window_left=-1, rope_positions=4096)
    a.update(kw)
    return psw.KvServer(**a)


def _tables(srv, reqs, fam):
    return srv.step_tables(reqs, fam)[:4]


def test_admit_commit_counts_pages_as_ceilings():
    srv = _server()
    r = srv.request()
    srv.admit(r, 40)                      # ceil(40/16) = 3 pages per family
    st = r.state()
    assert (st.frontier, st.pending, st.pending_tokens) == (0, 1, 40)
    assert (st.local_reserved, st.global_reserved) == (3, 3)
    assert srv.free_pages() == (61, 61)
    srv.commit(r)
    st = r.state()
    assert (st.frontier, st.local_held, st.global_held, st.pending) == (40, 3, 3, 0)
    # decode steps: a page only when the KV length crosses a multiple of 16
    for kv in range(41, 50):
        srv.admit(r, 1)
        want = math.ceil(kv / 16) - r.state().local_held
        assert r.state().local_reserved == want and r.state().global_reserved == want
        srv.commit(r)
    assert r.state().frontier == 49 and r.state().local_held == 4
    srv.release(r)
    assert srv.free_pages() == (64, 64)
    srv.close()


def test_different_page_sizes_per_family():
    srv = _server(local_page_size=16, global_page_size=32)
    r = srv.request()
    srv.admit(r, 33)
    assert (r.state().local_reserved, r.state().global_reserved) == (3, 2)
    srv.commit(r)
    srv.release(r)
    srv.close()


def test_refused_global_side_leaves_both_pools_untouched():
    """A forced partial failure: the local pool can grant the step, the global
    pool cannot; both pools end exactly as before (same free ids, same order)."""
    srv = _server(local_pages=10, global_pages=4)
    a = srv.request()
    srv.admit(a, 32)                       # 2 + 2 pages
    srv.commit(a)
    before = srv.free_pages()
    assert before == (8, 2)
    b = srv.request()
    assert _code(lambda: srv.admit(b, 40)) == "PSW_E_RANGE"   # needs 3 + 3
    assert srv.free_pages() == before
    st = b.state()
    assert (st.frontier, st.pending, st.local_held, st.global_held) == (0, 0, 0, 0)
    # the ids a fitting step now gets are the ones it would have got before
    c = srv.request()
    srv.admit(c, 32)
    qo, kvp, idx_l, last = _tables(srv, [c], psw.KV_LOCAL)
    assert list(idx_l) == [2, 3]           # 0, 1 went to request a
    srv.abort(c)
    for r in (a, b, c):
        srv.release(r)
    assert srv.free_pages() == (10, 4)
    srv.close()


def test_refused_local_side_takes_nothing():
    srv = _server(local_pages=2, global_pages=10)
    r = srv.request()
    assert _code(lambda: srv.admit(r, 40)) == "PSW_E_RANGE"
    assert srv.free_pages() == (2, 10)
    srv.release(r)
    srv.close()


def test_abort_returns_the_reservation_and_keeps_the_frontier():
    srv = _server()
    r = srv.request()
    srv.admit(r, 20)
    srv.commit(r)
    srv.admit(r, 20)                       # 40 -> 3 pages: one more each
    qo, kvp, idx, last = _tables(srv, [r], psw.KV_GLOBAL)
    assert list(qo) == [0, 20] and list(last) == [8]
    srv.abort(r)                           # the step failed
    st = r.state()
    assert (st.frontier, st.local_held, st.pending) == (20, 2, 0)
    assert srv.free_pages() == (62, 62)
    # a retry sees the same start position and gets the same page
    srv.admit(r, 20)
    _, _, idx2, _ = _tables(srv, [r], psw.KV_GLOBAL)
    np.testing.assert_array_equal(idx, idx2)
    srv.commit(r)
    assert r.state().frontier == 40
    srv.release(r)
    srv.close()


def test_window_and_rope_bounds_checked_before_anything_moves():
    srv = _server(window_left=31, rope_positions=1000)
    r = srv.request()
    assert _code(lambda: srv.admit(r, 33)) == "PSW_E_RANGE"    # would cross the window
    assert srv.free_pages() == (64, 64) and r.state().pending == 0
    srv.admit(r, 32)                                           # exactly the window
    srv.commit(r)
    assert _code(lambda: srv.admit(r, 1)) == "PSW_E_RANGE"
    srv.release(r)
    srv2 = _server(rope_positions=50)
    r2 = srv2.request()
    assert _code(lambda: srv2.admit(r2, 51)) == "PSW_E_RANGE"
    srv2.admit(r2, 50)
    srv2.commit(r2)
    srv2.release(r2)
    srv.close()
    srv2.close()


def test_request_of_another_server_is_rejected():
    s1, s2 = _server(), _server()
    r = s1.request()
    assert _code(lambda: s2.admit(r, 4)) == "PSW_E_PLAN"
    assert _code(lambda: s2.release(r)) == "PSW_E_PLAN"
    s1.admit(r, 4)
    assert _code(lambda: s2.step_tables([r], psw.KV_LOCAL)) == "PSW_E_PLAN"
    s1.commit(r)
    s1.release(r)
    s1.close()
    s2.close()


def test_pending_step_rules():
    srv = _server()
    r = srv.request()
    assert _code(lambda: srv.commit(r)) == "PSW_E_PLAN"
    assert _code(lambda: srv.abort(r)) == "PSW_E_PLAN"
    assert _code(lambda: srv.admit(r, 0)) == "PSW_E_SHAPE"
    srv.admit(r, 3)
    assert _code(lambda: srv.admit(r, 3)) == "PSW_E_PLAN"
    q = srv.request()
    assert _code(lambda: srv.step_tables([r, q], psw.KV_LOCAL)) == "PSW_E_PLAN"   # q has none
    assert _code(lambda: srv.step_tables([r, r], psw.KV_LOCAL)) == "PSW_E_SHAPE"
    assert _code(lambda: srv.step_tables([r], 2)) == "PSW_E_SHAPE"
    # a server with live requests refuses to go away
    assert _code(lambda: srv.close()) == "PSW_E_PLAN"
    srv.release(r)                         # releases the reservation too
    srv.release(q)
    assert srv.free_pages() == (64, 64)
    srv.close()


def test_server_desc_rejects():
    for kw, status in ((dict(local_pages=0), "PSW_E_SHAPE"),
                       (dict(global_page_size=0), "PSW_E_SHAPE"),
                       (dict(window_left=-2), "PSW_E_RANGE"),
                       (dict(rope_positions=0), "PSW_E_SHAPE"),
                       (dict(local_pages=1 << 31), "PSW_E_OVERFLOW")):
        assert _code(lambda: _server(**kw)) == status


def test_batch_tables_are_valid_plan_metadata():
    """Several requests at different frontiers: the tables describe every
    request's KV after the step, pages disjoint across requests, and a plan
    accepts them."""
    srv = _server(local_pages=200, global_pages=200)
    rng = np.random.default_rng(7)
    reqs = [srv.request() for _ in range(5)]
    for r in reqs:
        srv.admit(r, int(rng.integers(1, 100)))
        srv.commit(r)
    steps = [int(rng.integers(1, 40)) for _ in reqs]
    for r, n in zip(reqs, steps):
        srv.admit(r, n)
    for fam in (psw.KV_LOCAL, psw.KV_GLOBAL):
        qo, kvp, idx, last = _tables(srv, reqs, fam)
        assert list(np.diff(qo)) == steps
        assert len(set(idx.tolist())) == len(idx)                 # no page in two requests
        for b, r in enumerate(reqs):
            st = r.state()
            kv = st.frontier + st.pending_tokens
            npg = kvp[b + 1] - kvp[b]
            assert npg == math.ceil(kv / 16)
            assert (npg - 1) * 16 + last[b] == kv and 1 <= last[b] <= 16
        plan = psw.Plan(qo, kvp, idx, last, num_qo_heads=16, num_kv_heads=8 if fam == 0 else 1,
                        head_dim=256 if fam == 0 else 512, page_size=16, num_pages=200,
                        stream=0)
        info = plan.info()
        assert info["total_qo"] == sum(steps)
        plan.close()
    for r in reqs:
        srv.commit(r)
        srv.release(r)
    assert srv.free_pages() == (200, 200)
    srv.close()


def test_local_ring_keeps_at_most_its_pages():
    """With a local ring of 4 pages (64 slots) and window 31 the local family
    stops growing at 4 pages and the KV length runs past the window; the
    global family keeps every page."""
    srv = _server(window_left=31, local_ring_pages=4)
    r = srv.request()
    srv.admit(r, 40)
    assert (r.state().local_reserved, r.state().global_reserved) == (3, 3)
    srv.commit(r)
    srv.admit(r, 30)                                  # post 70: local 4 (ring), global 5
    assert (r.state().local_reserved, r.state().global_reserved) == (1, 2)
    qo, kvp, idx, last, kvl = srv.step_tables([r], psw.KV_LOCAL)
    assert list(kvl) == [70] and list(last) == [(70 - 1) % 16 + 1] and kvp[-1] == 4
    plan = psw.Plan(qo, kvp, idx, last, num_qo_heads=16, num_kv_heads=8, head_dim=256,
                    page_size=16, num_pages=64, stream=0, kv_len=kvl)
    assert plan.info()["max_kv_len"] == 70
    plan.close()
    srv.commit(r)
    srv.admit(r, 30)                                  # post 100: no new local page
    assert (r.state().local_reserved, r.state().global_reserved) == (0, 2)
    srv.commit(r)
    assert (r.state().frontier, r.state().local_held, r.state().global_held) == (100, 4, 7)
    # window 31 + 34 queries need 65 slots: the ring holds 64
    assert _code(lambda: srv.admit(r, 34)) == "PSW_E_RANGE"
    srv.admit(r, 33)
    srv.abort(r)
    srv.release(r)
    assert srv.free_pages() == (64, 64)
    srv.close()


def test_local_ring_needs_a_window():
    assert _code(lambda: _server(window_left=-1, local_ring_pages=4)) == "PSW_E_RANGE"
    assert _code(lambda: _server(window_left=10, local_ring_pages=-1)) == "PSW_E_RANGE"
