"""Host-side boundary tests (no GPU needed): the C-ABI library loads, exports
every symbol the header declares, and rejects bad input before any launch.

Reject contract: PR "feat(kernels): Rust wrapper for the hd256 windowed paged
prefill", Verification (out-of-pool page ids, final-page lengths above the
page size, i32 overflow of batch lengths and a zero KV-head count are errors
raised before any launch, as are inconsistent layouts, bad layer indices and
non-finite scales) and Description (bounds committed only after an update fully
succeeds; the plan's tile cross-checked against the kernel's).  Prep rejects:
issue "gemma4: serving prep needs pool-write forms", Proposed Plan.

Every call below fails validation, which runs before any HIP call, so nothing
here touches a device.  Device pointers are fake non-null addresses that are
never dereferenced.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import paged_sliding_window_page_amd as psw

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "psw.h")
FAKE = 0x1000  # never dereferenced: every call here is rejected on the host


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|void|char\s*\*|const char\s*\*)\s*\*?\s*"
                       r"([A-Za-z_][A-Za-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_symbols_exported():
    names = _declared()
    assert len(names) >= 14, names
    lib = ctypes.CDLL(psw.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in psw.h but not exported"
    assert sorted(psw.EXPORTS) == names


def test_version():
    assert "gfx950" in psw.version()


def _plan_args(**over):
    a = dict(qo_indptr=[0, 5, 9], kv_page_indptr=[0, 2, 3], kv_page_indices=[3, 1, 0],
             kv_last_page_len=[4, 16], num_qo_heads=16, num_kv_heads=8, head_dim=256,
             page_size=16, num_pages=4)
    a.update(over)
    return a


def _plan(**over):
    a = _plan_args(**over)
    return psw.Plan(a.pop("qo_indptr"), a.pop("kv_page_indptr"), a.pop("kv_page_indices"),
                    a.pop("kv_last_page_len"), stream=0, **a)


def _code(fn):
    with pytest.raises(psw.PswError) as e:
        fn()
    return e.value.status


# ------------------------------------------------------------------ plan ----

def test_plan_info_records_bounds():
    p = _plan()
    info = p.info()
    assert info["batch"] == 2 and info["total_qo"] == 9 and info["total_pages"] == 3
    assert info["max_page_id"] == 3 and info["max_last_page_len"] == 16
    assert info["max_kv_len"] == 20 and info["max_qo_len"] == 5
    assert info["group"] == 2 and info["tile_q"] == 128 and info["generation"] == 1


@pytest.mark.parametrize("over,status", [
    (dict(kv_page_indices=[3, 4, 0]), "PSW_E_RANGE"),            # page id outside the pool
    (dict(kv_page_indices=[3, -1, 0]), "PSW_E_RANGE"),
    (dict(kv_last_page_len=[17, 16]), "PSW_E_RANGE"),             # past page_size
    (dict(kv_last_page_len=[0, 16]), "PSW_E_RANGE"),
    (dict(num_kv_heads=0), "PSW_E_HEADS"),                        # zero KV heads
    (dict(num_qo_heads=12, num_kv_heads=8), "PSW_E_HEADS"),       # not a multiple
    (dict(qo_indptr=[0, 5, 5]), "PSW_E_SHAPE"),                   # qo_len 0
    (dict(qo_indptr=[1, 5, 9]), "PSW_E_SHAPE"),
    (dict(kv_page_indptr=[0, 2, 2]), "PSW_E_SHAPE"),              # request without pages
    (dict(qo_indptr=[0, 30, 31]), "PSW_E_SHAPE"),                 # kv_len < qo_len
    (dict(page_size=12), "PSW_E_SHAPE"),
    (dict(page_size=2048), "PSW_E_SHAPE"),                        # past the largest page
    (dict(qo_indptr=[0], kv_page_indptr=[0], kv_page_indices=[],  # empty batch
          kv_last_page_len=[]), "PSW_E_SHAPE"),
    (dict(num_qo_heads=2 ** 31), "PSW_E_OVERFLOW"),
    (dict(tile_q_override=-1), "PSW_E_OVERFLOW"),
])
def test_plan_rejects(over, status):
    assert _code(lambda: _plan(**over)) == status


def test_plan_rejects_zero_kv_heads_before_division():
    # also with a query head count that would make any division meaningless
    assert _code(lambda: _plan(num_kv_heads=0, num_qo_heads=0)) == "PSW_E_HEADS"


def test_batch_past_i32_fails_instead_of_truncating():
    # 2^32 + 2 would truncate to a legal-looking 2
    assert _code(lambda: _plan(batch=2 ** 32 + 2)) == "PSW_E_OVERFLOW"


def test_kv_len_past_i32_fails():
    n = 2 ** 21 + 1    # pages of 1024 slots: kv_len just past INT32_MAX
    ids = np.zeros(n, np.int32)
    assert _code(lambda: _plan(qo_indptr=[0, 1], kv_page_indptr=[0, n], kv_page_indices=ids,
                               kv_last_page_len=[1024], page_size=1024,
                               num_pages=1)) == "PSW_E_OVERFLOW"


def test_tile_query_checks_in_i32_domain():
    assert psw.prefill_tile_q(2, 256) == 128
    assert psw.prefill_tile_q(16, 512) == 8     # 128 rows: 8 tokens x 16 heads
    assert psw.prefill_tile_q(1, 256) == 256
    assert _code(lambda: psw.prefill_tile_q(2 ** 32 + 2, 256)) == "PSW_E_OVERFLOW"
    assert _code(lambda: psw.prefill_tile_q(0, 256)) == "PSW_E_HEADS"
    assert _code(lambda: psw.prefill_tile_q(-4, 256)) == "PSW_E_HEADS"
    assert _code(lambda: psw.prefill_tile_q(3, 256)) == "PSW_E_UNSUPPORTED"
    assert _code(lambda: psw.prefill_tile_q(2, 128)) == "PSW_E_UNSUPPORTED"


def test_plan_update_is_all_or_nothing():
    p = _plan()
    before = p.info()
    bad = _plan_args(kv_page_indptr=[0, 2, 4], kv_page_indices=[3, 1, 2, 9])  # 9 past pool
    bad.update(qo_indptr=[0, 5, 30])
    assert _code(lambda: p.update(bad.pop("qo_indptr"), bad.pop("kv_page_indptr"),
                                  bad.pop("kv_page_indices"), bad.pop("kv_last_page_len"),
                                  **bad)) == "PSW_E_RANGE"
    assert p.info() == before
    bad2 = _plan_args(kv_last_page_len=[4, 17])
    assert _code(lambda: p.update(bad2.pop("qo_indptr"), bad2.pop("kv_page_indptr"),
                                  bad2.pop("kv_page_indices"), bad2.pop("kv_last_page_len"),
                                  **bad2)) == "PSW_E_RANGE"
    assert p.info() == before
    good = _plan_args(kv_page_indices=[2, 0, 1], kv_last_page_len=[1, 4])
    p.update(good.pop("qo_indptr"), good.pop("kv_page_indptr"), good.pop("kv_page_indices"),
             good.pop("kv_last_page_len"), **good)
    after = p.info()
    assert after["generation"] == before["generation"] + 1
    assert after["digest"] != before["digest"]
    assert after["max_page_id"] == 2 and after["max_last_page_len"] == 4


# ------------------------------------------------------------------ pool ----

def _pool(**over):
    a = dict(num_layers=2, num_pages=4, page_size=16, num_kv_heads=8, head_dim=256)
    a.update(over)
    numel = a["num_layers"] * a["num_pages"] * 2 * a["num_kv_heads"] * a["page_size"] * a["head_dim"]
    numel = over.pop("numel", numel) if "numel" in over else numel
    return psw.pool_desc(FAKE, numel=numel, **{k: v for k, v in a.items() if k != "numel"})


def test_pool_checks():
    psw.check_pool(_pool())
    assert _code(lambda: psw.check_pool(_pool(numel=123))) == "PSW_E_SHAPE"
    assert _code(lambda: psw.check_pool(_pool(num_kv_heads=0))) == "PSW_E_HEADS"
    assert _code(lambda: psw.check_pool(_pool(page_size=24))) == "PSW_E_SHAPE"
    big = psw.pool_desc(FAKE, numel=1, num_layers=2 ** 30, num_pages=2 ** 30, page_size=16,
                        num_kv_heads=8, head_dim=256)
    assert _code(lambda: psw.check_pool(big)) == "PSW_E_OVERFLOW"
    # a page of 4 GiB or more: 2 (K, V) x 4096 heads x 1024 slots x 256 dims x 2 B
    huge = _pool(num_layers=1, num_pages=1, num_kv_heads=4096, page_size=1024)
    assert _code(lambda: psw.check_pool(huge)) == "PSW_E_UNSUPPORTED"
    psw.check_pool(_pool(num_layers=1, num_pages=1, num_kv_heads=2047, page_size=1024))


# ------------------------------------------------------------- attention ----

class _T:
    """Stands in for a tensor: a fake address and a dtype."""
    def __init__(self, dtype=None):
        import torch
        self.dtype = dtype or torch.float32

    def data_ptr(self):
        return FAKE


def _attn(plan, pool, layer=0, scale=1.0, wl=1023, stream=0, q=None, o=None):
    return psw.paged_prefill_window_hd256(plan, pool, layer, q or _T(), scale, wl, o or _T(),
                                          stream=stream)


@pytest.mark.parametrize("kw,status", [
    (dict(layer=2), "PSW_E_RANGE"),
    (dict(layer=-1), "PSW_E_RANGE"),
    (dict(scale=math.inf), "PSW_E_SCALE"),
    (dict(scale=math.nan), "PSW_E_SCALE"),
    (dict(wl=-2), "PSW_E_RANGE"),
    (dict(stream=0x77), "PSW_E_PLAN"),      # not the plan's stream
])
def test_attention_rejects(kw, status):
    assert _code(lambda: _attn(_plan(), _pool(), **kw)) == status


def test_attention_rejects_contradictory_layouts():
    plan = _plan()
    assert _code(lambda: _attn(plan, _pool(num_kv_heads=4))) == "PSW_E_PLAN"
    assert _code(lambda: _attn(plan, _pool(page_size=32))) == "PSW_E_PLAN"
    assert _code(lambda: _attn(plan, _pool(head_dim=512))) == "PSW_E_PLAN"
    # pool smaller than the plan's page ids: max page id 3 >= 3 pages
    assert _code(lambda: _attn(plan, _pool(num_pages=3))) == "PSW_E_RANGE"
    assert _code(lambda: _attn(plan, _pool(numel=5))) == "PSW_E_SHAPE"
    # the hd512 entry refuses an hd256 plan
    assert _code(lambda: psw.paged_prefill_hd512(plan, _pool(), 0, _T(), 1.0, _T(),
                                                 stream=0)) == "PSW_E_PLAN"


def test_attention_rejects_plan_tiled_under_override():
    plan = _plan(tile_q_override=32)
    assert plan.info()["tile_q"] == 32
    assert _code(lambda: _attn(plan, _pool())) == "PSW_E_PLAN"


def test_attention_rejects_null_pointers():
    plan = _plan()
    pool = _pool()
    code = _code(lambda: psw._check(psw._prefill256(plan.handle, ctypes.byref(pool), 0, None,
                                                    1.0, 10, FAKE, 0, 0)))
    assert code == "PSW_E_NULL"
    nob = psw.pool_desc(0, numel=pool.numel, num_layers=2, num_pages=4, page_size=16,
                        num_kv_heads=8, head_dim=256)
    assert _code(lambda: _attn(plan, nob)) == "PSW_E_NULL"
    assert _code(lambda: psw._check(psw._prefill256(None, ctypes.byref(pool), 0, FAKE, 1.0, 10,
                                                    FAKE, 0, 0))) == "PSW_E_NULL"


def test_attention_rejects_bad_output_dtype():
    plan = _plan()
    pool = _pool()
    assert _code(lambda: psw._check(psw._prefill256(plan.handle, ctypes.byref(pool), 0, FAKE, 1.0,
                                                    10, FAKE, 7, 0))) == "PSW_E_SHAPE"


# ------------------------------------------------------------------ prep ----

def _prep(plan, pool, positions=32, cos_numel=None, sin_numel=None, eps=1e-6, layer=1, stream=0):
    cn = positions * 128 if cos_numel is None else cos_numel
    sn = positions * 128 if sin_numel is None else sin_numel
    return psw._check(psw._prep256(plan.handle, ctypes.byref(pool), layer, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, FAKE, positions, cn, sn, eps, FAKE, stream))


@pytest.mark.parametrize("kw,status", [
    (dict(positions=19), "PSW_E_RANGE"),          # kv_len 20 -> last position 19
    (dict(cos_numel=32 * 128 - 1), "PSW_E_SHAPE"),
    (dict(sin_numel=31 * 128), "PSW_E_SHAPE"),
    (dict(eps=0.0), "PSW_E_SCALE"),
    (dict(eps=-1e-6), "PSW_E_SCALE"),
    (dict(eps=math.nan), "PSW_E_SCALE"),
    (dict(layer=2), "PSW_E_RANGE"),
    (dict(stream=5), "PSW_E_PLAN"),
])
def test_prep_rejects(kw, status):
    assert _code(lambda: _prep(_plan(), _pool(), **kw)) == status


def test_prep_rejects_page_written_twice():
    # both requests write page 1 (request 0 its tail, request 1 its only page)
    plan = _plan(kv_page_indices=[3, 1, 1])
    assert _code(lambda: _prep(plan, _pool())) == "PSW_E_SHAPE"


def test_prep_rejects_null_tables():
    plan = _plan()
    pool = _pool()
    code = _code(lambda: psw._check(psw._prep256(plan.handle, ctypes.byref(pool), 1, FAKE, FAKE,
                                                 FAKE, FAKE, FAKE, None, FAKE, 32, 4096, 4096,
                                                 1e-6, FAKE, 0)))
    assert code == "PSW_E_NULL"


def test_prep512_rejects_hd256_plan():
    plan = _plan()
    pool = _pool()
    code = _code(lambda: psw._check(psw._prep512(plan.handle, ctypes.byref(pool), 1, FAKE, FAKE,
                                                 FAKE, FAKE, 32, 32 * 256, 32 * 256, 1e-6, 0)))
    assert code == "PSW_E_PLAN"


def _prepq(plan, positions=32, cos_numel=None, sin_numel=None, eps=1e-6, stream=0, q_in=FAKE,
           w=FAKE, cos=FAKE, q_out=FAKE):
    cn = positions * 256 if cos_numel is None else cos_numel
    sn = positions * 256 if sin_numel is None else sin_numel
    return psw._check(psw._prepq512(None if plan is None else plan.handle, q_in, w, cos, FAKE,
                                    positions, cn, sn, eps, q_out, stream))


def _plan512(**over):
    return _plan(**_plan_args(num_kv_heads=1, head_dim=512, **over))


@pytest.mark.parametrize("kw,status", [
    (dict(positions=19), "PSW_E_RANGE"),          # kv_len 20 -> last position 19
    (dict(cos_numel=32 * 256 - 1), "PSW_E_SHAPE"),
    (dict(sin_numel=32 * 128), "PSW_E_SHAPE"),
    (dict(eps=0.0), "PSW_E_SCALE"),
    (dict(eps=math.inf), "PSW_E_SCALE"),
    (dict(stream=5), "PSW_E_PLAN"),
    (dict(q_in=None), "PSW_E_NULL"),
    (dict(w=None), "PSW_E_NULL"),
    (dict(cos=None), "PSW_E_NULL"),
    (dict(q_out=None), "PSW_E_NULL"),
])
def test_query_prep512_rejects(kw, status):
    assert _code(lambda: _prepq(_plan512(), **kw)) == status


def test_query_prep512_rejects_null_plan_and_hd256_plan():
    assert _code(lambda: _prepq(None)) == "PSW_E_NULL"
    assert _code(lambda: _prepq(_plan())) == "PSW_E_PLAN"


def test_decode_entries_reject_multi_token_plans_and_bad_modes():
    plan = _plan()                                  # qo_len 5 and 4
    pool = _pool()
    assert _code(lambda: psw._check(psw._decode256(plan.handle, ctypes.byref(pool), 0, FAKE, 1.0,
                                                   -1, FAKE, 1, 0))) == "PSW_E_SHAPE"
    assert _code(lambda: plan.set_decode_mode(3)) == "PSW_E_SHAPE"
    assert _code(lambda: psw._check(psw._decode_mode(None, 0))) == "PSW_E_NULL"
    plan.set_decode_mode(psw.DECODE_DIRECT)
    one = _plan(qo_indptr=[0, 1, 2])
    # validation still runs after the token check: a wrong stream is rejected
    assert _code(lambda: psw._check(psw._decode256(one.handle, ctypes.byref(pool), 0, FAKE, 1.0,
                                                   -1, FAKE, 1, 5))) == "PSW_E_PLAN"


def _decode_plan(kv, hq, hkv, d):
    kvp, idx, last, nxt = [0], [], [], 0
    for k in kv:
        n = (k + 15) // 16
        idx += list(range(nxt, nxt + n))
        nxt += n
        kvp.append(kvp[-1] + n)
        last.append(k - (n - 1) * 16)
    return psw.Plan(list(range(len(kv) + 1)), kvp, idx, last, num_qo_heads=hq, num_kv_heads=hkv,
                    head_dim=d, page_size=16, num_pages=nxt, stream=0)


@pytest.mark.parametrize("hq,hkv,d", [(16, 8, 256), (16, 1, 512), (32, 1, 256)])
def test_decode_form_follows_the_mode(hq, hkv, d):
    """Split keeps partials even where every request is one split; direct is
    one work-group per (request, KV head); auto takes direct on short
    requests; a group of 32 (no direct form) always splits."""
    short = _decode_plan([40, 700, 129], hq, hkv, d)
    long_ = _decode_plan([40, 7000, 129], hq, hkv, d)
    group32 = hq // hkv == 32
    for plan in (short, long_):
        plan.set_decode_mode(psw.DECODE_SPLIT)
        assert plan.decode_form(200)[0] is False
        plan.set_decode_mode(psw.DECODE_DIRECT)
        direct, wgs = plan.decode_form(200)
        assert direct is (not group32)
        if not group32:
            assert wgs == 3 * hkv
    short.set_decode_mode(psw.DECODE_AUTO)
    assert short.decode_form(100)[0] is (not group32)      # at most 101 keys each
    assert short.decode_form(-1)[0] is False                # 700 keys
    long_.set_decode_mode(psw.DECODE_AUTO)
    assert long_.decode_form(-1)[0] is False
    assert _code(lambda: _plan().decode_form(-1)) == "PSW_E_SHAPE"


def test_decode_auto_form_thresholds():
    small = lambda kv, d, hkv: _decode_plan(kv, 16, hkv, d).decode_form(-1)[0]
    assert small([160] * 4, 256, 8) and not small([161] * 4, 256, 8)
    assert small([256] * 4, 512, 1) and not small([257] * 4, 512, 1)
    # 32 requests x 8 KV heads = 256 work-groups: direct up to 1024 keys
    assert small([1024] * 32, 256, 8) and not small([1025] * 32, 256, 8)
    assert not small([1024] * 31, 256, 8)


def test_rope_table_rejects():
    assert _code(lambda: psw.rope_tables(FAKE, FAKE, 0, 256, 1e4, stream=0)) == "PSW_E_SHAPE"
    assert _code(lambda: psw.rope_tables(FAKE, FAKE, 16, 255, 1e4, stream=0)) == "PSW_E_SHAPE"
    assert _code(lambda: psw.rope_tables(FAKE, FAKE, 16, 256, -1.0, stream=0)) == "PSW_E_SCALE"
    assert _code(lambda: psw.rope_tables(None, FAKE, 16, 256, 1e4, stream=0)) == "PSW_E_NULL"


# ------------------------------------------------------ resident windows ----

def _ring_plan(kv_len, qo=(5, 4), pages=([3, 1], [0]), last=None, hkv=8, d=256):
    kvp = [0]
    idx = []
    for p in pages:
        idx += list(p)
        kvp.append(kvp[-1] + len(p))
    if last is None:
        last = [(k - 1) % 16 + 1 for k in kv_len]
    qo_indptr = [0]
    for n in qo:
        qo_indptr.append(qo_indptr[-1] + n)
    return psw.Plan(qo_indptr, kvp, idx, last, num_qo_heads=16, num_kv_heads=hkv, head_dim=d,
                    page_size=16, num_pages=4, stream=0, kv_len=kv_len)


def test_ring_plan_checks_absolute_lengths():
    p = _ring_plan([100, 16])                 # request 0 wraps its 2 pages
    assert p.info()["max_kv_len"] == 100
    # a request that does not wrap must keep its derived length
    assert _code(lambda: _ring_plan([100, 15], last=[4, 16])) == "PSW_E_SHAPE"
    # a wrapped one must carry the slot of its last position
    assert _code(lambda: _ring_plan([100, 16], last=[16, 16])) == "PSW_E_SHAPE"
    assert _code(lambda: _ring_plan([3, 16], qo=(5, 4), last=[3, 16])) == "PSW_E_SHAPE"  # kv < qo


def test_ring_attention_needs_the_window_inside_the_ring():
    pool = _pool()
    plan = _ring_plan([100, 16])              # ring of 32 slots, 5 queries
    assert _code(lambda: _attn(plan, pool, wl=-1)) == "PSW_E_RANGE"    # no window
    assert _code(lambda: _attn(plan, pool, wl=28)) == "PSW_E_RANGE"    # 28 + 5 > 32
    # the global family has no window: a wrapped request is refused
    p512 = _ring_plan([100, 16], hkv=1, d=512)
    pool512 = _pool(num_kv_heads=1, head_dim=512)
    assert _code(lambda: psw.paged_prefill_hd512(p512, pool512, 0, _T(), 1.0, _T(),
                                                 stream=0)) == "PSW_E_RANGE"


def test_ring_prep_refuses_a_step_longer_than_its_ring():
    plan = _ring_plan([100, 16], qo=(40, 4))  # 40 positions into 32 slots
    assert _code(lambda: _prep(plan, _pool(), positions=128)) == "PSW_E_RANGE"


def test_mfma_clock_probe_rejects_null():
    # checked before any device call, so it runs without a GPU
    assert _code(lambda: psw._check(psw._mfma_clock(None, None))) == "PSW_E_NULL"


# ------------------------------------------------------- allocation-free decode ----

def test_noalloc_decode_refuses_a_batch_past_its_workspace():
    """One request of 140M keys: its 8.75M page ids alone need 35 MB of the
    32 MiB static workspace, so the call is refused before any HIP call."""
    kv = 140_000_000
    n_pages = (kv + 15) // 16
    ids = np.arange(n_pages, dtype=np.int32)
    plan = psw.Plan([0, 1], [0, n_pages], ids, [kv - (n_pages - 1) * 16], num_qo_heads=16,
                    num_kv_heads=1, head_dim=512, page_size=16, num_pages=n_pages, stream=0)
    pool = psw.pool_desc(FAKE, numel=n_pages * 2 * 16 * 512, num_layers=1, num_pages=n_pages,
                         page_size=16, num_kv_heads=1, head_dim=512)
    code = _code(lambda: psw._check(psw._decode512_noalloc(plan.handle, ctypes.byref(pool), 0, FAKE,
                                                           1.0, FAKE, 1, 0)))
    assert code == "PSW_E_RANGE"
    assert "workspace" in psw.last_error()
    plan.close()


def test_noalloc_decode_rejects_like_the_allocating_entry():
    plan = _plan(qo_indptr=[0, 5, 9])   # prefill batch: not a decode plan
    pool = psw.pool_desc(FAKE, numel=4 * 2 * 8 * 16 * 256, num_layers=1, num_pages=4,
                         page_size=16, num_kv_heads=8, head_dim=256)
    code = _code(lambda: psw._check(psw._decode512_noalloc(plan.handle, ctypes.byref(pool), 0,
                                                           FAKE, 1.0, FAKE, 1, 0)))
    assert code == "PSW_E_PLAN"   # an hd256 plan on the hd512 entry
