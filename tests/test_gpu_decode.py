"""GPU parity of one-token decode through the prefill entries, against the fp64
oracle, through the C ABI.

Decode is the prefill entry called with one query per request (PR
"feat(gemma4): paged KV serving across both attention families", Description).
The library runs it either as one work-group per request or as equal shares
of the batch's keys (pieces of cut requests write partials that a merge
combines); these cases cover the
page-size modes of the decode kernel (pages of 8, 16 and >= 32 slots), the GQA
group widths (up to 16 query heads per KV head in the decode kernel, 32 through
the general split kernel), windows that start mid-tile, NaN outside the keys
a request may read, and the full-size 64-request batch as a whole.
Gate and tolerances: tests/gpu_util.py.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (SENTINEL, bits_tensor, check_close, flat_k_index, flat_v_index, geom_of,
                      oracle_attention, run_attention, say)

pytestmark = pytest.mark.gpu

LOCAL = synth.LOCAL
GLOBAL = synth.GLOBAL


def _case(hd, seed, kv, **kw):
    a = dict(LOCAL if hd == 256 else GLOBAL)
    a.update(kw)
    return synth.attention_case(seed, [1] * len(kv), kv, **a)


KV_MIX = [1, 2, 15, 16, 17, 31, 32, 33, 64, 65, 300, 1500]


@pytest.mark.parametrize("hd", [256, 512])
@pytest.mark.parametrize("page_size", [8, 16, 32, 64, 1024])
def test_decode_page_sizes(hd, page_size):
    case = _case(hd, 61, KV_MIX, page_size=page_size)
    wl = 100 if hd == 256 else -1
    gpu = run_attention(case, window_left=wl, label=f"decode P={page_size}")
    check_close(gpu, oracle_attention(case, window_left=wl), f"decode hd{hd} P={page_size}")


@pytest.mark.parametrize("hq,hkv", [(4, 4), (16, 8), (16, 4), (8, 1), (16, 1), (32, 1)])
def test_decode_group_sizes(hq, hkv):
    case = _case(256, 63, [40, 700, 129], num_qo_heads=hq, num_kv_heads=hkv)
    gpu = run_attention(case, window_left=200, label=f"decode group {hq // hkv}")
    check_close(gpu, oracle_attention(case, window_left=200), f"decode group {hq // hkv}")


@pytest.mark.parametrize("hd,page_size", [(256, 8), (256, 32), (512, 16), (512, 8)])
def test_decode_group32_page_sizes(hd, page_size):
    """The group-32 decode (split mode of the attention kernel) at page sizes
    other than 16, and at head_dim 512 (32 Q heads on one KV head)."""
    case = _case(hd, 65, [40, 700, 129, 1], num_qo_heads=32, num_kv_heads=1,
                 page_size=page_size)
    wl = 200 if hd == 256 else -1
    gpu = run_attention(case, window_left=wl, label=f"decode hd{hd} group 32 P={page_size}")
    check_close(gpu, oracle_attention(case, window_left=wl),
                f"decode hd{hd} group 32 P={page_size}")


@pytest.mark.parametrize("wl", [-1, 0, 1, 30, 31, 32, 33, 63, 64, 1023, 10 ** 6])
def test_decode_window_edges(wl):
    case = _case(256, 67, KV_MIX)
    gpu = run_attention(case, window_left=wl, label=f"decode wl={wl}")
    check_close(gpu, oracle_attention(case, window_left=wl), f"decode wl={wl}")


def _poison_outside(case, wl):
    """Pool bits with NaN in every page outside the tables, every slot past a
    request's KV length and every key before its window."""
    g = geom_of(case)
    bits = oracle.bf16_bits(case.pool).copy()
    used = set(case.table.kv_page_indices.tolist())
    by_page = bits.reshape(g.num_layers, g.num_pages, -1)
    for p in range(g.num_pages):
        if p not in used:
            by_page[:, p] = SENTINEL
    t = case.table
    d = np.arange(g.head_dim)
    P = g.page_size
    for b, kv in enumerate(case.kv_lens):
        pages = t.kv_page_indices[t.kv_page_indptr[b]:t.kv_page_indptr[b + 1]]
        first = 0 if wl < 0 else max(0, kv - 1 - wl)
        dead = list(range(first)) + list(range(kv, len(pages) * P))
        for key in dead:
            page, slot = int(pages[key // P]), key % P
            for hh in range(g.num_kv_heads):
                bits[flat_k_index(g, case.layer, page, hh, slot, d)] = SENTINEL
                bits[flat_v_index(g, case.layer, page, hh, d, slot)] = SENTINEL
    return bits


@pytest.mark.parametrize("hd,page_size", [(256, 16), (256, 8), (256, 64), (512, 16)])
def test_decode_nan_outside_the_keys_never_leaks(hd, page_size):
    case = _case(hd, 71, [1, 37, 70, 100, 250], page_size=page_size, num_pages=120)
    wl = 45 if hd == 256 else -1
    bits = _poison_outside(case, wl)
    clean = run_attention(case, window_left=wl, label="decode clean")
    dirty = run_attention(case, window_left=wl, pool=bits_tensor(bits), label="decode poisoned")
    np.testing.assert_array_equal(dirty, clean)
    check_close(clean, oracle_attention(case, window_left=wl), "decode poison case")


@pytest.mark.parametrize("hd", [256, 512])
def test_decode_full_size(hd):
    """The 64-request decode batch (KV ~ U[512, 8192], pool of 32768 pages)
    in the launch configuration the benchmark times: every request and head
    against the oracle."""
    dev = torch.device("cuda", 0)
    case = synth.decode_batch(hd, dev)
    wl = 1023 if hd == 256 else -1
    gpu = run_attention(case, window_left=wl, pool=case.pool, label=f"decode full hd{hd}")
    say("[gpu] copying the pool to the host for the oracle")
    host = synth.AttentionCase(**{**case.__dict__, "pool": case.pool.cpu()})
    del case
    ref = oracle_attention(host, window_left=wl, threads=8)
    check_close(gpu, ref, f"decode full hd{hd}")


def _run_decode_entry(case, mode, window_left, out_dtype):
    """The dedicated decode entries with the plan's decode form forced."""
    import paged_sliding_window_page_amd as psw
    from gpu_util import make_plan, pool_desc_of, to_np64
    dev = torch.device("cuda", 0)
    say(f"[gpu] decode entry mode={mode} D={case.head_dim} kv={case.kv_lens[:6]} "
        f"wl={window_left} out={out_dtype}")
    pool_d = case.pool.to(dev)
    q_d = case.q.to(dev)
    o_d = torch.full((q_d.shape[0], case.num_qo_heads, case.head_dim), float("nan"),
                     dtype=out_dtype, device=dev)
    plan = make_plan(case)
    plan.set_decode_mode(mode)
    pd = pool_desc_of(case, pool_d)
    if case.head_dim == 256:
        psw.paged_decode_window_hd256(plan, pd, case.layer, q_d, 1.0, window_left, o_d)
    else:
        psw.paged_decode_hd512(plan, pd, case.layer, q_d, 1.0, o_d)
    torch.cuda.synchronize()
    plan.close()
    return to_np64(o_d)


@pytest.mark.parametrize("hd", [256, 512])
@pytest.mark.parametrize("mode", [0, 1, 2])   # auto, split, direct (one work-group per request)
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_decode_entries_each_form(hd, mode, out_dtype):
    case = _case(hd, 71, KV_MIX + [512, 513, 4000])
    wl = 300 if hd == 256 else -1
    gpu = _run_decode_entry(case, mode, wl, out_dtype)
    check_close(gpu, oracle_attention(case, window_left=wl), f"decode entry hd{hd} mode {mode}")


@pytest.mark.parametrize("hd", [256, 512])
def test_decode_merge_past_256_requests(hd):
    """Split form on 300 requests: the merge runs in launches of 256 requests
    (each request's split list travels in its launch's arguments), so the cut
    requests past the first 256 go through a second launch."""
    kv = [24 + (97 * i) % 200 for i in range(300)]
    case = _case(hd, 81, kv)
    wl = 100 if hd == 256 else -1
    gpu = _run_decode_entry(case, 1, wl, torch.float32)
    check_close(gpu, oracle_attention(case, window_left=wl, threads=8),
                f"decode 300 requests hd{hd}")


@pytest.mark.parametrize("hd", [256, 512])
def test_decode_forms_agree_on_short_requests(hd):
    """Short requests (the automatic choice takes the direct form): direct and
    split give the same result within the gate, and both match the oracle."""
    case = _case(hd, 73, [3, 64, 200, 511, 512] * 4)
    wl = 1023 if hd == 256 else -1
    direct = _run_decode_entry(case, 2, wl, torch.float32)
    split = _run_decode_entry(case, 1, wl, torch.float32)
    ref = oracle_attention(case, window_left=wl)
    check_close(direct, ref, "direct")
    check_close(split, ref, "split")


@pytest.mark.parametrize("hd", [256, 512])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_decode_shares_span_requests(hd, out_dtype):
    """Split form on a batch whose equal shares cross request boundaries: 150
    short requests (1..200 keys) around three long ones, so work-groups run
    several whole requests in a row (each writing O itself) next to pieces of
    the long requests (partials, merged afterwards); the exchange-buffer parity
    carries over between the items of a work-group."""
    g = np.random.default_rng(5)
    kv = [int(x) for x in g.integers(1, 201, 150)]
    kv[10], kv[75], kv[140] = 3000, 9000, 5000
    case = _case(hd, 79, kv, num_pages=sum((k + 15) // 16 for k in kv) + 8)
    wl = 700 if hd == 256 else -1
    gpu = _run_decode_entry(case, 1, wl, out_dtype)
    check_close(gpu, oracle_attention(case, window_left=wl), f"decode shares hd{hd}")
