"""GPU parity of the attention entries against the fp64 oracle, through the C ABI.

Contract under test: windowed paged prefill at head_dim 256 and full paged
prefill at head_dim 512 (PR "feat(kernels): Rust wrapper for the hd256 windowed
paged prefill", Description; PR "feat(gemma4): paged KV serving across both
attention families", Description, including decode through the prefill entry at
one token).  Gate and tolerances: tests/gpu_util.py.
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


def _local(seed, qo, kv, **kw):
    a = dict(LOCAL)
    a.update(kw)
    return synth.attention_case(seed, qo, kv, **a)


# ------------------------------------------------ hd256 windowed prefill ----

def test_single_request_64_tokens_fp32_out():
    """One request of 64 tokens at start 0, 16 Q / 8 KV heads, pool of 32 pages
    under a random permutation, window_left 1023, sm_scale 1, fp32 output."""
    case = _local(1, [64], [64], num_pages=32)
    gpu = run_attention(case, window_left=1023, out_dtype=torch.float32, label="1x64")
    check_close(gpu, oracle_attention(case, window_left=1023), "1x64 fp32")


@pytest.mark.parametrize("qo,kv", [
    ([1, 2, 63, 64, 65], [1, 2, 63, 64, 65]),
    ([37], [1037]),
    ([20, 50, 1], [45, 50, 700]),
    ([130, 7], [300, 500]),
])
def test_ragged_batches(qo, kv):
    case = _local(3 + len(qo), qo, kv)
    for wl in (1023, -1):
        gpu = run_attention(case, window_left=wl, label=f"ragged {qo}")
        check_close(gpu, oracle_attention(case, window_left=wl), f"ragged wl={wl}")


@pytest.mark.parametrize("wl", [-1, 0, 1, 15, 16, 17, 63, 64, 65, 200, 299, 300, 10 ** 6])
def test_window_edges(wl):
    case = _local(9, [100, 40], [300, 77])
    gpu = run_attention(case, window_left=wl, label=f"wl={wl}")
    check_close(gpu, oracle_attention(case, window_left=wl), f"wl={wl}")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 4), (8, 1), (16, 1), (32, 1)])
def test_group_sizes(hq, hkv):
    case = _local(11, [70, 3], [200, 40], num_qo_heads=hq, num_kv_heads=hkv)
    gpu = run_attention(case, window_left=50, label=f"group {hq // hkv}")
    check_close(gpu, oracle_attention(case, window_left=50), f"group {hq // hkv}")


@pytest.mark.parametrize("page_size", [8, 32, 64, 256, 1024])
def test_page_sizes(page_size):
    case = _local(13, [90, 33], [150, 200], page_size=page_size)
    gpu = run_attention(case, window_left=70, label=f"P={page_size}")
    check_close(gpu, oracle_attention(case, window_left=70), f"P={page_size}")


def test_sm_scale_values():
    case = _local(15, [50], [80])
    for scale in (0.0, 0.0625, -1.0, 3.0):
        gpu = run_attention(case, window_left=30, sm_scale=scale, label=f"scale {scale}")
        check_close(gpu, oracle_attention(case, window_left=30, sm_scale=scale), f"scale {scale}")


def test_shared_pages_across_requests():
    """Two requests reading the same physical pages (attention only reads)."""
    case = _local(17, [40, 40], [100, 100], num_pages=14)
    t = case.table
    ids = t.kv_page_indices.copy()
    ids[7:14] = ids[0:7]
    table = synth.PageTable(t.kv_page_indptr, ids, t.kv_last_page_len)
    case.q[40:] = case.q[:40]
    gpu = run_attention(case, window_left=-1, table=table, label="shared pages")
    check_close(gpu, oracle_attention(case, window_left=-1, table=table), "shared pages")
    np.testing.assert_array_equal(gpu[:40], gpu[40:])


def _poisoned(case):
    """Pool bits with NaN in every page outside the tables and every slot past a
    request's KV length."""
    g = geom_of(case)
    bits = oracle.bf16_bits(case.pool).copy()
    used = set(case.table.kv_page_indices.tolist())
    by_page = bits.reshape(g.num_layers, g.num_pages, -1)
    for p in range(g.num_pages):
        if p not in used:
            by_page[:, p] = SENTINEL
    t = case.table
    d = np.arange(g.head_dim)
    for b in range(len(case.kv_lens)):
        last_page = t.kv_page_indices[t.kv_page_indptr[b + 1] - 1]
        for slot in range(int(t.kv_last_page_len[b]), g.page_size):
            for hh in range(g.num_kv_heads):
                bits[flat_k_index(g, case.layer, last_page, hh, slot, d)] = SENTINEL
                bits[flat_v_index(g, case.layer, last_page, hh, d, slot)] = SENTINEL
    return bits


@pytest.mark.parametrize("hd", [256, 512])
def test_nan_outside_the_keys_never_leaks(hd):
    fam = LOCAL if hd == 256 else GLOBAL
    case = synth.attention_case(19, [33, 70, 1], [45, 70, 99], num_pages=40, **fam)
    bits = _poisoned(case)
    wl = 20 if hd == 256 else -1
    clean = run_attention(case, window_left=wl, label="clean")
    dirty = run_attention(case, window_left=wl, pool=bits_tensor(bits), label="poisoned")
    np.testing.assert_array_equal(dirty, clean)
    check_close(clean, oracle_attention(case, window_left=wl), "poison case")


def test_page_permutation_is_bitwise_invariant():
    case = _local(23, [64, 100], [200, 100], num_pages=40)
    base = run_attention(case, window_left=99, label="perm base")
    g = geom_of(case)
    bits = oracle.bf16_bits(case.pool).reshape(g.num_layers, g.num_pages, -1)
    perm = np.random.default_rng(1).permutation(g.num_pages)
    moved = np.empty_like(bits)
    moved[:, perm] = bits
    t = case.table
    t2 = synth.PageTable(t.kv_page_indptr, perm[t.kv_page_indices].astype(np.int32),
                         t.kv_last_page_len)
    out = run_attention(case, window_left=99, pool=bits_tensor(moved.reshape(-1)), table=t2,
                        label="perm moved")
    np.testing.assert_array_equal(out, base)


def test_saturated_window_is_bitwise_full_causal():
    case = _local(29, [100, 20], [260, 33])
    full = run_attention(case, window_left=-1, label="full")
    for wl in (259, 260, 10 ** 6):
        np.testing.assert_array_equal(run_attention(case, window_left=wl, label=f"sat {wl}"), full)


def test_fp32_and_bf16_outputs_agree():
    case = _local(31, [90], [400])
    f32 = run_attention(case, window_left=128, out_dtype=torch.float32, label="f32")
    b16 = run_attention(case, window_left=128, out_dtype=torch.bfloat16, label="bf16")
    np.testing.assert_array_equal(
        torch.from_numpy(f32).to(torch.float32).to(torch.bfloat16).float().numpy(),
        b16.astype(np.float32))


def test_batch8_windowed_prefill_full_size():
    """8 requests, lengths ~ U[128, 2048] at start 0, pool of 4096 pages with
    random non-overlapping tables, window_left 1023, in the launch the benchmark
    times: the whole output tensor against the oracle."""
    g = synth.generator(2)
    lens = synth.uniform_lengths(8, 128, 2048, g)
    case = _local(2, lens, lens, num_pages=4096)
    gpu = run_attention(case, window_left=1023, label="b8 full size")
    ref = oracle_attention(case, window_left=1023, threads=8)
    check_close(gpu, ref, "b8 whole tensor")


# ------------------------------------------------ hd512 full prefill ----

def _global_case(seed, qo, kv, **kw):
    """16 Q / 1 KV heads at head_dim 512; V pages hold the raw K normalised
    without a weight (eps 1e-6), as the global family stores them, computed by
    the oracle."""
    a = dict(GLOBAL)
    a.update(kw)
    case = synth.attention_case(seed, qo, kv, **a)
    g = geom_of(case)
    kb, vb = oracle.kv_blocks(oracle.bf16_bits(case.pool).copy(), g)
    raw = oracle.bits_to_f64(kb)                        # [L, N, H, P, D]
    v = raw * oracle.inv_rms(raw, 1e-6)
    vb[...] = oracle.f64_to_bf16_bits(np.swapaxes(v, -1, -2))
    full = np.concatenate([kb.reshape(g.num_layers, g.num_pages, 1, -1),
                           vb.reshape(g.num_layers, g.num_pages, 1, -1)], axis=2).reshape(-1)
    case.pool = bits_tensor(full)
    return case


@pytest.mark.parametrize("qo,kv", [([300, 1, 64], [300, 50, 129]), ([17], [1000]), ([8], [8])])
def test_hd512_full_prefill(qo, kv):
    case = _global_case(37, qo, kv)
    gpu = run_attention(case, label="hd512")
    check_close(gpu, oracle_attention(case), f"hd512 {qo}")


@pytest.mark.parametrize("page_size", [8, 32, 64, 1024])
def test_hd512_page_sizes(page_size):
    """Page sizes other than 16 (per-round page lookup, a tile spanning part of
    a page or several pages)."""
    case = _global_case(39, [90, 33, 1], [150, 200, 77], page_size=page_size)
    gpu = run_attention(case, label=f"hd512 P={page_size}")
    check_close(gpu, oracle_attention(case), f"hd512 P={page_size}")


@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 1), (8, 2), (32, 1)])
def test_hd512_group_sizes(hq, hkv):
    """GQA groups other than 16 at head_dim 512: a work-group's 128 query rows
    are 128 / group tokens x the group's heads, 32 / group tokens per wave."""
    case = _global_case(43, [70, 1, 33], [70, 129, 300], num_qo_heads=hq, num_kv_heads=hkv)
    gpu = run_attention(case, label=f"hd512 group {hq // hkv}")
    check_close(gpu, oracle_attention(case), f"hd512 group {hq // hkv}")


@pytest.mark.parametrize("page_size", [16, 32])
def test_hd512_fp32_output(page_size):
    case = _global_case(47, [100, 7], [230, 64], page_size=page_size)
    f32 = run_attention(case, out_dtype=torch.float32, label=f"hd512 fp32 P={page_size}")
    check_close(f32, oracle_attention(case), f"hd512 fp32 P={page_size}")
    b16 = run_attention(case, out_dtype=torch.bfloat16, label=f"hd512 bf16 P={page_size}")
    np.testing.assert_array_equal(
        torch.from_numpy(f32).to(torch.float32).to(torch.bfloat16).float().numpy(),
        b16.astype(np.float32))


def test_hd512_full_size():
    """4 requests x 4096 tokens, causal, pool of 2048 pages, in the launch the
    benchmark times: the whole output tensor (262144 rows) against the oracle."""
    case = _global_case(3, [4096] * 4, [4096] * 4, num_pages=2048)
    gpu = run_attention(case, label="hd512 4x4096")
    ref = oracle_attention(case, threads=4)
    check_close(gpu, ref, "hd512 whole tensor")


# ------------------------------------------------ decode via the prefill entry ----

@pytest.mark.parametrize("hd", [256, 512])
def test_decode_batch(hd):
    """One query per request, KV lengths ~ U[100, 3000]: split-KV decode path."""
    gen = synth.generator(5)
    kv = synth.uniform_lengths(16, 100, 3000, gen)
    if hd == 256:
        case = _local(5, [1] * 16, kv)
        wl = 1023
    else:
        case = _global_case(5, [1] * 16, kv)
        wl = -1
    gpu = run_attention(case, window_left=wl, label=f"decode hd{hd}")
    check_close(gpu, oracle_attention(case, window_left=wl), f"decode hd{hd}")


@pytest.mark.parametrize("hd", [256, 512])
def test_decode_matches_prefill_rows(hd):
    """A one-token call whose KV ends at position p reproduces row p of a
    prefill over the same pages (within tolerance: different kernels)."""
    kv = 600
    if hd == 256:
        case = _local(41, [kv], [kv])
        wl = 255
    else:
        case = _global_case(41, [kv], [kv])
        wl = -1
    full = run_attention(case, window_left=wl, label="prefill rows")
    ids = case.table.kv_page_indices
    positions = [0, 15, 16, 17, 255, 256, 599]
    qo_indptr = np.arange(len(positions) + 1, dtype=np.int32)
    n_pages = [p // 16 + 1 for p in positions]
    indptr = np.concatenate([[0], np.cumsum(n_pages)]).astype(np.int32)
    indices = np.concatenate([ids[:n] for n in n_pages]).astype(np.int32)
    last = np.array([p - (n - 1) * 16 + 1 for p, n in zip(positions, n_pages)], np.int32)
    dec = synth.AttentionCase(case.num_qo_heads, case.num_kv_heads, case.head_dim, 16,
                              case.num_pages, 1, 0, [1] * len(positions),
                              [p + 1 for p in positions], qo_indptr,
                              synth.PageTable(indptr, indices, last), case.q[positions],
                              case.pool)
    out = run_attention(dec, window_left=wl, label="decode rows")
    check_close(out, full[positions], "decode vs prefill")
    check_close(out, oracle_attention(dec, window_left=wl), "decode vs oracle")


def test_pool_past_2gib_uses_64bit_offsets():
    """Pages past the 2 GiB mark of a 2.1 GiB pool (hd256, 8 KV heads)."""
    num_pages = 16500   # 128 KiB per page -> 2.16 GB
    small = _local(43, [50, 1], [120, 300], num_pages=30)
    used = small.table.kv_page_indices
    high = (num_pages - 30 + used).astype(np.int32)        # all above page 16384
    dev = torch.device("cuda", 0)
    pool = torch.zeros(num_pages * 2 * 8 * 16 * 256, dtype=torch.bfloat16, device=dev)
    per_page = 2 * 8 * 16 * 256
    src = small.pool.view(30, per_page)
    pool.view(num_pages, per_page)[num_pages - 30:] = src.to(dev)
    big = synth.AttentionCase(16, 8, 256, 16, num_pages, 1, 0, small.qo_lens, small.kv_lens,
                              small.qo_indptr,
                              synth.PageTable(small.table.kv_page_indptr, high,
                                              small.table.kv_last_page_len),
                              small.q, pool)
    say("[gpu] 2 GiB pool case")
    gpu = run_attention(big, window_left=1023, pool=pool, label="2GiB")
    check_close(gpu, oracle_attention(small, window_left=1023), ">2GiB pool")


def test_hd512_pool_past_4gib_uses_64bit_page_offsets():
    """hd512 prefill reading pages past the 4 GiB mark of a 4.6 GB pool (page
    byte offsets are page id x 32 KiB: past 2^32 from page 131072 on)."""
    num_pages = 140000
    small = _global_case(45, [70, 5], [150, 90], num_pages=20)
    used = small.table.kv_page_indices
    high = (num_pages - 20 + used).astype(np.int32)        # all above page 131072
    dev = torch.device("cuda", 0)
    per_page = 2 * 1 * 16 * 512
    pool = torch.zeros(num_pages * per_page, dtype=torch.bfloat16, device=dev)
    pool.view(num_pages, per_page)[num_pages - 20:] = small.pool.view(20, per_page).to(dev)
    big = synth.AttentionCase(16, 1, 512, 16, num_pages, 1, 0, small.qo_lens, small.kv_lens,
                              small.qo_indptr,
                              synth.PageTable(small.table.kv_page_indptr, high,
                                              small.table.kv_last_page_len),
                              small.q, pool)
    say("[gpu] 4 GiB hd512 pool case")
    gpu = run_attention(big, pool=pool, label="4GiB hd512")
    check_close(gpu, oracle_attention(small), ">4GiB hd512 pool")
