"""GPU parity of the fused pool-write prep entries and the RoPE tables.

Contract under test (issue "gemma4: serving prep needs pool-write forms --
hd256 QKV in one pass, hd512 V alongside K", Proposed Plan and Acceptance
Criteria): Q values against the oracle's contiguous rows, rotated K and
weightless-normed V at the offsets the pool layout gives, the layer offset,
and untouched memory everywhere else (placement compared bit for bit); for
hd512, V equals the raw K normalised with K's own denominator.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import paged_sliding_window_page_amd as psw
from gpu_util import SENTINEL, check_close, flat_k_index, flat_v_index, say, to_np64

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _tables(positions, head_dim, theta=1e4):
    c = torch.empty(positions, head_dim // 2, dtype=torch.float32, device=DEV)
    s = torch.empty_like(c)
    psw.rope_tables(c, s, positions, head_dim, theta)
    return c, s


def test_rope_tables_match_fp64_angles():
    for d in (256, 512):
        c, s = _tables(16384, d)
        torch.cuda.synchronize()
        p = np.arange(16384, dtype=np.float64)[:, None]
        i = np.arange(d // 2, dtype=np.float64)[None, :]
        ang = p * 10000.0 ** (-2.0 * i / d)
        # fp32 rounding of the fp64 value: within one fp32 ulp
        np.testing.assert_allclose(c.cpu().numpy(), np.cos(ang), rtol=0, atol=1.2e-7)
        np.testing.assert_allclose(s.cpu().numpy(), np.sin(ang), rtol=0, atol=1.2e-7)


def _geom(case, d):
    return oracle.PoolGeometry(case.num_layers, case.num_pages, case.num_kv_heads,
                               case.page_size, d)


def _written_index(case, g):
    """Flat indices of every pool element the prep must write, from the oracle's
    placement and the test's own flat-index formula."""
    t = case.table
    page, slot = oracle.expected_pool_writes(g, case.layer, case.qo_indptr, t.kv_page_indptr,
                                             t.kv_page_indices, t.kv_last_page_len)
    d = np.arange(g.head_dim)
    kidx, vidx = [], []
    for hh in range(g.num_kv_heads):
        kidx.append(flat_k_index(g, case.layer, page[:, None], hh, slot[:, None], d[None, :]))
        vidx.append(flat_v_index(g, case.layer, page[:, None], hh, d[None, :], slot[:, None]))
    # [T, H, D] each
    return np.stack(kidx, axis=1), np.stack(vidx, axis=1), page, slot


def _run_prep(case, d, label):
    g = _geom(case, d)
    say(f"[gpu] prep hd{d} {label} tokens={sum(case.qo_lens)} pages={case.num_pages} "
        f"layers={case.num_layers}")
    pool = torch.full((g.numel,), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    c, s = _tables(case.rope_positions, d, case.rope_theta)
    plan = psw.Plan(case.qo_indptr, case.table.kv_page_indptr, case.table.kv_page_indices,
                    case.table.kv_last_page_len, num_qo_heads=case.num_qo_heads,
                    num_kv_heads=case.num_kv_heads, head_dim=d, page_size=case.page_size,
                    num_pages=case.num_pages)
    pd = psw.pool_desc(pool, num_layers=case.num_layers, num_pages=case.num_pages,
                       page_size=case.page_size, num_kv_heads=case.num_kv_heads, head_dim=d)
    q_out = None
    if d == 256:
        q_out = torch.full(case.q_in.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        psw.qkv_norm_rope_paged_prefill_hd256(plan, pd, case.layer, case.q_in.to(DEV),
                                              case.k_in.to(DEV), case.v_in.to(DEV),
                                              case.q_norm_w.to(DEV), case.k_norm_w.to(DEV),
                                              c, s, case.eps, q_out)
    else:
        psw.k_v_norm_rope_paged_prefill_hd512(plan, pd, case.layer, case.k_in.to(DEV),
                                              case.k_norm_w.to(DEV), c, s, case.eps)
    torch.cuda.synchronize()
    plan.device_errors()
    plan.close()
    return g, pool, q_out


def _check_prep(case, d, g, pool, q_out, sample_tokens=None):
    kidx, vidx, page, slot = _written_index(case, g)
    bits = pool.view(torch.int16)
    changed = bits != SENTINEL
    n_changed = int(changed.sum().item())
    kflat = torch.from_numpy(kidx.reshape(-1)).to(DEV)
    vflat = torch.from_numpy(vidx.reshape(-1)).to(DEV)
    # placement, bit-exact: exactly the expected elements changed, nothing else
    assert bool(changed[kflat].all()) and bool(changed[vflat].all()), "an expected slot is untouched"
    assert n_changed == kidx.size + vidx.size, (n_changed, kidx.size + vidx.size)
    say(f"  placement exact: {n_changed} elements written, all in the expected slots")
    pos = oracle.token_positions(case.qo_indptr, case.table.kv_page_indptr,
                                 case.table.kv_last_page_len, case.page_size)
    toks = np.arange(len(pos)) if sample_tokens is None else np.asarray(sample_tokens)
    k_got = to_np64(pool[torch.from_numpy(kidx[toks].reshape(-1)).to(DEV)]).reshape(kidx[toks].shape)
    v_got = to_np64(pool[torch.from_numpy(vidx[toks].reshape(-1)).to(DEV)]).reshape(vidx[toks].shape)
    if d == 256:
        q_ref, k_ref, v_ref = oracle.qkv_prep_hd256(case.q_in[toks], case.k_in[toks],
                                                    case.v_in[toks], case.q_norm_w,
                                                    case.k_norm_w, pos[toks], case.eps,
                                                    case.rope_theta)
        q_got = to_np64(q_out[torch.from_numpy(toks).to(DEV)])
        check_close(q_got, q_ref, "q_out")
        exact = np.mean(oracle.f64_to_bf16_bits(q_ref) ==
                        oracle.bf16_bits(q_out[torch.from_numpy(toks).to(DEV)].cpu()))
        say(f"  q_out bitwise equal to RNE(oracle): {exact:.6f}")
    else:
        k_ref, v_ref = oracle.kv_prep_hd512(case.k_in[toks], case.k_norm_w, pos[toks], case.eps,
                                            case.rope_theta)
    check_close(k_got, k_ref, "K block")
    check_close(v_got, v_ref, "V block")
    for name, got, ref in (("K", k_got, k_ref), ("V", v_got, v_ref)):
        gb = oracle.f64_to_bf16_bits(got)  # got is exactly bf16-representable
        say(f"  {name} bitwise equal to RNE(oracle): {np.mean(gb == oracle.f64_to_bf16_bits(ref)):.6f}")


@pytest.mark.parametrize("qo,start", [([40], [0]), ([5, 33, 16, 1], [11, 0, 48, 300]),
                                      ([17], [15]), ([1], [0])])
def test_hd256_prep_placement_and_values(qo, start):
    case = synth.prep_case(50 + len(qo), qo, start, head_dim=256, num_kv_heads=8, num_layers=3,
                           layer=1, extra_pages=5, rope_positions=512)
    g, pool, q_out = _run_prep(case, 256, f"{qo}@{start}")
    _check_prep(case, 256, g, pool, q_out)


@pytest.mark.parametrize("qo,start", [([40], [0]), ([5, 33, 16, 1], [11, 0, 48, 300])])
def test_hd512_prep_placement_and_values(qo, start):
    case = synth.prep_case(60 + len(qo), qo, start, head_dim=512, num_kv_heads=1, num_layers=3,
                           layer=2, extra_pages=5, with_q_v=False, rope_positions=512)
    g, pool, _ = _run_prep(case, 512, f"{qo}@{start}")
    _check_prep(case, 512, g, pool, None)


@pytest.mark.parametrize("d", [256, 512])
@pytest.mark.parametrize("page_size", [8, 32, 64])
def test_prep_page_sizes(d, page_size):
    """Pages other than 16 slots: items of up to 8 tokens filling whole pages
    (8-slot pages), or several items per page starting mid-page (32 and 64),
    so the dim-major V stores take both their 8-slot-run form and the
    element-wise one."""
    case = synth.prep_case(80 + page_size, [5, 33, 16, 1, 70], [11, 0, 48, 300, 3], head_dim=d,
                           num_kv_heads=8 if d == 256 else 1, num_layers=2, layer=1,
                           page_size=page_size, extra_pages=3, with_q_v=d == 256,
                           rope_positions=512)
    g, pool, q_out = _run_prep(case, d, f"P={page_size}")
    _check_prep(case, d, g, pool, q_out)


def test_hd512_unit_weight_position_zero_k_equals_v_bitwise():
    case = synth.prep_case(71, [3], [0], head_dim=512, num_kv_heads=1, num_layers=1, layer=0,
                           with_q_v=False, rope_positions=64)
    case.k_norm_w = torch.ones(512, dtype=torch.bfloat16)
    g, pool, _ = _run_prep(case, 512, "w=1")
    kidx, vidx, _, _ = _written_index(case, g)
    k0 = pool[torch.from_numpy(kidx[0].reshape(-1)).to(DEV)].view(torch.int16).cpu().numpy()
    v0 = pool[torch.from_numpy(vidx[0].reshape(-1)).to(DEV)].view(torch.int16).cpu().numpy()
    np.testing.assert_array_equal(k0, v0)


@pytest.mark.parametrize("d", [256, 512])
def test_prep_8192_tokens_layer3_of_8(d):
    """8192 tokens at start 0 into layer 3 of an 8-layer pool of 1024 pages
    (random permutation), tables for 16384 positions: placement bit-exact over the
    whole pool, values of every token."""
    kw = dict(num_kv_heads=8) if d == 256 else dict(num_kv_heads=1, with_q_v=False)
    case = synth.prep_case(4, [8192], [0], head_dim=d, num_layers=8, layer=3, num_pages=1024,
                           rope_positions=16384, **kw)
    g, pool, q_out = _run_prep(case, d, "8192")
    _check_prep(case, d, g, pool, q_out)


def _run_query_prep(case, label):
    say(f"[gpu] query prep hd512 {label} tokens={sum(case.qo_lens)}")
    c, s = _tables(case.rope_positions, 512, case.rope_theta)
    plan = psw.Plan(case.qo_indptr, case.table.kv_page_indptr, case.table.kv_page_indices,
                    case.table.kv_last_page_len, num_qo_heads=case.num_qo_heads,
                    num_kv_heads=case.num_kv_heads, head_dim=512, page_size=case.page_size,
                    num_pages=case.num_pages)
    q_out = torch.full(case.q_in.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    psw.q_norm_rope_prefill_hd512(plan, case.q_in.to(DEV), case.q_norm_w.to(DEV), c, s,
                                  case.eps, q_out)
    torch.cuda.synchronize()
    plan.device_errors()
    plan.close()
    return q_out


@pytest.mark.parametrize("qo,start", [([40], [0]), ([5, 33, 16, 1], [11, 0, 48, 300]),
                                      ([1], [0]), ([17], [15])])
def test_hd512_query_prep_values(qo, start):
    """Global-family Q prep: every row written (no NaN left of the fill), values
    against the oracle at the token's position."""
    case = synth.prep_case(90 + len(qo), qo, start, head_dim=512, num_kv_heads=1,
                           with_q_v=False, with_q=True, rope_positions=512)
    q_out = _run_query_prep(case, f"{qo}@{start}")
    assert not bool(torch.isnan(q_out).any()), "a query row was not written"
    pos = oracle.token_positions(case.qo_indptr, case.table.kv_page_indptr,
                                 case.table.kv_last_page_len, case.page_size)
    ref = oracle.q_prep_hd512(case.q_in, case.q_norm_w, pos, case.eps, case.rope_theta)
    check_close(to_np64(q_out), ref, "q_out hd512")
    exact = np.mean(oracle.f64_to_bf16_bits(ref) == oracle.bf16_bits(q_out.cpu()))
    say(f"  q_out bitwise equal to RNE(oracle): {exact:.6f}")


def test_hd512_query_prep_8192_tokens():
    """8192 tokens x 16 heads at start 0, tables for 16384 positions: every row
    written, values of every row against the oracle."""
    case = synth.prep_case(5, [8192], [0], head_dim=512, num_kv_heads=1, num_pages=1024,
                           with_q_v=False, with_q=True, rope_positions=16384)
    q_out = _run_query_prep(case, "8192")
    assert not bool(torch.isnan(q_out).any()), "a query row was not written"
    toks = np.arange(8192)
    ref = oracle.q_prep_hd512(case.q_in, case.q_norm_w, toks, case.eps, case.rope_theta)
    check_close(to_np64(q_out), ref, "q_out hd512 whole tensor")


def test_global_layer_write_side_then_attention():
    """One global layer end to end from the raw projections: Q prep and K/V prep
    write the query buffer and the pool, then full attention reads both; the
    oracle chain rounds every stored row to bf16 like the GPU stores do."""
    # every key is written by this prep (start 0), so attention reads no unwritten slot
    case = synth.prep_case(83, [70, 190], [0, 0], head_dim=512, num_kv_heads=1, num_layers=2,
                           layer=1, with_q_v=False, with_q=True, rope_positions=1024,
                           extra_pages=3)
    g, pool, _ = _run_prep(case, 512, "layer chain")
    q_dev = _run_query_prep(case, "layer chain")
    t = case.table
    acase = synth.AttentionCase(16, 1, 512, 16, case.num_pages, 2, 1, case.qo_lens, case.kv_lens,
                                case.qo_indptr, t, q_dev.cpu(), pool)
    from gpu_util import run_attention
    gpu = run_attention(acase, pool=pool, label="layer chain attention")
    pos = oracle.token_positions(case.qo_indptr, t.kv_page_indptr, t.kv_last_page_len,
                                 case.page_size)
    q_ref = oracle.bits_to_f64(oracle.f64_to_bf16_bits(
        oracle.q_prep_hd512(case.q_in, case.q_norm_w, pos, case.eps, case.rope_theta)))
    k_ref, v_ref = oracle.kv_prep_hd512(case.k_in, case.k_norm_w, pos, case.eps, case.rope_theta)
    store = np.zeros(g.numel, dtype=np.float64)
    page, slot = oracle.expected_pool_writes(g, 1, case.qo_indptr, t.kv_page_indptr,
                                             t.kv_page_indices, t.kv_last_page_len)
    oracle.apply_pool_writes(store, g, 1, page, slot,
                             oracle.bits_to_f64(oracle.f64_to_bf16_bits(k_ref)),
                             oracle.bits_to_f64(oracle.f64_to_bf16_bits(v_ref)))
    ref = oracle.paged_attention(oracle.f64_to_bf16_bits(q_ref), oracle.f64_to_bf16_bits(store),
                                 g, 1, case.qo_indptr, t.kv_page_indptr, t.kv_page_indices,
                                 t.kv_last_page_len, 1.0, -1)
    check_close(gpu, ref, "Q prep + K/V prep -> attention")


def test_prep_then_attention_hd512_chain():
    """The global family's write side feeding its read side: prep writes K and V
    for 300 tokens, then full attention reads them back through the same pages."""
    case = synth.prep_case(81, [300], [0], head_dim=512, num_kv_heads=1, num_layers=2, layer=1,
                           with_q_v=False, rope_positions=1024, extra_pages=3)
    g, pool, _ = _run_prep(case, 512, "chain")
    q = synth.normal_bf16((300, 16, 512), 0.25, synth.generator(82))
    acase = synth.AttentionCase(16, 1, 512, 16, case.num_pages, 2, 1, [300], [300],
                                case.qo_indptr, case.table, q, pool)
    from gpu_util import run_attention
    gpu = run_attention(acase, pool=pool, label="chain attention")
    # oracle chain: prep rows (rounded to bf16 as stored) then attention
    pos = np.arange(300)
    k_ref, v_ref = oracle.kv_prep_hd512(case.k_in, case.k_norm_w, pos, case.eps, case.rope_theta)
    store = np.zeros(g.numel, dtype=np.float64)
    t = case.table
    page, slot = oracle.expected_pool_writes(g, 1, case.qo_indptr, t.kv_page_indptr,
                                             t.kv_page_indices, t.kv_last_page_len)
    oracle.apply_pool_writes(store, g, 1, page, slot,
                             oracle.bits_to_f64(oracle.f64_to_bf16_bits(k_ref)),
                             oracle.bits_to_f64(oracle.f64_to_bf16_bits(v_ref)))
    ref = oracle.paged_attention(q, oracle.f64_to_bf16_bits(store), g, 1, case.qo_indptr,
                                 t.kv_page_indptr, t.kv_page_indices, t.kv_last_page_len, 1.0, -1)
    check_close(gpu, ref, "prep -> attention")
