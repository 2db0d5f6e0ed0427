"""The allocation-free decode entry (paged_decode_hd512_noalloc) against the
entry it varies (paged_decode_hd512), through the C ABI: two calls in a row on
the library's static workspace, the second with a smaller batch, each equal to
the allocating entry bit for bit (same kernels, same schedule) and to the
oracle within the gate.  (The refusal of a batch past the workspace is a host
check, tested without a GPU in test_abi_cpu.py.)  The decode
contract is the prefill entry at one token (PR "feat(gemma4): paged KV serving
across both attention families", Description)."""
import numpy as np
import pytest
import torch

import synth
import paged_sliding_window_page_amd as psw
from gpu_util import check_close, make_plan, oracle_attention, pool_desc_of, say, to_np64

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _global_case(seed, kv, **kw):
    return synth.attention_case(seed, [1] * len(kv), kv, **{**synth.GLOBAL, **kw})


def _both(case):
    say(f"[gpu] no-alloc decode batch={len(case.kv_lens)} kv={case.kv_lens[:6]}")
    pool = case.pool.to(DEV)
    q = case.q.to(DEV)
    pd = pool_desc_of(case, pool)
    outs = []
    for fn in (psw.paged_decode_hd512, psw.paged_decode_hd512_noalloc):
        o = torch.full((q.shape[0], 16, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
        plan = make_plan(case)
        plan.set_decode_mode(psw.DECODE_SPLIT)   # the form with partials and a merge
        fn(plan, pd, case.layer, q, 1.0, o)
        torch.cuda.synchronize()
        plan.close()
        outs.append(to_np64(o))
    return outs


def test_noalloc_decode_matches_allocating_entry_twice():
    g = np.random.default_rng(9)
    big = _global_case(91, [int(x) for x in g.integers(300, 6000, 24)])
    small = _global_case(92, [int(x) for x in g.integers(1, 900, 5)])
    for case in (big, small):
        ref_entry, got = _both(case)
        np.testing.assert_array_equal(got, ref_entry)
        check_close(got, oracle_attention(case), f"no-alloc decode batch {len(case.kv_lens)}")
