"""Helpers for the GPU parity tests: move synthetic cases to the device, call
the library through its C ABI, and compare against the fp64 oracle.

Acceptance gate for floating-point outputs (bf16 or fp32 outputs alike):
  * element-wise |gpu - ref| <= max(2e-2, 1.01 * half_ulp_bf16(ref)): 2e-2
    absolute, widened only where rounding the output itself to bf16 can already
    exceed 2e-2.  For |x| in [2^e, 2^(e+1)) bf16 numbers are 2^(e-7) apart, so
    one round-to-nearest step is at most 2^(e-8); that passes 2e-2 only from
    |x| >= 8 (half-ulp 2^-5), and below 8 the gate is the plain 2e-2.  The
    factor 1.01 leaves room for the fp32 arithmetic before the rounding
    (relative error ~1e-6, against 1e-2 of a half-ulp);
  * relative RMS ||gpu - ref||_2 / ||ref||_2 <= 1e-2 over the whole tensor
    given (callers pass whole output tensors).
The reference is the unrounded float64 oracle.  Placement is compared bit for
bit.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import paged_sliding_window_page_amd as psw

ABS_TOL = 2e-2
REL_RMS_TOL = 1e-2
SENTINEL = 0x7FA5   # a NaN payload no valid computation produces


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits_tensor(bits: np.ndarray) -> torch.Tensor:
    """bf16 torch tensor (CPU) from uint16 bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16)


def to_np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 numbers in the binade of |x|: 2^(e-8) for |x| in
    [2^e, 2^(e+1)) (8 significant bits), the largest error of one
    round-to-nearest step to bf16.  Zero and subnormal magnitudes take the
    spacing of the smallest normal binade."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.maximum(a, np.finfo(np.float32).tiny))  # a = m * 2^e, m in [0.5, 1)
    return np.ldexp(1.0, e - 9)


def gate(ref: np.ndarray) -> np.ndarray:
    """Element-wise absolute bound of the acceptance gate."""
    return np.maximum(ABS_TOL, 1.01 * half_ulp_bf16(ref))


def check_close(gpu: np.ndarray, ref: np.ndarray, label: str = ""):
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.isfinite(ref).all(), "reference has non-finite values"
    assert np.isfinite(gpu).all(), f"{label}: GPU output has non-finite values"
    err = np.abs(gpu - ref)
    tol = gate(ref)
    bad = err > tol
    rel = float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300))
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    say(f"  {label}: max|err| {err.max():.3e} rel_rms {rel:.3e} worst at {tuple(int(i) for i in worst)}")
    assert not bad.any(), (f"{label}: {int(bad.sum())} elements past tolerance, worst "
                           f"{err[worst]:.4e} (ref {ref[worst]:.4e}) at {worst}")
    assert rel <= REL_RMS_TOL, f"{label}: relative RMS {rel:.3e} > {REL_RMS_TOL}"
    return float(err.max()), rel


def geom_of(case) -> oracle.PoolGeometry:
    return oracle.PoolGeometry(case.num_layers, case.num_pages, case.num_kv_heads,
                               case.page_size, case.head_dim)


def make_plan(case, table=None, qo_indptr=None, stream=None):
    t = table or case.table
    return psw.Plan(case.qo_indptr if qo_indptr is None else qo_indptr, t.kv_page_indptr,
                    t.kv_page_indices, t.kv_last_page_len, num_qo_heads=case.num_qo_heads,
                    num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                    page_size=case.page_size, num_pages=case.num_pages, stream=stream)


def pool_desc_of(case, pool_dev):
    return psw.pool_desc(pool_dev, num_layers=case.num_layers, num_pages=case.num_pages,
                         page_size=case.page_size, num_kv_heads=case.num_kv_heads,
                         head_dim=case.head_dim)


def run_attention(case, window_left=-1, sm_scale=1.0, out_dtype=torch.bfloat16, pool=None,
                  table=None, label=""):
    """Runs the matching attention entry on cuda:0; returns float64 numpy output."""
    say(f"[gpu] attention {label} D={case.head_dim} Hq={case.num_qo_heads} Hkv={case.num_kv_heads} "
        f"qo={case.qo_lens[:8]} kv={case.kv_lens[:8]} wl={window_left} P={case.page_size}")
    dev = torch.device("cuda", 0)
    pool_t = (case.pool if pool is None else pool)
    pool_d = pool_t.to(dev) if pool_t.device.type == "cpu" else pool_t
    q_d = case.q.to(dev)
    o_d = torch.full((q_d.shape[0], case.num_qo_heads, case.head_dim), float("nan"),
                     dtype=out_dtype, device=dev)
    plan = make_plan(case, table=table)
    pd = pool_desc_of(case, pool_d)
    if case.head_dim == 256:
        psw.paged_prefill_window_hd256(plan, pd, case.layer, q_d, sm_scale, window_left, o_d)
    else:
        assert window_left == -1
        psw.paged_prefill_hd512(plan, pd, case.layer, q_d, sm_scale, o_d)
    torch.cuda.synchronize()
    out = to_np64(o_d)
    plan.close()
    return out


def oracle_attention(case, window_left=-1, sm_scale=1.0, pool=None, table=None, samples=None,
                     threads=1):
    """The oracle's output for the case (every row, or only ``samples``).
    ``threads`` > 1 runs the requests in a thread pool (numpy releases the GIL
    in its array kernels), each request computed by the same oracle call."""
    t = table or case.table
    pl = case.pool if pool is None else pool

    def run(requests=None):
        return oracle.paged_attention(case.q, pl, geom_of(case), case.layer, case.qo_indptr,
                                      t.kv_page_indptr, t.kv_page_indices, t.kv_last_page_len,
                                      sm_scale, window_left, samples=samples, requests=requests)

    if threads <= 1 or samples is not None:
        return run()
    from concurrent.futures import ThreadPoolExecutor
    batch = len(case.qo_indptr) - 1
    out = None
    with ThreadPoolExecutor(threads) as ex:
        for b, part in zip(range(batch), ex.map(lambda r: run([r]), range(batch))):
            q0, q1 = int(case.qo_indptr[b]), int(case.qo_indptr[b + 1])
            if out is None:
                out = part
            else:
                out[q0:q1] = part[q0:q1]
            say(f"  oracle: request {b} done")
    return out


def flat_k_index(g, layer, page, head, slot, d):
    """Flat pool index of a K element (K block [H][P][D] first in each page)."""
    blk = g.num_kv_heads * g.page_size * g.head_dim
    return ((layer * g.num_pages + page) * 2) * blk + (head * g.page_size + slot) * g.head_dim + d


def flat_v_index(g, layer, page, head, d, slot):
    """Flat pool index of a V element (V block [H][D][P], after the K block)."""
    blk = g.num_kv_heads * g.page_size * g.head_dim
    return (((layer * g.num_pages + page) * 2 + 1) * blk + (head * g.head_dim + d) * g.page_size
            + slot)
