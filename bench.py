"""Benchmark of the paged sliding-window hot path on one MI355X.

One step runs every row of the hot path once, each on its own seeded synthetic
workload (inputs resident in HBM before timing starts), all on one stream:

  prep_hd256           fused Q/K/V norm+RoPE+scatter, 8192 tokens, layer 3 of 8
  prep_hd512           fused K/V (V = weightless norm of raw K), 8192 tokens
  prep_q_hd512         the global family's Q norm+RoPE, 8192 tokens x 16 heads
  prefill_window_hd256_1x64
                       windowed paged prefill, one request of 64 tokens, 32-page
                       pool, window 1023, fp32 output (launch-latency bound)
  prefill_window_hd256 windowed paged prefill, 8 requests ~ U[128, 2048], window 1023
  prefill_hd512        full paged prefill, 4 x 4096 tokens, 16 Q / 1 KV heads
  decode_local_hd256   one-token decode through the prefill entry, 64 requests,
                       KV ~ U[512, 8192], window 1023
  decode_global_hd512  the same requests on the global family, full attention

`ms_per_step` is the wall time of one such step (K steps after W warmup
steps).  The per-row figures come from each row launched K more times in a
block of its own, timed with HIP events on that stream: the K launches of a
compute-bound row back to back between one pair of events (their mean).  An
HBM-bound row's launches each follow a read of a 1 GiB buffer so that their
bytes come from HBM, not from the 256 MB last-level cache; N = max(K, 30)
(flush, launch) pairs between one pair of events, minus N flushes between
another, give the launches' own duration (the median of an event pair around
each single launch, which adds the launch's dispatch latency, is reported
beside it as ms_event_median).

The JSON line's `value` is the windowed paged prefill's algorithmic TFLOP/s on
the batch-8 workload (only (query, key) pairs inside the window count).  Per-row
figures (TFLOP/s against the bf16 MFMA peak, GB/s against HBM) are under
`rows`; `cpu_baseline` times the fp64 oracle on a bounded sample of the same
workload on this host.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--rows a,b] [--no-cpu]

`roofline.clock_mhz_under_mfma` is the shader clock measured with every CU
issuing bf16 MFMAs (psw_measure_mfma_clock, median of three) and
`roofline.frac_clock_adjusted` the prefill's fraction of the peak scaled to
that clock; `roofline.frac` stays against the published (2.4 GHz) peak.

`roofline.traffic` is the measured HBM traffic of one launch of the prefill
kernel, read from profiles/hbm_traffic.md when that summary was taken from the
current kernel sources (their digest is recorded there), else null.  The
summary is written by

    python bench.py --pmc-summary FETCH.csv WRITE.csv --copy-mib 256

from two rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE) of
`bench.py --copy-mib 256 ...`: each counter is scaled by what it reads for the
plain device copy that --copy-mib runs first (a known number of bytes).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
NOMINAL_MHZ = 2400.0   # shader clock the published MFMA peak is quoted at
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "windowed paged prefill TFLOP/s (% MFMA peak); seq_len-1 decode KV GB/s"
HEAD_KERNEL = "prefill256_pp_kernel<true, true>"   # bf16 output, 16-slot pages
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")
CALIB_KERNEL = "neg_kernel"   # the plain device copy run by --copy-mib


def source_digest():
    """sha256 over the kernel sources (every file of the package's csrc/)."""
    import hashlib
    d = os.path.join(ROOT, "paged_sliding_window_page_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), "rb") as fh:
            h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()


def short_kernel_name(name):
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    name = name.replace("psw_dev::", "").split("(")[0]
    return name


def pmc_summary(fetch_csv, write_csv, copy_mib):
    """Markdown summary of two rocprofv3 counter runs, bytes per dispatch."""
    import csv
    import collections
    import statistics

    def per_kernel(path, counter):
        per = collections.defaultdict(float)
        name = {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                per[r["Dispatch_Id"]] += float(r["Counter_Value"])
                name[r["Dispatch_Id"]] = r["Kernel_Name"]
        out = collections.defaultdict(list)
        for d, v in per.items():
            out[short_kernel_name(name[d])].append(v)
        return out

    fk = per_kernel(fetch_csv, "FETCH_SIZE")
    wk = per_kernel(write_csv, "WRITE_SIZE")
    calib = [k for k in fk if CALIB_KERNEL in k]
    if not calib:
        raise SystemExit(f"no {CALIB_KERNEL} dispatch in {fetch_csv}: run bench.py with --copy-mib")
    copy_bytes = float(copy_mib) * (1 << 20)
    f_fac = copy_bytes / (statistics.median(fk[calib[0]]) * 1024.0)
    w_fac = copy_bytes / (statistics.median(wk[calib[0]]) * 1024.0)
    lines = ["# HBM traffic per launch, from hardware counters", "",
             f"source_digest: {source_digest()}",
             f"calibration: plain copy of {copy_mib} MiB ({calib[0]}): "
             f"bytes read = FETCH_SIZE KiB x 1024 x {f_fac:.3f}, "
             f"bytes written = WRITE_SIZE KiB x 1024 x {w_fac:.3f}", "",
             "| kernel | dispatches | FETCH_SIZE KiB (median) | WRITE_SIZE KiB (median) "
             "| read MB | written MB | traffic_bytes |", "|---|---|---|---|---|---|---|"]
    for k in sorted(fk):
        if k not in wk or not (k.startswith("prefill") or k.startswith("attention")
                               or k.startswith("decode") or k.startswith("merge")
                               or k.startswith("prep")):
            continue
        fm = statistics.median(fk[k])
        wm = statistics.median(wk[k])
        rd = fm * 1024.0 * f_fac
        wr = wm * 1024.0 * w_fac
        lines.append(f"| `{k}` | {len(fk[k])} | {fm:.1f} | {wm:.1f} | {rd / 1e6:.2f} | "
                     f"{wr / 1e6:.2f} | {int(round(rd + wr))} |")
    return "\n".join(lines) + "\n"


def read_traffic(kernel):
    """Measured bytes per launch of `kernel`, if the summary matches the sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            text = fh.read()
    except OSError:
        return None
    digest = None
    for line in text.splitlines():
        if line.startswith("source_digest:"):
            digest = line.split(":", 1)[1].strip()
        if line.startswith(f"| `{kernel}` |") and digest == source_digest():
            return int(line.rstrip(" |").split("|")[-1])
    return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------ algorithmic work ----

def attention_flops(qo_lens, kv_lens, num_qo_heads, head_dim, window_left):
    """4 * D * H_q * sum over queries of the number of visible keys."""
    pairs = 0
    for qo, kv in zip(qo_lens, kv_lens):
        p = np.arange(kv - qo, kv, dtype=np.int64)
        vis = p + 1 if window_left < 0 else np.minimum(p, window_left) + 1
        pairs += int(vis.sum())
    return 4.0 * head_dim * num_qo_heads * pairs


def decode_bytes(kv_lens, num_qo_heads, num_kv_heads, head_dim, window_left, page_size=16):
    keys = 0
    pages = 0
    for kv in kv_lens:
        n = kv if window_left < 0 else min(kv, window_left + 1)
        keys += n
        pages += (n + page_size - 1) // page_size + 1
    kvb = keys * num_kv_heads * head_dim * 2 * 2
    qo = len(kv_lens) * num_qo_heads * head_dim * 2 * 2
    return float(kvb + qo + pages * 4)


def prep_bytes(tokens, head_dim, hq, hkv, with_q_v):
    half = head_dim // 2
    tables = tokens * half * 4 * 2
    if with_q_v:
        rd = tokens * (hq + 2 * hkv) * head_dim * 2
        wr = tokens * (hq + 2 * hkv) * head_dim * 2
        w = 2 * head_dim * 2
    else:
        rd = tokens * hkv * head_dim * 2
        wr = tokens * 2 * hkv * head_dim * 2
        w = head_dim * 2
    return float(rd + wr + tables + w)


# ------------------------------------------------------------------ workloads ----

class Row:
    def __init__(self, name, run, work, unit, bound, desc, hbm=False):
        self.name, self.run, self.work, self.unit = name, run, work, unit
        self.bound, self.desc, self.hbm = bound, desc, hbm


def build_rows(torch, psw, synth, dev, want):
    rows = []
    stream = torch.cuda.current_stream()

    def plan_of(qo_indptr, table, hq, hkv, d, num_pages):
        return psw.Plan(qo_indptr, table.kv_page_indptr, table.kv_page_indices,
                        table.kv_last_page_len, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d,
                        page_size=16, num_pages=num_pages, stream=stream)

    def tables(d):
        c = torch.empty(16384, d // 2, dtype=torch.float32, device=dev)
        s = torch.empty_like(c)
        psw.rope_tables(c, s, 16384, d, 1e4)
        return c, s

    # ---- prep (8192 tokens, start 0, layer 3 of 8, 1024-page pools) ----
    if "prep_hd256" in want or "prep_hd512" in want:
        for d, name in ((256, "prep_hd256"), (512, "prep_hd512")):
            if name not in want:
                continue
            hkv = 8 if d == 256 else 1
            case = synth.prep_case(4, [8192], [0], head_dim=d, num_kv_heads=hkv, num_layers=8,
                                   layer=3, num_pages=1024, with_q_v=(d == 256))
            numel = 8 * 1024 * 2 * hkv * 16 * d
            pool = torch.zeros(numel, dtype=torch.bfloat16, device=dev)
            pd = psw.pool_desc(pool, num_layers=8, num_pages=1024, page_size=16,
                               num_kv_heads=hkv, head_dim=d)
            plan = plan_of(case.qo_indptr, case.table, 16, hkv, d, 1024)
            c, s = tables(d)
            k_in = case.k_in.to(dev)
            k_w = case.k_norm_w.to(dev)
            if d == 256:
                q_in, v_in = case.q_in.to(dev), case.v_in.to(dev)
                q_w = case.q_norm_w.to(dev)
                q_out = torch.empty_like(q_in)

                def run(plan=plan, pd=pd, q_in=q_in, k_in=k_in, v_in=v_in, q_w=q_w, k_w=k_w,
                        c=c, s=s, q_out=q_out):
                    psw.qkv_norm_rope_paged_prefill_hd256(plan, pd, 3, q_in, k_in, v_in, q_w,
                                                          k_w, c, s, 1e-6, q_out)
            else:
                def run(plan=plan, pd=pd, k_in=k_in, k_w=k_w, c=c, s=s):
                    psw.k_v_norm_rope_paged_prefill_hd512(plan, pd, 3, k_in, k_w, c, s, 1e-6)
            work = prep_bytes(8192, d, 16, hkv, d == 256)
            rows.append(Row(name, run, work, "GB/s", "hbm",
                            f"fused prep hd{d}, 8192 tokens at start 0, layer 3 of 8, "
                            f"1024-page pool, RoPE theta 1e4 over 16384 positions", hbm=True))

    # ---- global-family query prep, 8192 tokens x 16 heads ----
    if "prep_q_hd512" in want:
        case = synth.prep_case(5, [8192], [0], head_dim=512, num_kv_heads=1, num_pages=1024,
                               with_q_v=False, with_q=True)
        plan = plan_of(case.qo_indptr, case.table, 16, 1, 512, 1024)
        c, s = tables(512)
        q_in, q_w = case.q_in.to(dev), case.q_norm_w.to(dev)
        q_out = torch.empty_like(q_in)

        def run(plan=plan, q_in=q_in, q_w=q_w, c=c, s=s, q_out=q_out):
            psw.q_norm_rope_prefill_hd512(plan, q_in, q_w, c, s, 1e-6, q_out)
        # Q read and written once, one cos and one sin row per token, the weight
        work = float(2 * 8192 * 16 * 512 * 2 + 8192 * 256 * 4 * 2 + 512 * 2)
        rows.append(Row("prep_q_hd512", run, work, "GB/s", "hbm",
                        "query prep hd512, 8192 tokens x 16 heads at start 0, RoPE theta 1e4 "
                        "over 16384 positions", hbm=True))

    # ---- windowed prefill hd256, one request of 64 tokens, fp32 output ----
    if "prefill_window_hd256_1x64" in want:
        case = synth.attention_case(1, [64], [64], num_pages=32, **synth.LOCAL)
        pool = case.pool.to(dev)
        q = case.q.to(dev)
        o = torch.empty(q.shape, dtype=torch.float32, device=dev)
        plan = plan_of(case.qo_indptr, case.table, 16, 8, 256, 32)
        pd = psw.pool_desc(pool, num_layers=1, num_pages=32, page_size=16, num_kv_heads=8,
                           head_dim=256)

        def run(plan=plan, pd=pd, q=q, o=o):
            psw.paged_prefill_window_hd256(plan, pd, 0, q, 1.0, 1023, o)
        rows.append(Row("prefill_window_hd256_1x64", run,
                        attention_flops([64], [64], 16, 256, 1023), "TFLOP/s", "mfma",
                        "hd256 windowed paged prefill, 1 request of 64 tokens at start 0, "
                        "16Q/8KV, page 16, pool 32 pages (random permutation), window_left "
                        "1023, sm_scale 1, fp32 out"))

    # ---- windowed prefill hd256, batch 8 ----
    if "prefill_window_hd256" in want:
        lens = synth.uniform_lengths(8, 128, 2048, synth.generator(2))
        case = synth.attention_case(2, lens, lens, num_pages=4096, **synth.LOCAL)
        pool = case.pool.to(dev)
        q = case.q.to(dev)
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        plan = plan_of(case.qo_indptr, case.table, 16, 8, 256, 4096)
        pd = psw.pool_desc(pool, num_layers=1, num_pages=4096, page_size=16, num_kv_heads=8,
                           head_dim=256)

        def run(plan=plan, pd=pd, q=q, o=o):
            psw.paged_prefill_window_hd256(plan, pd, 0, q, 1.0, 1023, o)
        rows.append(Row("prefill_window_hd256", run,
                        attention_flops(lens, lens, 16, 256, 1023), "TFLOP/s", "mfma",
                        f"hd256 windowed paged prefill, batch 8, seq_len {lens}, 16Q/8KV, "
                        f"page 16, pool 4096 pages, window_left 1023, sm_scale 1, bf16 out"))
        rows[-1].case = case

    # ---- full prefill hd512, 4 x 4096 ----
    if "prefill_hd512" in want:
        case = synth.attention_case(3, [4096] * 4, [4096] * 4, num_pages=2048, fill_pool=False,
                                    **synth.GLOBAL)
        # fill the pool as serving does, with the hd512 prep writing K and V
        # (V = weightless norm of the raw K) from raw K ~ N(0, 0.25^2)
        pool = torch.zeros(case.pool.numel(), dtype=torch.bfloat16, device=dev)
        pd = psw.pool_desc(pool, num_layers=1, num_pages=2048, page_size=16, num_kv_heads=1,
                           head_dim=512)
        plan = plan_of(case.qo_indptr, case.table, 16, 1, 512, 2048)
        raw_k = synth.normal_bf16((16384, 1, 512), 0.25, synth.generator(33, dev), device=dev)
        w = torch.ones(512, dtype=torch.bfloat16, device=dev)
        c, s = tables(512)
        psw.k_v_norm_rope_paged_prefill_hd512(plan, pd, 0, raw_k, w, c, s, 1e-6)
        q = case.q.to(dev)
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)

        def run(plan=plan, pd=pd, q=q, o=o):
            psw.paged_prefill_hd512(plan, pd, 0, q, 1.0, o)
        rows.append(Row("prefill_hd512", run,
                        attention_flops([4096] * 4, [4096] * 4, 16, 512, -1), "TFLOP/s", "mfma",
                        "hd512 full paged prefill, 4 x 4096 tokens, 16Q/1KV, causal, page 16, "
                        "pool 2048 pages, sm_scale 1, bf16 out"))

    # ---- decode through the prefill entry, 64 requests, both families ----
    if "decode_local_hd256" in want or "decode_global_hd512" in want:
        for d, name in ((256, "decode_local_hd256"), (512, "decode_global_hd512")):
            if name not in want:
                continue
            case = synth.decode_batch(d, dev)
            kv, hkv = case.kv_lens, case.num_kv_heads
            pool = case.pool
            q = case.q.to(dev)
            o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
            plan = plan_of(case.qo_indptr, case.table, 16, hkv, d, 32768)
            pd = psw.pool_desc(pool, num_layers=1, num_pages=32768, page_size=16,
                               num_kv_heads=hkv, head_dim=d)
            wl = 1023 if d == 256 else -1
            if d == 256:
                def run(plan=plan, pd=pd, q=q, o=o):
                    psw.paged_prefill_window_hd256(plan, pd, 0, q, 1.0, 1023, o)
            else:
                def run(plan=plan, pd=pd, q=q, o=o):
                    psw.paged_prefill_hd512(plan, pd, 0, q, 1.0, o)
            rows.append(Row(name, run, decode_bytes(kv, 16, hkv, d, wl), "GB/s", "hbm",
                            f"decode (seq_len 1) hd{d}, 64 requests, KV ~ U[512, 8192], "
                            f"{'window 1023' if wl >= 0 else 'full'}, 32768-page pool", hbm=True))
    return rows


def cpu_model():
    """The host CPU's model string (first "model name" of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_threads():
    """Threads the oracle's array library runs with (its BLAS pool)."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(synth, oracle, case, min_s=10.0, budget_s=25.0):
    """fp64 oracle on the batch-8 windowed workload, request by request
    (shortest first), in whole passes over the batch until at least min_s
    have been spent (or, within a pass, budget_s); returns algorithmic
    TFLOP/s on that sample.  The oracle runs in numpy: its matrix products use
    the BLAS thread pool (sized by the host's environment, e.g.
    OMP_NUM_THREADS), the rest one thread."""
    import torch
    cores = cpu_threads()
    g = oracle.PoolGeometry(1, case.num_pages, 8, 16, 256)
    done, flops, passes = [], 0.0, 0
    t0 = time.perf_counter()
    order = np.argsort(case.qo_lens)       # shortest first so the sample stays bounded
    while time.perf_counter() - t0 < min_s:
        for b in order:
            oracle.paged_attention(case.q, case.pool, g, 0, case.qo_indptr,
                                   case.table.kv_page_indptr, case.table.kv_page_indices,
                                   case.table.kv_last_page_len, 1.0, 1023, requests=[int(b)])
            done.append(int(b))
            flops += attention_flops([case.qo_lens[b]], [case.kv_lens[b]], 16, 256, 1023)
            if time.perf_counter() - t0 > budget_s:
                break
        passes += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    lens = sorted(int(case.qo_lens[b]) for b in set(done))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(done)} request evaluations ({passes} pass(es) over the batch-8 "
                      f"windowed workload, seq_len {lens}), all 16 heads, fp64, {dt:.1f} s",
            "wall_s": round(dt, 3), "os_cpu_count": os.cpu_count(),
            "torch_threads": torch.get_num_threads(), "blas_threads": int(cores),
            "cpu_model": cpu_model()}


def decode_sweep():
    """Split vs direct decode forms over batch x KV length, both families
    (median of 30 launches each, HIP events around the entry call, merge
    included); prints a markdown table."""
    import torch
    import synth
    import paged_sliding_window_page_amd as psw
    dev = torch.device("cuda", 0)
    print("| family | batch | KV keys | split (us) | direct (us) | faster |")
    print("|---|---|---|---|---|---|")
    for hd, geo, wl in ((256, synth.LOCAL, 1023), (512, synth.GLOBAL, -1)):
        for batch in (1, 8, 64):
            for kv in (64, 256, 512, 1024, 2048, 8192):
                case = synth.attention_case(11, [1] * batch, [kv] * batch, fill_pool=False, **geo)
                pool = torch.randn(case.pool.numel(), device=dev).mul_(0.25).to(torch.bfloat16)
                q = case.q.to(dev)
                o = torch.empty(batch, 16, hd, dtype=torch.bfloat16, device=dev)
                plan = psw.Plan(case.qo_indptr, case.table.kv_page_indptr,
                                case.table.kv_page_indices, case.table.kv_last_page_len,
                                num_qo_heads=16, num_kv_heads=geo["num_kv_heads"], head_dim=hd,
                                page_size=16, num_pages=case.num_pages)
                pd = psw.pool_desc(pool, num_layers=1, num_pages=case.num_pages, page_size=16,
                                   num_kv_heads=geo["num_kv_heads"], head_dim=hd)
                res = []
                for mode in (psw.DECODE_SPLIT, psw.DECODE_DIRECT):
                    plan.set_decode_mode(mode)

                    def run():
                        if hd == 256:
                            psw.paged_decode_window_hd256(plan, pd, 0, q, 1.0, wl, o)
                        else:
                            psw.paged_decode_hd512(plan, pd, 0, q, 1.0, o)
                    for _ in range(3):
                        run()
                    ts = []
                    for _ in range(30):
                        a = torch.cuda.Event(enable_timing=True)
                        b = torch.cuda.Event(enable_timing=True)
                        a.record()
                        run()
                        b.record()
                        torch.cuda.synchronize()
                        ts.append(a.elapsed_time(b) * 1e3)
                    res.append(float(np.median(ts)))
                plan.close()
                keys = min(kv, wl + 1) if wl >= 0 else kv
                print(f"| hd{hd} | {batch} | {keys} | {res[0]:.1f} | {res[1]:.1f} | "
                      f"{'direct' if res[1] < res[0] else 'split'} |", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--rows", type=str, default="")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first copy a buffer of this many MiB (device to device) three "
                         "times: the reference for scaling hardware byte counters")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the traffic summary of two rocprofv3 counter runs and exit")
    ap.add_argument("--decode-sweep", action="store_true",
                    help="time the split and direct decode forms over batch x KV length and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        if args.copy_mib <= 0:
            raise SystemExit("--pmc-summary needs the --copy-mib size the runs used")
        print(pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.copy_mib), end="")
        return
    if args.decode_sweep:
        decode_sweep()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import paged_sliding_window_page_amd as psw

    all_rows = ["prep_hd256", "prep_hd512", "prep_q_hd512", "prefill_window_hd256_1x64",
                "prefill_window_hd256", "prefill_hd512", "decode_local_hd256",
                "decode_global_hd512"]
    want = set(args.rows.split(",")) if args.rows else set(all_rows)
    dev = torch.device("cuda", 0)
    # cache flush before every HBM-bound row: a 1 GiB read evicts the L2s and
    # the 256 MB last-level cache.  A read, not a write: rewriting the buffer
    # leaves dirty lines behind whose write-back then lands inside the timed
    # kernel (12.2 vs 16.0 us for the hd512 prep row).
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
    log("building workloads ...")
    rows = build_rows(torch, psw, synth, dev, want)
    rows.sort(key=lambda r: all_rows.index(r.name))
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)   # reads and writes copy_mib MiB
        del src, dst
    torch.cuda.synchronize()
    log("warmup ...")
    for _ in range(args.warmup):
        for r in rows:
            r.run()
    torch.cuda.synchronize()

    # whole-path steps: every row once per step; their wall time is ms_per_step
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for r in rows:
            if r.hbm:
                flush.sum()
            r.run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-row figures: each row launched `steps` times in a block of its own.
    # A row that is not HBM-bound runs its launches back to back between one
    # pair of HIP events: the mean launch duration (an event pair around each
    # launch adds ~2-5 us of dispatch and event overhead to every launch).  An
    # HBM-bound row reads the flush buffer before every launch: it is timed
    # as N x (flush, launch) between one event pair minus N x flush between
    # another (N = max(steps, 30)), which leaves the launches' own duration
    # (it agrees with the kernel trace within ~2%); the median of an event
    # pair around each single launch is reported beside it.  The MFMA-bound
    # prefills take a fixed number of shader cycles per launch, so their
    # times follow the shader clock, which the part sets between about 1.6
    # and 2.1 GHz under load (hardware counters: the hd512 prefill at
    # 1.08-1.26 ms for 2.00-2.03 M cycles); runs that include the HBM-bound
    # rows and their flush reads tend to the lower clocks.
    evs = {r.name: [] for r in rows}
    loops = {}
    n_loop = max(args.steps, 30)
    for r in rows:
        r.run()
        if r.hbm:
            for _ in range(args.steps):
                flush.sum()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                r.run()
                e1.record()
                evs[r.name].append((e0, e1))
            pair = []
            for with_row in (True, False):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(n_loop):
                    flush.sum()
                    if with_row:
                        r.run()
                e1.record()
                pair.append((e0, e1))
            loops[r.name] = pair
        else:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                r.run()
            e1.record()
            evs[r.name].append((e0, e1))
    torch.cuda.synchronize()

    out_rows = {}
    for r in rows:
        ms = np.array([a.elapsed_time(b) for a, b in evs[r.name]])
        if r.hbm:
            (a0, a1), (b0, b1) = loops[r.name]
            t_ms = (a0.elapsed_time(a1) - b0.elapsed_time(b1)) / n_loop
            timing = (f"{n_loop} x (flush, launch) minus {n_loop} x flush, each between one "
                      f"pair of HIP events")
        else:
            t_ms, timing = float(ms[0]) / args.steps, "mean over back-to-back launches"
        rate = r.work / (t_ms * 1e-3) / (1e12 if r.unit == "TFLOP/s" else 1e9)
        peak = PEAK_BF16_TFLOPS if r.unit == "TFLOP/s" else PEAK_HBM_GBS
        out_rows[r.name] = {"achieved": round(rate, 3), "unit": r.unit, "peak": peak,
                            "frac": round(rate / peak, 4), "bound": r.bound,
                            "ms": round(t_ms, 4), "timing": timing,
                            "work": r.work, "workload": r.desc}
        if r.hbm:
            # an event pair around each single launch, dispatch latency included
            out_rows[r.name]["ms_event_median"] = round(float(np.median(ms)), 4)
            out_rows[r.name]["ms_event_p10"] = round(float(np.percentile(ms, 10)), 4)
            out_rows[r.name]["ms_event_p90"] = round(float(np.percentile(ms, 90)), 4)
        log(f"{r.name:24s} {t_ms * 1e3:9.1f} us  {rate:9.2f} {r.unit:8s} "
            f"({100 * rate / peak:5.1f}% of peak)")

    head = "prefill_window_hd256"
    res = {"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded), random page tables",
           "config": {"workload": "hd256 windowed paged prefill, batch 8, seq_len ~ U[128, 2048] "
                                  "(seed 2), 16 Q / 8 KV heads, head_dim 256, page 16, "
                                  "pool 4096 pages, window_left 1023, sm_scale 1",
                      "rows": sorted(out_rows)},
           "rows": out_rows}
    if head in out_rows:
        h = out_rows[head]
        res["value"] = h["achieved"]
        res["roofline"] = {"bound": "mfma", "achieved": h["achieved"], "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": h["frac"],
                           "traffic": read_traffic(HEAD_KERNEL), "kernel": HEAD_KERNEL,
                           "algorithmic_flops_per_launch": h["work"]}
        # the MFMA peak is quoted at the nominal 2.4 GHz; under matrix load the
        # shader clock settles lower, so the clock-adjusted fraction is given too
        mhz = float(np.median([psw.measure_mfma_clock() for _ in range(3)]))
        res["roofline"]["clock_mhz_under_mfma"] = round(mhz, 1)
        res["roofline"]["frac_clock_adjusted"] = round(
            h["achieved"] / (PEAK_BF16_TFLOPS * mhz / NOMINAL_MHZ), 4)
        if not args.no_cpu:
            import oracle
            case = next(r for r in rows if r.name == head).case
            log("timing the fp64 oracle on a bounded sample ...")
            res["cpu_baseline"] = cpu_baseline(synth, oracle, case)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
