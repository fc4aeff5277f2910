"""Throughput of the DSA forward path on one MI355X.

A step is one pass of the whole path over one sequence's queries: pool the
indexer keys, score each query against each pool before it (a chunk of
queries at a time), keep the top-k pools per query (int32 ids), and run
sparse attention over the kept tokens.  Inputs are seeded synthetic tensors
resident in HBM before the timed region (the page's own throughput figures
come from synthetic runs with untrained weights).

Prints one JSON line: queries/s for the whole path, TFLOP/s of the
algorithmic work, the roofline of the dominant kernel (from HIP events around
every launch inside the timed region), and the CPU oracle timed on a bounded
sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
MALL_BYTES = 256 << 20        # MI355X last-level (Infinity) cache
# L2 read bandwidth from the unit counts and clock: 8 XCDs x 16 L2 channels
# x 128 bytes per clock x 2.4 GHz (no published figure; the in-run probe
# reads about 85% of it)
PEAK_L2_GBS = 8 * 16 * 128 * 2.4
METRIC = "DSA fwd queries/sec at S=128k (indexer+topk+attn); TFLOP/s vs MFMA peak"


KERNEL_SOURCES = {
    "index_score": ["index_score.hip", "common.h"],
    "index_score_full": ["index_score.hip", "common.h"],
    "topk_select": ["topk_select.hip", "common.h"],
    "sparse_attn": ["sparse_attn.hip", "common.h"],
    "pool_keys": ["index_score.hip", "common.h"],
    "attn_bwd_dq": ["sparse_attn_bwd.hip", "common.h"],
    "attn_bwd_dkv": ["sparse_attn_bwd.hip", "common.h"],
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "long_context_sparse_dsa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the kernel source as it is now (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return t["hbm_bytes_per_launch"]


KERNEL_KINDS = [("pool_keys", "pool_keys"), ("pack_queries", "pack_queries"),
                ("index_score", "index_score"), ("topk_select", "topk_select"),
                ("sparse_attn_kernel", "sparse_attn"), ("attn_bwd_dq", "attn_bwd_dq"),
                ("bwd_select_bits", "attn_bwd_select"), ("attn_bwd_dkv", "attn_bwd_dkv")]


def kernel_kind(name: str):
    # the bf16 scorer with the correction term (its last template argument,
    # LO, is true) is the library's "index_score_full" kind
    if "index_score_bf16_kernel" in name and name.split("(")[0].rstrip().endswith("true>"):
        return "index_score_full"
    for key, kind in KERNEL_KINDS:
        if key in name:
            return kind
    return None


def _counter_rows(d: str):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"{d}: expected one counter_collection.csv, found {len(files)}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def traffic_summary(workload, fetch_dir, write_dir, cal_fetch_dir, cal_write_dir):
    """HBM bytes per launch and kernel kind from two rocprofv3 runs of one
    bench.py step (--pmc FETCH_SIZE, then --pmc WRITE_SIZE), each scaled by
    what the same counter reads for the 1 GiB copy of --copy-calibration.
    Writes profiles/traffic_<kind>_<workload>.json (read by the bench's
    roofline) and prints the summary table."""
    def per_kind(d, counter):
        tot, n = {}, {}
        for r in _counter_rows(d):
            if r["Counter_Name"] != counter:
                continue
            k = kernel_kind(r["Kernel_Name"])
            if k is None:
                continue
            tot[k] = tot.get(k, 0.0) + float(r["Counter_Value"]) * 1024.0
            n[k] = n.get(k, 0) + 1
        return tot, n

    def calibration(d, counter):
        # the largest single dispatch of the calibration run is the 1 GiB copy
        v = max(float(r["Counter_Value"]) for r in _counter_rows(d) if r["Counter_Name"] == counter)
        return (1 << 30) / (v * 1024.0)
    ff, wf = calibration(cal_fetch_dir, "FETCH_SIZE"), calibration(cal_write_dir, "WRITE_SIZE")
    fb, fn = per_kind(fetch_dir, "FETCH_SIZE")
    wb, _ = per_kind(write_dir, "WRITE_SIZE")
    print(f"FETCH_SIZE factor {ff:.4f}, WRITE_SIZE factor {wf:.4f} (1 GiB copy)\n")
    print("| kernel | launches | fetched B/launch (calibrated) | written B/launch (calibrated) |")
    print("|---|---|---|---|")
    order = [kind for _, kind in KERNEL_KINDS]
    order.insert(order.index("index_score") + 1, "index_score_full")
    for k in [kind for kind in order if kind in fb]:
        f = fb[k] * ff / fn[k]
        w = wb.get(k, 0.0) * wf / fn[k]
        print(f"| {k} | {fn[k]} | {f:.4g} | {w:.4g} |")
        if k in KERNEL_SOURCES:
            with open(os.path.join(ROOT, "profiles", f"traffic_{k}_{workload}.json"), "w") as fh:
                json.dump({"kernel": k, "workload": workload, "launches_per_step": fn[k],
                           "fetch_bytes_per_launch": f, "write_bytes_per_launch": w,
                           "hbm_bytes_per_launch": f + w, "fetch_factor": ff, "write_factor": wf,
                           "source_sha256": kernel_source_hash(k),
                           "summary": f"profiles/l2_egress_traffic_{workload}.md"}, fh, indent=1)


def trace_summary(d):
    """Markdown table of a rocprofv3 --kernel-trace --stats run."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"{d}: expected one kernel_stats.csv, found {len(files)}")
    with open(files[0]) as fh:
        rows = list(csv.DictReader(fh))
    print("| kernel | calls | total ms | average us | min us | max us | % |")
    print("|---|---|---|---|---|---|---|")
    for r in rows:
        name = r["Name"].replace("dsa::(anonymous namespace)::", "").replace("dsa::", "")
        name = name[:90]
        print(f"| `{name}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
              f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
              f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")


def copy_calibration():
    """A plain device copy of known size, for scaling the FETCH_SIZE and
    WRITE_SIZE counters: the counter values of this run divided by the bytes
    copied give the factor."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n,
                      "launches": 3}), flush=True)


def measure_peaks():
    """The chip's sustained rates on this machine, from the probes in
    libdsa_peaks.so (a bf16 and an fp8 matrix-core loop, a 1 GiB device
    copy), each the best of three launches timed with events on the current
    stream.  Reported beside the published peaks; the roofline fractions stay
    against the published ones."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "long_context_sparse_dsa_amd", "libdsa_peaks.so"))
    lib.dsa_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    lib.dsa_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.c_void_p]
    lib.dsa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    sink = torch.empty(1024 * 256, dtype=torch.float32, device="cuda")
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)

    def best(launch):
        rates = []
        for rep in range(4):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            work = launch()
            b.record(stream)
            b.synchronize()
            if rep:  # the first launch warms up
                rates.append(work / (a.elapsed_time(b) * 1e-3))
        return max(rates)

    def mfma(kind):
        fl = ctypes.c_double(0)
        if lib.dsa_probe_mfma(kind, 40000, ctypes.c_void_p(sink.data_ptr()), ctypes.byref(fl), sp):
            raise RuntimeError("mfma probe launch failed")
        return fl.value

    def copy():
        if lib.dsa_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n,
                              sp):
            raise RuntimeError("copy probe launch failed")
        return 2.0 * n
    def read(buf, nbytes, passes):
        if lib.dsa_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, passes,
                              ctypes.c_void_p(sink.data_ptr()), sp):
            raise RuntimeError("read probe launch failed")
        return float(nbytes) * passes
    l2_bytes = 16 << 20  # 2 MiB per XCD of the 4 MiB L2s
    out = {"mfma_bf16_tflops": best(lambda: mfma(0)) / 1e12,
           "mfma_fp8_tflops": best(lambda: mfma(1)) / 1e12,
           "copy_read_plus_write_gbs": best(copy) / 1e9,
           "l2_read_gbs": best(lambda: read(src, l2_bytes, 256)) / 1e9,
           "hbm_read_gbs": best(lambda: read(src, n, 4)) / 1e9,
           "published": {"mfma_bf16_tflops": PEAK_BF16_TFLOPS, "mfma_fp8_tflops": PEAK_FP8_TFLOPS,
                         "hbm_gbs": PEAK_HBM_GBS},
           "probe": "matrix-core loops (bf16 32x32x16, scaled fp8 32x32x64; 4 independent "
                    "chains per wave, 4 waves per SIMD), a 1 GiB device copy, 256 passes of "
                    "reads over 16 MiB (L2-resident) and 4 passes over 1 GiB (memory), best "
                    "of 3 launches after a warm-up"}
    del src, dst, sink
    return out


def step_stats(times_ms):
    t = sorted(times_ms)
    return {"ms_per_step_median": t[len(t) // 2] if len(t) % 2 else 0.5 * (t[len(t) // 2 - 1]
                                                                          + t[len(t) // 2]),
            "ms_per_step_min": t[0]}


def score_paths(wl, chunk_q, fp8):
    """Per query chunk of the indexer call without score_out: which scorer
    kernel the library runs.  Mirrors the library's rule (bf16 chunks whose
    first and last rows together see more than 32 k pools are scored without
    the correction term and bounded; chunks whose rows all see at most k
    pools are not scored).  Returns (bounded chunks, full chunks, pairs of
    each); the bench checks the launch counts against the library's."""
    nb = nf = 0
    pb = pf = 0
    for c0 in range(0, wl.s_q, chunk_q):
        rows = min(chunk_q, wl.s_q - c0)
        t = wl.q_pos0 + c0 + np.arange(rows, dtype=np.int64)
        n = np.minimum(t // 4, wl.n_pools)
        if n[-1] == 0 or n[-1] <= wl.k_pools:
            continue
        if not fp8 and n[0] + n[-1] > 2 * 16 * wl.k_pools:
            nb, pb = nb + 1, pb + int(n.sum())
        elif fp8:
            nb, pb = nb + 1, pb + int(n.sum())
        else:
            nf, pf = nf + 1, pf + int(n.sum())
    return nb, nf, pb, pf


def work_counts(wl):
    """Algorithmic work of one step (closed forms over the query positions)."""
    t = wl.q_pos0 + np.arange(wl.s_q, dtype=np.int64)
    n = np.minimum(t // 4, wl.n_pools)
    pairs = int(n.sum())
    kept = np.minimum(n, wl.k_pools)
    tail = np.minimum(wl.n_tail, t % 4) if wl.n_tail else np.zeros_like(t)
    if wl.n_tail:
        tail = np.where(t - 1 < wl.s_k, tail, 0)
    tokens = int((4 * kept + tail).sum())
    f_score = 2.0 * wl.h_idx * wl.d_idx * pairs
    f_attn = 2.0 * wl.h * (wl.d + wl.dv) * tokens
    b_attn = (tokens * (wl.d + wl.dv) * 2 + wl.s_q * wl.h * (wl.d + wl.dv) * 2
              + wl.s_q * wl.k_pools * 4)
    b_select = pairs * 4 + wl.s_q * wl.k_pools * 4
    b_pool = wl.n_pools * 4 * wl.d_idx * 2 + wl.n_pools * 4 * wl.d_idx * 2
    # attention backward, per token visit: the query-major pass recomputes
    # S = q k^T and dP = dout v^T and forms dq += dS k; the key-major pass
    # recomputes S and dP and forms dk += dS^T q and dv += P^T dout
    f_bwd_dq = 2.0 * wl.h * (2 * wl.d + wl.dv) * tokens
    f_bwd_dkv = 2.0 * wl.h * (2 * wl.d + 2 * wl.dv) * tokens
    # query-major pass bytes: the gathered key and value rows, q, out, dout,
    # lse, ids, and dq written in fp32
    b_bwd_dq = (tokens * (wl.d + wl.dv) * 2 + wl.s_q * wl.h * (wl.d + 2 * wl.dv) * 2
                + wl.s_q * wl.h * 4 + wl.s_q * wl.k_pools * 4 + wl.s_q * wl.h * wl.d * 4)
    return dict(pairs=pairs, tokens=tokens, f_score=f_score, f_attn=f_attn, b_attn=b_attn,
                b_select=b_select, b_pool=b_pool, f_bwd_dq=f_bwd_dq, f_bwd_dkv=f_bwd_dkv,
                b_bwd_dq=b_bwd_dq)


def cpu_baseline(wl, x, target_s: float, gate=None, fp8=False, gpu=None):
    """The oracle as it stands, on a strided sample of query rows.

    gpu (optional): host copies of the timed run's ids ("idx") and attention
    output ("out").  The oracle's ids of the sampled rows are then compared
    with them under the boundary rule of the test suite, and the oracle's
    attention on the GPU's ids with the GPU's output, so the line carries the
    parity of the very call it timed (returned as a second value)."""
    from oracle import oracle
    threads = os.cpu_count() or 1
    last = {}

    def run(rows):
        t0 = time.perf_counter()
        if fp8:
            idx, _ = oracle.index_topk_fp8(x["q_idx8"], x["k_idx8"], x["w"], wl.k_pools,
                                           q_pos0=wl.q_pos0, rows=rows, gate=gate)
        else:
            idx, _ = oracle.index_topk(x["q_idx"], x["k_idx"], x["w"], wl.k_pools,
                                       q_pos0=wl.q_pos0, rows=rows, gate=gate)
        oracle.sparse_attn(x["q"], x["k"], x["v"], idx, wl.k_pools, q_pos0=wl.q_pos0, rows=rows,
                           n_tail=wl.n_tail, scale=float(np.float32(1 / math.sqrt(wl.d))))
        last["rows"], last["idx"] = rows, idx
        return time.perf_counter() - t0

    def strided(r):
        return np.linspace(0, wl.s_q - 1, r).round().astype(np.int64)

    # two probes separate the fixed cost (pooling every key) from the
    # per-row cost, so that the timed sample lands near target_s
    probe = max(threads, 8)
    t1 = run(strided(probe))
    t4 = run(strided(4 * probe))
    per_row = max((t4 - t1) / (3 * probe), 1e-6)
    fixed = max(t1 - probe * per_row, 0.0)
    r = int(max(probe, min(wl.s_q, (target_s - fixed) / per_row)))
    rows = strided(r)
    t = run(rows)
    base = {"value": r / t, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{r} query rows evenly spaced over the {wl.s_q} queries of {wl.name} "
                      f"(pooling of all keys included), {t:.1f} s"}
    if gpu is None:
        return base, None
    return base, timed_call_parity(wl, x, gate, fp8, gpu, last["rows"], last["idx"])


def timed_call_parity(wl, x, gate, fp8, gpu, rows, ora_idx):
    """Boundary-rule comparison of the timed call's ids with the oracle's on
    the baseline's rows, the structural check of every id row, and the
    attention output on up to 256 of the rows (oracle fed the GPU's ids)."""
    from oracle import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import parity
    pos = wl.q_pos0 + np.arange(wl.s_q)
    out = {"rows": int(len(rows)), "rule": "ids equal the oracle's except pools within "
           "1e-3 |s_k| + 1e-6 max s of the k-th score; attention within 2e-2 absolute"}
    try:
        parity.validate_index_rows(gpu["idx"], pos, wl.n_pools, wl.k_pools)
        g = gpu["idx"][rows]
        differ = np.array([set(a.tolist()) != set(b.tolist()) for a, b in zip(g, ora_idx)])
        st = {"swaps": 0, "rows_with_swaps": 0, "worst_row": 0}
        if differ.any():
            # dense oracle scores only for the rows whose sets differ
            dr = rows[differ]
            if fp8:
                s_o = oracle.index_scores_fp8(x["q_idx8"], x["k_idx8"], x["w"], q_pos0=wl.q_pos0,
                                              rows=dr, gate=gate)
            else:
                s_o = oracle.index_scores(x["q_idx"], x["k_idx"], x["w"], q_pos0=wl.q_pos0,
                                          rows=dr, gate=gate)
            st = parity.check_index_rows(g[differ], ora_idx[differ], s_o, wl.q_pos0 + dr,
                                         wl.n_pools, wl.k_pools)
        out.update(swaps=st["swaps"], rows_with_swaps=st["rows_with_swaps"],
                   worst_row=st["worst_row"])
        ar = rows[np.linspace(0, len(rows) - 1, min(256, len(rows))).round().astype(np.int64)]
        o_o, lse_o = oracle.sparse_attn(x["q"], x["k"], x["v"], gpu["idx"][ar], wl.k_pools,
                                        q_pos0=wl.q_pos0, rows=ar, n_tail=wl.n_tail,
                                        scale=float(np.float32(1 / math.sqrt(wl.d))))
        err = np.abs(gpu["out"][ar].astype(np.float64) - o_o).max()
        assert err <= parity.ATTN_ABS, f"attention error {err}"
        out.update(attn_rows=int(len(ar)), attn_max_abs_err=float(err), ok=True)
    except AssertionError as e:
        out.update(ok=False, error=str(e)[:300])
    return out


def backward(args, wl, x, g, gate, chunk_q, ws, idx, out, stream):
    """Times dsa_sparse_attn_bwd on the ids, output and lse of one forward
    pass of the same workload (made before the timed region)."""
    import torch
    from long_context_sparse_dsa_amd import dsa, inputs
    if gate is None:
        dsa.dsa_index_score_topk(g["q_idx"], g["k_idx"], g["w"], wl.k_pools, q_pos0=wl.q_pos0,
                                 chunk_q=chunk_q, idx_out=idx, workspace=ws, stream=stream)
    else:
        dsa.dsa_index_score_topk_gated(g["q_idx"], g["k_idx"], gate, g["w"], wl.k_pools,
                                       q_pos0=wl.q_pos0, chunk_q=chunk_q, idx_out=idx,
                                       workspace=ws, stream=stream)
    o, lse = dsa.dsa_sparse_attn_fwd(g["q"], g["k"], g["v"], idx, q_pos0=wl.q_pos0,
                                     n_tail=wl.n_tail, out=out, want_lse=True, stream=stream)
    dout = inputs.make_dout(wl).to(o.device)
    del ws
    dev = o.device
    dq = torch.empty((wl.s_q, wl.h, wl.d), dtype=torch.float32, device=dev)
    dk = torch.empty((wl.s_k, wl.d), dtype=torch.float32, device=dev)
    dv = torch.empty((wl.s_k, wl.dv), dtype=torch.float32, device=dev)
    nbytes, bwd_chunk = dsa.dsa_sparse_attn_bwd_workspace_size(wl.s_q, wl.s_k, wl.h,
                                                               args.bwd_chunk_q)
    bws = dsa.new_workspace(nbytes, dev)

    def step():
        dsa.dsa_sparse_attn_bwd(g["q"], g["k"], g["v"], idx, o, dout, lse, q_pos0=wl.q_pos0,
                                n_tail=wl.n_tail, chunk_q=bwd_chunk, dq=dq, dk=dk, dv=dv,
                                workspace=bws, stream=stream)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")
    dsa.dsa_profile_read()
    dsa.dsa_profile_enable(True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dsa.dsa_profile_enable(False)
    stats = dsa.dsa_profile_read()
    ms = (t1 - t0) * 1e3 / args.steps
    per_step = step_stats([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    log(f"timed {args.steps} backward steps: {ms:.3f} ms/step ({per_step}); kernels {stats}")
    w = work_counts(wl)
    stages = {}
    for name, (launches, total) in stats.items():
        st = {"ms_per_step": total / args.steps, "launches_per_step": launches / args.steps}
        t_s = total / 1e3
        if name == "attn_bwd_dq":
            # the forward's gather: served by the L2s when every key and
            # value row fits the last-level cache, else by memory
            a = w["b_bwd_dq"] * args.steps / t_s / 1e9
            l2 = wl.s_k * (wl.d + wl.dv) * 2 <= MALL_BYTES
            peak = PEAK_L2_GBS if l2 else PEAK_HBM_GBS
            st.update(bound="l2" if l2 else "hbm", achieved=a, peak=peak, unit="GB/s",
                      frac=a / peak, tflops=w["f_bwd_dq"] * args.steps / t_s / 1e12)
        elif name == "attn_bwd_dkv":
            a = w["f_bwd_dkv"] * args.steps / t_s / 1e12
            st.update(bound="mfma", achieved=a, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                      frac=a / PEAK_BF16_TFLOPS)
        if "bound" in st:
            st["traffic"] = measured_traffic(name, wl.name)
            st["source_sha256"] = kernel_source_hash(name)
        stages[name] = st
    dominant = max(stats, key=lambda k: stats[k][1]) if stats else None
    flops = w["f_bwd_dq"] + w["f_bwd_dkv"]
    result = {
        "metric": "DSA sparse-attention backward queries/sec (dq, dk, dv)",
        "value": wl.s_q / (ms / 1e3), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, **per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "s_q": wl.s_q, "s_k": wl.s_k, "q_pos0": wl.q_pos0,
                   "k_pools": wl.k_pools, "attention": f"{wl.h}x{wl.d}", "kv_heads": 1,
                   "n_tail": wl.n_tail, "bwd_chunk_q": bwd_chunk},
        "tflops": flops / (ms / 1e3) / 1e12,
        "roofline": dict(stages[dominant], kernel=dominant) if dominant in stages
        and "bound" in stages[dominant] else None,
        "stages": stages,
        "work": {"tokens": w["tokens"], "f_bwd_dq": w["f_bwd_dq"], "f_bwd_dkv": w["f_bwd_dkv"],
                 "b_bwd_dq": w["b_bwd_dq"]},
        "peak_mem_gib": torch.cuda.max_memory_allocated() / 2 ** 30,
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="s128k")
    ap.add_argument("--chunk-q", type=int, default=0)
    ap.add_argument("--bwd-chunk-q", type=int, default=0,
                    help="queries per transposition chunk of the backward (0 = the library's "
                         "default)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the in-run matrix-core and copy probes")
    ap.add_argument("--gated", action="store_true",
                    help="gated pooling: per-token k-pool gates weight each key of a pool")
    ap.add_argument("--fp8", action="store_true",
                    help="the fp8 E4M3 indexer (workloads that carry E4M3 indexer inputs)")
    ap.add_argument("--backward", action="store_true",
                    help="time the sparse-attention backward (dq, dk, dv) instead of the "
                         "forward path; the forward's ids, output and lse are made first")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR",
                                                           "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                    help="(host only) turn rocprofv3 FETCH_SIZE / WRITE_SIZE runs of one step "
                         "of --workload into profiles/traffic_<kernel>_<workload>.json")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="(host only) table of a rocprofv3 --kernel-trace --stats run")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.traffic_summary:
        traffic_summary(args.workload, *args.traffic_summary)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_sparse_dsa_amd import dsa, inputs

    wl = inputs.WORKLOADS[args.workload]
    dsa.load_library()
    dev = torch.device("cuda")
    log(f"workload {wl}")
    t0 = time.time()
    x = inputs.make_inputs(wl)
    log(f"inputs generated in {time.time() - t0:.1f} s")
    if args.fp8 and "q_idx8" not in x:
        print(f"workload {wl.name} has no fp8 indexer inputs", file=sys.stderr)
        sys.exit(2)
    g = {k: v.to(dev) for k, v in x.items() if not k.endswith("8")}
    if args.fp8:
        g["q_idx"], g["k_idx"] = x["q_idx8"].to(dev), x["k_idx8"].to(dev)
    gate = inputs.make_gates(wl).to(dev) if args.gated else None
    ws_bytes, chunk_q = dsa.dsa_index_workspace_size(
        wl.s_q, wl.s_k, wl.h_idx, wl.d_idx, wl.k_pools, 4, args.chunk_q,
        dsa.DSA_FP8_E4M3 if args.fp8 else dsa.DSA_BF16)
    ws = dsa.new_workspace(ws_bytes, dev)
    idx = torch.empty((wl.s_q, wl.k_pools), dtype=torch.int32, device=dev)
    out = torch.empty((wl.s_q, wl.h, wl.dv), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    if args.backward:
        backward(args, wl, x, g, gate, chunk_q, ws, idx, out, stream)
        return

    def step():
        if gate is None:
            dsa.dsa_index_score_topk(g["q_idx"], g["k_idx"], g["w"], wl.k_pools,
                                     q_pos0=wl.q_pos0, chunk_q=chunk_q, idx_out=idx,
                                     workspace=ws, stream=stream)
        else:
            dsa.dsa_index_score_topk_gated(g["q_idx"], g["k_idx"], gate, g["w"], wl.k_pools,
                                           q_pos0=wl.q_pos0, chunk_q=chunk_q, idx_out=idx,
                                           workspace=ws, stream=stream)
        dsa.dsa_sparse_attn_fwd(g["q"], g["k"], g["v"], idx, q_pos0=wl.q_pos0,
                                n_tail=wl.n_tail, out=out, stream=stream)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")
    dsa.dsa_profile_read()
    dsa.dsa_profile_enable(True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dsa.dsa_profile_enable(False)
    stats = dsa.dsa_profile_read()
    ms = (t1 - t0) * 1e3 / args.steps
    per_step = step_stats([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    log(f"timed {args.steps} steps: {ms:.3f} ms/step ({per_step}); kernels {stats}")

    w = work_counts(wl)
    qps = wl.s_q / (ms / 1e3)
    tflops = (w["f_score"] + w["f_attn"]) / (ms / 1e3) / 1e12
    # the two scorer kernels and their algorithmic flops
    nb, nf, pb, pf = score_paths(wl, chunk_q, args.fp8)
    f_path = {"index_score": 2.0 * wl.h_idx * wl.d_idx * pb,
              "index_score_full": 2.0 * wl.h_idx * wl.d_idx * pf}
    for name, n_exp in (("index_score", nb), ("index_score_full", nf)):
        got = stats.get(name, (0, 0.0))[0]
        if got != n_exp * args.steps:
            raise SystemExit(f"{name}: {got} launches in {args.steps} steps, expected "
                             f"{n_exp * args.steps} (the scorer path rule changed?)")
    stages = {}
    for name, (launches, total) in stats.items():
        stages[name] = {"ms_per_step": total / args.steps, "launches_per_step": launches / args.steps}
    rl = {}
    for name, (launches, total) in stats.items():
        t_s = total / 1e3
        if name in f_path:
            a = f_path[name] * args.steps / t_s / 1e12
            peak = PEAK_FP8_TFLOPS if args.fp8 else PEAK_BF16_TFLOPS
            rl[name] = {"bound": "mfma", "achieved": a, "peak": peak,
                        "unit": "TFLOP/s", "frac": a / peak, "traffic": None}
        elif name == "sparse_attn":
            a = w["b_attn"] * args.steps / t_s / 1e9
            if wl.s_k * (wl.d + wl.dv) * 2 <= MALL_BYTES:
                # every gathered key/value row is cache-resident: counters
                # show the gather served by the L2s (one L2 request per
                # 128-byte line of a gathered row, 89% hits at 128k), so
                # the roof is the L2 read bandwidth
                f = w["f_attn"] * args.steps / t_s / 1e12
                rl[name] = {"bound": "l2", "achieved": a, "peak": PEAK_L2_GBS, "unit": "GB/s",
                            "frac": a / PEAK_L2_GBS, "traffic": None, "tflops": f}
            else:
                rl[name] = {"bound": "hbm", "achieved": a, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": a / PEAK_HBM_GBS, "traffic": None}
        elif name == "topk_select":
            a = w["b_select"] * args.steps / t_s / 1e9
            rl[name] = {"bound": "hbm", "achieved": a, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": a / PEAK_HBM_GBS, "traffic": None}
        elif name == "pool_keys":
            a = w["b_pool"] * args.steps / t_s / 1e9
            rl[name] = {"bound": "hbm", "achieved": a, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": a / PEAK_HBM_GBS, "traffic": None}
        if name in rl:
            rl[name]["traffic"] = None if args.fp8 or args.gated else \
                measured_traffic(name, wl.name)
            rl[name]["source_sha256"] = kernel_source_hash(name)
        stages[name].update(rl.get(name, {}))
    dominant = max(stats, key=lambda k: stats[k][1]) if stats else None

    result = {
        "metric": METRIC, "value": qps, "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "s_q": wl.s_q, "s_k": wl.s_k, "q_pos0": wl.q_pos0,
                   "indexer": f"{wl.h_idx}x{wl.d_idx}", "pool": 4, "k_pools": wl.k_pools,
                   "attention": f"{wl.h}x{wl.d}", "kv_heads": 1, "n_tail": wl.n_tail,
                   "chunk_q": chunk_q, "pooling": "gated" if args.gated else "mean",
                   "indexer_dtype": "e4m3" if args.fp8 else "bf16"},
        **per_step,
        "tflops": tflops, "tflops_frac_of_bf16_peak": tflops / PEAK_BF16_TFLOPS,
        "roofline": dict(rl[dominant], kernel=dominant) if dominant in rl else None,
        "stages": stages,
        "work": {"pairs": w["pairs"], "tokens": w["tokens"], "f_score": w["f_score"],
                 "f_score_bounded": f_path["index_score"],
                 "f_score_full": f_path["index_score_full"],
                 "f_attn": w["f_attn"], "b_attn": w["b_attn"], "b_select": w["b_select"]},
        "peak_mem_gib": torch.cuda.max_memory_allocated() / 2 ** 30,
    }
    if not args.no_peaks:
        result["peaks_measured"] = pk = measure_peaks()
        log(f"measured peaks: {pk}")
        # each stage's rate against the probe of its own roof, too
        probe_of = {"mfma": "mfma_fp8_tflops" if args.fp8 else "mfma_bf16_tflops",
                    "hbm": "hbm_read_gbs", "l2": "l2_read_gbs"}
        for st in stages.values():
            if "bound" in st and st["bound"] in probe_of:
                if st["bound"] == "mfma" and st is not stages.get("index_score") \
                        and st is not stages.get("index_score_full"):
                    continue
                st["frac_of_measured_peak"] = st["achieved"] / pk[probe_of[st["bound"]]]
        if result["roofline"] is not None:
            result["roofline"]["frac_of_measured_peak"] = \
                stages[result["roofline"]["kernel"]].get("frac_of_measured_peak")
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        gpu_out = {"idx": idx.cpu().numpy(), "out": out.float().cpu().numpy()}
        result["cpu_baseline"], result["parity"] = cpu_baseline(
            wl, x, args.cpu_seconds, None if gate is None else gate.cpu().numpy(), fp8=args.fp8,
            gpu=gpu_out)
        log(f"parity of the timed call: {result['parity']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
