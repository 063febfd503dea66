"""Benchmark of the MSA forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload chunk_16k_at_1m]
                    [--sched auto|kv_outer|q_outer] [--no-cpu] [--no-legs] [--no-decode] [--no-train]
                    [--no-topk] [--crossover]
    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR --pmc-kernel K --pmc-workload W   (no GPU)
    python bench.py --summarize-stats STATS_DIR                                          (no GPU)

One step = msa_forward (index scores + Top-k, inversion, attention, combine)
over one batch of the seeded synthetic workload, inputs already in HBM.
``value`` is the metric "effective TFLOP/s over the selected tokens": 4*d
flops per (query head, selected visible key) -- what the attention computes
-- divided by the whole forward step time, on the 1M-token-context workload
(16384 new queries at the end of a 1,048,576-token cache).  Each timed step
is preceded by a 1 GiB scrub write, so it starts with cold caches; the same
steps back to back (warm) are reported beside it.

Also on the line, never as ``value``:
  * ``roofline`` of the dominant kernel of the headline step against its
    bound (the index tile: MFMA, with the method's flops), with
    ``frac_of_achievable`` against ``achievable_peaks``: what a 2 GiB device
    copy, a 2 GiB fill and the library's best bf16 matmul (of three shapes)
    reach on the same GPU;
  * ``selection_check``: the GPU's selection of sampled rows against the
    fp64 oracle (exact, tie-band and failing rows);
  * legs: prefill_32k and the skewed 128k prefill (with block-popularity
    figures), the decode step (16 sequences x 1M tokens; microseconds per
    token), the standalone Top-k, the training kernels;
  * ``cpu_baseline``: the oracle timed on a bounded sample of the headline
    workload, on all host threads and on one; the oracle's selection checks
    of the headline and of each prefill leg are made in this leg (and skipped
    with it, --no-cpu).
Per-kernel times come from hipEvents that libmsa records around each launch
on the launch stream.
"""
import argparse
import csv
import gc
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MSA fwd effective TFLOP/s (selected tokens) & decode µs/token @1M ctx"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
HEADLINE = "chunk_16k_at_1m"
SCRUB_BYTES = 1 << 30


# ---- work and bytes of the method ------------------------------------------

def selected_tokens(wl, ids):
    """Sum over (b, i, g) of the visible tokens of the selected blocks."""
    Bk = wl.block_size
    pos = wl.q_offset + torch.arange(wl.n_q, device=ids.device, dtype=torch.int64).view(1, -1, 1, 1)
    j = ids.to(torch.int64)
    start = j * Bk
    n = torch.minimum(pos - start + 1, torch.full_like(start, Bk))
    n = torch.minimum(n, wl.n_k - start)
    n = torch.where(j >= 0, n.clamp(min=0), torch.zeros_like(n))
    return int(n.sum().item())


def attention_flops(wl, ids):
    """4*d per (query head, selected visible key): QK^T and PV."""
    G = wl.h_q // wl.h_kv
    return 4.0 * wl.d * G * selected_tokens(wl, ids)


def index_flops(wl):
    """2*d_idx per (query, group, candidate key): every token of the blocks j < L(i)."""
    L = (wl.q_offset + np.arange(wl.n_q, dtype=np.int64)) // wl.block_size
    return 2.0 * wl.d_idx * wl.h_kv * wl.batch * float(L.sum()) * wl.block_size


def method_bytes(wl, ids):
    """HBM bytes the attention step cannot avoid: Q in, every selected K/V
    block once per (b, g), O and lse out."""
    e = 2 if wl.dtype == "bf16" else 4
    valid = ids >= 0
    flat = (torch.arange(wl.batch * wl.h_kv, device=ids.device).view(wl.batch, 1, wl.h_kv, 1) * wl.nblk
            + ids.clamp(min=0).long())
    uniq = int(torch.unique(flat[valid]).numel())
    q = wl.batch * wl.n_q * wl.h_q * wl.d * e
    kv = uniq * wl.block_size * wl.d * e * 2
    o = wl.batch * wl.n_q * wl.h_q * (wl.d * e + 4)
    return q + kv + o


def impl_bytes(wl, ids):
    """What this implementation's KV-outer pass and combine move by design
    (each selected (query, group, block) reads the group's G query rows and
    writes G partial rows; the combine reads the partials back)."""
    e = 2 if wl.dtype == "bf16" else 4
    G = wl.h_q // wl.h_kv
    nnz = int((ids >= 0).sum().item())
    part_row = wl.d * e + 4
    return {"attn_kvouter": nnz * G * (wl.d * e + part_row), "combine": nnz * G * part_row}


# ---- timing ----------------------------------------------------------------

def _scrub_buffer():
    return torch.empty(SCRUB_BYTES, dtype=torch.uint8, device="cuda")


_LAST_STEP_MS = []  # per-step times of the last cold (scrubbed) timing


def step_spread(per):
    """min / median / max of per-step times (ms)."""
    return {"min": float(np.min(per)), "median": float(np.median(per)), "max": float(np.max(per)),
            "steps": len(per)} if per else None


def time_steps(fn, steps, warmup, scrub=None):
    """Warm-up, then exactly `steps` timed calls of fn between two device
    synchronisations.  With `scrub`, each call is preceded by a 1 GiB write
    (cold caches) and only the calls are timed (events around each); without,
    the calls run back to back.  Returns (ms per step, wall ms per step,
    {kernel: (avg ms per launch, launches per step)})."""
    from block_sparse_long_bk_amd import api
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    api.profile_reset()
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    api.profile_enable(True)
    t0 = time.perf_counter()
    if scrub is None:
        ev[0][0].record(st)
        for _ in range(steps):
            fn()
        ev[-1][1].record(st)
    else:
        for a, b in ev:
            api.profile_enable(False)
            scrub.fill_(1)
            api.profile_enable(True)
            a.record(st)
            fn()
            b.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    api.profile_enable(False)
    if scrub is None:
        ms = ev[0][0].elapsed_time(ev[-1][1]) / steps
    else:
        per = [a.elapsed_time(b) for a, b in ev]
        _LAST_STEP_MS[:] = per
        ms = float(np.mean(per))
    kern = {k: (t / n, n / steps) for k, (t, n) in api.profile_read().items() if n}
    return ms, wall * 1e3 / steps, kern


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


TRAFFIC_SOURCES = {
    "index_tile_topk": ["block_sparse_long_bk_amd/csrc/index.hip", "block_sparse_long_bk_amd/csrc/msa_device.h",
                        "block_sparse_long_bk_amd/csrc/msa_internal.h"],
    "attn_kvouter": ["block_sparse_long_bk_amd/csrc/attention.hip", "block_sparse_long_bk_amd/csrc/attn_common.h",
                     "block_sparse_long_bk_amd/csrc/msa_device.h", "block_sparse_long_bk_amd/csrc/msa_internal.h"],
}
# rocprofv3 kernel names of the profiled launch names
TRACE_NAME = {"index_tile_topk": "k_index_tile", "attn_kvouter": "k_attn_kvouter", "combine": "k_combine",
              "index_scan": "k_index_scan", "topk_rows": "k_topk", "attn_qouter": "k_attn_qouter"}


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source (else None)."""
    try:
        rec = json.load(open(os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash(rec.get("sources", [])):
        return None
    return rec.get("bytes_per_launch")


def roofline(kernel, avg_ms, *, flops=None, nbytes=None, peak_tflops=PEAK_BF16_TFLOPS, workload=None, method=None):
    """Roofline entry of one kernel: MFMA-bound with the method's flops, or
    HBM-bound with the method's bytes, per launch over its measured average."""
    if flops is not None:
        ach = flops / avg_ms / 1e9
        r = {"bound": "mfma", "achieved": ach, "peak": peak_tflops, "unit": "TFLOP/s", "frac": ach / peak_tflops,
             "method_flops_per_launch": flops}
    else:
        ach = nbytes / avg_ms / 1e6
        r = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
             "method_bytes_per_launch": nbytes}
    r["kernel"] = kernel
    r["avg_launch_ms"] = avg_ms
    tr = measured_traffic(kernel, workload) if workload else None
    r["traffic"] = tr
    if tr is not None and method:
        r["traffic_over_method_bytes"] = tr / method
    return r


# ---- the oracle on sampled rows ----------------------------------------------

def sample_queries(wl, n):
    """Evenly spaced queries plus the first, the last and those around block
    boundaries."""
    Bk = wl.block_size
    qs = set(np.linspace(0, wl.n_q - 1, max(n - 8, 2)).astype(int).tolist()) | {0, wl.n_q - 1}
    for p in np.linspace(wl.q_offset, wl.q_offset + wl.n_q - 1, 3).astype(int):
        b = (p // Bk) * Bk
        for pos in (b - 1, b, b + 1):
            if wl.q_offset <= pos < wl.q_offset + wl.n_q:
                qs.add(int(pos - wl.q_offset))
    return np.array(sorted(qs)[:max(n, 2)], dtype=np.int64)


def oracle_rows(wl, x_host, qi, threads=None):
    """Index scores, selection and attention of the rows (0, qi) in fp64.
    Returns (ids, scores, seconds, flops of the attention over those rows)."""
    from oracle import oracle as O
    if threads:
        O.set_num_threads(threads)
    prob = O.problem_of(wl.with_(batch=1))
    rows = np.stack([np.zeros_like(qi), qi], axis=1)
    t0 = time.perf_counter()
    s = O.block_scores(prob, x_host["iq"], x_host["ik"], rows)
    ids = O.select(prob, s, rows)
    O.attend(prob, x_host["q"], x_host["k"], x_host["v"], ids, rows)
    dt = time.perf_counter() - t0
    pos = torch.from_numpy(wl.q_offset + qi).view(-1, 1, 1)
    j = torch.from_numpy(ids).to(torch.int64)
    n = torch.minimum(pos - j * wl.block_size + 1, torch.full_like(j, wl.block_size))
    n = torch.where(j >= 0, n.clamp(min=0), torch.zeros_like(n))
    flops = 4.0 * wl.d * (wl.h_q // wl.h_kv) * float(n.sum())
    return ids, s, dt, flops


def host_inputs(x):
    return {k: v[:1].cpu() for k, v in x.items()}


def selection_check(wl, ids_gpu, qi, ids_o, s_o):
    from tests.parity import check_selection
    got = ids_gpu[0, torch.from_numpy(qi).to(ids_gpu.device)].cpu().numpy()
    rows = np.stack([np.zeros_like(qi), qi], axis=1)
    res = check_selection(wl.with_(batch=1), got, ids_o, s_o, rows=rows)
    return {"rows": int(len(qi) * wl.h_kv), "exact": res["exact"], "tie_band": res["tie"], "fail": res["fail"]}


def cpu_baseline(wl, xh, n_sample, n_sample_1t):
    """The oracle as it stands, timed on a bounded sample of the workload's
    queries (all their heads and groups): on every host thread, and on one."""
    from oracle import oracle as O
    qi = sample_queries(wl, n_sample)
    threads = O.num_threads()
    ids, s, dt, fl = oracle_rows(wl, xh, qi, threads)
    qi1 = qi[np.linspace(0, len(qi) - 1, n_sample_1t).astype(int)]
    _, _, dt1, fl1 = oracle_rows(wl, xh, qi1, 1)
    O.set_num_threads(threads)
    per_q = dt / len(qi)
    return ({"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
             "sample": f"{len(qi)} of {wl.n_q} queries of {wl.name} (first, last, block boundaries, evenly spaced), "
                       f"all {wl.h_q} heads: index scores, Top-k and attention in fp64, {dt:.1f} s",
             "seconds": dt, "extrapolated_full_step_s": per_q * wl.n_q * wl.batch,
             "value_1thread": fl1 / dt1 / 1e12, "seconds_1thread": dt1,
             "sample_1thread": f"{len(qi1)} of those queries on one thread", "host": _host_info()},
            qi, ids, s)


# Oracle coverage per workload for the full protocol run (--cpu-protocol):
# "all" = every query; a number = that many sampled queries.
PROTOCOL = (("tiny_f32_4k", "all", 4096), ("prefill_32k", "all", 2048), ("skewed_prefill_128k", 1024, 256),
            ("decode_16x1m", "all", 1), ("chunk_16k_at_1m", 256, 64))


def protocol_queries(wl, cover):
    """Every query, or a stratified sample: for the skewed prefill a quarter
    in the first 16 blocks, a quarter in the last 16 and the rest evenly
    spaced with the block boundaries; otherwise sample_queries."""
    if cover == "all":
        return np.arange(wl.n_q, dtype=np.int64)
    if wl.hot_frac > 0 and wl.q_offset == 0:
        head = min(16 * wl.block_size, wl.n_q)
        qs = set(np.linspace(0, head - 1, cover // 4).astype(int).tolist())
        qs |= set(np.linspace(wl.n_q - head, wl.n_q - 1, cover // 4).astype(int).tolist())
        qs |= set(sample_queries(wl, cover - len(qs)).tolist())
        return np.array(sorted(qs), dtype=np.int64)
    return sample_queries(wl, cover)


def _host_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "affinity": aff}


def cpu_baseline_protocol(args):
    """The oracle timed per stage (index scores + selection, then attention)
    with the query coverage of the measurement protocol, and every covered
    GPU row of msa_forward checked against it: selection row by row, then the
    attention output, lse and per-row rel-L2 (from the oracle's selection
    where a row lies in the tie band)."""
    from oracle import oracle as O
    from tests.parity import TOL, check_selection
    from block_sparse_long_bk_amd import api, inputs
    info = dict(_host_info(), threads=O.num_threads())
    print(f"[protocol] host {info}", flush=True)
    res = {"host": info, "workloads": {}}
    for name, cover, chunk in PROTOCOL:
        wl = inputs.WORKLOADS[name]
        x = inputs.generate(wl, device="cuda")
        p = api.problem_of(wl, sched="auto")
        ids, out, lse = api.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"])
        torch.cuda.synchronize()
        prob = O.problem_of(wl.with_(batch=1))
        tol = TOL[wl.dtype]
        st = dict(rows=0, exact=0, tie=0, fail=0, t_select=0.0, t_attend=0.0, flops=0.0, queries=0,
                  max_abs=0.0, d2=0.0, r2=0.0, worst_row=0.0, lse_abs=0.0, lse_pattern_ok=True)
        qi_all = protocol_queries(wl, cover)
        for b in range(wl.batch):
            xh = {k: v[b:b + 1].cpu() for k, v in x.items()}
            ids_b, out_b, lse_b = ids[b].cpu(), out[b].cpu(), lse[b].cpu()
            for c0 in range(0, len(qi_all), chunk):
                qi = qi_all[c0:c0 + chunk]
                rows = np.stack([np.zeros_like(qi), qi], axis=1)
                t0 = time.perf_counter()
                s_o = O.block_scores(prob, xh["iq"], xh["ik"], rows)
                ids_o = O.select(prob, s_o, rows)
                t1 = time.perf_counter()
                o_o, l_o = O.attend(prob, xh["q"], xh["k"], xh["v"], ids_o, rows)
                t2 = time.perf_counter()
                st["t_select"] += t1 - t0
                st["t_attend"] += t2 - t1
                st["queries"] += len(qi)
                got = ids_b[torch.from_numpy(qi)].numpy()
                sel = check_selection(wl.with_(batch=1), got, ids_o, s_o, rows=rows)
                for k in ("exact", "tie", "fail"):
                    st[k] += sel[k]
                st["rows"] += len(qi) * wl.h_kv
                pos = torch.from_numpy(wl.q_offset + qi).view(-1, 1, 1)
                j = torch.from_numpy(ids_o).to(torch.int64)
                n = torch.minimum(pos - j * wl.block_size + 1, torch.full_like(j, wl.block_size))
                n = torch.where(j >= 0, n.clamp(min=0), torch.zeros_like(n))
                st["flops"] += 4.0 * wl.d * (wl.h_q // wl.h_kv) * float(n.sum())
                o_g = out_b[torch.from_numpy(qi)].to(torch.float64).numpy()
                l_g = lse_b[torch.from_numpy(qi)].to(torch.float64).numpy()
                if not np.array_equal(got, ids_o):
                    # tie-band rows: the attention of the oracle's selection
                    tbl = ids[b:b + 1].clone()
                    tbl[0, torch.from_numpy(qi).cuda()] = torch.from_numpy(ids_o).cuda()
                    o2, l2 = api.sparse_attention(api.problem_of(wl.with_(batch=1), sched="auto"),
                                                  x["q"][b:b + 1], x["k"][b:b + 1], x["v"][b:b + 1], tbl)
                    o_g = o2[0, torch.from_numpy(qi).cuda()].cpu().to(torch.float64).numpy()
                    l_g = l2[0, torch.from_numpy(qi).cuda()].cpu().to(torch.float64).numpy()
                diff = o_g - o_o
                st["max_abs"] = max(st["max_abs"], float(np.max(np.abs(diff))))
                st["d2"] += float(np.sum(diff * diff))
                st["r2"] += float(np.sum(o_o * o_o))
                a2 = o_g.reshape(-1, wl.d)
                b2 = o_o.reshape(-1, wl.d)
                nb = np.linalg.norm(b2, axis=1)
                nd = np.linalg.norm(a2 - b2, axis=1)
                rel = np.where(nb > 0, nd / np.where(nb > 0, nb, 1.0), np.where(nd == 0, 0.0, np.inf))
                st["worst_row"] = max(st["worst_row"], float(rel.max()))
                fin = np.isfinite(l_o)
                st["lse_pattern_ok"] &= bool(np.array_equal(np.isneginf(l_g), np.isneginf(l_o))
                                             and np.all(np.isfinite(l_g[fin])))
                if fin.any():
                    st["lse_abs"] = max(st["lse_abs"], float(np.max(np.abs(l_g[fin] - l_o[fin]))))
                print(f"[protocol] {name} b={b} queries {c0}..{c0 + len(qi) - 1}: select {t1 - t0:.1f} s, "
                      f"attend {t2 - t1:.1f} s, selection {sel['exact']}/{len(qi) * wl.h_kv} exact "
                      f"{sel['tie']} tie {sel['fail']} fail", flush=True)
            del xh
        rl2 = (st["d2"] / st["r2"]) ** 0.5 if st["r2"] > 0 else 0.0
        per_q = (st["t_select"] + st["t_attend"]) / st["queries"]
        total_q = wl.n_q * wl.batch
        res["workloads"][name] = {
            "coverage": (f"every query ({total_q})" if cover == "all"
                         else f"{len(qi_all)} of {wl.n_q} queries, stratified"),
            "queries": st["queries"], "seconds_select": st["t_select"], "seconds_attend": st["t_attend"],
            "oracle_TFLOPs": st["flops"] / (st["t_select"] + st["t_attend"]) / 1e12,
            "full_config_s": per_q * total_q, "full_config_s_is": "measured" if cover == "all" else "extrapolated",
            "selection": {"rows": st["rows"], "exact": st["exact"], "tie_band": st["tie"], "fail": st["fail"]},
            "attention": {"max_abs": st["max_abs"], "rel_l2": rl2, "worst_row_rel_l2": st["worst_row"],
                          "lse_max_abs": st["lse_abs"], "lse_neg_inf_pattern": st["lse_pattern_ok"],
                          "within_tolerance": bool(st["fail"] == 0 and st["max_abs"] <= tol["max_abs"]
                                                   and rl2 <= tol["rel_l2"]
                                                   and st["worst_row"] <= tol["row_rel_l2"]
                                                   and st["lse_abs"] <= tol["lse_abs"] and st["lse_pattern_ok"]),
                          "tolerance": tol},
        }
        print(f"[protocol] {name}: {json.dumps(res['workloads'][name])}", flush=True)
        del x, ids, out, lse
        gc.collect()
        torch.cuda.empty_cache()
    return res


# ---- legs --------------------------------------------------------------------

def achievable_peaks():
    """What this GPU reaches on plain work, as a second reference beside the
    published peaks: a 2 GiB device-to-device copy (read + write GB/s, like
    the mixed traffic of the KV-outer pass), a 2 GiB fill (write only), and
    the installed library's dense bf16 matmul at three shapes (TFLOP/s at
    whatever clock the chip holds under it; the best is the reference)."""
    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    src = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    copy_gbs = 2 * src.numel() / timed(lambda: dst.copy_(src), 5) / 1e6
    write_gbs = dst.numel() / timed(lambda: dst.fill_(1), 5) / 1e6
    rows = dst.view(torch.float32).view(-1, 4096)  # the filled buffer: defined values
    read_gbs = dst.numel() / timed(lambda: rows.sum(dim=1), 5) / 1e6
    del src, dst, rows
    torch.cuda.empty_cache()
    mm = {}
    for m, n, k in ((8192, 8192, 8192), (16384, 16384, 8192), (32768, 8192, 8192)):
        a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(k, n, device="cuda", dtype=torch.bfloat16)
        mm[f"{m}x{n}x{k}"] = 2.0 * m * n * k / timed(lambda: torch.matmul(a, b), 8) / 1e9
        del a, b
        torch.cuda.empty_cache()
    return {"copy_GBs": copy_gbs, "write_GBs": write_gbs, "read_GBs": read_gbs,
            "bf16_matmul_TFLOPs": max(mm.values()), "bf16_matmul_by_shape": mm,
            "note": "2 GiB device copy (read + write), 2 GiB fill (write only), row sums of 2 GiB (read only) and "
                    "the best of torch.matmul bf16 at three shapes on this GPU"}


def add_achievable(line, peaks):
    """frac_of_achievable beside frac for every roofline entry of the line:
    MFMA-bound kernels against the best library matmul, HBM-bound ones
    against the read stream (the decode scan only reads)."""
    if not peaks:
        return

    def visit(d):
        if isinstance(d, dict):
            if d.get("bound") in ("mfma", "hbm") and d.get("achieved") is not None:
                ref = peaks["bf16_matmul_TFLOPs"] if d["bound"] == "mfma" else peaks["read_GBs"]
                d["frac_of_achievable"] = d["achieved"] / ref
            for v in d.values():
                visit(v)
        elif isinstance(d, list):
            for v in d:
                visit(v)
    visit(line)


def chunk_workspace_bytes(p, n_chunk):
    """Workspace bytes that make the attention run in query chunks of (about)
    n_chunk queries: the library takes the largest chunk that fits."""
    from block_sparse_long_bk_amd import api
    full, least = api.workspace_size(p, api.OP_FORWARD)
    if n_chunk >= p.n_q:
        return full
    per_q = (full - least) / max(p.n_q - 256, 1)  # the least workspace holds a 256-query chunk
    return int(least + per_q * (n_chunk - 256)) + (1 << 20)


def run_forward(wl, args, sched="auto", cold=True):
    from block_sparse_long_bk_amd import api, inputs
    x = inputs.generate(wl, device="cuda")
    p = api.problem_of(wl, sched=sched)
    if getattr(args, "chunk_queries", 0):
        ws = torch.empty(chunk_workspace_bytes(p, args.chunk_queries), dtype=torch.uint8, device="cuda")
    else:
        ws = api.alloc_workspace(p, api.OP_FORWARD)
    ids = torch.empty((wl.batch, wl.n_q, wl.h_kv, wl.topk), dtype=torch.int32, device="cuda")
    out = torch.empty_like(x["q"])
    lse = torch.empty((wl.batch, wl.n_q, wl.h_q), dtype=torch.float32, device="cuda")

    def step():
        api.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], ids=ids, out=out, lse=lse, ws=ws)

    step()
    torch.cuda.synchronize()
    r = dict(wl=wl, x=x, ids=ids, out=out, lse=lse, ws_bytes=ws.numel(),
             fl_attn=attention_flops(wl, ids), fl_idx=index_flops(wl), mbytes=method_bytes(wl, ids),
             ibytes=impl_bytes(wl, ids))
    if cold:
        scrub = _scrub_buffer()
        r["ms"], r["wall_ms"], r["kern"] = time_steps(step, args.steps, args.warmup, scrub=scrub)
        r["cold_steps"] = step_spread(_LAST_STEP_MS)
        del scrub
    r["ms_warm"], _, r["kern_warm"] = time_steps(step, args.steps, 1)
    if not cold:
        r["ms"], r["wall_ms"], r["kern"] = r["ms_warm"], None, r["kern_warm"]
    del ws
    return r


def kernels_ms(kern):
    return {k: round(v[0], 4) for k, v in kern.items()}


def forward_summary(r):
    wl, kern = r["wl"], r["kern"]
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    attn_ms = sum(v[0] * v[1] for k, v in kern.items() if k.startswith(("inv_", "attn_")) or k == "combine")
    out = {"workload": wl.name, "ms_per_step": r["ms"], "ms_per_step_warm": r["ms_warm"],
           "effective_TFLOPs": r["fl_attn"] / r["ms"] / 1e9,
           "effective_TFLOPs_warm": r["fl_attn"] / r["ms_warm"] / 1e9,
           "attention_tflops_per_step": r["fl_attn"] / 1e12, "index_tflops_per_step": r["fl_idx"] / 1e12,
           "sparse_attention_TFLOPs": r["fl_attn"] / attn_ms / 1e9 if attn_ms else None,
           "kernels_ms": kernels_ms(kern), "kernels_ms_warm": kernels_ms(r["kern_warm"]),
           "kernel_launches_per_step": {k: v[1] for k, v in kern.items()},
           "method_bytes_attention": r["mbytes"], "workspace_bytes": r["ws_bytes"]}
    if r.get("cold_steps"):
        out["cold_step_ms"] = r["cold_steps"]
    it = [k for k in kern if k.startswith("index_tile")]
    if it:
        out["index_tile"] = roofline(it[0], kern[it[0]][0], flops=r["fl_idx"], peak_tflops=peak, workload=wl.name)
    if "attn_kvouter" in kern:
        ms = kern["attn_kvouter"][0] * kern["attn_kvouter"][1]
        out["attn_kvouter"] = roofline("attn_kvouter", ms, flops=r["fl_attn"], peak_tflops=peak, workload=wl.name,
                                       method=r["mbytes"])
        out["attn_kvouter"]["design_bytes_per_launch"] = r["ibytes"]["attn_kvouter"]
        out["attn_kvouter"]["design_GBs"] = r["ibytes"]["attn_kvouter"] / ms / 1e6
    if "combine" in kern:
        out["combine_GBs"] = r["ibytes"]["combine"] / kern["combine"][0] / kern["combine"][1] / 1e6
    return out


def skew_figures(wl, ids, kern):
    """Block popularity of the selection and what KV-outer makes of it."""
    from block_sparse_long_bk_amd import inputs
    G = wl.h_q // wl.h_kv
    qi = min(2048 // G, 1024)  # (query, slot) entries per KV-outer work item
    flat = ids.view(wl.batch, wl.n_q, wl.h_kv, wl.topk).permute(0, 2, 1, 3).reshape(wl.batch * wl.h_kv, -1).long()
    cnt = torch.stack([torch.bincount(r[r >= 0], minlength=wl.nblk) for r in flat])  # [B*Hkv, nblk]
    sel = cnt[cnt > 0].double()
    items = torch.ceil(cnt.double() / qi)
    hot = inputs.hot_blocks(wl, "cuda")[0] if wl.hot_frac > 0 else None
    out = {"picks_per_selected_block": {"mean": float(sel.mean()), "p50": float(sel.quantile(0.5)),
                                        "p99": float(sel.quantile(0.99)), "max": int(sel.max())},
           "work_items": {"total": int(items.sum()), "max_per_block": int(items.max()),
                          "p99_per_block": float(items[cnt > 0].quantile(0.99))},
           "entries_per_item": qi}
    if hot is not None:
        on_hot = cnt[:, hot].sum()
        out["hot_blocks"] = int(hot.numel())
        out["share_of_picks_on_hot_blocks"] = float(on_hot / cnt.sum())
        out["picks_per_hot_block"] = {"mean": float(cnt[:, hot].double().mean()), "max": int(cnt[:, hot].max())}
    sel_keys = selected_tokens(wl, ids) * G
    if "attn_kvouter" in kern:
        out["kvouter_ns_per_1k_query_head_keys"] = kern["attn_kvouter"][0] * kern["attn_kvouter"][1] * 1e9 / sel_keys
    return out


def run_training(args, r):
    """The training-side kernels on the same workload and selection: the
    Main Branch backward and the Index-Branch KL loss with its gradients.
    Effective TFLOP/s count the products over the selected, unmasked tokens:
    backward 5 x 2d per (query head, key) (S, dP, dV, dK, dQ); KL 2d per
    (query head, key) for the Main Branch probabilities plus 4 x 2 d_idx per
    (query group, key) (index scores twice, d iq, d ik)."""
    from block_sparse_long_bk_amd import api, inputs
    wl, x, ids = r["wl"], r["x"], r["ids"]
    p = api.problem_of(wl)
    dout = inputs.generate(wl, device="cuda", tensors=("dout",))["dout"]
    sel = selected_tokens(wl, ids)
    G = wl.h_q // wl.h_kv
    ws = api.alloc_workspace(p, api.OP_BACKWARD)
    dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])

    def bwd():
        api.sparse_attention_backward(p, x["q"], x["k"], x["v"], r["out"], r["lse"], dout, ids, dq, dk, dv, ws=ws)

    bwd()
    ms_b, _, kern_b = time_steps(bwd, max(3, args.steps // 2), 1)
    fl_b = 10.0 * wl.d * G * sel
    del ws, dq, dk, dv, dout
    torch.cuda.empty_cache()
    ws = api.alloc_workspace(p, api.OP_INDEXER_KL)
    kl = torch.empty((wl.batch, wl.n_q, wl.h_kv), dtype=torch.float32, device="cuda")
    d_iq, d_ik = torch.empty_like(x["iq"]), torch.empty_like(x["ik"])

    def klstep():
        api.indexer_kl(p, x["q"], x["k"], x["iq"], x["ik"], r["lse"], ids, 1.0, kl, d_iq, d_ik, ws=ws)

    klstep()
    ms_k, _, kern_k = time_steps(klstep, max(3, args.steps // 2), 1)
    fl_k = (2.0 * wl.d * G + 8.0 * wl.d_idx) * sel
    del ws, kl, d_iq, d_ik
    torch.cuda.empty_cache()
    return {
        "backward": {"workload": wl.name, "ms_per_step": ms_b, "effective_TFLOPs": fl_b / ms_b / 1e9,
                     "tflops_per_step": fl_b / 1e12, "mfma_frac": fl_b / ms_b / 1e9 / PEAK_BF16_TFLOPS,
                     "kernels_ms": kernels_ms(kern_b)},
        "indexer_kl": {"workload": wl.name, "ms_per_step": ms_k, "effective_TFLOPs": fl_k / ms_k / 1e9,
                       "tflops_per_step": fl_k / 1e12, "kernels_ms": kernels_ms(kern_k)},
    }


def run_decode(args, idx_format="plain", kv_format="plain"):
    """decode_16x1m forward steps (cold: a 1 GiB scrub before each).
    idx_format "mxfp8": the idx_k cache is quantised once (untimed) to MXFP8
    by msa_mxfp8_quantize and the index scan reads codes + scales
    (d_idx + d_idx/32 bytes per key) instead of bf16; kv_format "mxfp8": K
    and V too (d + d/32 bytes per key and tensor)."""
    from block_sparse_long_bk_amd import api, inputs
    wl = inputs.WORKLOADS["decode_16x1m"]
    x = inputs.generate(wl, device="cuda")
    p = api.problem_of(wl, sched="auto", idx_format=idx_format, kv_format=kv_format)
    ik = x["ik"]
    if idx_format == "mxfp8":
        ik = api.mxfp8_quantize(x["ik"])
        del x["ik"]
    if kv_format == "mxfp8":
        for t in ("k", "v"):
            x[t] = api.mxfp8_quantize(x[t])
    ws = api.alloc_workspace(p, api.OP_FORWARD)
    ids = torch.empty((wl.batch, wl.n_q, wl.h_kv, wl.topk), dtype=torch.int32, device="cuda")
    out = torch.empty_like(x["q"])

    def step():
        api.forward(p, x["q"], x["k"], x["v"], x["iq"], ik, ids=ids, out=out, want_lse=False, ws=ws)

    step()
    torch.cuda.synchronize()
    steps = max(3, args.steps)
    scrub = _scrub_buffer()
    ms, _, kern = time_steps(step, steps, args.warmup, scrub=scrub)
    spread = step_spread(_LAST_STEP_MS)
    del scrub
    ms_w, _, _ = time_steps(step, steps, 1)
    # algorithmic bytes: idx_k of every candidate block, the selected K/V
    # tokens, the index and attention queries, block scores, ids and outputs
    L = (wl.q_offset + wl.n_q - 1) // wl.block_size
    e = 2
    key_bytes = wl.d_idx + wl.d_idx // 32 if idx_format == "mxfp8" else wl.d_idx * e
    b_idx = wl.batch * L * wl.block_size * wl.h_kv * key_bytes
    sel = selected_tokens(wl, ids)
    b_kv = sel * (wl.d + wl.d // 32 if kv_format == "mxfp8" else wl.d * e) * 2
    b_small = wl.batch * (wl.h_kv * wl.d_idx + 2 * wl.h_q * wl.d) * e + wl.batch * wl.h_kv * L * 4 * 2
    total = b_idx + b_kv + b_small
    res = {"workload": wl.name, "idx_format": idx_format, "kv_format": kv_format,
           "us_per_token": ms * 1e3 / (wl.batch * wl.n_q), "ms_per_step": ms,
           "us_per_token_warm": ms_w * 1e3 / (wl.batch * wl.n_q), "algorithmic_bytes": total,
           "hbm_GBs": total / ms / 1e6, "hbm_frac": total / ms / 1e6 / PEAK_HBM_GBS,
           "kernels_ms": kernels_ms(kern), "cold_step_ms": spread}
    if "index_scan" in kern:
        res["index_scan"] = roofline("index_scan", kern["index_scan"][0], nbytes=b_idx, workload=wl.name)
    del x, ws, ik
    torch.cuda.empty_cache()
    return res


def run_topk(args, cands=(1024, 2048, 4096, 8191), topk=16):
    """msa_topk_from_scores on its own (the pages benchmark their Top-k
    kernel separately): rows of C candidate blocks (C*128 context tokens) for
    the decode case (16 sequences x 8 groups = 128 rows) and for a prefill
    chunk's worth of rows (262,144 = 256 x 8 x 128), torch.topk on the same
    rows beside it for scale (it neither forces the local block nor breaks
    ties by the lower id)."""
    from block_sparse_long_bk_amd import api
    res = []
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    for C in cands:
        for case, B, nq in (("decode_128_rows", 16, 1), ("prefill_262144_rows", 256, 128)):
            rows = B * 8 * nq
            if case.startswith("prefill") and C > 4096:
                continue
            n_k = (C + 1) * 128
            p = api.problem(B, nq, n_k, 64, 8, 128, 128, topk, dtype="bf16", q_offset=C * 128)
            S = torch.randn((B, 8, nq, C + 1), generator=g, device="cuda", dtype=torch.float32)
            ids = torch.empty((B, nq, 8, topk), dtype=torch.int32, device="cuda")
            ms, _, kern = time_steps(lambda: api.topk_from_scores(p, S, ids), 10, 2)
            Sv = S[..., :C].reshape(rows, C)
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.topk(Sv, topk - 1, dim=1)
            ev0.record()
            for _ in range(10):
                torch.topk(Sv, topk - 1, dim=1)
            ev1.record()
            torch.cuda.synchronize()
            t_ms = ev0.elapsed_time(ev1) / 10
            res.append({"case": case, "rows": rows, "candidates": C, "context_tokens": C * 128,
                        "us": kern["topk_rows"][0] * 1e3, "scores_GBs": rows * C * 4 / kern["topk_rows"][0] / 1e6,
                        "torch_topk_us": t_ms * 1e3})
            del S, ids, Sv
    torch.cuda.empty_cache()
    return res


def run_crossover(args, chunks=(256, 512, 1024, 1460, 2048, 4096, 16384)):
    """KV-outer vs query-outer attention time on the last `c` queries of the
    1M-token chunked-prefill cache (2 % hot blocks).  reuse = c*k*Bk/Nk is the
    average number of reads of a KV token, the quantity whose crossover the
    Fireworks note on KV-stationary attention puts near 2.85."""
    from block_sparse_long_bk_amd import api, inputs
    base = inputs.WORKLOADS["chunk_16k_at_1m"]
    x = inputs.generate(base, device="cuda")
    rows = []
    for c in chunks:
        wl = base.with_(n_q=c, q_offset=base.n_k - c)
        q, iq = x["q"][:, -c:].contiguous(), x["iq"][:, -c:].contiguous()
        p0 = api.problem_of(wl)
        ids = api.index_topk(p0, iq, x["ik"])
        torch.cuda.synchronize()
        fl = attention_flops(wl, ids)
        rec = {"n_q": c, "reuse": c * wl.topk * wl.block_size / wl.n_k}
        for sched in ("kv_outer", "q_outer"):
            p = api.problem_of(wl, sched=sched)
            ws = api.alloc_workspace(p, api.OP_ATTENTION)
            out = torch.empty_like(q)

            def step():
                api.sparse_attention(p, q, x["k"], x["v"], ids, out=out, want_lse=False, ws=ws)

            ms, _, _ = time_steps(step, 5, 2)
            rec[sched + "_ms"] = ms
            rec[sched + "_TFLOPs"] = fl / ms / 1e9
            del ws, out
        rec["kv_over_q_speedup"] = rec["q_outer_ms"] / rec["kv_outer_ms"]
        rows.append(rec)
    del x
    torch.cuda.empty_cache()
    return rows


# ---- rocprofv3 summaries (no GPU) ---------------------------------------------

def _pmc_rows(d):
    fs = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    assert fs, f"no counter_collection.csv under {d}"
    rows = []
    for f in fs:
        rows += list(csv.DictReader(open(f)))
    return rows


def summarize_pmc(fetch_dir, write_dir, kernel, workload):
    """Per-launch HBM bytes of each kernel from a FETCH_SIZE and a WRITE_SIZE
    run (KiB per dispatch), each scaled by what the counter reads for the
    plain 1 GiB device copy in the same run; writes the traffic record of
    `kernel` and prints a markdown table."""
    per = {}
    for d, cname in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        for r in _pmc_rows(d):
            if r.get("Counter_Name") != cname:
                continue
            name = r["Kernel_Name"]
            key = (name, r.get("Dispatch_Id") or r.get("Correlation_Id"))
            per.setdefault(cname, {}).setdefault(name, {}).setdefault(key, 0.0)
            per[cname][name][key] += float(r["Counter_Value"]) * 1024.0
    # the 1 GiB calibration copy (--calib-copy-mib 1024) is the largest dispatch
    # of the runtime's device-to-device copy kernel
    fac = {}
    for cname in ("FETCH_SIZE", "WRITE_SIZE"):
        vals = [v for n in per[cname] if "copybuffer" in n.lower() for v in per[cname][n].values()]
        assert vals, f"no calibration copy in the {cname} run"
        fac[cname] = float(1 << 30) / max(vals)
    lines = ["| kernel | launches | scaled read GB | scaled write GB | total GB |", "|---|---:|---:|---:|---:|"]
    rec_bytes = None
    for name in sorted(per["FETCH_SIZE"], key=lambda n: -np.mean(list(per["FETCH_SIZE"][n].values()))):
        f = np.mean(list(per["FETCH_SIZE"][name].values())) * fac["FETCH_SIZE"]
        w = np.mean(list(per.get("WRITE_SIZE", {}).get(name, {0: 0.0}).values())) * fac["WRITE_SIZE"]
        short = _short(name)
        lines.append(f"| {short} | {len(per['FETCH_SIZE'][name])} | {f / 1e9:.3f} | {w / 1e9:.3f} | {(f + w) / 1e9:.3f} |")
        if TRACE_NAME.get(kernel, kernel) in name:
            rec_bytes = f + w if rec_bytes is None else max(rec_bytes, f + w)
    print(f"factors: FETCH_SIZE x {fac['FETCH_SIZE']:.3f}, WRITE_SIZE x {fac['WRITE_SIZE']:.3f}")
    print("\n".join(lines))
    if rec_bytes is not None and kernel in TRAFFIC_SOURCES:
        rec = {"kernel": kernel, "workload": workload, "bytes_per_launch": rec_bytes,
               "fetch_factor": fac["FETCH_SIZE"], "write_factor": fac["WRITE_SIZE"],
               "sources": TRAFFIC_SOURCES[kernel], "source_hash": source_hash(TRAFFIC_SOURCES[kernel])}
        path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")
        json.dump(rec, open(path, "w"), indent=1)
        print(f"wrote {path}")


KERNELS = ("k_index_tile", "k_index_scan", "k_attn_kvouter", "k_attn_qouter", "k_combine", "k_inv_hist",
           "k_inv_colscan", "k_inv_blkscan", "k_inv_scatter", "k_inv_items", "k_topk_rows", "k_topk_wg",
           "k_bwd_rowdot", "k_bwd_split", "k_bwd_fused", "k_bwd_dq_sum", "k_bwd_dkdv_reduce", "k_kl_lse",
           "k_kl_lse_sum", "k_kl_main", "k_kl_main8", "k_kl_finish", "k_kl_dik_reduce", "k_mxfp8_quantize",
           "k_fill_neg_inf")


def _short(name):
    """The library's kernel name inside a mangled or demangled symbol."""
    for k in sorted(KERNELS, key=len, reverse=True):
        if k in name:
            return k
    return name.split("(")[0].split("<")[0].split("::")[-1][:48] or "(unnamed)"


def summarize_stats(d):
    """Markdown table of a rocprofv3 --stats kernel summary."""
    fs = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    assert fs, f"no kernel_stats.csv under {d}"
    rows = list(csv.DictReader(open(fs[0])))
    print("| kernel | calls | avg us | min us | max us | total ms |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = _short(r["Name"])
        print(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
              f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['TotalDurationNs']) / 1e6:.2f} |")


def summarize_sq(dir_a, dir_b):
    """Per-kernel SQ figures from two rocprofv3 --pmc passes over the same
    command: pass A with SQ_WAVE_CYCLES, SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_WAIT_INST_ANY, SQ_INSTS_MFMA, SQ_INSTS_VALU, GRBM_GUI_ACTIVE; pass B
    with SQ_WAIT_INST_LDS, SQ_ACTIVE_INST_LDS, SQ_LDS_BANK_CONFLICT.  Counters
    are chip totals per dispatch; the k-th dispatch of a kernel in pass B is
    matched with its k-th dispatch in pass A.  Per dispatch: clock =
    GRBM_GUI_ACTIVE / 8 XCDs / dispatch time; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES
    / (1024 SIMDs x GRBM_GUI_ACTIVE / 8); VALU per MFMA = (SQ_INSTS_VALU -
    SQ_INSTS_MFMA) / SQ_INSTS_MFMA; waits as fractions of SQ_WAVE_CYCLES; LDS
    conflicts = SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS.  Prints min-max over
    the dispatches of each library kernel."""
    def dispatches(d):
        per = {}
        for r in _pmc_rows(d):
            key = r.get("Dispatch_Id") or r.get("Correlation_Id")
            e = per.setdefault(key, {"name": _short(r["Kernel_Name"]), "c": {},
                                     "ns": float(r["End_Timestamp"]) - float(r["Start_Timestamp"])})
            e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        out = {}
        for key in sorted(per, key=lambda k: int(k)):
            e = per[key]
            if e["name"].startswith("k_"):
                out.setdefault(e["name"], []).append(e)
        return out
    A, B = dispatches(dir_a), dispatches(dir_b)

    def rng(v, fmt):
        v = [x for x in v if x is not None and math.isfinite(x)]
        if not v:
            return "–"
        lo, hi = min(v), max(v)
        return fmt.format(lo) if fmt.format(lo) == fmt.format(hi) else fmt.format(lo) + "–" + fmt.format(hi)
    print("| kernel | dispatches | dispatch ms | clock GHz | MFMA busy | VALU / MFMA | wait on a dependency | "
          "wait on LDS | LDS bank conflicts |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|---:|")
    for name, da in sorted(A.items(), key=lambda kv: -sum(e["ns"] for e in kv[1])):
        db = B.get(name, [])
        ms, clk, busy, vpm, wdep, wlds, conf = [], [], [], [], [], [], []
        for i, e in enumerate(da):
            c = e["c"]
            act = c.get("GRBM_GUI_ACTIVE", 0.0) / 8
            ms.append(e["ns"] / 1e6)
            # (the GRBM window also covers the dispatch itself: no clock for short ones)
            clk.append(act / e["ns"] if e["ns"] > 1e5 and act else None)
            busy.append(c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (1024 * act) if act else None)
            nm = c.get("SQ_INSTS_MFMA", 0.0)
            vpm.append((c.get("SQ_INSTS_VALU", 0.0) - nm) / nm if nm else None)
            wc = c.get("SQ_WAVE_CYCLES", 0.0)
            wdep.append(c.get("SQ_WAIT_INST_ANY", 0.0) / wc if wc else None)
            if i < len(db):
                cb = db[i]["c"]
                wlds.append(cb.get("SQ_WAIT_INST_LDS", 0.0) / wc if wc else None)
                al = cb.get("SQ_ACTIVE_INST_LDS", 0.0)
                conf.append(cb.get("SQ_LDS_BANK_CONFLICT", 0.0) / al if al else None)
        print(f"| {name} | {len(da)} | {rng(ms, '{:.3f}')} | {rng(clk, '{:.2f}')} | {rng(busy, '{:.3f}')} | "
              f"{rng(vpm, '{:.1f}')} | {rng(wdep, '{:.2f}')} | {rng(wlds, '{:.3f}')} | {rng(conf, '{:.2f}')} |")


# ---- main --------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--sched", default="auto", choices=["auto", "kv_outer", "q_outer"])
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-legs", action="store_true", help="skip the prefill_32k and skewed_prefill_128k legs")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-train", action="store_true", help="skip the backward and indexer-loss legs")
    ap.add_argument("--no-topk", action="store_true", help="skip the standalone Top-k timing")
    ap.add_argument("--chunk-queries", type=int, default=0,
                    help="give the forward only the workspace for attention chunks of about this many queries")
    ap.add_argument("--cpu-sample", type=int, default=256, help="oracle queries of the headline workload")
    ap.add_argument("--cpu-sample-1thread", type=int, default=3, help="of those, timed again on one thread")
    ap.add_argument("--cpu-protocol", action="store_true",
                    help="only the oracle with the protocol's coverage per workload (every query of the tiny "
                         "and 32K prefills, all decode sequences), timed per stage, every covered row checked")
    ap.add_argument("--crossover", action="store_true",
                    help="also time both attention schedules on query chunks at the end of a 1M-token cache")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (reference for HBM counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--pmc-kernel", default="index_tile_topk")
    ap.add_argument("--pmc-workload", default=HEADLINE)
    ap.add_argument("--summarize-stats", metavar="STATS_DIR")
    ap.add_argument("--summarize-sq", nargs=2, metavar=("PASS_A_DIR", "PASS_B_DIR"))
    ap.add_argument("--legs", default="prefill_32k,skewed_prefill_128k",
                    help="comma-separated prefill legs (the backward and indexer loss run with prefill_32k)")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.pmc_kernel, args.pmc_workload)
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats)
        return
    if args.summarize_sq:
        summarize_sq(*args.summarize_sq)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this MSA forward path is built and measured on a single GPU "
              "(one GPU's share of the work at its real shape); --gpus must be 1", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from block_sparse_long_bk_amd import inputs

    if args.cpu_protocol:
        print(json.dumps({"cpu_baseline_protocol": cpu_baseline_protocol(args)}), flush=True)
        return
    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # the probes stay out of profiled runs: their 2 GiB copy would pass for the
    # calibration copy of a counter run
    peaks = None if (args.no_legs or args.calib_copy_mib) else achievable_peaks()
    wl = inputs.WORKLOADS[args.workload]
    r = run_forward(wl, args, sched=args.sched)
    fs = forward_summary(r)
    kern = r["kern"]
    value = r["fl_attn"] / r["ms"] / 1e9  # TFLOP/s, cold caches
    dom = max(kern, key=lambda k: kern[k][0] * kern[k][1])
    roof = fs.get("index_tile") if dom.startswith("index_tile") else fs.get(dom)
    if roof is None:
        roof = {"bound": None, "kernel": dom, "achieved": None, "peak": None, "unit": None, "frac": None,
                "traffic": None}
    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": r["ms"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "n_q": wl.n_q, "n_k": wl.n_k, "q_offset": wl.q_offset,
                   "block_size": wl.block_size, "topk": wl.topk, "h_q": wl.h_q, "h_kv": wl.h_kv, "d": wl.d,
                   "d_idx": wl.d_idx, "sched": args.sched, "hot_frac": wl.hot_frac,
                   "chunk_queries": args.chunk_queries or wl.n_q,
                   "caches": "cold (1 GiB scrub before each timed step)"},
        "roofline": roof,
        "achievable_peaks": peaks,
        "warm": {"value": fs["effective_TFLOPs_warm"], "ms_per_step": r["ms_warm"]},
        "headline": fs,
    }
    if not args.no_cpu:
        xh = host_inputs(r["x"])
        base, qi, ids_o, s_o = cpu_baseline(wl, xh, args.cpu_sample, args.cpu_sample_1thread)
        line["cpu_baseline"] = base
        line["selection_check"] = selection_check(wl, r["ids"], qi, ids_o, s_o)
        del xh
    del r
    torch.cuda.empty_cache()
    if not args.no_legs:
        for name in [n for n in args.legs.split(",") if n]:
            rl = run_forward(inputs.WORKLOADS[name], args, sched=args.sched)
            leg = forward_summary(rl)
            leg["skew"] = skew_figures(rl["wl"], rl["ids"], rl["kern"])
            if not args.no_cpu:
                # part of the CPU-baseline leg (the oracle runs only there):
                # the oracle's selection of 64 sampled queries of this workload
                xh = host_inputs(rl["x"])
                qi = sample_queries(rl["wl"], 64)
                ids_o, s_o, _, _ = oracle_rows(rl["wl"], xh, qi)
                chk = selection_check(rl["wl"], rl["ids"], qi, ids_o, s_o)
                line.setdefault("cpu_baseline", {}).setdefault("leg_selection_checks", {})[name] = chk
                leg["selection_check"] = chk
                del xh
            line[name] = leg
            if name == "prefill_32k" and not args.no_train:
                line.update(run_training(args, rl))
            del rl
            torch.cuda.empty_cache()
        a = line.get("prefill_32k", {}).get("skew", {})
        b = line.get("skewed_prefill_128k", {}).get("skew", {})
        if "kvouter_ns_per_1k_query_head_keys" in a and "kvouter_ns_per_1k_query_head_keys" in b:
            line["skewed_prefill_128k"]["kvouter_time_per_key_vs_prefill_32k"] = (
                b["kvouter_ns_per_1k_query_head_keys"] / a["kvouter_ns_per_1k_query_head_keys"])
    if args.crossover:
        line["crossover"] = run_crossover(args)
    if not args.no_decode:
        line["decode"] = run_decode(args)
        # the same decode step over an MXFP8 index-key cache (a different
        # cache format, reported beside the bf16 figure, never as `value`)
        line["decode_mxfp8"] = run_decode(args, idx_format="mxfp8")
        # and over an all-MXFP8 cache (index keys, K and V)
        line["decode_mxfp8_cache"] = run_decode(args, idx_format="mxfp8", kv_format="mxfp8")
    if not args.no_topk:
        line["topk_standalone"] = run_topk(args)
    add_achievable(line, peaks)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
