"""Benchmark of the MSA forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill_32k]
                    [--sched auto|kv_outer|q_outer] [--no-cpu] [--no-decode] [--no-train]

One step = msa_forward (index scores + Top-k, inversion, attention, combine)
over one batch of the seeded synthetic workload, inputs already in HBM.
Prints one JSON line.  ``value`` is effective TFLOP/s over the selected,
unmasked tokens, 4*d per (query head, key), divided by the whole forward
step time.  The decode leg (16 sequences x 1M cached tokens, one new token
each) reports microseconds per generated token.  The training legs time the
Main Branch backward and the Index-Branch KL loss on the same workload and
selection.  Per-kernel times come from
hipEvents that libmsa records around each launch on the launch stream.
"""
import argparse
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

from block_sparse_long_bk_amd import api, inputs  # noqa: E402

METRIC = "MSA fwd effective TFLOP/s (selected tokens) & decode µs/token @1M ctx"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")


def selected_tokens(wl, ids):
    """Sum over (b, i, g) of the visible tokens in the selected blocks."""
    Bk = wl.block_size
    pos = wl.q_offset + torch.arange(wl.n_q, device=ids.device, dtype=torch.int64).view(1, -1, 1, 1)
    j = ids.to(torch.int64)
    start = j * Bk
    n = torch.minimum(pos - start + 1, torch.full_like(start, Bk))
    n = torch.minimum(n, wl.n_k - start)
    n = torch.where(j >= 0, n.clamp(min=0), torch.zeros_like(n))
    return int(n.sum().item())


def attention_flops(wl, ids):
    G = wl.h_q // wl.h_kv
    return 4.0 * wl.d * G * selected_tokens(wl, ids)


def attention_bytes(wl, ids):
    """Algorithmic HBM bytes of the KV-outer attention and of the combine, per
    launch over the whole problem: every selected (b, i, g, block) moves the
    group's G query rows in and G partial rows (bf16/fp32 output + fp32 lse)
    out; each selected key block is read once per (b, g); the combine reads
    every partial, the block ids and writes the output and lse."""
    e = 2 if wl.dtype == "bf16" else 4
    G = wl.h_q // wl.h_kv
    valid = ids >= 0
    nnz = int(valid.sum().item())
    flat = (torch.arange(wl.batch * wl.h_kv, device=ids.device).view(wl.batch, 1, wl.h_kv, 1) * wl.nblk
            + ids.clamp(min=0).long())
    uniq = int(torch.unique(flat[valid]).numel())
    part_row = wl.d * e + 4
    kv = nnz * G * wl.d * e + nnz * G * part_row + uniq * wl.block_size * wl.d * e * 2 + nnz * 4
    comb = nnz * G * part_row + ids.numel() * 4 + wl.batch * wl.n_q * wl.h_q * (wl.d * e + 4)
    return {"attn_kvouter": kv, "combine": comb, "selected_group_blocks": nnz}


def index_flops(wl):
    L = (wl.q_offset + np.arange(wl.n_q, dtype=np.int64)) // wl.block_size
    return 2.0 * wl.d_idx * wl.h_kv * wl.batch * float(L.sum()) * wl.block_size


def time_steps(fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    api.profile_reset()
    api.profile_enable(True)
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(steps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    api.profile_enable(False)
    kern = {k: (ms / n, n / steps) for k, (ms, n) in api.profile_read().items() if n}
    return e0.elapsed_time(e1) / steps, wall * 1e3 / steps, kern


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


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


def cpu_baseline(wl, x, n_sample):
    """The fp64 oracle (as it stands) on an evenly spaced sample of queries."""
    from oracle import oracle as O

    h = {k: v.cpu() for k, v in x.items()}
    prob = O.problem_of(wl)
    qi = np.unique(np.linspace(0, wl.n_q - 1, n_sample).astype(np.int64))
    rows = np.stack([np.zeros_like(qi), qi], axis=1)
    t0 = time.perf_counter()
    s = O.block_scores(prob, h["iq"], h["ik"], rows)
    ids = O.select(prob, s, rows)
    O.attend(prob, h["q"], h["k"], h["v"], ids, rows)
    dt = time.perf_counter() - t0
    ids_t = torch.from_numpy(ids).view(len(qi), 1, wl.h_kv, wl.topk)
    # selected visible tokens for the sampled queries
    pos = torch.from_numpy(wl.q_offset + qi).view(-1, 1, 1, 1)
    j = ids_t.to(torch.int64)
    n = torch.minimum(pos - j * wl.block_size + 1, torch.full_like(j, wl.block_size))
    n = torch.where(j >= 0, n.clamp(min=0), torch.zeros_like(n))
    flops = 4.0 * wl.d * (wl.h_q // wl.h_kv) * float(n.sum())
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"{len(qi)} of {wl.n_q} queries (evenly spaced), all {wl.h_q} heads; index scores, "
                      f"Top-k and attention in fp64; {dt:.1f} s",
            "seconds": dt}


def run_prefill(args):
    wl = inputs.WORKLOADS[args.workload]
    x = inputs.generate(wl, device="cuda")
    p = api.problem_of(wl, sched=args.sched)
    ws = api.alloc_workspace(p, api.OP_FORWARD)
    ids = torch.empty((wl.batch, wl.n_q, wl.h_kv, wl.topk), dtype=torch.int32, device="cuda")
    out = torch.empty_like(x["q"])
    lse = torch.empty((wl.batch, wl.n_q, wl.h_q), dtype=torch.float32, device="cuda")

    def step():
        api.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], ids=ids, out=out, lse=lse, ws=ws)

    step()
    torch.cuda.synchronize()
    fl_attn = attention_flops(wl, ids)
    fl_idx = index_flops(wl)
    nbytes = attention_bytes(wl, ids)
    ms, wall_ms, kern = time_steps(step, args.steps, args.warmup)
    res = dict(wl=wl, x=x, ms=ms, wall_ms=wall_ms, kern=kern, fl_attn=fl_attn, fl_idx=fl_idx, ws=ws.numel(),
               bytes=nbytes, ids=ids, out=out, lse=lse)
    del ws
    return res


def run_training(args, r):
    """The training-side kernels on the same workload and selection: the
    Main Branch backward (msa_sparse_attention_backward) and the Index-Branch
    KL loss with its gradients (msa_indexer_kl).  Effective TFLOP/s count the
    products over the selected, unmasked tokens: backward 5 x 2d per (query
    head, key) (S, dP, dV, dK, dQ); KL 2d per (query head, key) for the Main
    Branch probabilities plus 4 x 2 d_idx per (query group, key) (index
    scores twice, d iq, d ik)."""
    wl, x, ids = r["wl"], r["x"], r["ids"]
    p = api.problem_of(wl, sched=args.sched)
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
        "backward": {"ms_per_step": ms_b, "effective_TFLOPs": fl_b / ms_b / 1e9, "tflops_per_step": fl_b / 1e12,
                     "mfma_frac": fl_b / ms_b / 1e9 / PEAK_BF16_TFLOPS,
                     "kernels_ms": {k: round(v[0], 4) for k, v in kern_b.items()}},
        "indexer_kl": {"ms_per_step": ms_k, "effective_TFLOPs": fl_k / ms_k / 1e9, "tflops_per_step": fl_k / 1e12,
                       "kernels_ms": {k: round(v[0], 4) for k, v in kern_k.items()}},
    }


def run_decode(args, idx_format="plain", kv_format="plain"):
    """decode_16x1m forward steps.  idx_format "mxfp8": the idx_k cache is
    quantised once (untimed) to MXFP8 by msa_mxfp8_quantize and the index scan
    reads codes + scales (d_idx + d_idx/32 bytes per key) instead of bf16;
    kv_format "mxfp8": K and V too (d + d/32 bytes per key and tensor)."""
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
    ms, wall_ms, kern = time_steps(step, steps, args.warmup)
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
    del x, ws, ik
    torch.cuda.empty_cache()
    return {"workload": wl.name, "idx_format": idx_format, "kv_format": kv_format, "us_per_token": ms * 1e3 / (wl.batch * wl.n_q), "ms_per_step": ms,
            "algorithmic_bytes": total, "hbm_GBs": total / ms / 1e6, "hbm_frac": total / ms / 1e6 / PEAK_HBM_GBS,
            "kernels_ms": {k: round(v[0], 4) for k, v in kern.items()}}


def run_crossover(args, chunks=(256, 512, 1024, 1460, 2048, 4096, 16384)):
    """KV-outer vs query-outer attention time on the last `c` queries of the
    1M-token chunked-prefill cache (2 % hot blocks).  reuse = c*k*Bk/Nk is the
    average number of reads of a KV token, the quantity whose crossover the
    Fireworks note on KV-stationary attention puts near 2.85."""
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_32k", choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--sched", default="auto", choices=["auto", "kv_outer", "q_outer"])
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-train", action="store_true", help="skip the backward and indexer-loss legs")
    ap.add_argument("--cpu-sample", type=int, default=8192)
    ap.add_argument("--crossover", action="store_true",
                    help="also time both attention schedules on query chunks at the end of a 1M-token cache")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this MSA forward path is built and measured on a single GPU "
              "(one GPU's share of the work at its real shape); --gpus must be 1", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    r = run_prefill(args)
    wl, kern = r["wl"], r["kern"]
    value = r["fl_attn"] / r["ms"] / 1e9  # TFLOP/s
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    dom = max(kern, key=lambda k: kern[k][0] * kern[k][1])
    # Algorithmic work of the dominant kernel per launch.  The KV-outer kernel
    # moves (Q rows + partials) ~ 2*(2D+4)*G bytes per selected (query, group,
    # block) against 4*D*G*128 flops: ~127 flop/B at d=128, below the MI355X
    # balance of ~312 flop/B, so its roof is HBM; the index kernel's is MFMA.
    bytes_kv = r["bytes"]["attn_kvouter"]
    if dom == "attn_kvouter":
        achieved = bytes_kv / kern[dom][1] / kern[dom][0] / 1e6
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    elif dom == "combine":
        achieved = r["bytes"]["combine"] / kern[dom][1] / kern[dom][0] / 1e6
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    elif dom.startswith("attn_"):
        achieved = r["fl_attn"] / kern[dom][1] / kern[dom][0] / 1e9
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s"}
    elif dom.startswith("index_tile"):
        achieved = r["fl_idx"] / kern[dom][0] / 1e9
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": None, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["kernel"] = dom
    roof["algorithmic_bytes_per_launch"] = bytes_kv if dom == "attn_kvouter" else None
    roof["frac"] = roof["achieved"] / roof["peak"] if roof["achieved"] else None
    roof["traffic"] = measured_traffic(dom, wl.name)
    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": r["ms"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "n_q": wl.n_q, "n_k": wl.n_k, "q_offset": wl.q_offset,
                   "block_size": wl.block_size, "topk": wl.topk, "h_q": wl.h_q, "h_kv": wl.h_kv, "d": wl.d,
                   "d_idx": wl.d_idx, "sched": args.sched, "hot_frac": wl.hot_frac},
        "roofline": roof,
        "attention_tflops_per_step": r["fl_attn"] / 1e12, "index_tflops_per_step": r["fl_idx"] / 1e12,
        "index_TFLOPs": None, "wall_ms_per_step": r["wall_ms"],
        "attn_kvouter_TFLOPs": (r["fl_attn"] / kern["attn_kvouter"][0] / 1e9) if "attn_kvouter" in kern else None,
        # the same work over the attention part of the step alone (inversion, attention, combine: the
        # msa_sparse_attention calls), i.e. without the index scoring and selection
        "sparse_attention_TFLOPs": r["fl_attn"] / sum(v[0] * v[1] for k, v in kern.items()
                                                      if k.startswith(("inv_", "attn_")) or k == "combine") / 1e9,
        "attn_kvouter_GBs": (r["bytes"]["attn_kvouter"] / kern["attn_kvouter"][0] / 1e6)
        if "attn_kvouter" in kern else None,
        "combine_GBs": (r["bytes"]["combine"] / kern["combine"][0] / 1e6) if "combine" in kern else None,
        "algorithmic_bytes": r["bytes"],
        "kernels_ms": {k: round(v[0], 4) for k, v in kern.items()},
        "kernel_launches_per_step": {k: v[1] for k, v in kern.items()},
        "workspace_bytes": r["ws"],
    }
    it = [k for k in kern if k.startswith("index_tile")]
    if it:
        line["index_TFLOPs"] = r["fl_idx"] / kern[it[0]][0] / 1e9
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl, r["x"], args.cpu_sample)
    if not args.no_train:
        # training-side kernels on the same workload (reported beside the
        # forward figure, never as `value`)
        line.update(run_training(args, r))
    del r
    torch.cuda.empty_cache()
    if args.crossover:
        line["crossover"] = run_crossover(args)
    if not args.no_decode:
        line["decode"] = run_decode(args)
        # the same decode step over an MXFP8 index-key cache (a different
        # cache format, reported beside the bf16 figure, never as `value`)
        line["decode_mxfp8"] = run_decode(args, idx_format="mxfp8")
        # and over an all-MXFP8 cache (index keys, K and V)
        line["decode_mxfp8_cache"] = run_decode(args, idx_format="mxfp8", kv_format="mxfp8")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
