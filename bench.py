#!/usr/bin/env python3
"""Benchmark of the MoBA forward pass on one MI355X.

One step = the whole forward pass over one batch (block table, pooled keys,
gate, dispatch, own-block and earlier-block attention, merge), launched through
the C ABI's stage entry points on torch's current stream so that each stage
can be bracketed by HIP events on that same stream. Inputs are seeded synthetic
tensors already resident in HBM when timing starts.

Prints one JSON line: the value is effective TFLOP/s, i.e. 4*d*sum over
(row, head) of the keys actually attended (earlier blocks in full, own block
causally) divided by the step time; "roofline" rates the dominant kernel (the
earlier-block attention) against the bf16 MFMA peak, with its measured HBM
traffic when that measurement belongs to the current kernel sources;
"cpu_baseline" times the CPU oracle on a bounded sample of the same workload.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

DEFAULT_WORKLOAD = "gqa32x8_t1m_b4096_k12_bf16"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
HEAD_DIM = 128

# HBM traffic of one launch of the earlier-block attention at the 1M-token
# workload: rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch, one counter
# per pass, averaged over the launches of one step), each scaled by the factor
# between the true bytes of a plain copy kernel and the same counter's reading
# for it (bench_support/hbm_copy.py). It describes the kernel
# sources whose SHA-256 is given; for any other sources traffic is reported as
# null until it is measured again.
MEASURED_TRAFFIC = {
    "workload": "gqa32x8_t1m_b4096_k12_bf16",
    "sources": ["block_sparse_long_moba_amd/csrc/attn.hip",
                "block_sparse_long_moba_amd/csrc/moba_internal.h"],
    "sha256": "1fe1c69cc251278854d90efb0865020158c4184c46a379604063f8adcc8aa746",
    "fetch_kib": 21416819.1, "write_kib": 25368006.1,
    "fetch_factor": 1.99998, "write_factor": 1.0,
}


def measured_traffic(workload):
    """Bytes per launch of the earlier-block attention, or None."""
    import hashlib
    m = MEASURED_TRAFFIC
    if m["sha256"] is None or workload != m["workload"]:
        return None
    h = hashlib.sha256()
    for rel in m["sources"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != m["sha256"]:
        return None
    return int(m["fetch_kib"] * 1024 * m["fetch_factor"] + m["write_kib"] * 1024 * m["write_factor"])


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def effective_flop(lengths, B, k, Hq, d=HEAD_DIM):
    """4*d*Hq*sum_t |I(t)|: earlier chosen blocks count B keys each, the own
    block counts the keys up to and including the query."""
    tot = 0
    for L in lengths:
        t = np.arange(L, dtype=np.int64)
        c = t // B
        tot += int(((np.minimum(k, c + 1) - 1) * B + (t % B) + 1).sum())
    return 4.0 * d * Hq * tot


def dense_flop(lengths, Hq, d=HEAD_DIM):
    return float(sum(2.0 * d * Hq * L * (L + 1) for L in lengths))


class Timer:
    """Pairs of HIP events (torch.cuda.Event records on the current stream)."""

    def __init__(self):
        self.pairs = {}

    def run(self, name, fn):
        import torch
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.pairs.setdefault(name, []).append((a, b))

    def totals(self):
        return {n: (sum(a.elapsed_time(b) for a, b in v), len(v)) for n, v in self.pairs.items()}


# Further workloads timed after the headline one, each reported under
# "workloads" with its own roofline and CPU baseline: the metric is quoted at
# 128K and 1M tokens; the 32K layer and the packed batch are the other
# single-GPU shapes of the same head layout.
ALSO_WORKLOADS = ["gqa32x8_t128k_b4096_k12_bf16", "gqa32x8_t32k_b512_k3_bf16",
                  "gqa32x8_varlen4_t256k_b4096_k12_bf16"]


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--also", default="auto",
                    help="comma-separated further workloads reported under \"workloads\" "
                    "(auto: %s after the default workload, none otherwise; none: skip)"
                    % ",".join(ALSO_WORKLOADS))
    ap.add_argument("--no-dense", action="store_true", help="skip the dense causal baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gate", choices=["mean", "window", "pooled"], default="mean",
                    help="gate variant (mean: top-k by mean-pooled keys; window: sliding window "
                    "with --n-sink initial blocks; pooled: mean top-k plus --extra-max / "
                    "--extra-min blocks by max- / min-pooled keys, topk + extras slots)")
    ap.add_argument("--n-sink", type=int, default=1)
    ap.add_argument("--extra-max", type=int, default=1)
    ap.add_argument("--extra-min", type=int, default=1)
    ap.add_argument("--decode", default=None, metavar="SxL",
                    help="time decode instead: S sequences with KV caches of L tokens each "
                    "(e.g. 1x1048576 or 32x32768), one new query per sequence")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward pass (dq, dk, dv; with --gate) instead of the forward")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows the CPU oracle times (0 = sized for about 15 s; 5 s for the "
                    "further workloads)")
    ap.add_argument("--flush", choices=["auto", "on", "off"], default="auto",
                    help="write a 512 MiB buffer between timed forward steps, outside the "
                    "steps' events, so that no step finds its inputs in L2 / MALL (auto: on "
                    "when q, k and v together are below 4 GiB)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured copy and GEMM ceilings")
    ap.add_argument("--max-workspace-gib", type=float, default=48.0,
                    help="largest forward workspace: the kv heads per pass are halved "
                    "from all of them until the workspace fits")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: there is no multi-GPU path (the forward pass would "
              "shard by kv-head group with no exchange between GPUs). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.decode:
        decode_bench(args)
        return
    if args.bwd:
        bwd_bench(args)
        return

    if args.also == "auto":
        also = ALSO_WORKLOADS if args.workload == DEFAULT_WORKLOAD and args.gate == "mean" else []
    elif args.also in ("", "none"):
        also = []
    else:
        also = [x for x in args.also.split(",") if x]
    from block_sparse_long_moba_amd import synth
    for name in [args.workload] + also:
        if name not in synth.WORKLOADS:
            print("unknown workload %s (known: %s)" % (name, ", ".join(synth.WORKLOADS)),
                  file=sys.stderr)
            sys.exit(2)

    head = forward_bench(args, args.workload, headline=True)
    res = {
        "metric": "MoBA fwd ms + effective TFLOP/s at 128K/1M tokens (8B heads), % MFMA peak",
        "value": head["value"], "unit": "TFLOP/s (effective)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": head["dtype"], "data": "synthetic (seeded N(0,1) q/k/v, per-block key offsets)",
        "config": head["config"],
    }
    res.update({k: v for k, v in head.items() if k not in ("value", "ms", "dtype", "config")})
    if also:
        res["workloads"] = {}
        for name in also:
            r = forward_bench(args, name, headline=False)
            res["workloads"][name] = {
                "value": r["value"], "unit": "TFLOP/s (effective)", "ms_per_step": r["ms"],
                "dtype": r["dtype"], "config": r["config"],
                "attention_mfma_frac": r["attention_mfma_frac"], "stage_ms": r["stage_ms"],
                "hbm": r["hbm"], "roofline": r["roofline"], "cpu_baseline": r["cpu_baseline"]}
    print(json.dumps(res), flush=True)


def forward_bench(args, name, headline):
    """Times the forward pass on workload `name`; with headline, also the
    dense causal baseline and the measured ceilings (unless switched off)."""
    import torch
    from block_sparse_long_moba_amd import moba, synth
    from block_sparse_long_moba_amd.tensors import to_device, workspace_view

    w = synth.WORKLOADS[name]
    B, k, Hq, Hkv = w.block_size, w.topk, w.num_q_heads, w.num_kv_heads
    if args.gate == "pooled":
        k += args.extra_max + args.extra_min  # slots: the mean gate's k plus the extra picks
    T = w.total_tokens
    log("workload %s: generating seeded inputs" % w.name)
    t0 = time.time()
    inp = synth.generate(w)
    log("inputs ready in %.1f s; uploading" % (time.time() - t0))
    torch.cuda.set_device(0)
    q, kk, v, cu = (to_device(x) for x in (inp.q, inp.k, inp.v, inp.cu_seqlens))
    shape = moba.shape_of(q, kk, cu, max_seqlen=max(w.lengths))
    P = Hkv
    while P > 1 and moba.moba_fwd_workspace_size(shape, B, k, P) > args.max_workspace_gib * 2**30:
        P //= 2
    lay = moba.moba_plan(shape, B, k, P)
    ws = torch.empty(lay.total_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda")
    passes = list(range(0, Hkv, lay.kv_heads_per_pass))
    log("workspace %.1f GiB, %d pass(es) of %d kv heads" % (lay.total_bytes / 2**30, len(passes),
                                                         lay.kv_heads_per_pass))

    def gate(g0):
        if args.gate == "window":
            moba.moba_gate_window(shape, B, k, args.n_sink, lay, ws, g0)
        elif args.gate == "pooled":
            moba.moba_gate_pooled(q, shape, B, k, args.extra_max, args.extra_min, lay, ws, g0)
        else:
            moba.moba_gate(q, shape, B, k, lay, ws, g0)

    def pools():
        if args.gate != "window":
            moba.moba_meanpool(kk, shape, B, lay, ws)
        if args.gate == "pooled":
            moba.moba_minmaxpool(kk, shape, B, lay, ws)

    def step(tm):
        tm.run("seqtable", lambda: moba.moba_seqtable(cu, shape, B, lay, ws))
        tm.run("meanpool", pools)
        for g0 in passes:
            tm.run("gate", lambda: gate(g0))
            tm.run("dispatch", lambda: moba.moba_dispatch(shape, B, k, lay, ws, g0))
            if w.dtype == "bf16":  # as moba_fwd runs it: the own block merged last
                tm.run("attn_prep", lambda: moba.moba_attn_prep(kk, v, shape, B, k, lay, ws, g0))
                tm.run("attn_hist", lambda: moba.moba_attn_fwd_hist(q, kk, shape, B, k, lay, ws,
                                                                     g0))
                tm.run("attn_own_merge", lambda: moba.moba_attn_fwd_own_merge(
                    q, kk, shape, B, k, lay, ws, out, lse, g0))
            else:
                tm.run("attn_diag", lambda: moba.moba_attn_fwd_diag(q, kk, v, shape, B, k, lay,
                                                                     ws, g0))
                tm.run("attn_hist", lambda: moba.moba_attn_fwd_hist(q, kk, shape, B, k, lay, ws,
                                                                     g0))
                tm.run("merge", lambda: moba.moba_merge(shape, B, k, lay, ws, out, lse, g0))

    # earlier-block rows dispatched per pass (for the dominant kernel's flops),
    # and whether the gate counted them (then the dispatch reads idx once)
    nbins = lay.kv_heads_per_pass * lay.num_blocks_bound
    hist_rows, gate_counted = [], []
    moba.moba_seqtable(cu, shape, B, lay, ws)
    pools()
    for g0 in passes:
        gate(g0)
        moba.moba_dispatch(shape, B, k, lay, ws, g0)
        torch.cuda.synchronize()
        words = workspace_view(ws, lay.bins_offset, 4 * nbins + 2 + 1, torch.int32)
        hist_rows.append(int(words[2 * nbins].item()) & 0xFFFFFFFF)  # offset[nbins]
        gate_counted.append(int(words[4 * nbins + 2].item()) != 0)

    log("warmup %d step(s)" % args.warmup)
    for _ in range(args.warmup):
        step(Timer())
    torch.cuda.synchronize()
    es = 2 if w.dtype == "bf16" else 4
    qkv_bytes = T * (Hq + 2 * Hkv) * HEAD_DIM * es
    flush = args.flush == "on" or (args.flush == "auto" and qkv_bytes < (4 << 30))
    fbuf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if flush else None
    log("timing %d step(s)%s" % (args.steps, " with a cache flush between steps" if flush else ""))
    tm = Timer()
    spans = []
    torch.cuda.synchronize()
    for i in range(args.steps):
        if fbuf is not None:
            fbuf.fill_(i & 255)  # between the steps' events: not timed
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step(tm)
        b.record()
        spans.append((a, b))
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in spans) / args.steps
    del fbuf
    stages = {n: (tot / args.steps, cnt) for n, (tot, cnt) in tm.totals().items()}
    log("step %.2f ms; stages %s" % (ms, {n: round(v[0], 3) for n, v in stages.items()}))

    if args.gate == "mean":
        eff = effective_flop(w.lengths, B, k, Hq)
    else:  # keys actually attended: dispatched earlier blocks in full, own block causally
        own = sum(int(((np.arange(L) % B) + 1).sum()) for L in w.lengths)
        eff = 4.0 * HEAD_DIM * (B * float(sum(hist_rows)) + Hq * own)
    value = eff / (ms * 1e-3) / 1e12
    # dominant kernel: earlier-block attention, MFMA bound
    hist_ms_total, hist_launches = tm.totals()["attn_hist"]
    hist_flop_per_step = 4.0 * HEAD_DIM * B * sum(hist_rows)
    hist_avg_ms = hist_ms_total / hist_launches
    hist_flop_per_launch = hist_flop_per_step / len(passes)
    achieved = hist_flop_per_launch / (hist_avg_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS
    traffic = measured_traffic(w.name)
    roofline = {"kernel": "attn_hist (earlier-block attention)", "bound": "mfma",
                "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "avg_launch_ms": round(hist_avg_ms, 4), "launches_per_step": len(passes),
                "flop_per_launch": hist_flop_per_launch}

    # memory-bound stages against the HBM roofline
    nb = sum(-(-L // B) for L in w.lengths)
    if args.gate == "window":   # no pooling; the gate writes idx only
        mp_bytes, gate_bytes = 0, T * Hq * k * 4
    elif args.gate == "pooled":  # k read twice (mean, max/min); q read by three rankings
        n_lists = (k - args.extra_max - args.extra_min) + args.extra_max + 1 + args.extra_min + 1
        mp_bytes = 2 * T * Hkv * HEAD_DIM * es + 3 * nb * Hkv * HEAD_DIM * 8
        gate_bytes = 3 * T * Hq * HEAD_DIM * es + T * Hq * (2 * n_lists + k) * 4
    else:
        mp_bytes = T * Hkv * HEAD_DIM * es + nb * Hkv * HEAD_DIM * 4
        gate_bytes = T * Hq * HEAD_DIM * es + T * Hq * k * 4
    # dispatch: idx read by the scatter pass (and by the count pass unless the
    # gate counted), items written
    n_hist = sum(hist_rows)
    idx_reads = sum(1 if c else 2 for c in gate_counted) / len(passes)
    disp_bytes = int(idx_reads * T * Hq * k * 4) + n_hist * 4
    # merge (float32): every valid slot's partial (row and lse) read, out and
    # lse written
    merge_bytes = (n_hist + T * Hq) * (HEAD_DIM * es + 4) + T * Hq * (HEAD_DIM * es + 4)
    # value transpose (bf16 stage of its own): values and keys read, vt written
    prep_bytes = 3 * T * Hkv * HEAD_DIM * es
    hbm = {}
    for sname, nbytes in (("meanpool", mp_bytes), ("gate", gate_bytes), ("dispatch", disp_bytes),
                          ("attn_prep", prep_bytes), ("merge", merge_bytes)):
        sm = stages[sname][0] if sname in stages else 0.0
        if nbytes == 0 or sm <= 0:
            continue
        hbm[sname] = {"ms": round(sm, 4), "GB/s": round(nbytes / (sm * 1e-3) / 1e9, 1),
                      "frac": round(nbytes / (sm * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    # attention: own and earlier blocks (bf16: with the merge, done by the
    # own-block kernel; float32: with the value transpose)
    attn_ms = sum(st[0] for name, st in stages.items()
                  if name.startswith("attn_") and name != "attn_prep")
    attn_eff = eff / (attn_ms * 1e-3) / 1e12

    dense = None
    if headline and not args.no_dense:
        log("dense causal baseline")
        dws = torch.empty(moba.moba_dense_causal_workspace_size(shape), dtype=torch.uint8,
                          device="cuda")
        dout = torch.empty_like(q)
        moba.moba_dense_causal_fwd(q, kk, v, cu, out=dout, workspace=dws,
                                   max_seqlen=max(w.lengths))
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        moba.moba_dense_causal_fwd(q, kk, v, cu, out=dout, workspace=dws,
                                   max_seqlen=max(w.lengths))
        b.record()
        torch.cuda.synchronize()
        dms = a.elapsed_time(b)
        dfl = dense_flop(w.lengths, Hq)
        dense = {"ms": round(dms, 3), "TFLOP/s": round(dfl / (dms * 1e-3) / 1e12, 1),
                 "mfma_frac": round(dfl / (dms * 1e-3) / 1e12 / peak, 4),
                 "speedup_moba_vs_dense": round(dms / ms, 3)}
        del dws, dout

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, w, args.cpu_rows, args.gate, k, args.n_sink, args.extra_max,
                           args.extra_min, seconds=15 if headline else 5)
        # the whole pass on the CPU, extrapolated from the sample by effective FLOP
        cpu["extrapolated_full_pass_s"] = round(eff / (cpu["value"] * 1e12), 1)

    # the least any forward pass must move: q, k, v read and out, lse written
    io_bytes = qkv_bytes + T * Hq * HEAD_DIM * es + T * Hq * 4
    minimal_io = {"bytes": io_bytes,
                  "ms_at_hbm_peak": round(io_bytes / (PEAK_HBM_GBS * 1e9) * 1e3, 3)}

    ceilings = None
    if headline and not args.no_ceilings:
        del ws, out, lse, q, kk, v
        ceilings = measured_ceilings(torch)
        ceilings["attn_hist_frac_of_gemm"] = round(achieved / ceilings["bf16_gemm_TFLOP/s"], 4)
        ceilings["attn_hist_frac_of_mfma_loop"] = round(
            achieved / ceilings["bf16_mfma_loop_TFLOP/s"], 4)
        ceilings["hbm_stages_frac_of_copy"] = {
            n: round(x["GB/s"] / ceilings["hbm_copy_GB/s"], 4) for n, x in hbm.items()}

    config = {"workload": w.name, "seq_lens": list(w.lengths), "total_tokens": T,
              "q_heads": Hq, "kv_heads": Hkv, "head_dim": HEAD_DIM, "block_size": B,
              "topk": k, "kv_heads_per_pass": lay.kv_heads_per_pass,
              "gate": {"mean": {"kind": "mean"},
                       "window": {"kind": "window", "n_sink": args.n_sink},
                       "pooled": {"kind": "pooled", "extra_max": args.extra_max,
                                  "extra_min": args.extra_min}}[args.gate],
              "parallelism": "single GPU"}
    return {
        "value": round(value, 3), "ms": round(ms, 3), "dtype": w.dtype, "config": config,
        "effective_flop": eff,
        "attention_effective_TFLOPs": round(attn_eff, 2),
        "attention_mfma_frac": round(attn_eff / peak, 4),
        "stage_ms": {n: round(v[0], 4) for n, v in stages.items()},
        "hbm": hbm,
        "dense_causal": dense,
        "roofline": roofline,
        "minimal_io": minimal_io,
        "measured_ceilings": ceilings,
        "cpu_baseline": cpu,
    }


def bwd_bench(args):
    """Backward pass of the workload (gate as --gate): D = <dO, O>, then per
    pass the gate and dispatch again, partial dq (own block, earlier blocks),
    their sum, and dk/dv; each stage bracketed by HIP events. The
    forward pass that produced out and lse runs once, untimed. Effective
    FLOP = 10*d per attended (row, head, key): the five products of the
    attention gradient (S recomputed, dP, dV, dK, dQ)."""
    import torch
    from block_sparse_long_moba_amd import moba, synth
    from block_sparse_long_moba_amd.tensors import to_device, workspace_view

    w = synth.WORKLOADS[args.workload]
    assert w.dtype == "bf16", "the backward pass is bf16 only"
    B, k, Hq, Hkv = w.block_size, w.topk, w.num_q_heads, w.num_kv_heads
    if args.gate == "pooled":
        k += args.extra_max + args.extra_min
    gate = {"mean": moba.gate_mean(), "window": moba.gate_window(args.n_sink),
            "pooled": moba.gate_pooled(args.extra_max, args.extra_min)}[args.gate]
    T = w.total_tokens
    log("bwd, workload %s: generating seeded inputs" % w.name)
    inp = synth.generate(w)
    torch.cuda.set_device(0)
    q, kk, v, cu = (to_device(x) for x in (inp.q, inp.k, inp.v, inp.cu_seqlens))
    shape = moba.shape_of(q, kk, cu, max_seqlen=max(w.lengths))
    P = Hkv
    while P > 1 and moba.moba_fwd_workspace_size(shape, B, k, P) > (48 << 30):
        P //= 2
    fws = torch.empty(moba.moba_fwd_workspace_size(shape, B, k, P), dtype=torch.uint8,
                      device="cuda")
    out, lse = moba.moba_fwd_gated(q, kk, v, cu, B, k, gate, fws, max_seqlen=max(w.lengths))
    torch.cuda.synchronize()
    del fws
    gen = torch.Generator(device="cuda").manual_seed(w.seed + 5)
    dout = torch.randn(q.shape, device="cuda", generator=gen).to(torch.bfloat16)
    P = Hkv
    while P > 1 and moba.moba_bwd_workspace_size(shape, B, k, P) > (64 << 30):
        P //= 2
    lay = moba.moba_bwd_plan(shape, B, k, P)
    ws = torch.empty(lay.total_bytes, dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(kk), torch.empty_like(v)
    passes = list(range(0, Hkv, lay.kv_heads_per_pass))
    log("bwd workspace %.1f GiB, %d pass(es) of %d kv heads" % (
        lay.total_bytes / 2**30, len(passes), lay.kv_heads_per_pass))

    def run_gate(g0):
        if args.gate == "window":
            moba.moba_gate_window(shape, B, k, args.n_sink, lay, ws, g0)
        elif args.gate == "pooled":
            moba.moba_gate_pooled(q, shape, B, k, args.extra_max, args.extra_min, lay, ws, g0)
        else:
            moba.moba_gate(q, shape, B, k, lay, ws, g0)

    def pools():
        if args.gate != "window":
            moba.moba_meanpool(kk, shape, B, lay, ws)
        if args.gate == "pooled":
            moba.moba_minmaxpool(kk, shape, B, lay, ws)

    def step(tm):
        tm.run("seqtable", lambda: moba.moba_seqtable(cu, shape, B, lay, ws))
        tm.run("meanpool", pools)
        tm.run("delta", lambda: moba.moba_bwd_delta(out, dout, shape, B, k, lay, ws))
        for g0 in passes:
            tm.run("gate", lambda: run_gate(g0))
            tm.run("dispatch", lambda: moba.moba_dispatch(shape, B, k, lay, ws, g0))
            tm.run("dq_diag", lambda: moba.moba_attn_bwd_dq(q, kk, v, dout, lse, shape, B, k,
                                                             lay, ws, g0, which=1))
            tm.run("dq_hist", lambda: moba.moba_attn_bwd_dq(q, kk, v, dout, lse, shape, B, k,
                                                             lay, ws, g0, which=2))
            tm.run("dq_sum", lambda: moba.moba_attn_bwd_dq_sum(shape, B, k, lay, ws, dq, g0))
            tm.run("dkdv", lambda: moba.moba_attn_bwd_dkdv(q, kk, v, dout, lse, shape, B, k, lay,
                                                            ws, dk, dv, g0))

    nbins = lay.kv_heads_per_pass * lay.num_blocks_bound
    hist_rows = []
    moba.moba_seqtable(cu, shape, B, lay, ws)
    pools()
    for g0 in passes:
        run_gate(g0)
        moba.moba_dispatch(shape, B, k, lay, ws, g0)
        torch.cuda.synchronize()
        off = workspace_view(ws, lay.bins_offset + 4 * nbins, nbins + 1, torch.int32)
        hist_rows.append(int(off[-1].item()) & 0xFFFFFFFF)

    log("warmup %d step(s)" % args.warmup)
    for _ in range(args.warmup):
        step(Timer())
    torch.cuda.synchronize()
    log("timing %d step(s)" % args.steps)
    tm = Timer()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step(tm)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    totals = tm.totals()
    stages = {n: tot / args.steps for n, (tot, cnt) in totals.items()}
    log("bwd step %.2f ms; stages %s" % (ms, {n: round(x, 3) for n, x in stages.items()}))

    d = HEAD_DIM
    own_pairs = Hq * sum(int(((np.arange(L) % B) + 1).sum()) for L in w.lengths)
    hist_pairs = B * float(sum(hist_rows))
    eff = 10.0 * d * (own_pairs + hist_pairs)
    # per-kernel algorithmic FLOP: dq = S, dP, dQ (6 d per pair); dk/dv = S, dP,
    # dV, dK (8 d per pair)
    kflop = {"dq_diag": 6.0 * d * own_pairs, "dq_hist": 6.0 * d * hist_pairs,
             "dkdv": 8.0 * d * (own_pairs + hist_pairs)}
    kernels = {}
    for name, fl in kflop.items():
        tot, cnt = totals[name]
        kernels[name] = {"ms_per_step": round(tot / args.steps, 3),
                         "avg_launch_ms": round(tot / cnt, 4),
                         "TFLOP/s": round(fl / (tot / args.steps * 1e-3) / 1e12, 2),
                         "frac": round(fl / (tot / args.steps * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                       4)}
    dom = max(kernels, key=lambda n: kernels[n]["ms_per_step"])
    roofline = {"kernel": dom, "bound": "mfma", "achieved": kernels[dom]["TFLOP/s"],
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": kernels[dom]["frac"],
                "traffic": None, "avg_launch_ms": kernels[dom]["avg_launch_ms"],
                "launches_per_step": len(passes),
                "flop_per_launch": kflop[dom] / len(passes)}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_bwd(
            inp, w, lambda rows: dout[torch.from_numpy(rows).cuda()].double().cpu().numpy(),
            args.cpu_rows, args.gate, k, args.n_sink, args.extra_max, args.extra_min)
    es = 2
    n_hist = float(sum(hist_rows))
    hbm_bytes = {"delta": 2 * T * Hq * d * es + T * Hq * 4,
                 "dq_sum": (n_hist + T * Hq) * d * 4 + T * Hq * k * 4 + T * Hq * d * es}
    hbm = {n: {"ms": round(stages[n], 4), "GB/s": round(b / (stages[n] * 1e-3) / 1e9, 1),
               "frac": round(b / (stages[n] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
           for n, b in hbm_bytes.items()}
    res = {
        "metric": "MoBA bwd ms + effective TFLOP/s (10*d per attended row-head-key), % MFMA peak",
        "value": round(eff / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s (effective)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v/dO, per-block key offsets)",
        "config": {"workload": w.name, "pass": "backward", "seq_lens": list(w.lengths),
                   "total_tokens": T, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "block_size": B, "topk": k, "kv_heads_per_pass": lay.kv_heads_per_pass,
                   "gate": {"mean": {"kind": "mean"},
                            "window": {"kind": "window", "n_sink": args.n_sink},
                            "pooled": {"kind": "pooled", "extra_max": args.extra_max,
                                       "extra_min": args.extra_min}}[args.gate],
                   "parallelism": "single GPU"},
        "effective_flop": eff,
        "stage_ms": {n: round(x, 4) for n, x in stages.items()},
        "kernels": kernels, "hbm": hbm, "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def decode_bench(args):
    """Decode: one new query per sequence over a KV cache (the 8B head shape,
    block 4096, top-k 12). Reports the latency of moba_decode and its HBM
    rate: the keys and values of the distinct blocks each (sequence, kv head)
    selected, read once, plus queries, pooled keys and outputs. The same call
    with topk covering every block is dense decode over the whole cache."""
    import torch
    from block_sparse_long_moba_amd import moba, synth
    from block_sparse_long_moba_amd.tensors import to_device, workspace_view

    S, L = (int(x) for x in args.decode.lower().split("x"))
    Hq, Hkv, B, k = 32, 8, 4096, 12
    log("decode: %d sequence(s) with caches of %d tokens: generating" % (S, L))
    inp = synth.custom([L] * S, Hq, Hkv, HEAD_DIM, "bf16", B, k, 91)
    cu = inp.cu_seqlens
    qd = np.stack([inp.q[cu[s + 1] - 1] for s in range(S)])
    q, kc, vc, cud = (to_device(x) for x in (qd, inp.k, inp.v, cu))
    inp_q_host, inp_k_host, inp_v_host = inp.q, inp.k, inp.v
    T = int(cu[-1])
    res = {}
    for name, topk in (("moba", k), ("dense", -(-L // B))):
        sh = moba.make_shape(T, S, Hq, Hkv, HEAD_DIM, "bf16", max_seqlen=L)
        ws = torch.empty(moba.moba_decode_workspace_size(sh, B, topk), dtype=torch.uint8,
                         device="cuda")
        moba.moba_decode_prepare(kc, cud, sh, B, topk, ws)
        out, lse = moba.moba_decode(q, kc, vc, sh, B, topk, ws)
        torch.cuda.synchronize()
        # selected blocks per (sequence, kv head): the kernel reads each once
        nb = -(-L // B)
        NBb = -(-T // B) + S
        table = (2 * 4 * (S + 1) + 15) // 16 * 16 + 16 * NBb
        align = lambda x: (x + 255) // 256 * 256
        off = align(align(table) + 8 * NBb * Hkv * HEAD_DIM)
        idx = workspace_view(ws, off, S * Hq * topk, torch.int32).view(S, Hkv, Hq // Hkv, topk)
        idx = idx.cpu().numpy()
        kv_bytes = 0
        for s in range(S):
            for g in range(Hkv):
                blocks = set(int(x) for x in idx[s, g].ravel() if x >= 0)
                kv_bytes += sum(min(B, L - j * B) for j in blocks) * HEAD_DIM * 2 * 2
        other = S * Hq * HEAD_DIM * 2 * 2 + S * Hq * (nb - 1) * HEAD_DIM * 4
        for _ in range(args.warmup):
            moba.moba_decode(q, kc, vc, sh, B, topk, ws, out=out, lse=lse)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            moba.moba_decode(q, kc, vc, sh, B, topk, ws, out=out, lse=lse)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / args.steps
        nbytes = kv_bytes + other
        res[name] = {"topk": topk, "ms": round(ms, 4), "hbm_bytes": nbytes,
                     "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        log("%s decode: %.4f ms, %.1f GB/s" % (name, ms, res[name]["GB/s"]))
        del ws
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        rows = np.asarray(cu[1:], dtype=np.int64) - 1  # the query is the last cache row
        log("cpu baseline: oracle prefill result at the %d last rows" % S)
        t0 = time.time()
        oracle.moba(inp_q_host, inp_k_host, inp_v_host, cu, B, k, rows=rows)
        dt = time.time() - t0
        cpu = {"value": round(dt * 1e3, 3), "unit": "ms", "cores": _threads(), "kind": "oracle",
               "sample": "the whole call: pooled keys of the cache's blocks, then selection "
                         "and attention of the %d queries" % S}
    line = {
        "metric": "MoBA decode latency (one query per sequence over its KV cache)",
        "value": res["moba"]["ms"], "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": False, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v, per-block key offsets)",
        "config": {"workload": "decode_%dx%d" % (S, L), "sequences": S, "cache_tokens": L,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": HEAD_DIM, "block_size": B,
                   "topk": k},
        "roofline": {"bound": "hbm", "achieved": res["moba"]["GB/s"], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": res["moba"]["frac"], "traffic": None},
        "dense_decode": res["dense"],
        "speedup_moba_vs_dense": round(res["dense"]["ms"] / res["moba"]["ms"], 3),
        "moba": res["moba"],
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def _threads():
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def measured_ceilings(torch):
    """Practical ceilings on this GPU, measured with torch (a measuring
    instrument here, not part of the path): HBM by a 4 GiB float32 copy
    (negation: every byte read once and written once), bf16 matrix-core
    throughput by an 8192^3 GEMM (hipBLASLt). Best of a few runs each."""
    def best_ms(fn, reps):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b))
        return min(out)
    n = 1 << 30
    src = torch.empty(n, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    copy_ms = best_ms(lambda: torch.neg(src, out=dst), 3)
    del src, dst
    m = 8192
    a = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    gemm_ms = best_ms(lambda: torch.mm(a, b), 5)
    del a, b
    # pure MFMA loop (libmoba_probe.so): 8 waves per CU, 4 independent chains
    probe = ctypes.CDLL(os.path.join(ROOT, "bench_support", "libmoba_probe.so"))
    probe.moba_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p]
    blocks = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    iters = 100000
    pout = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def run_probe():
        rc = probe.moba_probe_mfma_bf16(blocks, iters, ctypes.c_void_p(pout.data_ptr()),
                                        ctypes.c_void_p(stream))
        assert rc == 0, "MFMA probe launch failed (%d)" % rc
    mfma_ms = best_ms(run_probe, 3)
    mfma_flop = blocks * 4.0 * iters * 4 * 32768
    return {"hbm_copy_GB/s": round(2 * 4 * n / (copy_ms * 1e-3) / 1e9, 1),
            "bf16_gemm_TFLOP/s": round(2.0 * m ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
            "bf16_mfma_loop_TFLOP/s": round(mfma_flop / (mfma_ms * 1e-3) / 1e12, 1),
            "how": "4 GiB float32 negation (torch); 8192^3 bf16 torch.mm (hipBLASLt); "
                   "a loop of independent 32x32x16 bf16 MFMAs, 8 waves per CU "
                   "(libmoba_probe.so)"}


def cpu_baseline(inp, w, n_rows, gate="mean", k=None, n_sink=1, extra_max=1, extra_min=1,
                 seconds=15):
    """The fp64 oracle on a bounded sample of the same workload: the block
    representations the gate needs (pooled keys of every block), then the
    gate's selection and the attention for n sampled rows (all heads); with
    n_rows = 0 the sample is sized for about `seconds` of attention work."""
    import oracle
    B, Hq = w.block_size, w.num_q_heads
    k = w.topk if k is None else k
    rng = np.random.default_rng(w.seed + 77)
    T = w.total_tokens
    if n_rows <= 0:
        # about `seconds` of attention work at ~1.5 GFLOP/s per thread (fp64, plain loops)
        per_row = 4.0 * HEAD_DIM * Hq * (k * B)
        n_rows = int(max(8, min(T, seconds * 1.5e9 * _threads() / per_row)))
    rows = np.sort(rng.choice(T, size=min(n_rows, T), replace=False)).astype(np.int64)
    log("cpu baseline: oracle on %d sampled rows (%s gate)" % (len(rows), gate))
    t0 = time.time()
    if gate == "window":
        sel = oracle.select_window(inp.cu_seqlens, B, k, n_sink, Hq, rows=rows, total_tokens=T)
    else:
        kbar = oracle.meanpool(inp.k, inp.cu_seqlens, B)
        if gate == "pooled":
            kmax, kmin = oracle.minmaxpool(inp.k, inp.cu_seqlens, B)
            sel, _ = oracle.select_pooled(inp.q, kbar, kmax, kmin, inp.cu_seqlens, B, k,
                                          extra_max, extra_min, rows=rows)
        else:
            sel, _, _ = oracle.select(inp.q, kbar, inp.cu_seqlens, B, k, rows=rows)
    oracle.attend(inp.q, inp.k, inp.v, inp.cu_seqlens, B, k, sel, rows=rows)
    dt = time.time() - t0
    flop = 4.0 * HEAD_DIM * float(attended_keys(inp.cu_seqlens, B, sel, rows).sum())
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s (effective)",
            "cores": _threads(), "kind": "oracle", "seconds": round(dt, 2),
            "sample": "%d random rows x %d heads of %s (%s gate: block representations of all "
                      "blocks, then selection and attention for the sampled rows)"
                      % (len(rows), Hq, w.name, gate)}


def attended_keys(cu, B, sel, rows):
    """Keys attended per (sampled row, head) under selection sel[n][H][k]:
    earlier chosen blocks in full, the own block up to the row."""
    seq = np.searchsorted(cu, rows, side="right") - 1
    local = rows - cu[seq]
    c = local // B
    L = cu[seq + 1] - cu[seq]
    out = np.zeros(sel.shape[:2], dtype=np.int64)
    for i in range(sel.shape[0]):
        for h in range(sel.shape[1]):
            for j in sel[i, h]:
                if j < 0:
                    continue
                out[i, h] += (local[i] % B + 1) if j == c[i] else min(B, L[i] - j * B)
    return out


def cpu_baseline_bwd(inp, w, dout_rows_fn, n_rows, gate="mean", k=None, n_sink=1, extra_max=1,
                     extra_min=1):
    """The fp64 oracle's gradient on a bounded sample: dq of n sampled rows
    (all heads) over the gate's selection; 6 d per attended (row, head, key)
    (scores, dP and dq; the key-side gradients of a row cost the same again)."""
    import oracle
    B, Hq = w.block_size, w.num_q_heads
    k = w.topk if k is None else k
    rng = np.random.default_rng(w.seed + 78)
    T = w.total_tokens
    if n_rows <= 0:
        per_row = 6.0 * HEAD_DIM * Hq * (k * B)
        n_rows = int(max(8, min(T, 15 * 1.5e9 * _threads() / per_row)))
    rows = np.sort(rng.choice(T, size=min(n_rows, T), replace=False)).astype(np.int64)
    dout_rows = dout_rows_fn(rows)
    log("cpu baseline: oracle dq on %d sampled rows (%s gate)" % (len(rows), gate))
    t0 = time.time()
    if gate == "window":
        sel = oracle.select_window(inp.cu_seqlens, B, k, n_sink, Hq, rows=rows, total_tokens=T)
    else:
        kbar = oracle.meanpool(inp.k, inp.cu_seqlens, B)
        if gate == "pooled":
            kmax, kmin = oracle.minmaxpool(inp.k, inp.cu_seqlens, B)
            sel, _ = oracle.select_pooled(inp.q, kbar, kmax, kmin, inp.cu_seqlens, B, k,
                                          extra_max, extra_min, rows=rows)
        else:
            sel, _, _ = oracle.select(inp.q, kbar, inp.cu_seqlens, B, k, rows=rows)
    oracle.attend_bwd_dq_rows(inp.q, inp.k, inp.v, dout_rows, inp.cu_seqlens, B, k, sel, rows)
    dt = time.time() - t0
    flop = 6.0 * HEAD_DIM * float(attended_keys(inp.cu_seqlens, B, sel, rows).sum())
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s (6 d per attended pair)",
            "cores": _threads(), "kind": "oracle", "seconds": round(dt, 2),
            "sample": "dq of %d random rows x %d heads of %s (%s gate: block representations "
                      "of all blocks, selection, scores, dP and dq for the sampled rows)"
                      % (len(rows), Hq, w.name, gate)}


if __name__ == "__main__":
    main()
