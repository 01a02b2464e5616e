"""Benchmark of the one-GPU ring-attention forward.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--prefetch]
                    [--backward] [--no-cpu-baseline] [--dtype bf16|f16] [--key-padding FRAC]

A step is one ring_attn_forward call: every ring step of every virtual device
plus the fused finalize, on synthetic bf16 inputs already resident in HBM.
Without --prefetch the forward is two launches: the V^T pack, then one
launch of the step kernel that runs the whole ring (each workgroup walks its
query tile through its device's key/value blocks in ring order).  With
--prefetch it is the pack and one step-kernel launch per ring step, the next
blocks copied on a side stream.
Default workload: 32768 tokens, 32 heads, d = 128, 8 contiguous ring blocks of
4096, causal mask, scale 1/sqrt(128).  Throughput is causal-adjusted: FLOP =
4 * d * Hq * (allowed (query, key) pairs), i.e. only the two contractions over
pairs the mask lets through.  Prints one JSON line.

--backward times ring_attn_backward instead (the D = dout.out prep, the dq
kernel and the dk/dv kernel), with the forward's out and lse and a seeded
dout resident in HBM; FLOP = 10 * d * Hq * allowed pairs (the five
contractions of the backward: S, dP, dV, dK, dQ), fp32 gradients.

--dtype f16 runs the same shapes in fp16.  --key-padding FRAC adds a seeded
key-padding mask (about FRAC of the keys padded, plus a run of whole padded
tiles); the allowed pairs, and so the FLOP, then count real keys only.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak (AMD published figure)
PEAK_FP32_VECTOR_TFLOPS = 157.3  # MI355X fp32 vector peak (AMD published figure)
DEFAULT_WORKLOAD = "causal32k_h32_d128_8blk"
# the per-ring-step kernel that the prefetching forward launches once per step
STEP_KERNEL = "step_bf16_kernel<__bf16, 128, true, true, false>"
# The kernels' sources plus the driver that sets their launch order (a
# traffic record is only valid for the code and the order it was taken with).
KERNEL_SOURCES = ["ring_attention_step_amd/csrc/ring_fwd.hip", "ring_attention_step_amd/csrc/step_bf16.hip",
                  "ring_attention_step_amd/csrc/pack_vt.hip", "ring_attention_step_amd/csrc/plan.h",
                  "ring_attention_step_amd/csrc/kernels.h", "ring_attention_step_amd/csrc/api.hip"]
BWD_KERNEL_SOURCES = ["ring_attention_step_amd/csrc/backward.hip", "ring_attention_step_amd/csrc/bwd_kernels.h",
                      "ring_attention_step_amd/csrc/plan.h",
                      "ring_attention_step_amd/csrc/kernels.h", "ring_attention_step_amd/csrc/api.hip"]


def _code_only(text: str) -> str:
    """Source text without comments and blank space (comment edits leave the kernel unchanged)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def ring_kernel_name(w, key_padding=0.0) -> str:
    """The one-launch kernel instance a workload runs: element type, head
    dimension, key-padding mask, q-tile-major item order (striped blocks)."""
    e = "_Float16" if w.dtype == "f16" else "__bf16"
    b = lambda x: "true" if x else "false"
    return "ring_fwd_kernel<%s, %d, %s, %s>" % (e, w.d, b(key_padding > 0), b(w.layout == 1))


def bwd_kernel_names(w, key_padding=0.0, dkdv_only=False) -> str:
    """The backward kernel instances a workload runs (striped layouts take the
    tile-index-major item order)."""
    e = "_Float16" if w.dtype == "f16" else "__bf16"
    b = lambda x: "true" if x else "false"
    dkdv = "bwd_dkdv_kernel<%s, %d, %s>" % (e, w.d, b(w.layout == 1))
    if dkdv_only:
        return dkdv
    return "bwd_prep_kernel<%s> + bwd_dq_kernel<%s, %d, %s, %s> + %s" % (e, e, w.d, b(key_padding > 0),
                                                                        b(w.layout == 1), dkdv)


def kernel_source_sha(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for p in sources:
        with open(os.path.join(ROOT, p)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str, prefetch: bool, backward: bool = False):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, or None when it is missing or the kernel changed since."""
    name = "traffic_%s%s%s.json" % ("bwd_" if backward else "", workload, "_prefetch" if prefetch else "")
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_src_sha") != kernel_source_sha(BWD_KERNEL_SOURCES if backward else KERNEL_SOURCES):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, x, pairs_fn, n_tok=None):
    """The fp64 oracle, untuned, on a bounded sample of the workload's rows:
    every head at n_tok evenly spaced query tokens (full key sets)."""
    import numpy as np

    import oracle

    if n_tok is None:
        n_tok = int(os.environ.get("RING_BENCH_CPU_TOKENS", "1024"))
    n_tok = min(n_tok, w.T)
    toks = np.linspace(0, w.T - 1, n_tok).astype(np.int64)
    heads = np.repeat(np.arange(w.Hq), n_tok)
    rows_t = np.tile(toks, w.Hq)
    cu = x.get("cu_seqlens")
    t0 = time.perf_counter()
    oracle.forward(x["q"], x["k"], x["v"], n_blocks=w.n_blocks, layout=w.layout, mask=w.mask,
                   max_ring_passes=w.max_ring_passes, cu_seqlens=cu, scale=w.scale, rows=(heads, rows_t))
    dt = time.perf_counter() - t0
    pairs = pairs_fn(rows_t)
    flop = 4.0 * w.d * pairs
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "%d query rows (all %d heads x %d evenly spaced tokens, full key sets) of %s in %.2f s"
                      % (len(heads), w.Hq, n_tok, w.name, dt)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _resident_inputs(ra, W, w, key_padding):
    """The workload's seeded inputs on cuda:0, its plan, and the key-padding mask if asked for."""
    import torch

    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
    x = W.make_inputs(w)
    dev = torch.device("cuda:0")
    if w.packed:
        qkv = x["qkv"].to(dev)
        q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    else:
        q, k, v = x["q"].to(dev), x["k"].to(dev), x["v"].to(dev)
    cu = x.get("cu_seqlens")
    plan = ra.ring_attn_plan(w.T, w.n_blocks, layout=w.layout, mask_mode=w.mask,
                             max_ring_passes=w.max_ring_passes, cu_seqlens_host=cu, dtype=tdt, head_dim=w.d)
    key_valid = None
    if key_padding > 0:
        if w.mask != 1 or w.max_ring_passes < w.n_blocks:
            print("--key-padding is measured on full causal rings", file=sys.stderr)
            sys.exit(2)
        kv = W.random_key_valid(w.T, w.seed, key_padding)
        # allowed pairs per head: a real key t' is seen by the queries t >= t'
        plan["allowed_pairs"] = int((kv.to(torch.int64) * (w.T - torch.arange(w.T))).sum())
        key_valid = kv.to(dev)
    out = torch.empty(w.T, w.Hq, w.d, device=dev, dtype=q.dtype)
    lse = torch.empty(w.Hq, w.T, device=dev, dtype=torch.float32)
    return x, q, k, v, cu, out, lse, plan, torch.cuda.current_stream(), key_valid


def time_forward(ra, W, w, prefetch, steps, warmup, key_padding=0.0):
    """Inputs resident in HBM, `warmup` untimed forwards, then `steps` timed
    ones bracketed by synchronisations: wall and event time per forward."""
    import torch

    x, q, k, v, cu, out, lse, plan, stream, key_valid = _resident_inputs(ra, W, w, key_padding)
    n_docs = 0 if cu is None else cu.numel() - 1
    ws = torch.empty(ra.ring_attn_forward_workspace_size(q, k, w.n_blocks, n_docs, prefetch), device=q.device,
                     dtype=torch.uint8)

    def step():
        ra.ring_attn_forward(q, k, v, out, lse, n_blocks=w.n_blocks, layout=w.layout, mask_mode=w.mask,
                             max_ring_passes=w.max_ring_passes, cu_seqlens_host=cu, key_valid=key_valid,
                             scale=w.scale, prefetch=prefetch, workspace=ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # step-kernel launches per forward: the whole ring in one, or one per ring step with prefetch
    n_launch = min(w.max_ring_passes, w.n_blocks) if prefetch or w.dtype == "f32" else 1
    return {"ms_wall": wall * 1e3 / steps, "ms_event": ev0.elapsed_time(ev1) / steps,
            "flop": 4.0 * w.d * w.Hq * plan["allowed_pairs"], "plan": plan, "x": x, "n_launch": n_launch}


def per_config_lines(ra, W, args, headline):
    """Every workload of the benchmark table, each timed on its own (inputs
    resident, warmup, timed forwards) with its own bounded oracle CPU timing:
    the two fp32 worked examples (vector-ALU kernel), the three 16-bit
    long-context ones (matrix-core kernel), and the headline one with the
    side-stream prefetch on."""
    import torch

    lines = []
    plan_ = [(name, False) for name in W.WORKLOADS] + [(DEFAULT_WORKLOAD, True)]
    for name, prefetch in plan_:
        w = W.WORKLOADS[name]
        print("[bench] per-config: %s prefetch=%s" % (name, prefetch), file=sys.stderr, flush=True)
        if name == DEFAULT_WORKLOAD and not prefetch:
            ms, ms_ev, value = headline["ms_per_step"], headline["roofline"]["event_ms_per_step"], headline["value"]
            cpu = headline.get("cpu_baseline")
        else:
            steps = max(3, min(args.steps, 20))
            m = time_forward(ra, W, w, prefetch, steps, max(1, min(args.warmup, 3)))
            ms, ms_ev = m["ms_wall"], m["ms_event"]
            value = m["flop"] / (ms * 1e-3) / 1e12
            cpu = None
            if not args.no_cpu_baseline and not prefetch:
                small = w.T <= 4096
                cpu = cpu_baseline(w, m["x"], lambda toks, w=w, x=m["x"]: _pairs_of_rows(w, x, toks),
                                   n_tok=w.T if small else 48)
            del m
            torch.cuda.empty_cache()
        peak = PEAK_BF16_TFLOPS if w.dtype != "f32" else PEAK_FP32_VECTOR_TFLOPS
        lines.append({"workload": name, "dtype": w.dtype, "prefetch": prefetch, "ms_per_step": round(ms, 4),
                      "event_ms_per_step": round(ms_ev, 4), "value": round(value, 4), "unit": "TFLOP/s",
                      "peak": peak, "peak_kind": "bf16 MFMA" if w.dtype != "f32" else "fp32 vector ALU",
                      "frac": round(value / peak, 5), "cpu_baseline": cpu})
    return lines


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--prefetch", action="store_true")
    ap.add_argument("--backward", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time the headline workload only (no per_config lines), e.g. under a profiler")
    ap.add_argument("--dtype", choices=["bf16", "f16"], default="bf16",
                    help="16-bit input type (the workloads are quoted in bf16; f16 runs the same shapes)")
    ap.add_argument("--key-padding", type=float, default=0.0, metavar="FRAC",
                    help="add a seeded key-padding mask padding about FRAC of the keys (full causal rings only)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="instead of the benchmark, run a plain device copy of BYTES bytes 5 times "
                         "(reference reading for the HBM byte counters)")
    ap.add_argument("--overlap-report", metavar="TRACE_DIR",
                    help="print the per-step copy / compute table of the last prefetching forward in a rocprofv3 "
                         "kernel trace of 'bench.py --prefetch' (no GPU work)")
    args = ap.parse_args()
    if args.overlap_report:
        print(prefetch_overlap_report(args.overlap_report, args.workload))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the ring on one GPU (all ring blocks are virtual devices on it); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import ring_attention_step_amd as ra
    import workloads as W

    if args.copy_calibration:
        n = args.copy_calibration // 4 * 4
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)  # an element-wise kernel: reads n bytes, writes n bytes
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)
        return

    w = W.WORKLOADS[args.workload]
    if w.dtype != "bf16":
        print("bench workloads are the bf16 long-context ones (the fp32 worked examples are reported in "
              "per_config)", file=sys.stderr)
        sys.exit(2)
    w = dataclasses.replace(w, dtype=args.dtype)
    torch.cuda.set_device(torch.device("cuda:0"))
    if args.backward:
        return bench_backward(args, ra, W, w, *_resident_inputs(ra, W, w, args.key_padding))
    m = time_forward(ra, W, w, args.prefetch, args.steps, args.warmup, args.key_padding)
    if args.key_padding > 0:
        args.no_cpu_baseline = True  # the CPU baseline leg samples the unpadded workload
    # the counter record is the bf16 kernel without a key mask
    traffic = traffic_from_profile(w.name, args.prefetch) if args.dtype == "bf16" and args.key_padding == 0 else None
    achieved = m["flop"] / (m["ms_event"] * 1e-3) / 1e12
    value = m["flop"] / (m["ms_wall"] * 1e-3) / 1e12
    plan = m["plan"]
    res = {
        "metric": "causal-adjusted attention TFLOP/s and % bf16 MFMA peak, 32K ring fwd, 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_wall"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.T, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
                   "ring_blocks": w.n_blocks, "layout": ["contiguous", "striped"][w.layout],
                   "mask": ["none", "causal", "doc-causal"][w.mask], "max_ring_passes": w.max_ring_passes,
                   "prefetch": bool(args.prefetch), "key_padding": args.key_padding, "flop_per_step": m["flop"],
                   "allowed_pairs_per_head": plan["allowed_pairs"]},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        # achieved: the forward's FLOP over its event-timed duration on the
        # launch stream, which also holds the V^T pack (about 1% of it): a
        # slight underestimate of the step kernel's own rate.
        "roofline": {"bound": "mfma", "kernel": STEP_KERNEL if args.prefetch else ring_kernel_name(w, args.key_padding),
                     "achieved": round(achieved, 3),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "launches_per_step": m["n_launch"],
                     "event_ms_per_step": round(m["ms_event"], 4),
                     "timing": "hip events on the launch stream around the timed steps, incl. the V^T pack"},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_for(w, m["x"])
    if (not args.headline_only and args.workload == DEFAULT_WORKLOAD and not args.prefetch and args.dtype == "bf16"
            and args.key_padding == 0):
        del m
        res["per_config"] = per_config_lines(ra, W, args, res)
    print(json.dumps(res), flush=True)


def bench_backward(args, ra, W, w, x, q, k, v, cu, out, lse, plan, stream, key_valid=None):
    import torch

    dev = q.device
    n_docs = 0 if cu is None else cu.numel() - 1
    ws_f = torch.empty(ra.ring_attn_forward_workspace_size(q, k, w.n_blocks, n_docs, False), device=dev,
                       dtype=torch.uint8)
    ra.ring_attn_forward(q, k, v, out, lse, n_blocks=w.n_blocks, layout=w.layout, mask_mode=w.mask,
                         max_ring_passes=w.max_ring_passes, cu_seqlens_host=cu, key_valid=key_valid, scale=w.scale,
                         prefetch=False, workspace=ws_f, stream=stream)
    del ws_f
    dout = W.random_dout(w.T, w.Hq, w.d, args.dtype, w.seed).to(dev)
    dq = torch.empty(w.T, w.Hq, w.d, device=dev, dtype=torch.float32)
    dk = torch.empty(w.T, w.Hkv, w.d, device=dev, dtype=torch.float32)
    dv = torch.empty_like(dk)
    ws = torch.empty(ra.ring_attn_backward_workspace_size(q, w.n_blocks, n_docs), device=dev, dtype=torch.uint8)
    flop = 10.0 * w.d * w.Hq * plan["allowed_pairs"]

    def step():
        ra.ring_attn_backward(q, k, v, out, dout, lse, dq, dk, dv, n_blocks=w.n_blocks, layout=w.layout,
                              mask_mode=w.mask, max_ring_passes=w.max_ring_passes, cu_seqlens_host=cu,
                              key_valid=key_valid, scale=w.scale, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_event = ev0.elapsed_time(ev1) / args.steps
    ms_wall = wall * 1e3 / args.steps
    value = flop / (ms_wall * 1e-3) / 1e12
    achieved = flop / (ms_event * 1e-3) / 1e12
    res = {
        "metric": "causal-adjusted attention backward TFLOP/s and % bf16 MFMA peak, ring bwd, 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "backward", "tokens": w.T, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.d, "ring_blocks": w.n_blocks, "layout": ["contiguous", "striped"][w.layout],
                   "mask": ["none", "causal", "doc-causal"][w.mask], "max_ring_passes": w.max_ring_passes,
                   "grad_dtype": "f32", "key_padding": args.key_padding, "flop_per_step": flop, "allowed_pairs_per_head": plan["allowed_pairs"]},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        # the three backward kernels together, event-timed on the launch stream;
        # traffic: HBM bytes per launch of the dominant one (dk/dv) from the
        # committed counter record
        "roofline": {"bound": "mfma", "kernel": bwd_kernel_names(w, args.key_padding),
                     "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profile(w.name, False, backward=True)
                     if args.dtype == "bf16" and key_valid is None else None,
                     "traffic_kernel": bwd_kernel_names(w, args.key_padding, dkdv_only=True),
                     "event_ms_per_step": round(ms_event, 4),
                     "timing": "hip events on the launch stream around the timed backward calls"},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_backward(w, x, dout.cpu())
    print(json.dumps(res), flush=True)


def cpu_baseline_backward(w, x, dout):
    """The fp64 oracle's backward, untuned, on a bounded sample: dout kept on
    n_tok evenly spaced tokens of one head (zero elsewhere), that head and its
    kv head only; every term of those rows (dq rows, their dk / dv sums)."""
    import numpy as np

    import oracle

    n_tok = int(os.environ.get("RING_BENCH_CPU_BWD_TOKENS", "1024"))
    toks = np.linspace(0, w.T - 1, n_tok).astype(np.int64)
    h, g = 0, 0
    sub_g = dout.new_zeros(dout.shape[0], 1, dout.shape[2])
    sub_g[toks, 0] = dout[toks, h]
    t0 = time.perf_counter()
    oracle.backward(x["q"][:, [h]], x["k"][:, [g]], x["v"][:, [g]], sub_g, n_blocks=w.n_blocks, layout=w.layout,
                    mask=w.mask, max_ring_passes=w.max_ring_passes, cu_seqlens=x.get("cu_seqlens"), scale=w.scale,
                    rows=(np.zeros(n_tok, np.int64), toks), rows_dkdv=True)
    dt = time.perf_counter() - t0
    pairs = _pairs_of_rows(w, x, toks)
    return {"value": 10.0 * w.d * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": "backward terms of %d query rows (head 0, evenly spaced tokens, full key sets) of %s "
                      "in %.1f s, single thread (dk/dv sums are serial)" % (n_tok, w.name, dt)}


def _ring_step_pairs(w):
    """Active (device, block) pairs of each ring step for a workload without
    documents: contiguous causal skips blocks after the device's own, no mask
    and striped causal skip nothing."""
    N, P = w.n_blocks, min(w.max_ring_passes, w.n_blocks)
    if w.mask == 2:
        raise ValueError("the overlap report covers workloads without documents")
    return [sum(1 for i in range(N) if not (w.mask == 1 and w.layout == 0 and (i - s) % N > i)) for s in range(P)]


def prefetch_overlap_report(trace_dir, workload):
    """Per ring step of the last prefetching forward in a rocprofv3 kernel
    trace (--kernel-trace, csv): the step kernel's time, the time of the blit
    copies that fetch its key/value blocks (one K copy and one V^T copy per
    active pair, on the library's copy stream, in step order), and the time
    the compute stream sat idle between the previous step and this one.  The
    transfer is hidden when a step's copies finish while the step before it
    still computes (compute per block outlasting the send)."""
    import csv
    import glob

    w = __import__("workloads").WORKLOADS[workload]
    pairs = _ring_step_pairs(w)
    path = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)[0]
    rows = list(csv.DictReader(open(path)))
    kern = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in rows)
    steps = [k for k in kern if "step_bf16_kernel" in k[2] or "step_f32_kernel" in k[2]]
    copies = [k for k in kern if "__amd_rocclr_copyBuffer" in k[2]]
    n_steps, n_copy = len(pairs), 2 * sum(pairs[1:])
    if len(steps) < n_steps or len(copies) < n_copy:
        raise ValueError("trace holds %d step kernels and %d copies, a forward needs %d and %d"
                         % (len(steps), len(copies), n_steps, n_copy))
    steps, copies = steps[-n_steps:], copies[-n_copy:]
    lines = ["| step | pairs | compute ms | copy ms | copies end before the step starts | compute idle before the step, ms |",
             "|---|---|---|---|---|---|"]
    c0 = 0
    tot_copy = tot_comp = tot_idle = 0.0
    for s in range(n_steps):
        comp = (steps[s][1] - steps[s][0]) * 1e-6
        tot_comp += comp
        idle = (steps[s][0] - steps[s - 1][1]) * 1e-6 if s else 0.0
        if s == 0:
            lines.append("| 0 | %d | %.3f | (own block) | - | - |" % (pairs[0], comp))
            continue
        mine = copies[c0:c0 + 2 * pairs[s]]
        c0 += 2 * pairs[s]
        cp = sum(e - b for b, e, _ in mine) * 1e-6
        tot_copy += cp
        tot_idle += max(idle, 0.0)
        lines.append("| %d | %d | %.3f | %.3f | %s | %.3f |" % (s, pairs[s], comp, cp,
                                                             "yes" if max(e for _, e, _ in mine) <= steps[s][0] else "NO",
                                                             idle))
    span = (steps[-1][1] - min(steps[0][0], copies[0][0])) * 1e-6
    lines.append("")
    lines.append("forward span %.3f ms: step kernels %.3f ms, copies %.3f ms, compute idle between steps %.3f ms "
                 "(%.1f%% of the copy time)" % (span, tot_comp, tot_copy, tot_idle, 100.0 * tot_idle / max(tot_copy, 1e-9)))
    return "\n".join(lines)


def cpu_baseline_for(w, x):
    return cpu_baseline(w, x, lambda toks: _pairs_of_rows(w, x, toks))


def _pairs_of_rows(w, x, toks):
    """Allowed keys of each listed query token under the workload's mask and ring, summed."""
    import numpy as np

    tot = 0
    N, B, P = w.n_blocks, w.block, min(w.max_ring_passes, w.n_blocks)
    cu = x.get("cu_seqlens")
    for t in toks:
        t = int(t)
        lo, hi = 0, w.T - 1
        if w.mask:
            hi = t
        if w.mask == 2:
            c = cu.numpy()
            lo = int(c[np.searchsorted(c, t, side="right") - 1])
        bi = t % N if w.layout == 1 else t // B
        for s in range(P):
            j = (bi - s) % N
            if w.layout == 1:
                keys = np.arange(B) * N + j
                tot += int(((keys >= lo) & (keys <= hi)).sum())
            else:
                a, b = max(lo, j * B), min(hi, j * B + B - 1)
                tot += max(0, b - a + 1)
    return tot


if __name__ == "__main__":
    main()
