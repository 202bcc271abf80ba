#!/usr/bin/env python3
"""Throughput of the QSA prompt-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload (the headline): a prompt chunk of T=1984 query tokens at
pos0 0 through 12 layers, 2 KV groups x 12 query heads, head dim 256, int8
K/V codes with fp16 per-64-dim scales, budget 2051.  Every token sees at
most 1984 cells, so its ids are the identity, derived on the device, and
the host issues no selection call (the pages' host skips it for such
prompts); a step is then 12 back-to-back fused qsa_flash calls (each
enqueued as its two halves, see below), each on its own layer's seeded
inputs, resident in HBM before the timed region.  The value is query
tokens per second, T * steps / elapsed.

Other workloads (--workload):
  t512_pos0_x12, t1024_pos0_x12   the same at T = 512 / 1024;
  t1984_pos30000                  long context: per step one layer of
                                  qsa_topk (top 2051 of up to 31,984
                                  cells) + qsa_flash with explicit ids;
  decode4_pos8192                 4 tokens at position 8192: qsa_topk,
                                  split qsa_flash, qsa_merge (also
                                  decode1_pos512, decode8_pos2048 and
                                  decode8_pos30000);
  t1984_pos30000_split            the long-context prompt through the same
                                  split path (one wavefront per selected
                                  64-cell chunk, then the merge) instead
                                  of the fused row kernel;
  quantize_kv_31984               the K/V quantiser on the long-context
                                  cache: qsa_quantize of the fp16 K and V
                                  rows of 2 groups x 31,984 cells per step
                                  (cells quantised per second; roofline HBM
                                  on 512 B in + 264 B out per row).

One JSON line goes to stdout; progress goes to stderr.  A prompt step
enqueues each layer's fused qsa_flash as its two halves, qsa_flash_prepare
(the dequantisation prepass) and qsa_flash_attend.  Without --warmup the
warmup runs for 0.3 s, long enough for the GPU clock to settle under load
(with a few steps only it is still rising, and a short timed region reads
10% slow); without --steps the timed region lasts about 0.2 s (at least 20
steps).  Two timed regions of K steps follow: the first, with nothing
between kernels, gives value and ms_per_step; in the second, HIP events on
the launch stream bracket each step's dominant launches (the attend calls,
run back to back after every layer is prepared into its own workspace;
decode: the split qsa_flash call, repeated), for the roofline figures.  An
event between two kernels costs the stream a few microseconds and would
count the dispatch of the next kernel as part of it, which is why the
regions are apart.  The line carries
  roofline      that kernel against the resource that binds it: for prompt
                chunks whose tokens are all under budget the tile kernel
                shares every dequantised chunk among 120 queries, so its
                bound is fp16 MFMA (algorithmic flops / mean duration);
                row-gather workloads (tokens above budget, decode) are bound
                by HBM on the gathered bytes;
  gathered      algorithmic gathered bytes / the same duration, against the
                HBM peak (above 1 when chunks are shared from L2);
  mfma          algorithmic flops / the same duration;
  cpu_baseline  the fp64 oracle on this host, a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published
BYTES_PER_VISIT = 2 * 256 + 2 * 4 * 2   # int8 K + V codes, 4 fp16 K + 4 fp16 V scales
ID_BYTES_PER_VISIT = 4                  # int32 id read for rows above budget
ROW_BYTES = 2 * (12 * 256 * 2)          # fp16 Q in + fp16 O out per (token, group)
FLOPS_PER_VISIT = 12 * 256 * 2 * 2      # 12 heads x (QK^T + PV) x 2 flop per MAC
# The pages' own figure for this metric: 12 qsa_flash layers at T=1984, pos0
# 0 in 272.54 ms on an Apple M5 ("opus_r9_qsa", result table).  Context only.
PAGES_M5_TOKS = {1984: 1984 / 0.27254, 1024: 1024 / 0.07533, 512: 512 / 0.02068}

WORKLOADS = {
    "t1984_pos0_x12": dict(T=1984, pos0=0, layers=12, kind="prompt"),
    "t1024_pos0_x12": dict(T=1024, pos0=0, layers=12, kind="prompt"),
    "t512_pos0_x12": dict(T=512, pos0=0, layers=12, kind="prompt"),
    "t1984_pos30000": dict(T=1984, pos0=30000, layers=1, kind="prompt"),
    "decode4_pos8192": dict(T=4, pos0=8192, layers=1, kind="split"),
    "decode1_pos512": dict(T=1, pos0=512, layers=1, kind="split"),
    "decode8_pos2048": dict(T=8, pos0=2048, layers=1, kind="split"),
    "decode8_pos30000": dict(T=8, pos0=30000, layers=1, kind="split"),
    "t1984_pos30000_split": dict(T=1984, pos0=30000, layers=1, kind="split"),
    "quantize_kv_31984": dict(T=1984, pos0=30000, layers=1, kind="quantize"),
}
AUTO_WARMUP_S = 0.3  # default warmup: the GPU clock takes tens of ms under load to settle
AUTO_TIMED_S = 0.2    # default timed region length
MIN_STEPS = 20


def run_warmup(args, step, sync):
    """Runs the warmup steps: exactly args.warmup of them when given, else
    steps until AUTO_WARMUP_S has passed (at least 3).  Fills in args.warmup
    and, when not given, args.steps (enough steps for about AUTO_TIMED_S).
    Returns nothing; the caller's timed regions follow."""
    t0 = time.perf_counter()
    n = 0
    if args.warmup is not None:
        for _ in range(args.warmup):
            step()
        sync()
        n = args.warmup
    else:
        while n < 3 or time.perf_counter() - t0 < AUTO_WARMUP_S:
            step()
            n += 1
            if n % 8 == 0:
                sync()
        sync()
        args.warmup = n
    if args.steps is None:
        per_step = (time.perf_counter() - t0) / max(n, 1)
        args.steps = max(MIN_STEPS, min(5000, int(AUTO_TIMED_S / max(per_step, 1e-6))))


DECODE_REPEAT = 16  # split qsa_flash launches per kernel-timing step (decode)
QUANT_REPEAT = 8    # K and V qsa_quantize launch pairs per kernel-timing step
LAUNCH_TIMING = ("HIP events on the launch stream around each step's dominant launches, run "
                 "back to back (every layer prepared first; decode: the split flash call "
                 "%d times; quantiser: the step %d times), over a second timed region of K "
                 "steps; value and ms_per_step come from the first region, which has no "
                 "events" % (DECODE_REPEAT, QUANT_REPEAT))
QUANT_ROW_BYTES = 256 * 2 + 256 + 4 * 2  # fp16 row in; int8 codes + 4 fp16 scales out
# sources of the kernel whose HBM traffic each workload's record describes
TRAFFIC_SOURCES = {
    "t1984_pos0_x12": ("qsa_flash_tile.hip", "qsa_device.h"),
    "t1984_pos30000": ("qsa_flash_rows.hip", "qsa_device.h"),
    "quantize_kv_31984": ("qsa_quantize.hip", "qsa_device.h"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(T: int, pos0: int, budget: int, G: int = 2):
    """Cell-visits, bytes and flops the method moves per qsa_flash launch."""
    visits = 0
    id_visits = 0
    for t in range(T):
        nkv = pos0 + t + 1
        nsel = min(nkv, budget)
        visits += nsel * G
        if nkv > budget:
            id_visits += nsel * G
    by = visits * BYTES_PER_VISIT + id_visits * ID_BYTES_PER_VISIT + T * G * ROW_BYTES
    return visits, by, visits * FLOPS_PER_VISIT


def kernel_source_hash(names) -> str:
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "quantized_sparse_flash_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload, if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % workload)
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("{"):
                rec = json.loads(line)
    names = TRAFFIC_SOURCES.get(workload)
    if not rec or not names or rec.get("kernel_sources_sha256") != kernel_source_hash(names):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(T: int, pos0: int, layers: int, target_s: float = 12.0, max_layers: int = 3):
    """The fp64 oracle on this host: whole layers of the same workload until
    about target_s seconds have passed; scaled to query tokens/s for the
    workload's layer count."""
    import oracle
    import qsa_synth
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    done, t_total = 0, 0.0
    while done < min(max_layers, layers) and t_total < target_s:
        inp = qsa_synth.layer_inputs(T, pos0, layer=done)
        ids = None
        t0 = time.perf_counter()
        if inp.scores is not None:
            ids = oracle.select(T, pos0, inp.budget, inp.scores, 2, inp.n_cells)
        oracle.attend(inp, ids)
        t_total += time.perf_counter() - t0
        done += 1
    tok_s = T * done / t_total / layers
    return {"value": tok_s, "unit": "query-tokens/s (%d layers)" % layers, "cores": threads,
            "kind": "oracle",
            "sample": "%d of the %d layers (all %d tokens each, T=%d pos0=%d), fp64 oracle "
                      "selection + attention, %.1f s wall; scaled by 1/%d"
                      % (done, layers, T, T, pos0, t_total, layers)}


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: enough for about %.1f s, at least %d)"
                         % (AUTO_TIMED_S, MIN_STEPS))
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps (default: steps until %.2f s have passed, "
                         "which lets the GPU clock settle)" % AUTO_WARMUP_S)
    ap.add_argument("--workload", default="t1984_pos0_x12", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run one device copy of this many MiB before timing (a known-size "
                         "kernel for scaling FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the path is built and timed on a single "
              "MI355X (--gpus %d not supported)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import qsa_synth
    import quantized_sparse_flash_amd as qsa

    wl = WORKLOADS[args.workload]
    T, pos0, L, kind = wl["T"], wl["pos0"], wl["layers"], wl["kind"]
    qsa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy_mb:
        n = args.calib_copy_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("bench: calibration copy of %d MiB done" % args.calib_copy_mb)
    if kind == "quantize":
        bench_quantize(args, pos0 + T, dev)
        return

    log("bench: generating %d layer(s) of inputs (%s)" % (L, args.workload))
    layers = []
    for layer in range(L):
        inp = qsa_synth.layer_inputs(T, pos0, layer=layer)
        d = {k: torch.from_numpy(np.ascontiguousarray(getattr(inp, k))).to(dev)
             for k in ("q", "kq", "ksc", "vq", "vsc")}
        s = qsa.QsaShape(T=T, pos0=pos0, n_groups=2, budget=inp.budget, n_cells=inp.n_cells)
        d["scores"] = None if inp.scores is None else torch.from_numpy(inp.scores).to(dev)
        d["ids"] = None
        if inp.scores is not None:
            d["ids"] = torch.empty((T, 2, inp.budget), dtype=torch.int32, device=dev)
        d["out"] = torch.empty((T, s.n_heads, 256), dtype=torch.float16, device=dev)
        if kind == "split":
            d["part"] = torch.empty((T, s.n_part_chunks, s.n_heads, qsa.PART_STRIDE),
                                    dtype=torch.float32, device=dev)
        d["shape"] = s
        # a workspace of its own per layer (the kernel-timing region
        # prepares every layer before the attend launches run)
        need = qsa.qsa_flash_workspace_bytes(s)
        d["ws"] = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        layers.append(d)
    # one workspace serves every layer: the calls run in order on one stream
    ws = max((d["ws"] for d in layers if d["ws"] is not None), key=lambda t: t.numel(),
             default=None)
    torch.cuda.synchronize()
    budget = layers[0]["shape"].budget

    def step():
        for d in layers:
            s = d["shape"]
            if d["scores"] is not None:
                qsa.qsa_topk(s, d["scores"], d["ids"])
            if kind == "split":
                qsa.qsa_flash(s, d["q"], d["kq"], d["ksc"], d["vq"], d["vsc"], d["ids"], None,
                              d["part"])
                qsa.qsa_merge(s, d["part"], d["out"])
            else:
                qsa.qsa_flash_prepare(s, d["kq"], d["ksc"], d["vq"], d["vsc"], workspace=ws)
                qsa.qsa_flash_attend(s, d["q"], d["kq"], d["ksc"], d["vq"], d["vsc"], d["ids"],
                                     d["out"], workspace=ws)

    repeat = DECODE_REPEAT if T <= 8 else 1

    def step_timed(ev0, ev1) -> int:
        """The same step with its dominant launches back to back between two
        events: every layer is prepared (into its own workspace) before the
        attend launches run; a decode step's split qsa_flash call, which
        only rewrites its partials, runs DECODE_REPEAT times (once for
        prompt-sized splits).  Returns the number of launches between the
        events."""
        if kind == "split":
            for d in layers:
                if d["scores"] is not None:
                    qsa.qsa_topk(d["shape"], d["scores"], d["ids"])
            ev0.record()
            for _ in range(repeat):
                for d in layers:
                    qsa.qsa_flash(d["shape"], d["q"], d["kq"], d["ksc"], d["vq"], d["vsc"],
                                  d["ids"], None, d["part"])
            ev1.record()
            for d in layers:
                qsa.qsa_merge(d["shape"], d["part"], d["out"])
            return repeat * L
        for d in layers:
            s = d["shape"]
            if d["scores"] is not None:
                qsa.qsa_topk(s, d["scores"], d["ids"])
            qsa.qsa_flash_prepare(s, d["kq"], d["ksc"], d["vq"], d["vsc"], workspace=d["ws"])
        ev0.record()
        for d in layers:
            qsa.qsa_flash_attend(d["shape"], d["q"], d["kq"], d["ksc"], d["vq"], d["vsc"],
                                 d["ids"], d["out"], workspace=d["ws"])
        ev1.record()
        return L

    run_warmup(args, step, torch.cuda.synchronize)

    # timed region 1 (value, ms_per_step): K steps with nothing else on the
    # stream.  An event between two kernels costs the stream a few
    # microseconds and reads the next kernel's dispatch as part of its time,
    # so the launch durations come from a second region.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # timed region 2 (roofline): K more steps, HIP events on the launch
    # stream (torch's current stream) around each step's dominant launches
    ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
          for _ in range(args.steps)]
    n_launch = 0
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for k in range(args.steps):
        n_launch += step_timed(*ev[k])
    torch.cuda.synchronize()
    elapsed_ev = time.perf_counter() - t1
    mean_launch_s = sum(e0.elapsed_time(e1) for e0, e1 in ev) / n_launch / 1e3

    ms_per_step = elapsed / args.steps * 1e3
    value = T * args.steps / elapsed
    visits, by, flops = algorithmic(T, pos0, budget)
    gbs = by / mean_launch_s / 1e9
    tflops = flops / mean_launch_s / 1e12
    log("bench: %.3f ms/step (%.3f in the kernel-timing region), attention kernel mean %.1f us, "
        "%.0f GB/s algorithmic, %.1f TFLOP/s"
        % (ms_per_step, elapsed_ev / args.steps * 1e3, mean_launch_s * 1e6, gbs, tflops))

    traffic = measured_traffic(args.workload)
    identity_tile = pos0 + T <= budget and kind == "prompt"
    if identity_tile:
        roofline = {"bound": "mfma", "achieved": tflops, "peak": MFMA_F16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": tflops / MFMA_F16_PEAK_TFLOPS,
                    "traffic": traffic,
                    # the library takes 8-wave workgroups of 10 tokens when at
                    # least 256 of them cover the prompt, else 4-wave ones of 5
                    "kernel": "flash_tile_kernel<%d> (qsa_flash_attend)"
                              % (8 if 2 * -(-T // 10) >= 256 else 4),
                    "flops_per_launch": flops, "mean_launch_us": mean_launch_s * 1e6,
                    "launch_timing": LAUNCH_TIMING}
    else:
        roofline = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
                    "kernel": ("flash_rows_kernel<true> (split qsa_flash)" if kind == "split"
                               else "flash_rows_kernel<false> (qsa_flash_attend)"),
                    "algorithmic_bytes_per_launch": by, "mean_launch_us": mean_launch_s * 1e6,
                    "launch_timing": LAUNCH_TIMING}
        if kind == "split":
            # the (o, m, l) records the split call writes (and the merge
            # reads): one per (token, selected 64-cell chunk, head)
            n_rec = sum(-(-min(pos0 + t + 1, budget) // 64) for t in range(T)) * 2 * 12
            roofline["partial_bytes_per_launch"] = n_rec * qsa.PART_STRIDE * 4
    m5 = PAGES_M5_TOKS.get(T) if (pos0 == 0 and L == 12) else None
    steps_desc = {"prompt": "qsa_flash", "split": "qsa_topk + split qsa_flash + qsa_merge"}
    line = {
        "metric": "qsa_flash query-tokens/s at T=%d (%d layer%s)" % (T, L, "s" if L > 1 else ""),
        "value": value,
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (value / m5) if m5 else None,
        "dtype": "f16",
        "precision": "int8 K/V codes with fp16 scales, dequantised to fp16; fp16 Q, P and out; "
                     "fp16 MFMA with fp32 accumulation",
        "data": "synthetic (seeded: q N(0,1) fp16, codes U[-127,127], scales U[0.002,0.02]"
                "%s)" % (", scores N(0,1) fp32" if pos0 + T > budget else ""),
        "config": {"workload": "%s: T=%d pos0=%d, %d layer(s) of %s%s, 2 KV groups x 12 "
                               "heads, head dim 256, budget %d"
                               % (args.workload, T, pos0, L,
                                  "qsa_topk + " if (pos0 + T > budget and kind == "prompt")
                                  else "", steps_desc[kind], budget),
                   "T": T, "pos0": pos0, "layers": L, "n_groups": 2, "heads_per_group": 12,
                   "head_dim": 256, "budget": budget},
        "roofline": roofline,
        "gathered": {"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": by,
                     "cell_visits_per_launch": visits},
        "mfma": {"bound": "mfma", "achieved": tflops, "peak": MFMA_F16_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": tflops / MFMA_F16_PEAK_TFLOPS,
                 "flops_per_launch": flops},
    }
    if m5:
        line["vs_baseline_note"] = ("value / the pages' Apple M5 figure (%.0f query-tokens/s, "
                                    "12 layers at T=%d); another machine, context only" % (m5, T))
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle (bounded sample)")
        line["cpu_baseline"] = cpu_baseline(T, pos0, L)
    print(json.dumps(line), flush=True)


def bench_quantize(args, n_cells: int, dev) -> None:
    """qsa_quantize on the fp16 K and V rows of a 2-group cache of n_cells
    cells; one step quantises both tensors (two calls)."""
    import numpy as np
    import torch

    import qsa_synth
    import quantized_sparse_flash_amd as qsa

    G = 2
    rows = G * n_cells
    log("bench: generating fp16 K/V rows (%d cells x %d groups)" % (n_cells, G))
    xs = [torch.from_numpy(qsa_synth.kv_rows(rows, seed=s).reshape(G, n_cells, 256)).to(dev)
          for s in (1, 2)]
    codes = [torch.empty((G, n_cells, 256), dtype=torch.int8, device=dev) for _ in xs]
    scales = [torch.empty((G, n_cells, 4), dtype=torch.float16, device=dev) for _ in xs]

    def step():
        for i in range(2):
            qsa.qsa_quantize(xs[i], codes[i], scales[i])

    run_warmup(args, step, torch.cuda.synchronize)
    # value from K plain steps; launch durations from K more steps, each
    # repeated QUANT_REPEAT times between two events
    t0 = time.perf_counter()
    for k in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
          for _ in range(args.steps)]
    for k in range(args.steps):
        ev[k][0].record()
        for _ in range(QUANT_REPEAT):
            step()
        ev[k][1].record()
    torch.cuda.synchronize()
    mean_launch_s = (sum(e0.elapsed_time(e1) for e0, e1 in ev)
                     / (2 * QUANT_REPEAT * args.steps) / 1e3)
    by = rows * QUANT_ROW_BYTES
    gbs = by / mean_launch_s / 1e9
    value = rows * args.steps / elapsed
    log("bench: %.3f ms/step, quantize kernel mean %.1f us, %.0f GB/s"
        % (elapsed / args.steps * 1e3, mean_launch_s * 1e6, gbs))
    line = {
        "metric": "qsa_quantize cells/s (K and V rows of 2 groups)",
        "value": value,
        "unit": "cells/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "precision": "fp16 rows in, int8 codes + fp16 scales out; divisions and rounding "
                     "decisions in IEEE fp32",
        "data": "synthetic (seeded: fp16 N(0,1) x 10^U(-3,1) per 64-dim block)",
        "config": {"workload": "%s: qsa_quantize of K and V, 2 groups x %d cells x 256 dims"
                               % (args.workload, n_cells),
                   "n_cells": n_cells, "n_groups": G, "head_dim": 256},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic(args.workload),
                     "kernel": "quantize_kernel (qsa_quantize)",
                     "algorithmic_bytes_per_launch": by, "mean_launch_us": mean_launch_s * 1e6,
                     "launch_timing": LAUNCH_TIMING},
    }
    if not args.no_cpu_baseline:
        import oracle
        log("bench: timing the CPU oracle quantiser (bounded sample)")
        x0 = xs[0].cpu().numpy()
        done, t_total = 0, 0.0
        while t_total < 10.0 and done < 40:
            t1 = time.perf_counter()
            oracle.quantize(x0)
            t_total += time.perf_counter() - t1
            done += 1
        # a cell is one K row and one V row: K-only passes count half a cell per row
        line["cpu_baseline"] = {"value": done * rows / (2.0 * t_total), "unit": "cells/s",
                                "cores": 1, "kind": "oracle",
                                "sample": "%d passes of the oracle quantiser over the K rows "
                                          "(%d rows, single thread), %.1f s; scaled to K+V "
                                          "cells" % (done, rows, t_total)}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
