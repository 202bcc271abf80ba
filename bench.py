#!/usr/bin/env python3
"""Throughput of the QSA prompt-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one prompt chunk pushed through the whole path for 12 layers:
for the headline workload (T=1984 query tokens at pos0 0, 2 KV groups x 12
heads, head dim 256, int8 K/V with fp16 per-64-dim scales) every token is
under the 2051-cell budget, so its ids are the identity and are derived
inside the attention kernel; a step is then 12 back-to-back qsa_flash
dispatches, each over its own layer's seeded inputs (resident in HBM before
the timed region).  The value is query tokens per second:
T * steps / elapsed.

One JSON line goes to stdout; progress goes to stderr.  The line carries
`roofline` for the attention kernel (algorithmic gathered bytes per launch
over its mean launch time, measured with HIP events on the launch stream)
and `cpu_baseline` (the fp64 oracle on this host, a bounded sample).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published
LAYERS = 12
BYTES_PER_VISIT = 2 * 256 + 2 * 4 * 2   # int8 K + V codes, 4 fp16 K + 4 fp16 V scales
ID_BYTES_PER_VISIT = 4                  # int32 id read for rows above budget
ROW_BYTES = 2 * (12 * 256 * 2)          # fp16 Q in + fp16 O out per (token, group)
FLOPS_PER_VISIT = 12 * 256 * 2 * 2      # 12 heads x (QK^T + PV) x 2 flop per MAC


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


def cpu_baseline(T: int, pos0: int, target_s: float = 12.0, max_layers: int = 3):
    """The fp64 oracle on this host: whole layers of the same workload until
    about target_s seconds have passed; scaled to query tokens/s for 12
    layers."""
    import oracle
    import qsa_synth
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    done, t_total = 0, 0.0
    while done < max_layers and t_total < target_s:
        inp = qsa_synth.layer_inputs(T, pos0, layer=done)
        ids = None
        if inp.scores is not None:
            ids = oracle.select(T, pos0, inp.budget, inp.scores, 2, inp.n_cells)
        t0 = time.perf_counter()
        if ids is None:
            oracle.attend(inp, None)
        else:
            oracle.attend(inp, ids)
        t_total += time.perf_counter() - t0
        done += 1
    tok_s = T * done / t_total / LAYERS
    return {"value": tok_s, "unit": "query-tokens/s (12 layers)", "cores": threads,
            "kind": "oracle",
            "sample": "%d of the 12 layers (all %d tokens each, T=%d pos0=%d), fp64 oracle "
                      "attention, %.1f s wall; scaled by 1/12" % (done, T, T, pos0, t_total)}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--T", type=int, default=1984)
    ap.add_argument("--pos0", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the path is built and timed on a single "
              "MI355X (--gpus %d not supported)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import qsa_synth
    import quantized_sparse_flash_amd as qsa

    T, pos0 = args.T, args.pos0
    qsa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("bench: generating %d layers of inputs (T=%d pos0=%d)" % (LAYERS, T, pos0))
    layers = []
    for layer in range(LAYERS):
        inp = qsa_synth.layer_inputs(T, pos0, layer=layer)
        d = {k: torch.from_numpy(np.ascontiguousarray(getattr(inp, k))).to(dev)
             for k in ("q", "kq", "ksc", "vq", "vsc")}
        s = qsa.QsaShape(T=T, pos0=pos0, n_groups=2, budget=inp.budget, n_cells=inp.n_cells)
        d["ids"] = None
        if inp.scores is not None:
            sc = torch.from_numpy(inp.scores).to(dev)
            d["ids"] = torch.empty((T, 2, inp.budget), dtype=torch.int32, device=dev)
            qsa.qsa_topk(s, sc, d["ids"])
            del sc
        d["out"] = torch.empty((T, s.n_heads, 256), dtype=torch.float16, device=dev)
        d["shape"] = s
        layers.append(d)
    torch.cuda.synchronize()
    budget = layers[0]["shape"].budget

    def step(events=None):
        for i, d in enumerate(layers):
            if events is not None:
                events[i][0].record()
            qsa.qsa_flash(d["shape"], d["q"], d["kq"], d["ksc"], d["vq"], d["vsc"], d["ids"],
                          d["out"])
            if events is not None:
                events[i][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, per-launch events on the launch stream
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in range(LAYERS)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    launch_ms = [e[0].elapsed_time(e[1]) for row in ev for e in row]
    mean_launch_s = float(np.mean(launch_ms)) / 1e3

    ms_per_step = elapsed / args.steps * 1e3
    value = T * args.steps / elapsed
    visits, by, flops = algorithmic(T, pos0, budget)
    gbs = by / mean_launch_s / 1e9
    tflops = flops / mean_launch_s / 1e12
    log("bench: %.3f ms/step (12 layers), launch mean %.1f us, %.0f GB/s algorithmic, "
        "%.1f TFLOP/s" % (ms_per_step, mean_launch_s * 1e6, gbs, tflops))

    line = {
        "metric": "qsa_flash query-tokens/s at T=%d (12 layers)" % T,
        "value": value,
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 K/V codes, fp16 scales/Q/P/out, fp32 accumulate",
        "data": "synthetic (seeded: q N(0,1) fp16, codes U[-127,127], scales U[0.002,0.02])",
        "config": {"workload": "qsa_flash T=%d pos0=%d, 12 layers, 2 KV groups x 12 heads, "
                               "head dim 256, budget %d" % (T, pos0, budget),
                   "T": T, "pos0": pos0, "layers": LAYERS, "n_groups": 2,
                   "heads_per_group": 12, "head_dim": 256, "budget": budget},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "qsa flash attention",
                     "algorithmic_bytes_per_launch": by, "cell_visits_per_launch": visits,
                     "mean_launch_us": mean_launch_s * 1e6},
        "mfma": {"achieved": tflops, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": tflops / MFMA_F16_PEAK_TFLOPS, "flops_per_launch": flops},
    }
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle (bounded sample)")
        line["cpu_baseline"] = cpu_baseline(T, pos0)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
