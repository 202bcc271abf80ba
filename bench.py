#!/usr/bin/env python3
"""Throughput of the QSA prompt-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload (the headline): a prompt chunk of T=1984 query tokens at
pos0 0 through 12 layers, 2 KV groups x 12 query heads, head dim 256, int8
K/V codes with fp16 per-64-dim scales, budget 2051.  Every token sees at
most 1984 cells, so its ids are the identity, derived on the device, and
the host issues no selection call (the pages' host skips it for such
prompts); a step is then 12 back-to-back qsa_flash calls, each on its own
layer's seeded inputs, resident in HBM before the timed region.  The value
is query tokens per second, T * steps / elapsed.

Other workloads (--workload):
  t512_pos0_x12, t1024_pos0_x12   the same at T = 512 / 1024 (the default
                                  line also carries their figures, under
                                  "other_prompts");
  t1984_pos30000                  long context: per step one layer of
                                  qsa_topk (top 2051 of up to 31,984
                                  cells) + qsa_flash with explicit ids;
  decode4_pos8192                 4 tokens at position 8192: qsa_topk,
                                  split qsa_flash, qsa_merge (also
                                  decode1_pos512, decode8_pos2048 and
                                  decode8_pos30000);
  t1984_pos30000_split            the long-context prompt through the same
                                  split path instead of the fused one;
  t96_pos2050, t32_pos2050,       one layer of qsa_topk + qsa_flash whose
  t200_pos1900, t200_pos30000     rows above budget are few enough to run
                                  as row pieces plus the merge;
  quantize_kv_31984               the K/V quantiser on the long-context
                                  cache (cells quantised per second);
  score_t1984_pos30000            the selection scores of the long-context
                                  prompt (qsa_score, four values per cell).

One JSON line goes to stdout; progress goes to stderr.  Every C-ABI call of
a step is bound once (arguments checked and marshalled before timing) and
then only re-issued.  Without --warmup the warmup runs for 0.3 s, long
enough for the GPU clock to settle under load; without --steps the timed
region lasts about 0.2 s (at least 20 steps).  The default workload
measures its two extra prompts (T=512 and T=1024, 12 layers each) before
the headline, with the headline's inputs already on the device, so that
its warmup steps, however few, start from the clock the chip holds under
load.  Three timed regions follow:
  1. K steps back to back, nothing else on the stream: value, ms_per_step;
  2. the pages' protocol: SAMPLES single steps, each bracketed by HIP
     events, each preceded (outside the events) by a 1 GiB write that
     flushes the 256 MB Infinity Cache and the L2s: median and min ms per
     step ("samples");
  3. kernel timing, for the roofline: HIP events on the launch stream
     around K groups of back-to-back qsa_flash calls (one per layer; the
     whole call, every kernel it enqueues), and for prompts also around the
     attention kernel alone (every layer prepared first).  An event between
     two kernels costs the stream a few microseconds, which is why this
     region is apart from the first.
The line carries
  roofline      the qsa_flash call against the resource that binds it: fp16
                MFMA for prompt chunks (algorithmic flops / mean call
                duration), HBM for the K/V quantiser; traffic = counter HBM
                bytes per call from profiles/, null when the kernel sources
                changed since;
  attend_only   the attention kernel alone, same units (prompts);
  gathered      algorithmic gathered bytes / the call duration, against the
                HBM peak (above 1 when chunks are shared from L2);
  cpu_baseline  the fp64 oracle on this host, a bounded sample, plus one
                single-thread T=512 layer.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import subprocess
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
    # fused calls with few rows above budget (row pieces): the budget-crossing
    # chunks, a crossing after 151 tiled tokens, and 400 rows at long context
    "t96_pos2050": dict(T=96, pos0=2050, layers=1, kind="prompt"),
    "t32_pos2050": dict(T=32, pos0=2050, layers=1, kind="prompt"),
    "t200_pos1900": dict(T=200, pos0=1900, layers=1, kind="prompt"),
    "t200_pos30000": dict(T=200, pos0=30000, layers=1, kind="prompt"),
    "quantize_kv_31984": dict(T=1984, pos0=30000, layers=1, kind="quantize"),
    "score_t1984_pos30000": dict(T=1984, pos0=30000, layers=1, kind="score"),
}
# the default line also reports these (12 layers each, same protocol)
OTHER_PROMPTS = ("t512_pos0_x12", "t1024_pos0_x12")
AUTO_WARMUP_S = 0.3  # default warmup: the GPU clock takes tens of ms under load to settle
AUTO_TIMED_S = 0.2    # default timed region length
MIN_STEPS = 20
SAMPLES = 30          # single-step samples of the pages' protocol
FLUSH_BYTES = 1 << 30  # written before each sample: 4x the Infinity Cache

DECODE_REPEAT = 16  # split qsa_flash launches per kernel-timing step (decode)
QUANT_REPEAT = 8    # K and V qsa_quantize launch pairs per kernel-timing step
QUANT_ROW_BYTES = 256 * 2 + 256 + 4 * 2  # fp16 row in; int8 codes + 4 fp16 scales out
SCORE_INDEX_DIM = 4  # qsa_score vector length of the score workload (one value per 64-dim block)
SCORE_REPEAT = 8     # qsa_score launches per kernel-timing step
# sources of the kernels whose HBM traffic each workload's record describes
TRAFFIC_SOURCES = {
    "t1984_pos0_x12": ("qsa_flash_tile.hip", "qsa_device.h"),
    "t1984_pos30000": ("qsa_flash_rows.hip", "qsa_device.h"),
    "quantize_kv_31984": ("qsa_quantize.hip", "qsa_device.h"),
    "score_t1984_pos30000": ("qsa_score.hip", "qsa_device.h"),
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
    """HBM bytes per qsa_flash call from the committed rocprofv3 counter
    summary of this workload, if it was taken on the current kernel
    sources; else None."""
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


def run_warmup(args, step, sync):
    """Runs the warmup steps: exactly args.warmup of them when given, else
    steps until AUTO_WARMUP_S has passed (at least 3).  Returns (warmup
    steps run, timed steps to use)."""
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
    steps = args.steps
    if steps is None:
        per_step = (time.perf_counter() - t0) / max(n, 1)
        steps = max(MIN_STEPS, min(5000, int(AUTO_TIMED_S / max(per_step, 1e-6))))
    return n, steps


def single_thread_oracle_t512():
    """One T=512, pos0 0 layer of the fp64 oracle on one host thread (a child
    process with OMP_NUM_THREADS=1): seconds and query tokens/s."""
    code = ("import sys, time; sys.path.insert(0, %r); import oracle, qsa_synth; "
            "inp = qsa_synth.layer_inputs(512, 0, layer=0); t = time.perf_counter(); "
            "oracle.attend(inp, None); print(time.perf_counter() - t)" % ROOT)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=600)
    if r.returncode != 0:
        return None
    s = float(r.stdout.strip().splitlines()[-1])
    return {"value": 512 / s, "unit": "query-tokens/s (1 layer)", "cores": 1, "kind": "oracle",
            "sample": "one T=512 pos0 0 layer, fp64 oracle attention, one thread, %.2f s" % s}


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


class Timer:
    """HIP events on torch's current stream, which every bound call uses."""

    def __init__(self, torch):
        self.torch = torch

    def pair(self):
        E = self.torch.cuda.Event
        return E(enable_timing=True), E(enable_timing=True)


def load_workload(workload: str, dev) -> list:
    """The device inputs, outputs, workspaces and bound calls of every layer
    of a prompt or split workload."""
    import numpy as np
    import torch

    import qsa_synth
    import quantized_sparse_flash_amd as qsa

    wl = WORKLOADS[workload]
    T, pos0, L, kind = wl["T"], wl["pos0"], wl["layers"], wl["kind"]
    log("bench: generating %d layer(s) of inputs (%s)" % (L, workload))
    layers = []
    for layer in range(L):
        inp = qsa_synth.layer_inputs(T, pos0, layer=layer)
        d = {k: torch.from_numpy(np.ascontiguousarray(getattr(inp, k))).to(dev)
             for k in ("q", "kq", "ksc", "vq", "vsc")}
        s = qsa.QsaShape(T=T, pos0=pos0, n_groups=2, budget=inp.budget, n_cells=inp.n_cells)
        d["shape"] = s
        d["scores"] = None if inp.scores is None else torch.from_numpy(inp.scores).to(dev)
        d["ids"] = None
        if inp.scores is not None:
            d["ids"] = torch.empty((T, 2, inp.budget), dtype=torch.int32, device=dev)
        d["out"] = torch.empty((T, s.n_heads, 256), dtype=torch.float16, device=dev)
        need = qsa.qsa_flash_workspace_bytes(s)
        # a workspace of its own per layer (the attend-only region prepares
        # every layer before the attention launches run)
        d["ws"] = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        d["part"] = None
        if kind == "split":
            d["part"] = torch.empty((T, s.n_part_chunks, s.n_heads, qsa.PART_STRIDE),
                                    dtype=torch.float32, device=dev)
        d["topk"] = (qsa.bind_qsa_topk(s, d["scores"], d["ids"]) if d["scores"] is not None
                     else None)
        d["flash"] = qsa.bind_qsa_flash(s, d["q"], d["kq"], d["ksc"], d["vq"], d["vsc"],
                                        d["ids"], None if kind == "split" else d["out"],
                                        d["part"], d["ws"])
        d["merge"] = qsa.bind_qsa_merge(s, d["part"], d["out"]) if kind == "split" else None
        layers.append(d)
    torch.cuda.synchronize()
    return layers


def measure(workload: str, args, dev, flush, layers=None) -> dict:
    """Runs one prompt or split workload through the three timed regions
    (on the layers of load_workload, loaded here unless given)."""
    import torch

    import quantized_sparse_flash_amd as qsa

    wl = WORKLOADS[workload]
    T, pos0, L, kind = wl["T"], wl["pos0"], wl["layers"], wl["kind"]
    if layers is None:
        layers = load_workload(workload, dev)
    budget = layers[0]["shape"].budget

    def step():
        for d in layers:
            if d["topk"] is not None:
                d["topk"]()
            d["flash"]()
            if d["merge"] is not None:
                d["merge"]()

    n_warm, steps = run_warmup(args, step, torch.cuda.synchronize)

    # 1. value and ms_per_step: K steps with nothing else on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # 2. the pages' protocol: single steps after a cache flush, median + min
    tm = Timer(torch)
    samp = []
    for k in range(SAMPLES):
        flush.fill_(k & 0xFF)
        e0, e1 = tm.pair()
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        samp.append(e0.elapsed_time(e1))
    med, mn = statistics.median(samp), min(samp)

    # 3. kernel timing: every step's qsa_flash calls back to back
    repeat = DECODE_REPEAT if T <= 8 else 1
    ev = [tm.pair() for _ in range(steps)]
    for k in range(steps):
        for d in layers:
            if d["topk"] is not None:
                d["topk"]()
        ev[k][0].record()
        for _ in range(repeat):
            for d in layers:
                d["flash"]()
        ev[k][1].record()
        for d in layers:
            if d["merge"] is not None:
                d["merge"]()
    torch.cuda.synchronize()
    call_s = sum(a.elapsed_time(b) for a, b in ev) / (steps * repeat * L) / 1e3
    attend_s = None
    if kind == "prompt":
        # the attention kernel alone: every layer prepared into its own
        # workspace first, then the attend launches back to back
        ev = [tm.pair() for _ in range(steps)]
        for k in range(steps):
            for d in layers:
                if d["topk"] is not None:
                    d["topk"]()
                qsa.qsa_flash_prepare(d["shape"], d["kq"], d["ksc"], d["vq"], d["vsc"],
                                      workspace=d["ws"])
            ev[k][0].record()
            for d in layers:
                qsa.qsa_flash_attend(d["shape"], d["q"], d["kq"], d["ksc"], d["vq"], d["vsc"],
                                     d["ids"], d["out"], workspace=d["ws"])
            ev[k][1].record()
        torch.cuda.synchronize()
        attend_s = sum(a.elapsed_time(b) for a, b in ev) / (steps * L) / 1e3

    visits, by, flops = algorithmic(T, pos0, budget)
    ms_per_step = elapsed / steps * 1e3
    res = {"workload": workload, "T": T, "pos0": pos0, "layers": L, "kind": kind,
           "steps": steps, "warmup": n_warm, "ms_per_step": ms_per_step,
           "value": T * steps / elapsed, "budget": budget,
           "samples": {"n": SAMPLES, "median_ms": med, "min_ms": mn,
                       "tokens_per_s_at_median": T / (med / 1e3),
                       "flush_bytes_before_each": FLUSH_BYTES,
                       "what": "one step between HIP events, after a %d MiB write that flushes "
                               "the Infinity Cache and the L2s" % (FLUSH_BYTES >> 20)},
           "visits": visits, "bytes": by, "flops": flops, "call_s": call_s,
           "attend_s": attend_s}
    log("bench: %s %.3f ms/step, samples median %.3f / min %.3f ms, qsa_flash call %.1f us%s"
        % (workload, ms_per_step, med, mn, call_s * 1e6,
           "" if attend_s is None else ", attend kernel %.1f us" % (attend_s * 1e6)))
    del layers
    return res


def fused_kernels(T: int, pos0: int, budget: int, G: int = 2) -> str:
    """The kernels a fused qsa_flash call of this shape enqueues, for the
    bench line's label (the library's routing: tokens under budget on the
    tiled path; rows above budget as row pieces plus the merge when at most
    512 of them, every token so when the call has at most 256 rows, else
    one wavefront per row)."""
    t_id = max(0, min(T, budget - pos0))
    rows_above = (T - t_id) * G
    # 8-wave tiles of 128 queries when at least 256 of them cover the tokens
    tiled = "dequant_chunks_kernel + flash_tile_kernel<%d>" % (
        8 if G * -(-t_id * 12 // 128) >= 256 else 4)
    pieces = ("row pieces (flash_rows_staged_kernel<false, true>, or flash_split_kernel "
              "when each piece is one chunk) + merge_kernel")
    if rows_above == 0:
        return tiled
    if T * G <= 256:
        return pieces
    rest = pieces if rows_above <= 512 else "flash_rows_staged_kernel<false, false>"
    return tiled + " + " + rest if t_id else rest


def roofline_of(r: dict, traffic) -> dict:
    """The roofline object of a measured workload (see the module text)."""
    T, pos0, kind = r["T"], r["pos0"], r["kind"]
    tflops = r["flops"] / r["call_s"] / 1e12
    identity = pos0 + T <= r["budget"]
    if kind == "split":
        kern = "qsa_flash in split mode: flash_split_kernel"
    else:
        kern = "qsa_flash: " + fused_kernels(T, pos0, r["budget"])
    roof = {"bound": "mfma", "achieved": tflops, "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": tflops / MFMA_F16_PEAK_TFLOPS,
            "traffic": traffic, "kernel": kern, "flops_per_launch": r["flops"],
            "mean_launch_us": r["call_s"] * 1e6,
            "launch_timing": "HIP events on the launch stream around every step's qsa_flash "
                             "calls run back to back (the whole call: each kernel it "
                             "enqueues%s), over a timed region of its own"
                             % ("; decode: the split call %d times" % DECODE_REPEAT
                                if T <= 8 else "")}
    if traffic is not None:
        roof["traffic_gbs"] = traffic / r["call_s"] / 1e9
        roof["traffic_frac_of_hbm"] = roof["traffic_gbs"] / HBM_PEAK_GBS
    if not identity:
        # rows above budget gather their own cells: mostly from L2 and the
        # Infinity Cache (the gathered bytes exceed what HBM could deliver)
        roof["note"] = ("row gather: neither roofline binds; each row's cells are copied from "
                        "L2 and the Infinity Cache into LDS (see gathered and traffic) while "
                        "the VALU widens V to fp16; QK^T runs on the int8 MFMA, priced here "
                        "at the fp16 peak")
    return roof


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
    ap.add_argument("--no-other-prompts", action="store_true",
                    help="on the default workload, skip the T=512 / T=1024 figures")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run one device copy of this many MiB before timing (a known-size "
                         "kernel for scaling FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the path is built and timed on a single "
              "MI355X (--gpus %d not supported)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_sparse_flash_amd as qsa

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
    if WORKLOADS[args.workload]["kind"] == "quantize":
        bench_quantize(args, WORKLOADS[args.workload], dev)
        return
    if WORKLOADS[args.workload]["kind"] == "score":
        bench_score(args, WORKLOADS[args.workload], dev)
        return
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    # The default line's extra 12-layer prompts run first, right after the
    # headline's inputs are on the device, and the headline follows at once:
    # its warmup steps then start with the chip already at the clock it
    # holds under load (from idle the clock takes tens of ms to rise, longer
    # than a few warmup steps).
    other = None
    head_layers = None
    if args.workload == "t1984_pos0_x12" and not args.no_other_prompts:
        head_layers = load_workload(args.workload, dev)
        other = {}
        for wl in OTHER_PROMPTS:
            o = measure(wl, argparse.Namespace(steps=None, warmup=None), dev, flush)
            ro = roofline_of(o, None)
            other[wl] = {"value": o["value"], "unit": "query-tokens/s",
                         "ms_per_step": o["ms_per_step"], "samples": o["samples"],
                         "qsa_flash_call_us": o["call_s"] * 1e6,
                         "attend_kernel_us": o["attend_s"] * 1e6,
                         "mfma_frac": ro["frac"], "steps": o["steps"]}
    r = measure(args.workload, args, dev, flush, head_layers)
    del head_layers
    T, pos0, L, kind = r["T"], r["pos0"], r["layers"], r["kind"]
    call_s = r["call_s"]
    gbs = r["bytes"] / call_s / 1e9
    roof = roofline_of(r, measured_traffic(args.workload))
    m5 = PAGES_M5_TOKS.get(T) if (pos0 == 0 and L == 12) else None
    steps_desc = {"prompt": "qsa_flash", "split": "qsa_topk + split qsa_flash + qsa_merge"}
    budget = r["budget"]
    line = {
        "metric": "qsa_flash query-tokens/s at T=%d (%d layer%s)" % (T, L, "s" if L > 1 else ""),
        "value": r["value"],
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": r["steps"],
        "warmup": r["warmup"],
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (r["value"] / m5) if m5 else None,
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
        "samples": r["samples"],
        "roofline": roof,
        "gathered": {"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": r["bytes"],
                     "cell_visits_per_launch": r["visits"]},
    }
    if r["attend_s"] is not None:
        at = r["flops"] / r["attend_s"] / 1e12
        line["attend_only"] = {
            "bound": "mfma", "achieved": at, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": at / MFMA_F16_PEAK_TFLOPS, "mean_launch_us": r["attend_s"] * 1e6,
            "kernel": "the attention kernel of qsa_flash_attend (tile or rows kernel)",
            "launch_timing": "HIP events around every step's attend launches run back to "
                             "back, every layer prepared into its own workspace first"}
    if m5:
        line["vs_baseline_note"] = ("value / the pages' Apple M5 figure (%.0f query-tokens/s, "
                                    "12 layers at T=%d); another machine, context only" % (m5, T))
    if other is not None:
        line["other_prompts"] = other
    del flush
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle (bounded sample)")
        cb = cpu_baseline(T, pos0, L)
        if T == 1984 and pos0 == 0:
            cb["single_thread_t512"] = single_thread_oracle_t512()
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


def bench_quantize(args, wl, dev) -> None:
    """qsa_quantize on the fp16 K and V rows of a 2-group cache of n_cells
    cells; one step quantises both tensors (two calls)."""
    import torch

    import qsa_synth
    import quantized_sparse_flash_amd as qsa

    n_cells = wl["pos0"] + wl["T"]
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

    n_warm, steps = run_warmup(args, step, torch.cuda.synchronize)
    # value from K plain steps; launch durations from K more steps, each
    # repeated QUANT_REPEAT times between two events
    t0 = time.perf_counter()
    for k in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    tm = Timer(torch)
    ev = [tm.pair() for _ in range(steps)]
    for k in range(steps):
        ev[k][0].record()
        for _ in range(QUANT_REPEAT):
            step()
        ev[k][1].record()
    torch.cuda.synchronize()
    mean_launch_s = (sum(e0.elapsed_time(e1) for e0, e1 in ev)
                     / (2 * QUANT_REPEAT * steps) / 1e3)
    by = rows * QUANT_ROW_BYTES
    gbs = by / mean_launch_s / 1e9
    value = rows * steps / elapsed
    log("bench: %.3f ms/step, quantize kernel mean %.1f us, %.0f GB/s"
        % (elapsed / steps * 1e3, mean_launch_s * 1e6, gbs))
    line = {
        "metric": "qsa_quantize cells/s (K and V rows of 2 groups)",
        "value": value,
        "unit": "cells/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": n_warm,
        "ms_per_step": elapsed / steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "precision": "fp16 rows in, int8 codes + fp16 scales out; divisions and rounding "
                     "decisions in IEEE fp32",
        "data": "synthetic (seeded: fp16 N(0,1) x 10^U(-3,1) per 64-dim block)",
        "config": {"workload": "quantize_kv_31984: qsa_quantize of K and V, 2 groups x %d "
                               "cells x 256 dims" % n_cells,
                   "n_cells": n_cells, "n_groups": G, "head_dim": 256},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic("quantize_kv_31984"),
                     "kernel": "quantize_kernel (qsa_quantize)",
                     "algorithmic_bytes_per_launch": by, "mean_launch_us": mean_launch_s * 1e6,
                     "launch_timing": "HIP events around %d back-to-back K+V quantiser call "
                                      "pairs per step, over a timed region of its own"
                                      % QUANT_REPEAT},
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


def bench_score(args, wl, dev) -> None:
    """qsa_score for one long-context layer: the rows above budget get a
    score per visible cell from a SCORE_INDEX_DIM-value index query and
    pooled key; one call per step."""
    import torch

    import qsa_synth
    import quantized_sparse_flash_amd as qsa

    T, pos0, D, G, budget = wl["T"], wl["pos0"], SCORE_INDEX_DIM, 2, qsa_synth.BUDGET
    n_cells = pos0 + T
    log("bench: generating score inputs (T=%d pos0=%d, %d values per cell)" % (T, pos0, D))
    qidx_h, pooled_h = qsa_synth.score_inputs(T, pos0, D)
    qidx, pooled = torch.from_numpy(qidx_h).to(dev), torch.from_numpy(pooled_h).to(dev)
    scores = torch.empty((T, G, n_cells), dtype=torch.float32, device=dev)
    shape = qsa.QsaShape(T=T, pos0=pos0, n_groups=G, budget=budget, n_cells=n_cells)
    call = qsa.bind_qsa_score(shape, qidx, pooled, scores)
    n_scores = sum(G * (pos0 + t + 1) for t in range(T) if pos0 + t + 1 > budget)
    by = n_scores * 4 + qidx_h.nbytes + pooled_h.nbytes  # scores out, inputs read once
    flops = n_scores * 2 * D

    n_warm, steps = run_warmup(args, call, torch.cuda.synchronize)
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    tm = Timer(torch)
    ev = [tm.pair() for _ in range(steps)]
    for k in range(steps):
        ev[k][0].record()
        for _ in range(SCORE_REPEAT):
            call()
        ev[k][1].record()
    torch.cuda.synchronize()
    mean_launch_s = sum(e0.elapsed_time(e1) for e0, e1 in ev) / (SCORE_REPEAT * steps) / 1e3
    gbs = by / mean_launch_s / 1e9
    log("bench: %s %.3f ms/step, qsa_score kernel mean %.1f us, %.0f GB/s"
        % (args.workload, elapsed / steps * 1e3, mean_launch_s * 1e6, gbs))
    line = {
        "metric": "qsa_score query-tokens/s at T=%d (1 layer)" % T,
        "value": T * steps / elapsed,
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": n_warm,
        "ms_per_step": elapsed / steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "precision": "fp32 index queries and pooled keys, fp32 fused multiply-adds",
        "data": "synthetic (seeded: qidx and pooled N(0,1) fp32)",
        "config": {"workload": "%s: qsa_score, T=%d pos0=%d, 2 KV groups, %d values per cell, "
                               "budget %d" % (args.workload, T, pos0, D, budget),
                   "T": T, "pos0": pos0, "n_groups": G, "index_dim": D, "budget": budget},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic("score_t1984_pos30000"),
                     "kernel": "score4_kernel (qsa_score)",
                     "algorithmic_bytes_per_launch": by, "scores_per_launch": n_scores,
                     "flops_per_launch": flops, "mean_launch_us": mean_launch_s * 1e6,
                     "launch_timing": "HIP events around %d back-to-back qsa_score calls per "
                                      "step, over a timed region of its own" % SCORE_REPEAT},
    }
    if not args.no_cpu_baseline:
        import oracle
        log("bench: timing the CPU oracle's scores (bounded sample)")
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        done, t_total = 0, 0.0
        while done < 10 and t_total < 8.0:
            t1 = time.perf_counter()
            oracle.score(T, pos0, budget, qidx_h, pooled_h)
            t_total += time.perf_counter() - t1
            done += 1
        line["cpu_baseline"] = {"value": T * done / t_total, "unit": "query-tokens/s (1 layer)",
                                "cores": threads, "kind": "oracle",
                                "sample": "%d whole calls of the workload, fp64 oracle scores, "
                                          "%.1f s wall" % (done, t_total)}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
