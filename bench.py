#!/usr/bin/env python3
"""Benchmark: one paged-attention step (all layers) on one MI355X.

A step is one pass of the whole hot path over one batch: slot mapping once,
then for every layer the KV append followed by paged attention (decode +
split-KV merge, plus prefill chunks where the workload has them), all on one
stream, inputs resident in HBM.  By default each layer is one
pkv_append_attention_step call (the decode tokens are appended inside the
decode kernel); --separate runs pkv_kv_append + pkv_paged_attention_step.
Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--extra A,B]
                    [--separate] [--kv-dtype fp16|fp8]

The headline workload (default long_context: 16 layers of 4 sequences at
262,144 tokens, the largest configuration) is the line's top level; the
workloads named by --extra (default, with the default headline: qwen_ragged
and qwen_uniform) are measured in the same run and reported under
"workloads", each with its own roofline and cpu_baseline.

value      = decode tokens per second of the whole step (query tokens of the
             decode and multi-token-decode sequences x steps / wall time),
             wall time between synchronisations.
roofline   = the dominant kernel (paged decode + its merge): algorithmic
             bytes per launch (KV of every context, Q and O, block ids, and
             the appended rows when fused) over the launch's average
             duration from HIP events around back-to-back attention
             launches, against the 8 TB/s HBM peak; also against the rate of
             a plain device copy moving the same number of bytes
             (measured_copy_gbps, frac_of_measured_copy), and against the
             read rate of pkv_hbm_read_probe over the same tile size and
             bytes in a random order in a 4 GiB buffer (read_probe_gbps,
             frac_of_read_probe).  traffic = HBM bytes per launch from the
             committed rocprofv3 counter summary named in traffic_source
             (reported only while the decode kernel's sources still hash to
             the value recorded there; not measured in this run).
ms_per_step_median / _min = per-step durations from events between the timed
             steps.
prefill    = (steps with prefill chunks) the chunks alone timed the same
             way: flops per launch over launch time against the dense fp16
             MFMA peak; query_tokens_per_s counts every new token of the step.
cpu_baseline = the fp64 CPU oracle, timed on the host on a bounded sample of
             the same workload (a few layers of the step), scaled to a step;
             with the host's CPU model and the cores the process may use.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn step: KV-read HBM GB/s (% of peak) and decode tokens/s at 1 GPU"
HBM_PEAK_GBPS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0  # dense fp16 matrix-core peak (no sparsity)
DEFAULT_WORKLOAD = "long_context"
DEFAULT_EXTRA = ("qwen_ragged", "qwen_uniform")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--extra", default=None,
                    help="comma-separated workloads measured in the same run and reported "
                         "under 'workloads' (default: qwen_ragged,qwen_uniform with the "
                         "default headline and no overrides; 'none' for none)")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the HBM read-rate probe")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0 = workload's)")
    ap.add_argument("--batch", type=int, default=0, help="override the batch (uniform / long_context)")
    ap.add_argument("--ctx", type=int, default=0, help="override the context length (uniform / long_context)")
    ap.add_argument("--partition", type=int, default=0,
                    help="force split-KV partition tokens (multiple of 64; 0 = automatic)")
    ap.add_argument("--separate", action="store_true",
                    help="append and attention as two calls per layer (default: one fused call)")
    ap.add_argument("--schedule", choices=["auto", "on", "off"], default="auto",
                    help="decode on the balanced schedule (on), on the fixed partition grid "
                         "(off), or as the step chooses: the schedule only with prefill "
                         "chunks (auto)")
    ap.add_argument("--graph", action="store_true",
                    help="capture the whole step (all layers) once as a HIP graph and time "
                         "its replays")
    ap.add_argument("--one-call", action="store_true",
                    help="every layer of a step in one library call "
                         "(pkv_append_attention_layers) instead of one call per layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kv-dtype", choices=["fp16", "fp8"], default="fp16",
                    help="cache element type: fp16 (the workloads' own), or fp8 E4M3 codes "
                         "with fp32 row scales")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES (5 times), the "
                         "reference for scaling HBM traffic counters, and exit")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    return ap.parse_args()


def kv_row_bytes(wl, kv_dtype: str) -> int:
    """Cache bytes of one (token, KV head) row: d fp16 values, or d fp8 codes
    and one fp32 scale."""
    return wl.head_dim * 2 if kv_dtype == "fp16" else wl.head_dim + 4


def algorithmic_bytes_per_attention_launch(wl, fused: bool, kv_dtype: str = "fp16") -> int:
    """For the sequences whose attention streams the cache (decodes, and
    multi-token decodes whose G x n rows fit one tile): KV of every context +
    Q and O rows + block ids, one layer; when the call also appends their new
    tokens, + those fp16 K/V rows read, their cache rows written, and their
    slots."""
    m = wl.short_chunk()
    ctx = wl.context_lens[m].astype(np.int64)
    T = int(wl.new_tokens[m].sum())
    row = kv_row_bytes(wl, kv_dtype)
    kv = int(ctx.sum()) * wl.num_kv_heads * row * 2
    qo = 2 * T * wl.num_q_heads * wl.head_dim * 2
    ids = int((-(-ctx // wl.block_size)).sum()) * 4
    app = (2 * T * wl.num_kv_heads * (wl.head_dim * 2 + row) + 8 * T) if fused else 0
    return kv + qo + ids + app


def streamed_tokens(wl) -> int:
    """Query tokens of the sequences whose attention streams the cache: one
    per decode sequence, n per multi-token decode."""
    return int(wl.new_tokens[wl.short_chunk()].sum())


def measured_traffic(wl):
    """(HBM bytes per attention launch, summary path) from the committed
    rocprofv3 counter summary of this workload, or None when there is none
    or the decode kernel's sources changed since it was taken."""
    import hashlib
    rel = f"profiles/paged_decode_{wl.name}_hbm_traffic.txt"
    path = os.path.join(ROOT, rel)
    if not os.path.exists(path):
        return None
    fields = dict(line.split(": ", 1) for line in open(path) if ": " in line and not line.startswith(" "))
    h = hashlib.sha256()
    for f in ("paged_kv_decode_append_amd/csrc/decode.hip", "paged_kv_decode_append_amd/csrc/decode_block.h",
              "paged_kv_decode_append_amd/csrc/device_util.h"):
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if fields.get("kernel_source_sha256", "").strip() != h.hexdigest():
        return None
    return float(fields["traffic_bytes_per_launch"]), rel


def read_probe_rate(tile_bytes: int, bytes_per_launch: int, seed: int = 0):
    """GB/s that pkv_hbm_read_probe sustains reading `bytes_per_launch` per
    launch as whole `tile_bytes` tiles in a random order, from a buffer of at
    least 4 GiB (far beyond the last-level cache), successive launches taking
    the next tiles of one permutation; 10 launches back to back from one
    library call, HIP events on the launch stream."""
    import torch
    import paged_kv_decode_append_amd as pkv
    n = max(1, bytes_per_launch // tile_bytes)
    launches, warm = 10, 2
    # every launch reads tiles no earlier launch read: together they stay
    # within one permutation of a buffer of >= 4 GiB when it is large enough
    ntiles = max(n, (4 << 30) // tile_bytes)
    base = torch.zeros(ntiles * tile_bytes, dtype=torch.uint8, device="cuda")
    perm = np.random.default_rng(seed).permutation(ntiles).astype(np.int32)
    reps = -(-(launches + warm) * n // ntiles)
    ids = torch.from_numpy(np.tile(perm, reps)[: (launches + warm) * n].copy()).cuda()
    sink = torch.empty(pkv.PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    # the launches of one call run back to back (no host cost between them)
    pkv.hbm_read_probe(base, ids[: warm * n], tile_bytes, sink, launches=warm)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    pkv.hbm_read_probe(base, ids[warm * n:], tile_bytes, sink, launches=launches)
    b.record(stream)
    torch.cuda.synchronize()
    t = a.elapsed_time(b) * 1e-3 / launches
    del base, ids, sink
    torch.cuda.empty_cache()
    return {"read_probe_gbps": round(n * tile_bytes / t / 1e9, 1), "read_probe_tile_bytes": tile_bytes,
            "read_probe_bytes_per_launch": n * tile_bytes}


def host_description():
    """CPU model and the cores this process may run on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        cpus = sorted(os.sched_getaffinity(0))
    except AttributeError:
        cpus = list(range(os.cpu_count() or 1))
    runs, lo = [], None
    for k, c in enumerate(cpus):
        if lo is None:
            lo = c
        if k + 1 == len(cpus) or cpus[k + 1] != c + 1:
            runs.append(f"{lo}-{c}" if c != lo else f"{c}")
            lo = None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cpus": len(cpus),
            "affinity": ",".join(runs)}


def measured_copy_rate(nbytes: int) -> float:
    """GB/s of a plain device-to-device copy moving `nbytes` in total (half
    read, half written): the rate HBM gives a trivially streaming kernel of
    the same size, with its own launch ramp and drain."""
    import torch
    half = max(nbytes // 2, 1 << 20)
    src = torch.ones(half, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        dst.copy_(src)
    times = []
    for _ in range(20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e-3)
    return 2 * half / float(np.median(times)) / 1e9


def prefill_roofline(wl, caches, layers, outs):
    """The prefill chunks alone (split-KV prefill kernel + its merge), timed
    with HIP events over L back-to-back launches: achieved TFLOP/s against
    the dense fp16 MFMA peak."""
    import torch
    import paged_kv_decode_append_amd as pkv
    from paged_kv_decode_append_amd.step import Step

    B = wl.num_decode_seqs
    pre = Step(wl.block_tables[B:], wl.context_lens[B:], wl.new_tokens[B:], 0, wl.num_q_heads,
               wl.num_kv_heads, wl.head_dim, wl.scale)
    pre.plan()
    stream = torch.cuda.current_stream()

    def launch_all():
        for c, t, o in zip(caches, layers, outs):
            pkv.paged_attention_step(c, t["q"][B:], o[B:], pre.block_tables, pre.context_lens,
                                     pre.query_start_loc, 0, wl.scale, pre.max_context_len,
                                     pre.max_query_len, workspace=pre.workspace)

    launch_all()
    times = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        launch_all()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e-3 / wl.num_layers)
    t = float(np.mean(times))
    flops = wl.prefill_flops_per_layer()
    return {"bound": "mfma", "flop_per_launch": flops, "launch_us": round(t * 1e6, 2),
            "achieved": round(flops / t / 1e12, 2), "peak": MFMA_FP16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(flops / t / 1e12 / MFMA_FP16_PEAK_TFLOPS, 4),
            "kernel": "chunked-prefill attention on MFMA (+ its split-KV merge)"}


def cpu_baseline(wl, layer_tensors_dev, budget_s: float, kv_dtype: str = "fp16"):
    """Time the oracle (append replay + attention, fp64) on whole layers of
    the step until the budget is spent; scale to decode tokens/s of a step."""
    import torch
    import oracle
    from oracle import fp8 as ofp8

    qsl = wl.query_start_loc if wl.num_decode_seqs < wl.num_seqs else None
    slots = oracle.slot_mapping(wl.block_tables, wl.context_lens, qsl, wl.block_size)
    spent, layers = 0.0, 0
    for t in layer_tensors_dev:
        host = {k: (v.detach().cpu().view(torch.int16).numpy().view(np.uint16)
                    if v.dtype == torch.float16 else v.detach().cpu().numpy())
                for k, v in t.items()}
        t0 = time.perf_counter()
        if kv_dtype == "fp8":
            kc, vc, ks, vs = ofp8.kv_append(host["k_codes"], host["v_codes"], host["k_scale"],
                                            host["v_scale"], host["k_new"], host["v_new"], slots)
            oracle.paged_attention_fp8(host["q"], kc, vc, ks, vs, wl.block_tables,
                                       wl.context_lens, qsl, wl.scale)
        else:
            kp, vp = oracle.kv_append(host["k_pool"], host["v_pool"], host["k_new"],
                                      host["v_new"], slots)
            oracle.paged_attention(host["q"], kp, vp, wl.block_tables, wl.context_lens, qsl,
                                   wl.scale)
        spent += time.perf_counter() - t0
        layers += 1
        if spent >= budget_s:
            break
    per_step = spent / layers * wl.num_layers
    return {
        "value": streamed_tokens(wl) / per_step,
        "unit": "tokens/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{layers} of {wl.num_layers} layers of one {wl.name} step "
                  f"({spent:.1f} s), scaled to a whole step",
        **host_description(),
    }


def measure(args, name: str, with_cpu: bool, overrides=None) -> dict:
    """One workload: K timed steps, the attention launch's roofline, the
    prefill chunks' (when the step has them) and the oracle's baseline."""
    import torch
    import workloads
    import paged_kv_decode_append_amd as pkv
    from paged_kv_decode_append_amd.step import Step

    wl = workloads.WORKLOADS[name](**(overrides or {}))
    if args.kv_dtype == "fp8":
        layers = [workloads.layer_tensors_fp8(wl, l, device="cuda") for l in range(wl.num_layers)]
        caches = [pkv.KVCache(t["k_codes"], t["v_codes"], t["k_scale"], t["v_scale"])
                  for t in layers]
    else:
        layers = [workloads.layer_tensors(wl, l, device="cuda") for l in range(wl.num_layers)]
        caches = [pkv.KVCache(t["k_pool"], t["v_pool"]) for t in layers]
    outs = [torch.empty_like(t["q"]) for t in layers]
    step = Step.from_workload(wl, kv_partition_tokens=args.partition,
                              use_schedule={"auto": None, "on": True, "off": False}[args.schedule])
    torch.cuda.synchronize()

    fused = not args.separate

    def run_step():
        step.plan()
        for c, t, o in zip(caches, layers, outs):
            step.layer(c, t["q"], t["k_new"], t["v_new"], o, fused=fused)

    prepared = None
    if args.one_call:
        prepared = step.prepare_layers([(c, t["q"], t["k_new"], t["v_new"], o)
                                        for c, t, o in zip(caches, layers, outs)])
        run_step = prepared
    if args.graph:
        run_step()
        graph = step.capture([(c, t["q"], t["k_new"], t["v_new"], o)
                              for c, t, o in zip(caches, layers, outs)], fused=fused)
        run_step = graph.replay

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # Timed region: exactly K steps between synchronisations; an event between
    # steps (no synchronisation) gives the per-step spread.
    stream = torch.cuda.current_stream()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    marks[0].record(stream)
    for k in range(args.steps):
        run_step()
        marks[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    step_ms = [marks[k].elapsed_time(marks[k + 1]) for k in range(args.steps)]

    # Per-launch duration of the attention (decode + merge [+ prefill]) with HIP
    # events on the launch stream, in a separate pass so that events do not
    # perturb the step timing above: the L layers' attention calls run back
    # to back between two events (fused: the whole step is those calls; when
    # separate, each pass appends every layer first).
    reps = min(args.steps, 20)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for r in range(reps):
        step.plan()
        if not fused:
            for c, t in zip(caches, layers):
                pkv.kv_append(c, t["k_new"], t["v_new"], step.slot_mapping)
        ev[r][0].record(stream)
        if prepared is not None:
            prepared.attend()
        for c, t, o in zip(caches, layers, outs) if prepared is None else ():
            if fused:
                step.layer(c, t["q"], t["k_new"], t["v_new"], o, fused=True)
            else:
                pkv.paged_attention_step(c, t["q"], o, step.block_tables, step.context_lens,
                                         step.query_start_loc, step.num_decode_seqs, step.scale,
                                         step.max_context_len, step.max_query_len,
                                         workspace=step.workspace,
                                         kv_partition_tokens=step.kv_partition_tokens,
                                         schedule=step.schedule)
        ev[r][1].record(stream)
    torch.cuda.synchronize()
    attn_us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3 / wl.num_layers

    alg_bytes = algorithmic_bytes_per_attention_launch(wl, fused, args.kv_dtype)
    achieved = alg_bytes / (attn_us * 1e-6) / 1e9
    copy_gbps = measured_copy_rate(alg_bytes)
    long_chunks = not wl.short_chunk().all()
    prefill = prefill_roofline(wl, caches, layers, outs) if long_chunks else None
    kv_bytes_step = (int(wl.context_lens[wl.short_chunk()].astype(np.int64).sum()) *
                     wl.num_kv_heads * kv_row_bytes(wl, args.kv_dtype) * 2 * wl.num_layers)
    multi = wl.num_decode_seqs < int(wl.short_chunk().sum())
    over = " over an fp8 (E4M3) cache" if args.kv_dtype == "fp8" else ""
    quant = "quantizing " if args.kv_dtype == "fp8" else ""
    kernel = (f"paged decode attention{over} with the decode tokens' {quant}append fused in"
              if fused else f"paged decode attention{over}") + " (+ split-KV merge when split)"
    if multi:
        kernel += ("; multi-token decodes on the packed-row MFMA kernel (+ its merge)" +
                   (f" after their {quant}append" if fused else ""))
    # the committed counters were taken on the workload's own sizes, fused,
    # fp16, with the automatic plan
    traffic = (measured_traffic(wl) if fused and args.kv_dtype == "fp16" and not overrides
               and args.partition == 0 and args.schedule == "auto" else None)
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": traffic[0] if traffic else None,
        "traffic_source": (f"{traffic[1]} (rocprofv3 FETCH_SIZE + WRITE_SIZE of the same kernel "
                           "sources, scaled by a plain copy's counters; not measured in this run)"
                           if traffic else None),
        "kernel": kernel,
        "alg_bytes_per_launch": alg_bytes,
        "launch_us": round(attn_us, 2),
        "measured_copy_gbps": round(copy_gbps, 1),
        "frac_of_measured_copy": round(achieved / copy_gbps, 4),
    }
    if not args.no_read_probe:
        row_tile = 16 * (wl.head_dim * 2 if args.kv_dtype == "fp16" else wl.head_dim)
        probe = read_probe_rate(row_tile, alg_bytes)
        roofline.update(probe)
        roofline["frac_of_read_probe"] = round(achieved / probe["read_probe_gbps"], 4)
    result = {
        "metric": METRIC,
        "value": round(streamed_tokens(wl) / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(float(np.median(step_ms)), 4),
        "ms_per_step_min": round(float(np.min(step_ms)), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic: fp16 products with fp32 accumulation; fp8 codes are
        # widened to fp16 (exactly) before they are multiplied
        "dtype": "fp16" if args.kv_dtype == "fp16" else "fp16 (fp8_e4m3 KV codes widened)",
        "kv_dtype": "fp16" if args.kv_dtype == "fp16" else "fp8_e4m3",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "layers": wl.num_layers,
            "batch": wl.num_seqs,
            "decode_seqs": wl.num_decode_seqs,
            "query_tokens": wl.num_tokens,
            "q_heads": wl.num_q_heads,
            "kv_heads": wl.num_kv_heads,
            "head_dim": wl.head_dim,
            "block_size": wl.block_size,
            "context_tokens": int(wl.context_lens.sum()),
            "max_context": wl.max_context_len,
            "pool_blocks_per_layer": wl.num_blocks,
            "parallelism": "single-gpu",
            "append": ("fused into the decode kernel" if args.kv_dtype == "fp16"
                       else "quantizing, fused into the decode kernel") if fused
                      else "separate kernel",
            "kv_cache": "fp16" if args.kv_dtype == "fp16" else "fp8_e4m3 + fp32 row scales",
            "launch": ("one HIP graph per step" if args.graph else
                       "one library call per step" if args.one_call else
                       "one library call per layer"),
        },
        "roofline": roofline,
        "kv_read_gbps_step": round(kv_bytes_step / (ms_per_step * 1e-3) / 1e9, 1),
    }
    if prefill is not None:
        result["query_tokens_per_s"] = round(wl.num_tokens / (ms_per_step * 1e-3), 1)
        result["prefill"] = prefill
    if with_cpu:
        result["cpu_baseline"] = cpu_baseline(wl, layers, args.cpu_budget_s, args.kv_dtype)
    del layers, caches, outs, step, run_step, prepared
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return result


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: the benchmark measures a single device; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 5}))
        return
    if args.one_call and (args.separate or args.graph):
        print(json.dumps({"error": "--one-call is the fused eager step; drop --separate/--graph"}))
        sys.exit(2)

    import workloads
    if args.workload not in workloads.WORKLOADS:
        print(json.dumps({"error": f"unknown workload {args.workload}"}))
        sys.exit(2)
    overrides = {k: v for k, v in (("layers", args.layers), ("batch", args.batch),
                                    ("ctx_len", args.ctx)) if v}
    if args.extra is None:
        extra = list(DEFAULT_EXTRA) if args.workload == DEFAULT_WORKLOAD and not overrides else []
    else:
        extra = [w for w in args.extra.split(",") if w and w != "none"]
    for w in extra:
        if w not in workloads.WORKLOADS:
            print(json.dumps({"error": f"unknown workload {w}"}))
            sys.exit(2)
    with_cpu = not args.no_cpu_baseline
    result = measure(args, args.workload, with_cpu, overrides)
    if extra:
        result["workloads"] = {w: measure(args, w, with_cpu) for w in extra if w != args.workload}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
