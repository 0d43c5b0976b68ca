#!/usr/bin/env python3
"""Benchmark of the FlashAttention-2 forward (HIP path) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one fa2_fwd call over one batch of the workload (default: the
headline workload, long_causal = bf16 [B=2, H=16, N=8192, d=128], causal,
0.1% of Q/K entries x20, fp32 O).  Inputs are seeded, synthetic and already
resident in device memory when timing starts; successive steps rotate over
copies of the inputs and outputs that together span at least 512 MB (twice
the 256 MB last-level cache), so each step reads its inputs from HBM.  W
untimed steps, then K timed steps bracketed by device synchronisation; each
launch is also bracketed by HIP events recorded on the stream the kernel
runs on.

Prints ONE JSON line: throughput in TFLOP/s of credited work
(4*B*H*N^2*d, halved when causal), the roofline of the attention kernel
against the MI355X dense-bf16 matrix peak, the HBM traffic measured by
rocprofv3 counters (from the committed summary, if it matches the current
kernel source), and the fp64 CPU oracle timed on a bounded sample of the
same workload on the host cores.

With --kv-heads K (K dividing H) the key/value tensors have K heads and the
grouped-head entry points run (fa2_fwd_gqa / fa2_bwd_gqa); the credited work
is unchanged (it counts query heads).

With --window LEFT RIGHT the sliding-window entry points run
(fa2_fwd_window / fa2_bwd_window) and the credited work counts only the
visible (query, key) pairs: 4*d (forward) or 10*d (backward) flop per pair.

By default (--split auto) the forward asks fa2_split_plan for a schedule on
the device's compute units: where the grid of query tiles is too small and
uneven to fill the chip (few heads, long sequences, causal), heavy tiles'
key ranges are cut into chunks and a step is fa2_fwd_split (the forward
kernel over the chunks, then the merge of the partial results); otherwise
a step is fa2_fwd_window.  --split off always runs fa2_fwd_window.  Events
bracket the whole step, so with a split the kernel time includes the merge.

With --block-sparse DENSITY (forward) every head gets its own seeded random
mask of 128x128 blocks (--sparse-block ROWS KEYS to change), each set with probability DENSITY and the diagonal
blocks always set (workloads.make_block_mask, seed = --seed), combined with
the workload's causal flag; a step is fa2_fwd_sparse over the lists
fa2_sparse_plan built (outside the timed region), and the credited work
counts the visible pairs exactly (4*d flop per pair).

With --pass bwd a step is one fa2_bwd call (the D, dK/dV and dQ kernels) on
the same workload, with dO drawn from the seeded generator and O and LSE
from one fa2_fwd call made before timing; throughput is credited backward
work (10*B*H*N^2*d, halved when causal) and the CPU baseline times the fp64
gradient oracle.

With --fp8 (forward) a step is fa2_fp8_pack of Q and of K (rotation by a
seeded randomized Hadamard transform and E4M3 quantization, one scale per
(sequence, head)) followed by fa2_fwd_fp8 (Q K^T on FP8 matrix cores, P V in
bf16); `value` counts the whole step, the roofline the attention kernel
alone against the peak of its mix of work (half the flops at the FP8 rate,
half at the bf16 rate: 2 / (1/5033 + 1/2517) TFLOP/s).

With --pass decode a step is one fa2_decode_paged call on a synthetic
serving batch (DECODE_CONFIG: B sequences whose context lengths are drawn
uniformly from [L_min, L_max] by a seeded generator, one new token each,
H query heads on H_kv key/value heads, d = 128, pages of 64 keys in a
randomly permuted cache).  Decoding is bound by HBM: the line reports GB/s
of algorithmic traffic (each sequence's keys and values read once, Q read,
O and LSE written) against the 8 TB/s peak.

Extra modes used to produce committed profile summaries:
    --calibrate-copy      time a plain 1 GiB device copy (counter calibration)
    --summarize-pmc DIR   summarise rocprofv3 --pmc CSV output found under DIR
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOPs/s and % of MI355X bf16 MFMA peak, d=128 N=8k causal"
METRIC_BWD = "attention bwd TFLOPs/s and % of MI355X bf16 MFMA peak, d=128 N=8k causal"
# Dense bf16 matrix-core peak: 256 CUs x 4096 flop/clk/CU x 2.4 GHz.
PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
PEAK_F32_TFLOPS = 157.3
# Dense FP8 matrix-core peak (E4M3 x E4M3, fp32 accumulation): twice bf16.
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS
PEAK_HBM_GBS = 8000.0
# Sources (and the build script with its compile flags) behind each measured
# kernel: a profile summary stamped with the hash of its list is current only
# while none of them changes.
_CSRC = "exact_tiled_attention_33_amd/csrc/"
_COMMON = [_CSRC + "fa2_api.cpp", _CSRC + "fa2_launch.h", "exact_tiled_attention_33_amd/build_lib.py"]
KERNEL_SOURCES = [_CSRC + "fa2_fwd_bf16.hip", _CSRC + "fa2_fwd_f32.hip"] + _COMMON
BWD_SOURCES = [_CSRC + "fa2_bwd_bf16.hip"] + _COMMON
DECODE_SOURCES = [_CSRC + "fa2_decode.hip", _CSRC + "fa2_fwd_bf16.hip"] + _COMMON  # merge kernel in the latter
FP8_SOURCES = [_CSRC + "fa2_fp8.hip", _CSRC + "fa2_fwd_bf16.hip"] + _COMMON
CALIB_BYTES = 1 << 30
ROTATE_BYTES = 512 * 10**6  # rotated input/output sets span at least this (twice the 256 MB MALL)
METRIC_DECODE = "paged-KV decode, GB/s of key/value traffic vs MI355X HBM peak"
DECODE_CONFIG = {"B": 64, "H": 32, "H_kv": 8, "d": 128, "n_q": 1, "page_size": 64, "L_min": 1024, "L_max": 8192}


def idle_clock(fa2):
    """Shader clock (GHz) of 256 probe workgroups on an otherwise idle GPU."""
    try:
        return round(fa2.shader_clock_ghz(), 3)
    except Exception:  # pragma: no cover - diagnostic only
        return None


def warm_step_ms(events):
    """Median GPU time of one warm-up step (events recorded between steps),
    or 0.1 ms without warm-up steps."""
    if len(events) < 2:
        return 0.1
    return statistics.median(a.elapsed_time(b) for a, b in zip(events[:-1], events[1:]))


def start_probe(fa2, seconds):
    """One probe workgroup on a stream of its own, started just ahead of the
    timed launches, for 80% of the timed region's expected length `seconds`
    (so that it ends inside the region and the synchronisation that closes
    the region never waits for it); None if it cannot start."""
    try:
        p = fa2.ClockProbe(1)
        p.start(0.8 * seconds)
        return p
    except Exception:  # pragma: no cover - diagnostic only
        return None


def clock_report(idle_before, probe, idle_after):
    during = None
    if probe is not None:
        try:
            during = round(probe.ghz(), 3)
        except Exception:  # pragma: no cover
            during = None
    return {"during_timed_ghz": during, "idle_before_ghz": idle_before, "idle_after_ghz": idle_after,
            "probe": "fa2_clock_probe: shader cycles (s_memtime) against the 100 MHz reference (s_memrealtime); "
                     "during = one single-wave workgroup on its own stream over the first 80% of the timed region "
                     "(it takes one wave slot of the chip); idle = 256 workgroups for 50 us before and after it"}


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES if sources is None else sources):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, profile: str = None, sources=None):
    """HBM bytes per launch of the dominant kernel from profiles/<profile>_hbm.md
    (profile defaults to fa2_fwd_<workload>), if it was measured on the
    current sources of that kernel (default: the forward's); else None."""
    path = os.path.join(ROOT, "profiles", f"{profile or 'fa2_fwd_' + workload}_hbm.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash(sources):
        return None
    return float(m_bytes.group(1))


def cpu_baseline(w, q, k, v, budget_s: float = 12.0):
    """Time the fp64 oracle on whole heads of the workload until the budget
    is used (at least one head).  Returns the cpu_baseline object."""
    import numpy as np
    import torch

    import oracle.exact_attention as ref

    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done, t_total = 0, 0.0
    for b, h in heads:
        g = h * k.shape[1] // w.H  # key/value head of query head h
        qh = q[b, h].to("cpu", torch.float64).numpy()
        kh = k[b, g].to("cpu", torch.float64).numpy()
        vh = v[b, g].to("cpu", torch.float64).numpy()
        t0 = time.perf_counter()
        ref.attention_head(qh, kh, vh, w.scale, w.causal)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= budget_s:
            break
    import workloads

    flops = workloads.credited_flops(1, done, w.N, w.d, w.causal)
    return {
        "value": flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{done} of {w.B * w.H} (batch, head) pairs of {w.name}, whole heads "
                  f"(N={w.N}, d={w.d}, causal={w.causal}), fp64 numpy, {t_total:.1f} s",
        "seconds": t_total,
    }


def window_of(args, w):
    """(window_left, window_right) of the run: --window, else the workload's
    causal (-1, 0) or unmasked (-1, -1) form."""
    if args.window is not None:
        wl, wr = args.window
        if wl < -1 or wr < -1:
            raise SystemExit("bench.py: --window bounds must be >= -1")
        return wl, wr
    return (-1, 0) if w.causal else (-1, -1)


def kv_heads(args, w) -> int:
    """Key/value heads of the run: --kv-heads if given (grouped heads), else H."""
    hkv = args.kv_heads or w.H
    if hkv < 1 or w.H % hkv:
        raise SystemExit(f"bench.py: --kv-heads {hkv} must divide H = {w.H}")
    return hkv


def run_bench(args) -> dict:
    import torch

    import exact_tiled_attention_33_amd as fa2
    import workloads

    w = workloads.get(args.workload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    q, k, v = workloads.make_inputs(w, seed=args.seed, device=dev)
    hkv = kv_heads(args, w)
    k, v = k[:, :hkv].contiguous(), v[:, :hkv].contiguous()
    o_dtype = torch.bfloat16 if args.o_dtype == "bf16" else torch.float32
    o = torch.empty(w.shape, dtype=o_dtype, device=dev)
    lse = torch.empty(w.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)
    in_code = fa2.BF16 if w.dtype == "bf16" else fa2.F32
    o_code = fa2.BF16 if args.o_dtype == "bf16" else fa2.F32
    handle = stream.cuda_stream
    wl, wr = window_of(args, w)
    call_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                 w.B, w.H, hkv, w.N, w.d, wl, wr, w.scale, handle, in_code, o_code)
    schedule = {"split": False}
    if args.split == "auto" and w.dtype == "bf16" and args.block_sparse is None and not args.fp8:
        splan = fa2.split_plan(w.shape, window=(wl, wr), num_units=props.multi_processor_count)
        if splan.splits:
            items = splan.device_items(dev)
            workspace = torch.empty(splan.workspace_bytes, dtype=torch.uint8, device=dev)
            call_args = call_args + (items.data_ptr(), splan.n_items, splan.n_slots, workspace.data_ptr(),
                                     splan.workspace_bytes)
            lengths = splan.items[:, 2] - splan.items[:, 1]
            schedule = {"split": True, "items": splan.n_items, "partial_slots": splan.n_slots,
                        "workgroups": splan.n_items * w.B * w.H, "longest_chunk_key_tiles": int(lengths.max()),
                        "workspace_bytes": splan.workspace_bytes}
    fwd_call = fa2.fa2_fwd_split if schedule["split"] else fa2.fa2_fwd_window
    sparse_pairs = None
    fp8_kernel = None
    if args.fp8:
        if args.window is not None or args.block_sparse is not None or w.dtype != "bf16":
            raise SystemExit("bench.py: --fp8 takes a bf16 workload, causal or not, and no other variant")
        signs = workloads.make_signs(w.d, args.seed + 11)
        sg = [float(t) for t in signs.tolist()]
        q8 = torch.empty(q.shape, dtype=torch.uint8, device=dev)
        k8 = torch.empty(k.shape, dtype=torch.uint8, device=dev)
        qs = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        ks = torch.empty(k.shape[:2], dtype=torch.float32, device=dev)
        wsq = torch.empty(fa2.fa2_fp8_pack_workspace(w.B, w.H, w.N), dtype=torch.uint8, device=dev)
        wsk = torch.empty(fa2.fa2_fp8_pack_workspace(w.B, hkv, w.N), dtype=torch.uint8, device=dev)
        attn_args = (q8.data_ptr(), qs.data_ptr(), k8.data_ptr(), ks.data_ptr(), v.data_ptr(), o.data_ptr(),
                     lse.data_ptr(), w.B, w.H, hkv, w.N, w.d, int(w.causal), w.scale, handle, o_code)

        def fwd_call(*_):
            st = fa2.fa2_fp8_pack(q.data_ptr(), w.B, w.H, w.N, w.d, sg, q8.data_ptr(), qs.data_ptr(), wsq.data_ptr(),
                                  wsq.numel(), handle)
            if st == fa2.FA2_OK:
                st = fa2.fa2_fp8_pack(k.data_ptr(), w.B, hkv, w.N, w.d, sg, k8.data_ptr(), ks.data_ptr(),
                                      wsk.data_ptr(), wsk.numel(), handle)
            if st == fa2.FA2_OK:
                st = fa2.fa2_fwd_fp8(*attn_args)
            return st

        fp8_kernel = lambda: fa2.fa2_fwd_fp8(*attn_args)  # noqa: E731
        schedule = {"split": False, "fp8": {"rotation": "randomized Hadamard", "format": "E4M3",
                                            "scales": "one per (sequence, head)"}}
    if args.block_sparse is not None:
        if args.window is not None or w.dtype != "bf16":
            raise SystemExit("bench.py: --block-sparse takes a bf16 workload and no --window")
        bq, bk = args.sparse_block
        bmask = workloads.make_block_mask(w.H, -(-w.N // bq), -(-w.N // bk), args.block_sparse, seed=args.seed)
        sp = fa2.fa2_sparse_plan(w.N, bq, bk, bmask, w.causal)
        sp_ptr, sp_ent = sp.device_arrays(dev)
        call_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.H, hkv,
                     w.N, w.d, int(w.causal), w.scale, handle, in_code, o_code, w.H, sp_ptr.data_ptr(),
                     sp_ent.data_ptr() if sp_ent is not None else None, sp.n_entries)
        fwd_call = fa2.fa2_fwd_sparse
        sparse_pairs = w.B * sum(workloads.credited_pairs_block_sparse(w.N, bmask[h], bq, bk, w.causal)
                                 for h in range(w.H))
        dense_pairs = w.B * w.H * (w.N * (w.N + 1) // 2 if w.causal else w.N * w.N)
        schedule = {"split": False, "block_sparse": {"block": [bq, bk], "density": args.block_sparse,
                                                     "layouts": w.H, "key_tile_entries": sp.n_entries,
                                                     "visible_pair_fraction": round(sparse_pairs / dense_pairs, 4)}}
    # Successive steps rotate over copies of (Q, K, V, O, LSE) that together
    # exceed the 256 MB last-level cache (MALL) twice over, so that no step
    # finds its inputs left in that cache by the previous one and the bytes
    # moved are HBM bytes.  (The FP8 step packs from one Q, K into one code
    # buffer, so it keeps a single set.)
    set_bytes = sum(t.numel() * t.element_size() for t in (q, k, v, o, lse))
    n_sets = 1 if fp8_kernel is not None else min(8, max(1, -(-ROTATE_BYTES // set_bytes)))
    sets = [(q, k, v, o, lse)] + [(q.clone(), k.clone(), v.clone(), torch.empty_like(o), torch.empty_like(lse))
                                  for _ in range(n_sets - 1)]
    set_args = [tuple(t.data_ptr() for t in st) + tuple(call_args[5:]) for st in sets]
    torch.cuda.synchronize()

    def step(i):
        st = fwd_call(*set_args[i % n_sets])
        if st != fa2.FA2_OK:
            raise fa2.Fa2Error(st)

    wev = [torch.cuda.Event(enable_timing=True) for _ in range(args.warmup + 1)]
    wev[0].record(stream)
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
            wev[i + 1].record(stream)
    torch.cuda.synchronize()
    warm_ms = warm_step_ms(wev)

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    clk_before = idle_clock(fa2)
    probe = start_probe(fa2, args.steps * warm_ms * 1e-3)
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(args.warmup + i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock = clock_report(clk_before, probe, idle_clock(fa2))
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_launch_ms = sum(per_launch_ms) / len(per_launch_ms)
    span_ms = starts[0].elapsed_time(ends[-1])

    if sparse_pairs is not None:
        flops = 4.0 * w.d * sparse_pairs
    elif args.window is None:
        flops = workloads.credited_flops(w.B, w.H, w.N, w.d, w.causal)
    else:
        flops = 4.0 * w.B * w.H * w.d * workloads.credited_pairs(w.N, wl, wr)
    value = flops * args.steps / wall / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    fp8_timing = None
    if fp8_kernel is not None:
        # the attention kernel alone, on the packed inputs of the last step
        ks_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ke_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        for i in range(args.steps):
            ks_ev[i].record(stream)
            if fp8_kernel() != fa2.FA2_OK:
                raise fa2.Fa2Error(-1, "fa2_fwd_fp8")
            ke_ev[i].record(stream)
        torch.cuda.synchronize()
        step_ms = avg_launch_ms
        avg_launch_ms = sum(a.elapsed_time(b) for a, b in zip(ks_ev, ke_ev)) / args.steps
        peak = 2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS)
        fp8_timing = {"step_ms_avg": round(step_ms, 4), "attention_kernel_ms_avg": round(avg_launch_ms, 4),
                      "pack_ms_avg": round(step_ms - avg_launch_ms, 4)}
    # the counter summaries are taken on the plain forward with fp32 O
    plain_run = (hkv == w.H and args.window is None and not schedule["split"] and sparse_pairs is None
                 and fp8_kernel is None and args.o_dtype == "fp32")
    traffic = traffic_from_profiles(w.name) if plain_run else None
    prof = os.path.join("profiles", f"fa2_fwd_{w.name}_hbm.md")
    if traffic is not None:
        traffic_source = prof
    elif not plain_run:
        traffic_source = "none: counters are taken for the plain forward of the workload (fp32 O) only"
    elif not os.path.exists(os.path.join(ROOT, prof)):
        traffic_source = f"none: no {prof}"
    else:
        traffic_source = f"none: the kernel sources changed since {prof} was measured"
    plan = fa2.fa2_plan(w.B, w.H, w.N, w.d, int(w.causal), in_code)
    # Algorithmic bytes per launch: Q, K, V read once, O and LSE written once.
    esz = 2 if w.dtype == "bf16" else 4
    alg_bytes = (w.B * w.H * w.N * w.d * esz + 2 * w.B * hkv * w.N * w.d * esz
                 + w.B * w.H * w.N * w.d * (2 if args.o_dtype == "bf16" else 4) + w.B * w.H * w.N * 4)
    # The kernel is bound by whichever roof its arithmetic intensity is under.
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    hbm_bound = flops / alg_bytes < ridge
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(alg_bytes / (avg_launch_ms * 1e-3) / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(alg_bytes / (avg_launch_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    else:
        achieved = flops / (avg_launch_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1), "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
            "scale": w.scale, "in_dtype": w.dtype, "o_dtype": args.o_dtype, "kv_heads": hkv,
            "window": [wl, wr],
            "outlier_frac": w.outlier_frac, "outlier_mult": w.outlier_mult, "seed": args.seed,
            "dropout": 0.0, "backward": False, "parallelism": "single GPU",
        },
        "schedule": schedule,
        **({"fp8_timing": fp8_timing} if fp8_timing else {}),
        "pct_of_peak": round(100.0 * value / peak, 2),
        "roofline": {
            **roof,
            "traffic": traffic,
            "traffic_source": traffic_source,
            "kernel_ms_avg": round(avg_launch_ms, 4),
            "algorithmic_flops_per_launch": flops,
            "algorithmic_bytes_per_launch": alg_bytes,
            "arithmetic_intensity": round(flops / alg_bytes, 1),
            "ridge_flop_per_byte": round(ridge, 1),
            "achieved_tflops": round(flops / (avg_launch_ms * 1e-3) / 1e12, 2),
            "executed_flops_per_launch": plan["flops_executed"],
        },
        "timing": {"events_span_ms": round(span_ms, 4), "wall_s": round(wall, 4),
                   "per_launch_ms_min": round(min(per_launch_ms), 4),
                   "per_launch_ms_median": round(statistics.median(per_launch_ms), 4),
                   "per_launch_ms_max": round(max(per_launch_ms), 4),
                   "input_sets": n_sets, "input_set_bytes": set_bytes},
        "gpu": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                "cus": props.multi_processor_count},
        "shader_clock": clock,
        "kernel_source_sha256_16": kernel_source_hash(FP8_SOURCES if fp8_kernel is not None else None),
        "context_not_target": "pages (A100): FA1 25-40% of peak, FA2 50-73% of peak, up to 230 TFLOP/s",
    }
    if not args.no_cpu_baseline and args.window is None and sparse_pairs is None and fp8_kernel is None:
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, budget_s=args.cpu_budget)
    return result


def cpu_baseline_bwd(w, q, k, v, g, budget_s: float = 12.0):
    """Time the fp64 gradient oracle on whole heads until the budget is used
    (at least one head)."""
    import torch

    import oracle.attention_grad as gref
    import workloads

    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    done, t_total = 0, 0.0
    for b in range(w.B):
        for h in range(w.H):
            kvh = h * k.shape[1] // w.H  # key/value head of query head h
            arrs = [t[b, i].to("cpu", torch.float64).numpy() for t, i in ((q, h), (k, kvh), (v, kvh), (g, h))]
            t0 = time.perf_counter()
            gref.attention_grad_head(*arrs, w.scale, w.causal)
            t_total += time.perf_counter() - t0
            done += 1
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    flops = workloads.credited_bwd_flops(1, done, w.N, w.d, w.causal)
    return {
        "value": flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{done} of {w.B * w.H} (batch, head) pairs of {w.name}, whole heads "
                  f"(N={w.N}, d={w.d}, causal={w.causal}), fp64 numpy gradient oracle, {t_total:.1f} s",
        "seconds": t_total,
    }


def run_bench_bwd(args) -> dict:
    import torch

    import exact_tiled_attention_33_amd as fa2
    import workloads

    w = workloads.get(args.workload)
    if w.dtype != "bf16":
        raise SystemExit(f"bench.py --pass bwd: the backward pass covers bf16 workloads ({w.name} is not)")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    q, k, v = workloads.make_inputs(w, seed=args.seed, device=dev)
    hkv = kv_heads(args, w)
    k, v = k[:, :hkv].contiguous(), v[:, :hkv].contiguous()
    g = workloads.make_grad_output(w, seed=args.seed + 7919, device=dev)
    stream = torch.cuda.Stream(device=dev)
    wl, wr = window_of(args, w)
    with torch.cuda.stream(stream):
        o, lse = fa2.forward(q, k, v, scale=w.scale, stream=stream, window=(wl, wr))
    delta = torch.empty(w.shape[:3], dtype=torch.float32, device=dev)
    dq = torch.empty(w.shape, dtype=torch.float32, device=dev)
    dk, dv = (torch.empty(k.shape, dtype=torch.float32, device=dev) for _ in range(2))
    call_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), g.data_ptr(), lse.data_ptr(),
                 delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), w.B, w.H, hkv, w.N, w.d,
                 wl, wr, w.scale, stream.cuda_stream, fa2.BF16, fa2.F32, fa2.F32)
    torch.cuda.synchronize()

    def step():
        st = fa2.fa2_bwd_window(*call_args)
        if st != fa2.FA2_OK:
            raise fa2.Fa2Error(st, "fa2_bwd")

    wev = [torch.cuda.Event(enable_timing=True) for _ in range(args.warmup + 1)]
    wev[0].record(stream)
    for i in range(args.warmup):
        step()
        wev[i + 1].record(stream)
    torch.cuda.synchronize()
    warm_ms = warm_step_ms(wev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    clk_before = idle_clock(fa2)
    probe = start_probe(fa2, args.steps * warm_ms * 1e-3)
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock = clock_report(clk_before, probe, idle_clock(fa2))
    per_call_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_ms = sum(per_call_ms) / len(per_call_ms)
    pairs = workloads.credited_pairs(w.N, wl, wr)
    flops = 10.0 * w.B * w.H * w.d * pairs
    # executed: dK/dV recomputes S and dP (4 products), dQ does S, dP, dQ (3)
    executed = 14.0 * w.B * w.H * w.d * pairs
    value = flops * args.steps / wall / 1e12
    achieved = flops / (avg_ms * 1e-3) / 1e12
    # counters are taken per call (the three kernels) on the plain causal workload
    prof = os.path.join("profiles", f"fa2_bwd_{w.name}_hbm.md")
    counted_run = hkv == w.H and args.window is None
    traffic = traffic_from_profiles(w.name, f"fa2_bwd_{w.name}", BWD_SOURCES) if counted_run else None
    if traffic is not None:
        traffic_source = prof
    elif not counted_run:
        traffic_source = "none: counters are taken for the plain workload only"
    elif not os.path.exists(os.path.join(ROOT, prof)):
        traffic_source = f"none: no {prof}"
    else:
        traffic_source = f"none: the kernel sources changed since {prof} was measured"
    result = {
        "metric": METRIC_BWD,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
            "scale": w.scale, "in_dtype": w.dtype, "o_dtype": "fp32", "grad_dtype": "fp32", "kv_heads": hkv,
            "window": [wl, wr],
            "outlier_frac": w.outlier_frac, "outlier_mult": w.outlier_mult, "seed": args.seed,
            "dropout": 0.0, "backward": True, "parallelism": "single GPU",
        },
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": round(PEAK_BF16_TFLOPS, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "traffic_source": traffic_source,
            "scope": "one fa2_bwd call (D, dK/dV and dQ kernels), HIP events on its stream",
            "call_ms_avg": round(avg_ms, 4),
            "algorithmic_flops_per_call": flops,
            "executed_flops_per_call": executed,
        },
        "timing": {"wall_s": round(wall, 4), "per_call_ms_min": round(min(per_call_ms), 4),
                   "per_call_ms_max": round(max(per_call_ms), 4)},
        "gpu": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                "cus": props.multi_processor_count},
        "shader_clock": clock,
        "kernel_source_sha256_16": kernel_source_hash(BWD_SOURCES),
    }
    if not args.no_cpu_baseline and args.window is None:
        result["cpu_baseline"] = cpu_baseline_bwd(w, q, k, v, g, budget_s=args.cpu_budget)
    return result


def run_bench_decode(args) -> dict:
    import torch

    import exact_tiled_attention_33_amd as fa2
    import workloads

    cfg = dict(DECODE_CONFIG)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    g = torch.Generator().manual_seed(args.seed)
    lens = torch.randint(cfg["L_min"], cfg["L_max"] + 1, (cfg["B"],), generator=g).tolist()
    kc, vc, table = workloads.make_paged_cache(lens, cfg["H_kv"], cfg["d"], cfg["page_size"], seed=args.seed + 1,
                                               device=dev)
    q = torch.randn((cfg["B"], cfg["H"], cfg["n_q"], cfg["d"]), generator=g).to(torch.bfloat16).to(dev)
    ctx = torch.tensor(lens, dtype=torch.int32, device=dev)
    max_ctx = max(lens)
    split, ws_bytes = fa2.fa2_decode_paged_workspace(cfg["B"], cfg["H"], cfg["H_kv"], cfg["n_q"], cfg["d"], max_ctx,
                                                     args.split_keys, props.multi_processor_count)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    o_dtype = torch.bfloat16 if args.o_dtype == "bf16" else torch.float32
    o = torch.empty(q.shape, dtype=o_dtype, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)
    call_args = (q.data_ptr(), kc.data_ptr(), vc.data_ptr(), o.data_ptr(), lse.data_ptr(), cfg["B"], cfg["H"],
                 cfg["H_kv"], cfg["n_q"], cfg["d"], 1.0 / math.sqrt(cfg["d"]), table.data_ptr(), table.shape[1],
                 ctx.data_ptr(), max_ctx, cfg["page_size"], kc.shape[0], split, ws.data_ptr(), ws_bytes,
                 stream.cuda_stream, fa2.BF16, fa2.BF16 if args.o_dtype == "bf16" else fa2.F32)
    torch.cuda.synchronize()

    def step():
        st = fa2.fa2_decode_paged(*call_args)
        if st != fa2.FA2_OK:
            raise fa2.Fa2Error(st, "fa2_decode_paged")

    wev = [torch.cuda.Event(enable_timing=True) for _ in range(args.warmup + 1)]
    wev[0].record(stream)
    for i in range(args.warmup):
        step()
        wev[i + 1].record(stream)
    torch.cuda.synchronize()
    warm_ms = warm_step_ms(wev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    clk_before = idle_clock(fa2)
    probe = start_probe(fa2, args.steps * warm_ms * 1e-3)
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock = clock_report(clk_before, probe, idle_clock(fa2))
    per_launch_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    avg_ms = sum(per_launch_ms) / len(per_launch_ms)
    kv_bytes = 2 * sum(lens) * cfg["H_kv"] * cfg["d"] * 2
    rows = cfg["B"] * cfg["H"] * cfg["n_q"]
    alg_bytes = kv_bytes + rows * cfg["d"] * 2 + rows * cfg["d"] * (2 if args.o_dtype == "bf16" else 4) + rows * 4
    flops = 4.0 * cfg["H"] * cfg["d"] * sum(lens) * cfg["n_q"]
    gbs = alg_bytes / (avg_ms * 1e-3) / 1e9
    # counters are taken on this batch with the library's chunk and fp32 O
    prof = os.path.join("profiles", "fa2_decode_paged_hbm.md")
    counted_run = args.split_keys == 0 and args.o_dtype == "fp32" and args.seed == 0
    traffic = traffic_from_profiles("paged_decode", "fa2_decode_paged", DECODE_SOURCES) if counted_run else None
    if traffic is not None:
        traffic_source = prof
    elif not counted_run:
        traffic_source = "none: counters are taken for the default batch, chunk and fp32 O only"
    elif not os.path.exists(os.path.join(ROOT, prof)):
        traffic_source = f"none: no {prof}"
    else:
        traffic_source = f"none: the kernel sources changed since {prof} was measured"
    return {
        "metric": METRIC_DECODE,
        "value": round(alg_bytes * args.steps / wall / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "paged_decode", **cfg, "context_lens_sum": sum(lens), "max_context": max_ctx,
                   "split_keys": split, "o_dtype": args.o_dtype, "seed": args.seed, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic, "traffic_source": traffic_source,
                     "kernel_ms_avg": round(avg_ms, 4),
                     "algorithmic_bytes_per_launch": alg_bytes, "algorithmic_flops_per_launch": flops,
                     "arithmetic_intensity": round(flops / alg_bytes, 2)},
        "timing": {"per_launch_ms_min": round(min(per_launch_ms), 4),
                   "per_launch_ms_max": round(max(per_launch_ms), 4)},
        "gpu": {"name": props.name, "arch": getattr(props, "gcnArchName", ""), "cus": props.multi_processor_count},
        "shader_clock": clock,
        "kernel_source_sha256_16": kernel_source_hash(DECODE_SOURCES),
    }


def calibrate_copy(args) -> None:
    """A plain device-to-device copy of CALIB_BYTES, repeated: its counter
    readings calibrate FETCH_SIZE / WRITE_SIZE against known bytes."""
    import torch

    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": CALIB_BYTES, "repeats": args.steps}))


def summarize_pmc(root: str) -> None:
    """Average per-dispatch counter values (KiB) per kernel from rocprofv3
    --pmc CSV output under ``root``."""
    import csv

    rows = []
    for path in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    acc = {}
    for r in rows:
        name = r.get("Kernel_Name", "?")
        ctr = r.get("Counter_Name", "?")
        val = float(r.get("Counter_Value", "nan"))
        key = (name[:90], ctr)
        acc.setdefault(key, []).append(val)
    for (name, ctr), vals in sorted(acc.items()):
        print(f"{ctr}\t{len(vals)} dispatches\tmean {sum(vals) / len(vals):.1f} KiB\t{name}")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline one)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--o-dtype", choices=["fp32", "bf16"], default="fp32")
    ap.add_argument("--pass", dest="which", choices=["fwd", "bwd", "decode"], default="fwd",
                    help="fwd (default): the forward pass; bwd: the backward pass; decode: paged-KV decoding")
    ap.add_argument("--window", type=int, nargs=2, default=None, metavar=("LEFT", "RIGHT"),
                    help="sliding-window mask: key j visible to query i iff i-LEFT <= j <= i+RIGHT "
                         "(-1 = unbounded side); overrides the workload's causal flag")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="key/value heads (grouped heads; default: as many as query heads)")
    ap.add_argument("--split", choices=["auto", "off"], default="auto",
                    help="forward: split heavy query tiles' key ranges when the planner predicts a gain")
    ap.add_argument("--block-sparse", type=float, default=None, metavar="DENSITY",
                    help="forward: random 128x128 block mask per head with this block density")
    ap.add_argument("--fp8", action="store_true",
                    help="forward: FP8 Q K^T with incoherent processing (pack Q, K, then fa2_fwd_fp8)")
    ap.add_argument("--sparse-block", type=int, nargs=2, default=[128, 128], metavar=("ROWS", "KEYS"),
                    help="block size of the --block-sparse mask (rows a multiple of 32, keys of 64)")
    ap.add_argument("--split-keys", type=int, default=0,
                    help="decode: keys per chunk (a multiple of 64; 0 = the library's choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--summarize-pmc", default=None)
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs the attention forward on exactly one GPU; "
              f"--gpus {args.gpus} (WORLD_SIZE={world}) is not supported. "
              "Run with --gpus 1.", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        calibrate_copy(args)
        return 0
    import workloads

    if args.workload is None:
        args.workload = workloads.HEADLINE
    if args.which == "decode":
        result = run_bench_decode(args)
    else:
        result = run_bench_bwd(args) if args.which == "bwd" else run_bench(args)
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
