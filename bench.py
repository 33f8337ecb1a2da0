#!/usr/bin/env python3
"""Benchmark of sink-aware masked attention, forward + backward, on one GPU.

One step = one full pass of the hot path over the long-context workload
(B=1, Hq=64, Hkv=8, d=64, T=8192, two attention layers: a 128-token
sliding window with 4 prefix keys, and full causal): per layer the forward
kernel, then the backward phases (prepare, dQ, dK/dV, finish).  Inputs are
seeded synthetic bf16 tensors already resident in device memory; outputs
and workspace are preallocated.

Printed: one JSON line with useful (unmasked) TFLOP/s of the whole step
(4d FLOP per visible (q, k) pair forward, 10d backward), the fraction of
the bf16 dense MFMA peak, the roofline of the dominant kernel (timed live
with HIP events on the library's stream, on every EVENT_STRIDE-th timed
step), peak device memory, and the fp64 oracle timed on a bounded sample on
the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --workload decode_grpo_32   (rollout decode: its own JSON line,
                                                     effective HBM GB/s)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sink-attn fwd+bwd useful TFLOP/s and % bf16 MFMA peak at T=8192"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
NOMINAL_SCLK_GHZ = 2.4
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
WINDOW_INF = 2**31 - 1
CPU_SAMPLE_HEADS = 4
# HIP events (per-launch durations for the rooflines) are recorded on every
# EVENT_STRIDE-th timed step only: each record puts a few microseconds of GPU
# time between two kernels (with all twelve per long_8192 step on every step,
# the step measured 2.72-2.75 ms against 2.68 ms without them).
EVENT_STRIDE = 4
COPY_PROBE_BYTES = 256 * 2**20

KERNEL_SOURCES = {
    "sinkattn_fwd_bf16_d64": ["fwd_bf16.hip", "common.h", "mask_tiles.h"],
    "sinkattn_bwd_dkdv_bf16_d64": ["bwd_bf16.hip", "common.h", "mask_tiles.h"],
    "sinkattn_bwd_dq_bf16_d64": ["bwd_dq_bf16.hip", "common.h", "mask_tiles.h"],
    # the kernels of one library call, whose HBM traffic the decode and GRPO
    # lines report together
    "sinkattn_decode_call": ["decode_bf16.hip", "common.h", "mask_tiles.h"],
    "sinkattn_grpo_call": ["grpo.hip"],
}
# useful FLOP per visible pair of each kernel (d = head dim): forward QK^T and PV;
# dK/dV kernel S, dP, dV, dK; dQ kernel dQ (its recomputed S and dP are not useful work)
KERNEL_FLOP_PER_PAIR = {"sinkattn_fwd_bf16_d64": 4, "sinkattn_bwd_dkdv_bf16_d64": 8,
                        "sinkattn_bwd_dq_bf16_d64": 2}


def dq_window_kernel(seqlen: int, group: int, window: int, prefix: int) -> bool:
    """Whether the library runs its resident-tile window dQ kernel (suffix _win):
    the same test as the host launcher -- GQA groups of a multiple of 4, 32-key
    tiles (w < 1024) and at most 6 key tiles per 32-row block, i.e.
    ceil(min(p, T) / 32) + ceil(w / 32) + 1 <= 6."""
    if group % 4 or window >= 1024:
        return False
    return (min(prefix, seqlen) + 31) // 32 + (window + 31) // 32 + 1 <= 6


def kernel_variants(key_tile: int, query_tile: int, group: int = 1, win_dq: bool = False) -> dict:
    """Names of the kernels one layer launches, per timed phase, for the tile
    shapes the library reports (narrow tiles carry a suffix; the narrow
    forward takes four query heads per workgroup when the GQA group size is a
    multiple of 4, suffix _k32h; win_dq: the resident-tile window dQ kernel)."""
    if query_tile != 128:
        raise ValueError(f"no dK/dV kernel with {query_tile}-row query tiles")
    k32 = "_k32" if key_tile == 32 else ""
    fwd = "_k32h" if key_tile == 32 and group % 4 == 0 else k32
    return {"fwd_ms": "sinkattn_fwd_bf16_d64" + fwd,
            "bwd_dkdv_ms": "sinkattn_bwd_dkdv_bf16_d64",
            "bwd_dq_ms": "sinkattn_bwd_dq_bf16_d64" + ("_win" if win_dq else k32)}


def kernel_base(name: str) -> str:
    for suffix in ("_k32h", "_k32", "_win"):
        if name.endswith(suffix):
            return name[:-len(suffix)]
    return name


def visible_pairs_per_head(n: int, window: int, prefix: int) -> int:
    """Number of (q, k) pairs the mask leaves visible in one sequence of n
    tokens: row i sees min(i + 1, w + p + 1) keys."""
    c = min(window, n) + min(prefix, n) + 1
    if c >= n:
        return n * (n + 1) // 2
    return c * (c + 1) // 2 + (n - c) * c


def useful_pairs(inp) -> int:
    hq = inp.q.shape[-2]
    if inp.lengths is not None:
        per = sum(visible_pairs_per_head(n, inp.window, inp.prefix) for n in inp.lengths)
        return per * hq
    b, t = inp.q.shape[0], inp.q.shape[1]
    return b * hq * visible_pairs_per_head(t, inp.window, inp.prefix)


def kernel_source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel_base(kernel)]:
        with open(os.path.join(ROOT, "sink_aware_masked_sinkattn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def committed_traffic(kernel: str, workload: str, layer=None):
    """HBM bytes of one launch of `kernel` (on layer `layer` of an attention workload, whose
    summaries list one value per layer), from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", txt)
    key = "hbm_bytes_per_launch" + ("" if layer is None else rf"\[layer {layer}\]")
    val = re.search(key + r":\s*([0-9.eE+]+)", txt)
    if not sha or not val or sha.group(1) != kernel_source_sha(kernel):
        return None
    return float(val.group(1))


def committed_sclk(kernel: str, workload: str):
    """Shader clock (GHz) under this workload, measured for `kernel` from the SQ counters of
    the committed counter summary (SQ_BUSY_CYCLES per shader array over the kernel's time);
    the row of the kernel's longest grid. None without such a summary."""
    path = os.path.join(ROOT, "profiles", f"sq_counters_{workload}.md")
    if not os.path.exists(path):
        return None
    best = None
    for line in open(path):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) < 4 or cells[0] != kernel:
            continue
        try:
            t_us, ghz = float(cells[2]), float(cells[3])
        except ValueError:
            continue
        if best is None or t_us > best[0]:
            best = (t_us, ghz)
    return best[1] if best else None


def kernel_bytes(inp, kernel_base_name: str) -> int:
    """Algorithmic HBM bytes of one launch of a kernel on a layer: what it must read and
    write at least once.  Forward: Q, K, V in, O out (bf16), l out (fp32).  dQ kernel (with
    the row statistics): Q, K, V, dO, O in, dQ out (bf16), l in, L and D out (fp32).  dK/dV
    kernel: Q, K, V, dO in (bf16), L and D in (fp32), dK and dV out (bf16; the kernel keeps
    them in fp32 accumulators, an implementation choice, not counted)."""
    q, k = inp.q.numel(), inp.k.numel()
    rows = q // inp.q.shape[-1]               # (token, query head) rows
    if kernel_base_name == "sinkattn_fwd_bf16_d64":
        return 2 * (q + 2 * k + q) + 4 * rows
    if kernel_base_name == "sinkattn_bwd_dq_bf16_d64":
        return 2 * (4 * q + 2 * k) + 12 * rows
    if kernel_base_name == "sinkattn_bwd_dkdv_bf16_d64":
        return 2 * (2 * q + 4 * k) + 8 * rows
    raise KeyError(kernel_base_name)


def compulsory_bytes(inp) -> tuple:
    """HBM bytes the forward and the backward cannot avoid: forward reads Q, K, V and writes
    O (bf16) and l (fp32); backward reads Q, K, V, dO (bf16), L and D (fp32) and writes dQ, dK,
    dV (bf16)."""
    q, k = inp.q.numel(), inp.k.numel()
    rows = q // inp.q.shape[-1]               # (token, query head) rows
    fwd = 2 * (q + 2 * k + q) + 4 * rows
    bwd = 2 * (q + 2 * k + q) + 8 * rows + 2 * (q + 2 * k)
    return fwd, bwd


def cpu_baseline(layers, head_dim: int, min_seconds: float = 10.0):
    """The fp64 oracle as it stands, timed on a bounded sample: query heads of
    every layer in groups of CPU_SAMPLE_HEADS (each with its own kv head, forward
    + backward over the full sequence, or every packed sequence), group after
    group until at least `min_seconds` have passed (10-30 s on 16 host cores)."""
    import numpy as np  # noqa: F401
    import torch

    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max(i.get("num_threads", 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    hq = layers[0].q.shape[-2]
    group = hq // layers[0].k.shape[-2]
    flops = 0.0
    heads_done = 0
    t0 = time.perf_counter()
    while heads_done < hq and (heads_done == 0 or time.perf_counter() - t0 < min_seconds):
        heads = list(range(heads_done, min(hq, heads_done + CPU_SAMPLE_HEADS)))
        kvh = [h // group for h in heads]
        for inp in layers:
            q, do = (t[..., heads, :].to(torch.float64).numpy() for t in (inp.q, inp.do))
            k, v = (t[..., kvh, :].to(torch.float64).numpy() for t in (inp.k, inp.v))
            s = inp.sinks[heads].to(torch.float64).numpy()
            cu = inp.cu_seqlens.numpy() if inp.cu_seqlens is not None else None
            oracle.forward(q, k, v, s, inp.window, inp.prefix, inp.scale, cu_seqlens=cu)
            oracle.backward(q, k, v, s, do, inp.window, inp.prefix, inp.scale, cu_seqlens=cu)
            lens = inp.lengths if inp.lengths is not None else (inp.q.shape[1],) * inp.q.shape[0]
            flops += (14 * head_dim * len(heads) *
                      sum(visible_pairs_per_head(n, inp.window, inp.prefix) for n in lens))
        heads_done += len(heads)
    dt = time.perf_counter() - t0
    what = ("every packed sequence" if layers[0].lengths is not None
            else f"T={layers[0].q.shape[1]}")
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{heads_done} of {hq} query heads per layer ({len(layers)} "
                      f"layer(s), {what}), fwd+bwd in fp64; {dt:.1f} s",
            "seconds": round(dt, 3)}


DECODE_METRIC = "sink-attn decode: effective HBM GB/s of the visible K/V cache rows"


def decode_visible(n: int, window: int, prefix: int) -> int:
    """Keys the query at position n - 1 sees in a cache of n tokens."""
    if n <= 0:
        return 0
    return min(n, min(window, n - 1) + 1 + min(prefix, max(0, n - 1 - min(window, n - 1))))


def decode_cpu_baseline(layers, min_seconds: float = 10.0):
    """The fp64 oracle's decode over the whole workload (every sequence, both
    layers; inputs converted to fp64 beforehand), repeated until about
    `min_seconds` of CPU time."""
    import torch

    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max(i.get("num_threads", 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    prepared, step_bytes = [], 0
    for inp in layers:
        lens = inp.cache_seqlens.tolist()
        cap = max(lens)
        prepared.append((inp.q.to(torch.float64).numpy(),
                         inp.k_cache[:, :cap].to(torch.float64).numpy(),
                         inp.v_cache[:, :cap].to(torch.float64).numpy(), lens,
                         inp.sinks.to(torch.float64).numpy(), inp))
        hkv, d = inp.k_cache.shape[2], inp.k_cache.shape[3]
        step_bytes += sum(decode_visible(n, inp.window, inp.prefix) for n in lens) * hkv * d * 4
    reps = 0
    t0 = time.perf_counter()
    while True:
        for q, k, v, lens, s, inp in prepared:
            oracle.decode(q, k, v, lens, s, inp.window, inp.prefix, inp.scale)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": step_bytes * reps / dt / 1e9, "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"the whole workload (all sequences, both layers), fp64 decode, "
                      f"{reps} repetitions in {dt:.1f} s; GB/s of visible K/V rows",
            "seconds": round(dt, 3)}


def copy_probe(dev) -> None:
    """Copy a COPY_PROBE_BYTES buffer device to device three times: the
    reference that scales the hardware byte counters (FETCH_SIZE, WRITE_SIZE)
    of the same run to bytes."""
    import torch
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def run_decode(args) -> int:
    """One step = one decode call per layer of a decode workload (one new token
    for every sequence of the batch); inputs resident, outputs and workspace
    preallocated.  value = compulsory bytes (visible K/V rows, q, o, lse) of
    the step / step time."""
    import torch

    from sink_aware_masked_sinkattn_amd import (load_library, make_decode_problem,
                                                sinkattn_decode,
                                                sinkattn_decode_workspace_size)
    from workloads import DECODE_WORKLOADS, decode_workload_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    load_library()
    wl = DECODE_WORKLOADS[args.workload]
    layers = decode_workload_inputs(args.workload)
    dev = torch.device("cuda:0")
    runs = []
    for inp in layers:
        r = {"inp": inp, "q": inp.q.to(dev), "k": inp.k_cache.to(dev), "v": inp.v_cache.to(dev),
             "lens": inp.cache_seqlens.to(dev), "s": inp.sinks.to(dev)}
        r["o"] = torch.empty_like(r["q"])
        r["lse"] = torch.empty(r["q"].shape[:2], dtype=torch.float32, device=dev)
        pb = make_decode_problem(r["q"], r["k"], inp.window, inp.prefix, inp.scale)
        r["ws"] = torch.empty(max(1, sinkattn_decode_workspace_size(pb)), dtype=torch.uint8,
                              device=dev)
        vis = sum(decode_visible(n, inp.window, inp.prefix) for n in inp.cache_seqlens.tolist())
        hq, d = inp.q.shape[1], inp.q.shape[2]
        hkv = inp.k_cache.shape[2]
        r["bytes"] = vis * hkv * d * 2 * 2 + 2 * inp.q.numel() * 2 + inp.q.shape[0] * hq * 4
        r["flops"] = 4 * d * hq * vis
        runs.append(r)
    torch.cuda.synchronize()

    def step(events=None):
        for li, r in enumerate(runs):
            inp = r["inp"]
            if events:
                events[li][0].record()
            sinkattn_decode(r["q"], r["k"], r["v"], r["lens"], r["s"], inp.window, inp.prefix,
                            inp.scale, out=r["o"], lse=r["lse"], workspace=r["ws"])
            if events:
                events[li][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in runs]
              for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(events[i] if i % EVENT_STRIDE == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / K
    ev_steps = range(0, K, EVENT_STRIDE)
    per_layer = []
    for li, r in enumerate(runs):
        ms = sum(events[i][li][0].elapsed_time(events[i][li][1]) for i in ev_steps) / len(ev_steps)
        per_layer.append({"window": r["inp"].window if r["inp"].window < WINDOW_INF else "inf",
                          "prefix": r["inp"].prefix, "ms": round(ms, 5),
                          "bytes": r["bytes"], "gbs": round(r["bytes"] / (ms * 1e-3) / 1e9, 1),
                          "tflops": round(r["flops"] / (ms * 1e-3) / 1e12, 3)})
    total_bytes = sum(r["bytes"] for r in runs)
    value = total_bytes / (ms_per_step * 1e-3) / 1e9
    dom = max(range(len(runs)), key=lambda i: per_layer[i]["ms"])
    achieved = runs[dom]["bytes"] / (per_layer[dom]["ms"] * 1e-3) / 1e9
    # HBM bytes of one call of the dominant layer from the committed counter
    # summary (None if it was taken on other kernel sources)
    traffic = committed_traffic("sinkattn_decode_call", args.workload)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": "sinkattn_decode_stream_bf16_d64 + sinkattn_decode_combine_bf16_d64 "
                          f"(one sinkattn_decode call, layer {dom})",
                "avg_launch_ms": per_layer[dom]["ms"],
                "algorithmic_bytes_per_launch": runs[dom]["bytes"]}
    # every layer's call against HBM (a decode call reads each visible K/V row once)
    launches = [{"bound": "hbm", "achieved": p["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": round(p["gbs"] / PEAK_HBM_GBS, 4), "kernel": "one sinkattn_decode call",
                 "layer": li, "avg_launch_ms": p["ms"], "algorithmic_bytes_per_launch": p["bytes"]}
                for li, p in enumerate(per_layer)]
    if args.copy_probe:
        copy_probe(dev)
    cpu = None if args.no_cpu_baseline else decode_cpu_baseline(layers)
    out = {
        "metric": DECODE_METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": wl.batch, "cache_capacity": wl.capacity,
                   "cache_lengths": list(wl.lengths), "heads_q": wl.heads_q,
                   "heads_kv": wl.heads_kv, "head_dim": wl.head_dim,
                   "layers": [{"window": w if w < WINDOW_INF else "inf", "prefix": p}
                              for (w, p) in wl.layers],
                   "parallelism": "single GPU"},
        "per_layer": per_layer,
        "roofline": roofline,
        "roofline_per_launch": launches,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


GRPO_METRIC = "GRPO token loss + gradient: effective HBM GB/s of the compulsory bytes"


def grpo_bytes(inp) -> int:
    """Compulsory HBM bytes of one GRPO loss call: per token logp_new, logp_old (and logp_ref
    with a KL term) and the action mask read, the gradient written; per rollout the reward
    and the sequence offset read and the advantage written; the loss."""
    n, b = inp.logp_new.numel(), inp.rewards.numel()
    per_tok = 4 + 4 + (4 if inp.beta != 0.0 else 0) + 1 + 4
    return n * per_tok + b * (4 + 4 + 4) + 4 + 4


def grpo_cpu_baseline(inp, min_seconds: float = 10.0):
    """The fp64 oracle's GRPO loss over the whole workload, repeated until about
    `min_seconds` of CPU time."""
    import oracle
    args = (inp.logp_new.numpy(), inp.logp_old.numpy(), inp.logp_ref.numpy(),
            inp.action_mask.numpy(), inp.rewards.numpy(), inp.cu_seqlens.numpy(),
            inp.group_size, inp.eps_adv, inp.eps_clip, inp.beta, inp.kl_mode)
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.grpo_loss(*args)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": grpo_bytes(inp) * reps / dt / 1e9, "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"the whole workload ({inp.logp_new.numel()} tokens), fp64, {reps} "
                      f"repetitions in {dt:.1f} s; GB/s of the same compulsory bytes",
            "seconds": round(dt, 3)}


def run_grpo(args) -> int:
    """One step = one GRPO loss call (advantages, loss and per-token gradient) over the
    packed batch; inputs resident, outputs and workspace preallocated.  value = compulsory
    bytes / step time."""
    import torch

    from sink_aware_masked_sinkattn_amd import (load_library, make_grpo_problem,
                                                sinkattn_grpo_loss,
                                                sinkattn_grpo_workspace_size)
    from workloads import GRPO_WORKLOADS, grpo_workload_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    load_library()
    wl = GRPO_WORKLOADS[args.workload]
    inp = grpo_workload_inputs(args.workload)
    dev = torch.device("cuda:0")
    t = {k: getattr(inp, k).to(dev) for k in ("logp_new", "logp_old", "logp_ref", "action_mask",
                                              "rewards", "cu_seqlens")}
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    grad = torch.empty_like(t["logp_new"])
    adv = torch.empty_like(t["rewards"])
    pb = make_grpo_problem(inp.rewards.numel(), inp.group_size, inp.logp_new.numel(),
                           inp.eps_adv, inp.eps_clip, inp.beta, inp.kl_mode)
    ws = torch.empty(max(1, sinkattn_grpo_workspace_size(pb)), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev:
            ev[0].record()
        sinkattn_grpo_loss(t["logp_new"], t["logp_old"], t["logp_ref"], t["action_mask"],
                           t["rewards"], t["cu_seqlens"], inp.group_size, inp.eps_adv,
                           inp.eps_clip, inp.beta, inp.kl_mode, loss=loss, grad=grad,
                           advantages=adv, workspace=ws)
        if ev:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(events[i] if i % EVENT_STRIDE == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / K
    per_call = [events[i][0].elapsed_time(events[i][1]) for i in range(0, K, EVENT_STRIDE)]
    avg_ms = sum(per_call) / len(per_call)
    nbytes = grpo_bytes(inp)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    traffic = committed_traffic("sinkattn_grpo_call", args.workload)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": "grpo_rollout_stats + grpo_tokens + grpo_loss_sum "
                          "(one sinkattn_grpo_loss call)",
                "avg_launch_ms": round(avg_ms, 5), "median_call_ms":
                    round(statistics.median(per_call), 5),
                "algorithmic_bytes_per_launch": nbytes}
    launches = [dict(roofline)]   # one call, three kernels: reported together
    if args.copy_probe:
        copy_probe(dev)
    cpu = None if args.no_cpu_baseline else grpo_cpu_baseline(inp)
    out = {
        "metric": GRPO_METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "groups": wl.groups, "group_size": wl.group_size,
                   "rollout_lengths": list(wl.lengths), "tokens": inp.logp_new.numel(),
                   "optimised_tokens": int(inp.action_mask.sum()), "beta": wl.beta,
                   "kl_mode": wl.kl_mode, "eps_clip": wl.eps_clip, "parallelism": "single GPU"},
        "tokens_per_s": round(inp.logp_new.numel() / (ms_per_step * 1e-3), 1),
        "roofline": roofline,
        "roofline_per_launch": launches,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_8192")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, copy a 256 MiB buffer device-to-device 3 times: the "
                         "reference for scaling hardware byte counters (FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "the sink-attention path here is a single-GPU kernel library; multi-GPU sharding "
              "is described in the design notes but not built.", file=sys.stderr)
        return 2

    from workloads import DECODE_WORKLOADS, GRPO_WORKLOADS
    if args.workload in DECODE_WORKLOADS:
        return run_decode(args)
    if args.workload in GRPO_WORKLOADS:
        return run_grpo(args)

    import torch

    from sink_aware_masked_sinkattn_amd import (BWD_DKDV, BWD_DQ, BWD_FINISH, BWD_PREPARE,
                                                load_library, make_problem, sinkattn_bwd_phases,
                                                sinkattn_bwd_workspace_size, sinkattn_fwd,
                                                sinkattn_tile_config)
    from workloads import WORKLOADS, workload_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    load_library()
    wl = WORKLOADS[args.workload]
    layers = workload_inputs(args.workload)
    dev = torch.device("cuda:0")

    runs = []
    for inp in layers:
        r = {"inp": inp}
        r["q"], r["k"], r["v"], r["do"] = (t.to(dev) for t in (inp.q, inp.k, inp.v, inp.do))
        r["s"] = inp.sinks.to(dev)
        r["cu"] = inp.cu_seqlens.to(dev) if inp.cu_seqlens is not None else None
        r["ms"] = inp.max_seqlen if inp.cu_seqlens is not None else None
        runs.append(r)
    torch.cuda.synchronize()
    # device memory beyond the resident inputs: outputs, lse, workspace, transients
    base_alloc = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    for r in runs:
        inp = r["inp"]
        r["o"] = torch.empty_like(r["q"])
        pb = make_problem(r["q"], r["k"], inp.window, inp.prefix, inp.scale, r["cu"], r["ms"])
        lse_shape = (pb.heads_q, pb.total_tokens) if r["cu"] is not None else \
            (pb.batch, pb.heads_q, pb.seqlen)
        r["lse"] = torch.empty(lse_shape, dtype=torch.float32, device=dev)
        r["grads"] = (torch.empty_like(r["q"]), torch.empty_like(r["k"]),
                      torch.empty_like(r["v"]), torch.empty_like(r["s"]))
        r["ws"] = torch.empty(sinkattn_bwd_workspace_size(pb), dtype=torch.uint8, device=dev)
        r["pairs"] = useful_pairs(inp)
        group = pb.heads_q // pb.heads_kv
        # the library clamps w and p to the (longest) sequence length
        r["kernels"] = kernel_variants(*sinkattn_tile_config(pb), group,
                                       dq_window_kernel(pb.seqlen, group, min(inp.window, pb.seqlen),
                                                        min(inp.prefix, pb.seqlen)))
    torch.cuda.synchronize()

    def step(events=None):
        for li, r in enumerate(runs):
            inp = r["inp"]
            a = (r["q"], r["k"], r["v"], r["s"])
            ev = events[li] if events is not None else None
            if ev:
                ev[0].record()
            sinkattn_fwd(*a, inp.window, inp.prefix, inp.scale, r["cu"], r["ms"], out=r["o"],
                         lse=r["lse"])
            if ev:
                ev[1].record()
            bargs = (*a, r["o"], r["lse"], r["do"], inp.window, inp.prefix, inp.scale, r["cu"],
                     r["ms"])
            for j, ph in enumerate((BWD_PREPARE, BWD_DQ, BWD_DKDV, BWD_FINISH)):
                sinkattn_bwd_phases(ph, *bargs, workspace=r["ws"], grads=r["grads"])
                if ev:
                    ev[2 + j].record()

    step()
    torch.cuda.synchronize()
    peak_mem = torch.cuda.max_memory_allocated()
    inputs_bytes = sum(sum(t.numel() * t.element_size()
                           for t in (r["q"], r["k"], r["v"], r["do"], r["s"])) for r in runs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in runs]
              for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(events[i] if i % EVENT_STRIDE == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / K

    d = wl.head_dim
    per_layer = []
    for li, r in enumerate(runs):
        per_it = [[events[i][li][j].elapsed_time(events[i][li][j + 1]) for j in range(5)]
                  for i in range(0, K, EVENT_STRIDE)]
        ph = [sum(it[j] for it in per_it) / len(per_it) for j in range(5)]
        fwd_b, bwd_b = compulsory_bytes(r["inp"])
        per_layer.append({"window": r["inp"].window, "prefix": r["inp"].prefix,
                          "pairs": r["pairs"], "fwd_ms": ph[0], "bwd_prepare_ms": ph[1],
                          "bwd_dq_ms": ph[2], "bwd_dkdv_ms": ph[3], "bwd_finish_ms": ph[4],
                          "median_ms": {"fwd": round(statistics.median(it[0] for it in per_it), 4),
                                        "bwd": round(statistics.median(sum(it[1:]) for it in per_it), 4),
                                        "total": round(statistics.median(sum(it) for it in per_it), 4)},
                          "compulsory_gbs": {"fwd": round(fwd_b / (ph[0] * 1e-3) / 1e9, 1),
                                             "bwd": round(bwd_b / (sum(ph[1:]) * 1e-3) / 1e9, 1)}})
    total_flops = sum(14 * d * r["pairs"] for r in runs)
    value = total_flops / (ms_per_step * 1e-3) / 1e12

    # Roofline per launch: every kernel of every layer against the bound its own
    # arithmetic intensity sets (useful FLOP over algorithmic bytes, against the
    # ridge peak_flops / peak_bytes): MFMA above the ridge, HBM below.  The
    # headline roofline is the launch with the largest time per step.
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    launches = []
    for li, (p, r) in enumerate(zip(per_layer, runs)):
        p["kernels"] = r["kernels"]
        for ph, name in r["kernels"].items():
            base = kernel_base(name)
            t_s = p[ph] * 1e-3
            flop = KERNEL_FLOP_PER_PAIR[base] * d * p["pairs"]
            nbytes = kernel_bytes(r["inp"], base)
            if flop / nbytes >= ridge:
                rl = {"bound": "mfma", "achieved": round(flop / t_s / 1e12, 2),
                      "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
            else:
                rl = {"bound": "hbm", "achieved": round(nbytes / t_s / 1e9, 1),
                      "peak": PEAK_HBM_GBS, "unit": "GB/s"}
            rl["frac"] = round(rl["achieved"] / rl["peak"], 4)
            rl.update({"kernel": name, "layer": li, "avg_launch_ms": round(p[ph], 4),
                       "algorithmic_flop_per_launch": flop,
                       "algorithmic_bytes_per_launch": nbytes})
            launches.append(rl)
    dom = max(launches, key=lambda x: x["avg_launch_ms"])
    traffic = committed_traffic(dom["kernel"], args.workload, dom["layer"])
    roofline = {k: dom[k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    roofline.update({"traffic": traffic, "kernel": dom["kernel"], "layer": dom["layer"],
                     "avg_launch_ms": dom["avg_launch_ms"],
                     "algorithmic_flop_per_launch": dom["algorithmic_flop_per_launch"],
                     "algorithmic_bytes_per_launch": dom["algorithmic_bytes_per_launch"]})
    # diagnostic only: the 2516.6 TFLOP/s peak assumes 2.4 GHz; the committed SQ counter
    # summary measures the shader clock under this load, which lowers the attainable peak
    sclk = committed_sclk(dom["kernel"], args.workload)
    diagnostics = None
    if sclk:
        diagnostics = {"sclk_ghz_measured": sclk,
                       "sclk_source": f"profiles/sq_counters_{args.workload}.md",
                       "step_frac_of_peak_at_measured_sclk":
                           round(value / (PEAK_BF16_TFLOPS * sclk / NOMINAL_SCLK_GHZ), 4)}

    # the full-causal layer alone (the target configuration)
    causal = [p for p in per_layer if p["window"] >= 8192 and p["prefix"] == 0]
    causal_info = None
    if causal:
        p = causal[0]
        t_ms = (p["fwd_ms"] + p["bwd_prepare_ms"] + p["bwd_dkdv_ms"] + p["bwd_dq_ms"] +
                p["bwd_finish_ms"])
        t_bwd = t_ms - p["fwd_ms"]
        tf = 14 * d * p["pairs"] / (t_ms * 1e-3) / 1e12
        causal_info = {"ms": round(t_ms, 4), "useful_tflops": round(tf, 2),
                       "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                       "fwd_tflops": round(4 * d * p["pairs"] / (p["fwd_ms"] * 1e-3) / 1e12, 2),
                       "bwd_tflops": round(10 * d * p["pairs"] / (t_bwd * 1e-3) / 1e12, 2)}

    if args.copy_probe:
        copy_probe(dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(layers, d)

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": wl.batch, "seq_len": wl.seqlen,
                   "heads_q": wl.heads_q, "heads_kv": wl.heads_kv, "head_dim": wl.head_dim,
                   "layers": [{"window": w if w < WINDOW_INF else "inf", "prefix": p}
                              for (w, p) in wl.layers],
                   "parallelism": "single GPU"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "useful_flop_per_step": total_flops,
        "full_causal_layer": causal_info,
        "per_layer_ms": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in p.items()}
                         for p in per_layer],
        "roofline": roofline,
        "roofline_per_launch": launches,
        "cpu_baseline": cpu,
        "peak_mem_bytes": int(peak_mem - base_alloc),
        "peak_mem_including_inputs_bytes": int(peak_mem - base_alloc + inputs_bytes),
        "diagnostics": diagnostics,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
