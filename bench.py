#!/usr/bin/env python3
"""Benchmark one step of the paged-KV hot path on one MI355X.

A step is one pass of the whole hot path over one batch: the slot-mapped KV
write of the step's new tokens, then attention for every layer of the
workload (split-K decode + reduce, or the chunked-prefill kernel). Inputs are
seeded synthetic data (``synth``) already resident in HBM when timing starts.

Default workload: the Qwen3-0.6B-shaped decode step (B=4, Hq=16, Hkv=8,
D=128, bf16, 2048-token contexts with a 512-token shared prefix chain, a
2048 MiB pool). Its 26 MiB of live K/V would fit the GPU's last-level cache, so
the pool holds several independent batches ("waves", each with its own
prefix chain) and consecutive steps serve different ones; a step still
processes exactly one batch.

Prints one JSON line: the step throughput (``value``), a roofline entry for
the dominant kernel (its average launch time from HIP events recorded by the
library on the launch stream over the timed region) and the CPU oracle's rate
on a bounded sample of the same workload.

    python bench.py [--workload qwen3|mixed|hybrid|prefill|hprefill|mixedstep|tiny] [--kv bf16|fp8]
                    [--head-dim D] [--scrub] [--steps K] [--warmup W]

``--kv fp8`` runs the same workload over FP8 (E4M3) pools with per-layer
scales (quantizing write, FP8 decode/prefill); the decode byte count then
counts one byte per K/V element. ``--head-dim`` changes the workload's head
dimension (e.g. 512 for the Gemma-style hybrid decode or prefill).
``--scrub`` reads 1 GiB before every timed attention launch, so the
per-kernel times are taken with caches holding unrelated data.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "paged decode attn: KV GB/s & % HBM peak; prefill-chunk TFLOP/s & % MFMA"
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = {"decode_partial": ["decode.hip", "device.h"], "prefill": ["prefill.hip", "device.h"]}
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
DEFAULT_WAVES = {"qwen3": 16}
DEFAULT_STEPS = {"qwen3": 1000, "mixed": 200, "hybrid": 200, "prefill": 30, "hprefill": 30, "mixedstep": 100,
                 "tiny": 500}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def decode_bytes(wl, tabs, rows):
    """Algorithmic bytes of one decode step over ``rows`` (every layer):
    distinct live K/V token rows (shared prefix blocks once) + Q + O + the
    block-table entries the rows attend through."""
    esz = 2 if wl.dtype == "bf16" else 4
    kv_esz = 1 if wl.kv_dtype == "fp8" else esz
    total = 0
    for L in wl.layers:
        src = L.alias_of or L.name
        t = tabs[src]["tables"]
        seen = set()
        nblk = 0
        for b in rows:
            n = int(wl.seq_lens[b])
            lo = max(0, n - L.window) if L.window else 0
            for p in range(lo, n):
                seen.add((int(t[b][p // wl.block_size]), p % wl.block_size))
            nblk += -(-n // wl.block_size) - lo // wl.block_size
        kv = len(seen) * wl.hkv * wl.head_dim * kv_esz * 2
        qo = 2 * len(rows) * wl.hq * wl.head_dim * esz
        total += kv + qo + 4 * nblk
    return total


def decode_kv_bytes_per_layer(wl, tabs, rows):
    out = {}
    for L in wl.layers:
        out[L.name] = decode_bytes(_only(wl, L), tabs, rows)
    return out


def _only(wl, L):
    import copy

    w = copy.copy(wl)
    w.layers = [L]
    return w


def prefill_flops(wl, rows=None):
    """4 * D per (query head, visible key) pair: Q.K and P.V, multiply-adds x2,
    summed over the workload's layers (each with its own window)."""
    pairs = 0
    cu = np.concatenate([[0], np.cumsum(wl.chunk_lens)])
    for L in wl.layers:
        W = L.window
        for b in range(wl.batch):
            C = int(wl.chunk_lens[b])
            P = int(wl.seq_lens[b]) - C
            for i in range(C):
                if rows is not None and int(cu[b]) + i not in rows:
                    continue
                a = P + i
                lo = max(0, a - W + 1) if W else 0
                pairs += a + 1 - lo
    return 4.0 * wl.head_dim * wl.hq * pairs


def code_lines(text):
    """A source's code without its // comments, blank lines and indentation
    (the kernel's identity for recorded counters: editing a comment does not
    change the kernel)."""
    out = []
    for line in text.splitlines():
        code = line.split("//", 1)[0].strip()
        if code:
            out.append(code)
    return "\n".join(out)


def source_hash(kern):
    """sha256 of the code of the source files a kernel is built from."""
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kern]:
        with open(os.path.join(ROOT, "block_paged_kv_amd", "csrc", f)) as fh:
            h.update(code_lines(fh.read()).encode())
    return h.hexdigest()


def counter_traffic(kern, workload):
    """HBM bytes per launch recorded in profiles/<kern>_<workload>_hbm_counters.md
    (FETCH_SIZE and WRITE_SIZE, scaled by a copy of known size), or None when
    the file is missing or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kern}_{workload}_hbm_counters.md")  # workload: name[_dD][_fp8]
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.lstrip().startswith("- `"):
                k, v = line.split(":", 1)
                fields[k.strip(" -`")] = v.strip(" `\n")
    if fields.get("source_sha256") != source_hash(kern):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def launch_percentiles(pk, kern):
    """p10 / p50 / p90 of the kernel's per-launch durations (us) in the timed pass."""
    dur = pk.trace_durations(kern)
    if len(dur) == 0:
        return None
    return [round(float(x) * 1e3, 3) for x in np.percentile(np.asarray(dur), [10, 50, 90])]


def blas_threads():
    try:
        from threadpoolctl import threadpool_info

        return max([int(x.get("num_threads", 1)) for x in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        return 1


def cpu_baseline(wl, args):
    """Time the float64 oracle on a bounded sample of the same workload."""
    import oracle  # noqa: F401  (imported only on this leg)
    import runner
    from oracle import RefAllocator
    import synth

    tabs = synth.build_tables(RefAllocator, wl)
    pools = runner.oracle_setup(wl, tabs)
    budget = args.cpu_seconds
    if wl.kind == "decode":
        rows = list(range(wl.wave_size or wl.batch))
        sub = _subset(wl, rows)
        sub_pools = pools
        work = decode_bytes(wl, tabs, rows)
        unit, scale = "GB/s", 1e9
        sample = f"oracle decode of {len(rows)} rows (every layer), repeated"
        fn = lambda: runner.oracle_step(sub, sub_pools)  # noqa: E731
    elif wl.num_decode:
        # continuous-batching step: the oracle over the step's decode rows (the
        # metric's unit is their KV GB/s)
        rows = list(range(wl.num_decode))
        work = decode_bytes(wl, tabs, rows)
        unit, scale = "GB/s", 1e9
        sample = f"oracle over the {len(rows)} decode rows of the step (varlen prefill form), repeated"
        fn = lambda: runner.oracle_step(wl, pools, rows=rows)  # noqa: E731
    else:
        T = int(wl.chunk_lens.sum())
        rows = sorted(set(np.linspace(0, T - 1, 128).astype(int).tolist()))
        work = prefill_flops(wl, set(rows))
        unit, scale = "TFLOP/s", 1e12
        sample = f"oracle prefill of {len(rows)} query rows spread over the chunk, all heads, repeated"
        fn = lambda: runner.oracle_step(wl, pools, rows=rows)  # noqa: E731
    reps = 0
    t0 = time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget or reps >= 1000:
            break
    rate = work * reps / el / scale
    return {"value": rate, "unit": unit, "cores": blas_threads(), "kind": "oracle",
            "sample": f"{sample} {reps}x in {el:.1f} s on {len(os.sched_getaffinity(0))} host cores "
                      f"(BLAS threads {blas_threads()})"}


def copy_calibration():
    """A plain device-to-device copy of a known size, launched 5 times, so the
    HBM byte counters (FETCH_SIZE, WRITE_SIZE) of the kernels above can be
    scaled by what the same counters read for known traffic."""
    import torch

    nbytes = 256 << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}), flush=True)


def time_serial_mixed_step(pk, wl, dev, outs, ws, stream, steps):
    """ms per step of the same continuous-batching step with its two parts one
    after the other on one stream (decode rows, then the chunk rows), captured
    and replayed like the timed region: the reference for the concurrent call."""
    import torch

    import runner

    nd = wl.num_decode
    calls = []
    for L in wl.layers:
        if L.alias_of:
            continue
        d = dev[L.name]
        calls.append(pk.paged_kv_write(d["k_pool"], d["v_pool"], d["step_k"], d["step_v"], d["step_slots"],
                                       stream=stream, prepare=True))
    for L in wl.layers:
        d = dev[L.name]
        o = outs[L.name]
        calls.append(pk.paged_attn_decode(o[:nd], d["q"][:nd], d["k_pool"], d["v_pool"], d["tables"][:nd],
                                          dev["_seq_lens"][:nd], wl.scale, runner.decode_max_seq_len(wl),
                                          sliding_window=L.window, partition_tokens=wl.partition_tokens,
                                          workspace=ws, stream=stream, prepare=True))
        calls.append(pk.paged_attn_prefill_chunk(o, d["q"], d["k_pool"], d["v_pool"], d["tables"][nd:],
                                                 dev["_cu_q"][nd:], dev["_seq_lens"][nd:],
                                                 int(wl.chunk_lens.max()), wl.scale, sliding_window=L.window,
                                                 stream=stream, prepare=True))
    with torch.cuda.stream(stream):
        for c in calls:
            c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(steps):
            for c in calls:
                c()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def _subset(wl, rows):
    import copy

    sub = copy.copy(wl)
    sub.batch = len(rows)
    sub.seq_lens = wl.seq_lens[rows]
    sub.tokens = [wl.tokens[r] for r in rows]
    sub.layers = []
    for L in wl.layers:
        L2 = copy.copy(L)
        L2.q = L.q[rows]
        sub.layers.append(L2)
    return sub


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3", choices=["qwen3", "mixed", "hybrid", "prefill", "hprefill", "mixedstep", "tiny"])
    ap.add_argument("--waves", type=int, default=None, help="independent batches rotated through")
    ap.add_argument("--kv", default="bf16", choices=["bf16", "fp8"], help="KV pool element type")
    ap.add_argument("--head-dim", type=int, default=None, help="head_dim override (e.g. 512 for the hybrid decode)")
    ap.add_argument("--partition-tokens", type=int, default=None,
                    help="decode split-K partition size (default: the workload's, else the library rule)")
    ap.add_argument("--scrub", action="store_true",
                    help="read a 1 GiB buffer before every attention launch of the per-kernel timing pass, "
                         "so the roofline is taken with cold caches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (scales HBM byte counters)")
    args = ap.parse_args()

    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; a multi-GPU run is not available "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_paged_kv_amd as pk
    import runner
    import synth

    steps = args.steps or DEFAULT_STEPS[args.workload]
    waves = args.waves or DEFAULT_WAVES.get(args.workload, 1)
    kw = {"waves": waves} if args.workload == "qwen3" else {}
    if args.kv == "fp8":
        if args.workload == "tiny":
            print("bench.py: --kv fp8 needs a bf16 workload (not tiny)", file=sys.stderr)
            sys.exit(2)
        kw["kv_dtype"] = "fp8"
    fp8 = args.kv == "fp8"
    if args.head_dim:
        kw["head_dim"] = args.head_dim
    if args.partition_tokens is not None:
        kw["part"] = args.partition_tokens
    log(f"[bench] building workload {args.workload} ({kw})")
    wl = synth.make(args.workload, **kw)
    R = waves if args.workload == "qwen3" else 1
    mixed_step = wl.kind == "prefill" and wl.num_decode > 0
    wsz = wl.wave_size or wl.batch
    tabs = synth.build_tables(pk.Allocator, wl)
    log("[bench] writing cached context to device pools")
    dev = runner.gpu_setup(wl, tabs, fill=0.0)
    torch.cuda.synchronize()

    # Prepared calls for every step variant (one per wave), bound to a stream
    # of our own so they can be captured into a graph.
    stream = torch.cuda.Stream()
    calls = []
    if wl.kind == "decode":
        outs = {L.name: torch.empty((wsz,) + tuple(dev[L.name]["q"].shape[1:]), dtype=dev[L.name]["q"].dtype,
                                    device="cuda") for L in wl.layers}
    else:
        outs = {L.name: torch.empty_like(dev[L.name]["q"]) for L in wl.layers}
    ws = runner.gpu_workspace(_subset(wl, list(range(wsz))) if R > 1 else wl, dev)
    for r in range(R):
        rows = slice(r * wsz, (r + 1) * wsz)
        seq = []
        for L in wl.layers:
            if L.alias_of:
                continue
            d = dev[L.name]
            nt = wl.new_tokens
            t0 = sum(nt[:r * wsz])
            t1 = sum(nt[:(r + 1) * wsz])
            if fp8:
                seq.append(pk.paged_kv_write_fp8(d["k_pool"], d["v_pool"], d["step_k"][t0:t1],
                                                 d["step_v"][t0:t1], d["step_slots"][t0:t1], L.k_scale,
                                                 L.v_scale, stream=stream, prepare=True))
            else:
                seq.append(pk.paged_kv_write(d["k_pool"], d["v_pool"], d["step_k"][t0:t1],
                                             d["step_v"][t0:t1], d["step_slots"][t0:t1], stream=stream,
                                             prepare=True))
        for L in wl.layers:
            d = dev[L.name]
            if mixed_step:
                seq.append(pk.paged_attn_mixed(
                    outs[L.name], d["q"], d["k_pool"], d["v_pool"], d["tables"], dev["_cu_q"], dev["_seq_lens"],
                    wl.num_decode, int(wl.chunk_lens.max()), wl.scale, runner.decode_max_seq_len(wl),
                    sliding_window=L.window, partition_tokens=wl.partition_tokens, workspace=ws,
                    k_scale=L.k_scale, v_scale=L.v_scale, stream=stream, prepare=True))
            elif wl.kind == "decode" and fp8:
                seq.append(pk.paged_attn_decode_fp8(
                    outs[L.name], d["q"][rows], d["k_pool"], d["v_pool"], d["tables"][rows],
                    dev["_seq_lens"][rows], wl.scale, L.k_scale, L.v_scale, int(wl.seq_lens[rows].max()),
                    sliding_window=L.window, partition_tokens=wl.partition_tokens, workspace=ws,
                    stream=stream, prepare=True))
            elif wl.kind == "decode":
                seq.append(pk.paged_attn_decode(
                    outs[L.name], d["q"][rows], d["k_pool"], d["v_pool"], d["tables"][rows],
                    dev["_seq_lens"][rows], wl.scale, int(wl.seq_lens[rows].max()),
                    sliding_window=L.window, partition_tokens=wl.partition_tokens, workspace=ws,
                    stream=stream, prepare=True))
            elif fp8:
                seq.append(pk.paged_attn_prefill_chunk_fp8(
                    outs[L.name], d["q"], d["k_pool"], d["v_pool"], d["tables"], dev["_cu_q"],
                    dev["_seq_lens"], int(wl.chunk_lens.max()), wl.scale, L.k_scale, L.v_scale,
                    sliding_window=L.window, stream=stream, prepare=True))
            else:
                seq.append(pk.paged_attn_prefill_chunk(
                    outs[L.name], d["q"], d["k_pool"], d["v_pool"], d["tables"], dev["_cu_q"],
                    dev["_seq_lens"], int(wl.chunk_lens.max()), wl.scale, sliding_window=L.window,
                    stream=stream, prepare=True))
        calls.append(seq)

    def step(i):
        for c in calls[i % R]:
            c()

    stream.wait_stream(torch.cuda.current_stream())
    log(f"[bench] warmup {args.warmup} steps")
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()

    # Timed region 1 (throughput): `steps` consecutive steps captured as one
    # HIP graph, so host launch overhead is not part of a step. Falls back to
    # eager launches if capture is not possible.
    timing = "graph"
    graph = None
    if not args.eager:
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                for i in range(steps):
                    step(args.warmup + i)
            graph.replay()  # warm replay: instantiation and first-touch costs
            torch.cuda.synchronize()
        except Exception as e:  # noqa: BLE001
            log(f"[bench] graph capture failed ({e}); timing eager launches")
            graph = None
            timing = "eager"
    log(f"[bench] timing {steps} steps ({timing})")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        with torch.cuda.stream(stream):
            for i in range(steps):
                step(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps

    # Timed region 2 (per-kernel durations): the same steps launched eagerly,
    # the library recording a HIP event pair around every launch on the launch
    # stream (events inside a captured graph cannot be timed).
    log(f"[bench] per-kernel timing over {steps} eager steps{' (caches scrubbed)' if args.scrub else ''}")
    if args.scrub:
        # A read leaves the caches holding clean, unrelated lines (a write
        # would leave dirty ones whose write-back the next kernel would pay).
        scrub_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        sink = torch.zeros((), dtype=torch.float32, device="cuda")
    n_writes = sum(1 for L in wl.layers if not L.alias_of)
    pk.trace_reset()
    torch.cuda.synchronize()
    pk.trace_enable(True)
    with torch.cuda.stream(stream):
        for i in range(steps):
            for j, c in enumerate(calls[(args.warmup + i) % R]):
                if args.scrub and j >= n_writes:
                    pk.trace_enable(False)
                    sink.copy_(scrub_buf.sum())
                    pk.trace_enable(True)
                c()
    torch.cuda.synchronize()
    pk.trace_enable(False)

    extra = {}
    if mixed_step:
        # Decode rows' KV bytes over the step time is the value; the chunk's
        # prefill carries the dominant kernel's roofline, the decode partial a
        # second one (both timed while they share the device).
        dec_rows = list(range(wl.num_decode))
        T = int(wl.chunk_lens.sum())
        dwork = decode_bytes(wl, tabs, dec_rows)
        pwork = prefill_flops(wl, set(range(wl.num_decode, T)))
        value = dwork / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        kern = "prefill"
        k_ms, k_n = pk.trace_query(kern)
        work = pwork
        achieved = pwork * steps / (k_ms * 1e-3) / 1e12
        peak, bound, runit = MFMA_BF16_PEAK_TFLOPS, "mfma", "TFLOP/s"
        d_ms, d_n = pk.trace_query("decode_partial")
        d_ach = dwork * steps / (d_ms * 1e-3) / 1e9
        serial_ms = time_serial_mixed_step(pk, wl, dev, outs, ws, stream, steps)
        extra = {
            "roofline_decode": {"kernel": "decode_partial", "bound": "hbm", "achieved": round(d_ach, 3),
                                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(d_ach / HBM_PEAK_GBS, 4),
                                "avg_launch_us": round(d_ms * 1e3 / max(d_n, 1), 3), "work_per_step": dwork},
            "prefill_tflops_in_step": round(pwork / (ms_per_step * 1e-3) / 1e12, 3),
            "serial_ms_per_step": round(serial_ms, 6),
            "speedup_vs_serial": round(serial_ms / ms_per_step, 4),
        }
    elif wl.kind == "decode":
        per_wave = [decode_bytes(wl, tabs, list(range(r * wsz, (r + 1) * wsz))) for r in range(R)]
        work = float(np.mean([per_wave[(args.warmup + i) % R] for i in range(steps)]))
        value = work / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        kern = "decode_partial"
        k_ms, k_n = pk.trace_query(kern)
        achieved = work * steps / (k_ms * 1e-3) / 1e9  # all partial launches of the region
        peak, bound, runit = HBM_PEAK_GBS, "hbm", "GB/s"
    else:
        work = prefill_flops(wl)
        value = work / (ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        kern = "prefill"
        k_ms, k_n = pk.trace_query(kern)
        achieved = work * steps / (k_ms * 1e-3) / 1e12
        peak, bound, runit = MFMA_BF16_PEAK_TFLOPS, "mfma", "TFLOP/s"
    kernels = {}
    for name in pk.KERNELS:
        ms, n = pk.trace_query(name)
        if n:
            kernels[name] = {"launches": n, "avg_us": round(ms * 1e3 / n, 3)}
    if len(wl.layers) > 1:
        # attention launches cycle through the layers in order within a step
        dur = pk.trace_durations(kern)
        kernels[f"{kern}_by_layer_avg_us"] = {
            L.name: round(float(np.mean(dur[i::len(wl.layers)])) * 1e3, 3) for i, L in enumerate(wl.layers)}
    log(f"[bench] kernels: {kernels}")

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": {"qwen3": "qwen3-0.6b-shaped decode step", "mixed": "mixed-length continuous-batching decode",
                         "hybrid": "gemma-style hybrid sliding/full/kv-shared decode",
                         "prefill": "chunked prefill over cached prefix",
                         "hprefill": "gemma-style hybrid sliding/full/kv-shared chunked prefill",
                         "mixedstep": "continuous-batching step: decode rows + a prefill chunk in one call",
                         "tiny": "tiny fp32 decode"}[args.workload],
            "batch": int(wsz), "num_q_heads": wl.hq, "num_kv_heads": wl.hkv, "head_dim": wl.head_dim,
            "block_size": wl.block_size, "max_seq_len": wl.max_seq_len,
            "layers": [L.name for L in wl.layers], "waves_rotated": R,
            "pool_blocks": [L.num_blocks for L in wl.layers if not L.alias_of],
            "kv_dtype": "fp8_e4m3" if fp8 else wl.dtype,
        },
        "roofline": {
            "kernel": kern,
            "bound": bound,
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": runit,
            "frac": round(achieved / peak, 4),
            "traffic": counter_traffic(kern, args.workload + (f"_d{args.head_dim}" if args.head_dim else "")
                                       + ("_fp8" if fp8 else "")),
            "avg_launch_us": round(k_ms * 1e3 / max(k_n, 1), 3),
            "launch_us_p10_p50_p90": launch_percentiles(pk, kern),
            "launches": k_n,
            "work_per_step": work,
        },
        "kernels": kernels,
        "timing": timing,
        "kernel_timing_caches": "scrubbed (1 GiB read before each attention launch)" if args.scrub else "warm",
    }
    result.update(extra)
    if mixed_step:
        result["config"]["decode_rows"] = wl.num_decode
        result["config"]["chunk_tokens"] = [int(c) for c in wl.chunk_lens[wl.num_decode:]]
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(wl, args)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
