#!/usr/bin/env python3
"""Benchmark the paged-KV hot path on one MI355X.

A step is one pass of the whole hot path over one batch: the slot-mapped KV
write of the step's new tokens, then attention for every layer of the
workload (split-K decode + reduce, or the chunked-prefill kernel). Inputs are
seeded synthetic data (``synth``) already resident in HBM when timing starts.

Default (``--workload headline``): the two halves of the metric in one line.
  * Decode: the Gemma-style hybrid step (B=8, Hq=8, Hkv=1, head_dim 256, bf16,
    32768-token rows; a sliding layer with W=512 and its own pool, a full layer,
    a KV-shared layer reading the full layer's pool), the largest decode
    configuration. ``value`` is its step throughput (algorithmic bytes per
    step time) and ``roofline`` its decode kernels (partial + reduce).
  * Prefill: the 2048-token chunk over a 63488-token paged prefix (Hq=32,
    Hkv=8, head_dim 128), reported as ``roofline_prefill``.
Other workloads run alone with ``--workload NAME``.

Kernel times come from HIP events the library records around each launch on
the launch stream (``paged_trace_*``), over at least 50 steps launched eagerly
with a 1 GiB read before every attention launch, so the caches hold unrelated
data (``--warm`` drops the scrub); the same steps back to back without it are
reported as ``roofline_warm``. The step throughput times K steps captured as
one HIP graph. ``cpu_baseline`` times the float64 oracle on a bounded sample.

    python bench.py [--workload headline|qwen3|mixed|hybrid|prefill|hprefill|mixedstep|tiny]
                    [--kv bf16|fp8] [--head-dim D] [--partition-tokens P] [--warm]
                    [--shard N] [--steps K] [--warmup W]

``--kv fp8`` runs the same workload over FP8 (E4M3) pools with per-layer
scales (quantizing write, FP8 decode/prefill); the decode byte count then
counts one byte per K/V element. ``--head-dim`` changes the workload's head
dimension (e.g. 512 for the Gemma-style hybrid decode or prefill).
``--shard N`` times one GPU's share of an N-GPU run of the workload (its KV
heads split N ways when they divide, else its rows) on this one GPU; the line
then reports that GPU's throughput on its share.
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
KERNEL_SOURCES = {"decode_partial": ["decode.hip", "device.h"], "decode_reduce": ["decode.hip", "device.h"],
                  "prefill": ["prefill.hip", "device.h"]}
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
DEFAULT_WAVES = {"qwen3": 16}
DEFAULT_STEPS = {"qwen3": 1000, "mixed": 200, "hybrid": 200, "prefill": 30, "hprefill": 30, "mixedstep": 100,
                 "tiny": 500}
MIN_KERNEL_STEPS = 50           # eager steps of each per-kernel timing pass
WORKLOAD_TITLES = {
    "qwen3": "qwen3-0.6b-shaped decode step (B=4, Hq=16, Hkv=8, D=128, 2048-token rows, 512-token shared prefix)",
    "mixed": "mixed-length continuous-batching decode (B=32, Hq=32, Hkv=8, D=128, rows U[128, 8192], 4 prefixes)",
    "hybrid": "gemma-style hybrid decode: sliding (W=512) + full + kv-shared layers "
              "(B=8, Hq=8, Hkv=1, D=256, 32768-token rows)",
    "prefill": "chunked prefill: a 2048-token chunk over a 63488-token paged prefix (Hq=32, Hkv=8, D=128)",
    "hprefill": "gemma-style hybrid chunked prefill: sliding + full + kv-shared layers",
    "mixedstep": "continuous-batching step: decode rows + a prefill chunk in one call",
    "tiny": "tiny fp32 decode",
}


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
    fp8 = wl.kv_dtype == "fp8"
    calls = []
    for L in wl.layers:
        if L.alias_of:
            continue
        d = dev[L.name]
        if fp8:
            calls.append(pk.paged_kv_write_fp8(d["k_pool"], d["v_pool"], d["step_k"], d["step_v"], d["step_slots"],
                                               L.k_scale, L.v_scale, stream=stream, prepare=True))
        else:
            calls.append(pk.paged_kv_write(d["k_pool"], d["v_pool"], d["step_k"], d["step_v"], d["step_slots"],
                                           stream=stream, prepare=True))
    for L in wl.layers:
        d = dev[L.name]
        o = outs[L.name]
        msl = runner.decode_max_seq_len(wl)
        chunk = int(wl.chunk_lens.max())
        if fp8:
            calls.append(pk.paged_attn_decode_fp8(o[:nd], d["q"][:nd], d["k_pool"], d["v_pool"], d["tables"][:nd],
                                                  dev["_seq_lens"][:nd], wl.scale, L.k_scale, L.v_scale, msl,
                                                  sliding_window=L.window, partition_tokens=wl.partition_tokens,
                                                  workspace=ws, stream=stream, prepare=True))
            calls.append(pk.paged_attn_prefill_chunk_fp8(o, d["q"], d["k_pool"], d["v_pool"], d["tables"][nd:],
                                                         dev["_cu_q"][nd:], dev["_seq_lens"][nd:], chunk, wl.scale,
                                                         L.k_scale, L.v_scale, sliding_window=L.window,
                                                         stream=stream, prepare=True))
        else:
            calls.append(pk.paged_attn_decode(o[:nd], d["q"][:nd], d["k_pool"], d["v_pool"], d["tables"][:nd],
                                              dev["_seq_lens"][:nd], wl.scale, msl, sliding_window=L.window,
                                              partition_tokens=wl.partition_tokens, workspace=ws, stream=stream,
                                              prepare=True))
            calls.append(pk.paged_attn_prefill_chunk(o, d["q"], d["k_pool"], d["v_pool"], d["tables"][nd:],
                                                     dev["_cu_q"][nd:], dev["_seq_lens"][nd:], chunk, wl.scale,
                                                     sliding_window=L.window, stream=stream, prepare=True))
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


def counter_traffic_step(kern_counts, tag):
    """HBM bytes of one step's launches of the given kernels ({kernel: launches
    per step}) from the recorded counters, or None if any is missing or stale."""
    tot = 0
    for kern, n in kern_counts.items():
        t = counter_traffic(kern, tag)
        if t is None:
            return None
        tot += t * n
    return tot


def timed_pass(pk, stream, calls, first, steps, n_writes, scrub):
    """Launch ``steps`` steps eagerly with the library's launch events on;
    with ``scrub``, read 1 GiB before every attention launch (a read leaves
    the caches holding clean, unrelated lines; a write would leave dirty ones
    whose write-back the next kernel would pay). Returns {kernel: [ms, ...]}."""
    import torch

    R = len(calls)
    if scrub:
        scrub_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        sink = torch.zeros((), dtype=torch.float32, device="cuda")
    pk.trace_reset()
    torch.cuda.synchronize()
    pk.trace_enable(True)
    with torch.cuda.stream(stream):
        for i in range(steps):
            for j, c in enumerate(calls[(first + i) % R]):
                if scrub and j >= n_writes:
                    pk.trace_enable(False)
                    sink.copy_(scrub_buf.sum())
                    pk.trace_enable(True)
                c()
    torch.cuda.synchronize()
    pk.trace_enable(False)
    return {k: list(pk.trace_durations(k)) for k in pk.KERNELS}


def _pcts(ms):
    if not ms:
        return None
    return [round(float(x) * 1e3, 3) for x in np.percentile(np.asarray(ms), [10, 50, 90])]


def roofline_entry(kernels, durations, steps, work_per_step, bound, traffic=None, extra=None):
    """Roofline of the kernels named in ``kernels`` taken together: their
    summed launch durations per step against the step's algorithmic work."""
    total_ms = sum(sum(durations.get(k, [])) for k in kernels)
    per_step_ms = total_ms / max(steps, 1)
    if bound == "hbm":
        achieved = work_per_step / (per_step_ms * 1e-3) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
    else:
        achieved = work_per_step / (per_step_ms * 1e-3) / 1e12
        peak, unit = MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    e = {"kernel": "+".join(kernels), "bound": bound, "achieved": round(achieved, 3), "peak": peak,
         "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic,
         "kernel_us_per_step": round(per_step_ms * 1e3, 3),
         "avg_launch_us": {k: round(float(np.mean(durations[k])) * 1e3, 3) for k in kernels if durations.get(k)},
         "launch_us_p10_p50_p90": {k: _pcts(durations.get(k)) for k in kernels if durations.get(k)},
         "launches": {k: len(durations.get(k, [])) for k in kernels},
         "work_per_step": work_per_step}
    if extra:
        e.update(extra)
    return e


# (rows, query heads, KV heads) of each workload at its full size.
FULL_SHAPES = {"tiny": (2, 4, 2), "qwen3": (4, 16, 8), "mixed": (32, 32, 8), "hybrid": (8, 8, 1),
               "prefill": (1, 32, 8), "hprefill": (4, 8, 1), "mixedstep": (32, 32, 8)}


def shard_overrides(name, n):
    """Shape overrides for one GPU's share of an n-GPU run, and how it splits:
    the KV heads n ways when they divide (each GPU holds Hkv/n heads of every
    pool and the matching query heads; nothing is exchanged inside attention),
    else the rows (each GPU owns its requests' pools and tables)."""
    if n <= 1:
        return {}, None
    B, hq, hkv = FULL_SHAPES[name]
    if hkv % n == 0:
        return {"hq": hq // n, "hkv": hkv // n}, "kv_heads"
    if B % n == 0:
        return {"batch": B // n}, "rows"
    print(f"bench.py: {name} splits neither its {hkv} KV heads nor its {B} rows {n} ways", file=sys.stderr)
    sys.exit(2)


def run_part(pk, args, name, steps, warmup):
    """Build workload ``name``, time its steps (graph) and its kernels (eager,
    scrubbed and warm); return the fields of a bench line for it."""
    import torch

    import runner
    import synth

    waves = args.waves or DEFAULT_WAVES.get(name, 1)
    kw = {"waves": waves} if name == "qwen3" else {}
    fp8 = args.kv == "fp8"
    if fp8:
        if name == "tiny":
            print("bench.py: --kv fp8 needs a bf16 workload (not tiny)", file=sys.stderr)
            sys.exit(2)
        kw["kv_dtype"] = "fp8"
    if args.head_dim:
        kw["head_dim"] = args.head_dim
    if args.partition_tokens is not None:
        kw["part"] = args.partition_tokens
    shard_kw, shard_split = shard_overrides(name, args.shard)
    kw.update(shard_kw)
    log(f"[bench] building workload {name} ({kw})")
    wl = synth.make(name, **kw)
    R = waves if name == "qwen3" else 1
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
    # The prefill's key-split workspace (None when the library does not split
    # these shapes on this device: query tiles enough to fill it).
    pws = runner.prefill_workspace(wl) if wl.kind == "prefill" and not mixed_step else None
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
                    sliding_window=L.window, workspace=pws, stream=stream, prepare=True))
            else:
                seq.append(pk.paged_attn_prefill_chunk(
                    outs[L.name], d["q"], d["k_pool"], d["v_pool"], d["tables"], dev["_cu_q"],
                    dev["_seq_lens"], int(wl.chunk_lens.max()), wl.scale, sliding_window=L.window,
                    workspace=pws, stream=stream, prepare=True))
        calls.append(seq)

    def step(i):
        for c in calls[i % R]:
            c()

    stream.wait_stream(torch.cuda.current_stream())
    log(f"[bench] {name}: warmup {warmup} steps")
    with torch.cuda.stream(stream):
        for i in range(warmup):
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
                    step(warmup + i)
            graph.replay()  # warm replay: instantiation and first-touch costs
            torch.cuda.synchronize()
        except Exception as e:  # noqa: BLE001
            log(f"[bench] graph capture failed ({e}); timing eager launches")
            graph = None
            timing = "eager"
    log(f"[bench] {name}: timing {steps} steps ({timing})")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        with torch.cuda.stream(stream):
            for i in range(steps):
                step(warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    del graph

    # Timed regions 2 and 3 (per-kernel durations): the same steps launched
    # eagerly, first with the caches scrubbed before every attention launch,
    # then back to back (warm).
    ksteps = max(steps, MIN_KERNEL_STEPS)
    n_writes = sum(1 for L in wl.layers if not L.alias_of)
    log(f"[bench] {name}: per-kernel timing over {ksteps} eager steps, scrubbed"
        + ("" if args.warm else " and warm"))
    dur_cold = timed_pass(pk, stream, calls, warmup, ksteps, n_writes, scrub=not args.warm)
    dur_warm = dur_cold if args.warm else timed_pass(pk, stream, calls, warmup, ksteps, n_writes, scrub=False)
    caches = "warm (back to back)" if args.warm else "scrubbed (1 GiB read before each attention launch)"

    tag = (name + (f"_d{args.head_dim}" if args.head_dim else "") + ("_fp8" if fp8 else "")
           + (f"_shard{args.shard}" if shard_split else ""))
    nl = len(wl.layers)
    part = {"name": name, "wl": wl, "tabs": tabs, "ms_per_step": ms_per_step, "timing": timing,
            "ksteps": ksteps, "caches": caches}
    extra = {}
    if mixed_step:
        dec_rows = list(range(wl.num_decode))
        T = int(wl.chunk_lens.sum())
        dwork = decode_bytes(wl, tabs, dec_rows)
        pwork = prefill_flops(wl, set(range(wl.num_decode, T)))
        part["value"], part["unit"] = dwork / (ms_per_step * 1e-3) / 1e9, "GB/s"
        part["roofline"] = roofline_entry(["prefill"], dur_cold, ksteps, pwork, "mfma",
                                          counter_traffic_step({"prefill": nl}, tag))
        part["roofline_warm"] = roofline_entry(["prefill"], dur_warm, ksteps, pwork, "mfma")
        serial_ms = time_serial_mixed_step(pk, wl, dev, outs, ws, stream, steps)
        extra = {
            "roofline_decode": roofline_entry(["decode_partial", "decode_reduce"], dur_cold, ksteps, dwork, "hbm"),
            "prefill_tflops_in_step": round(pwork / (ms_per_step * 1e-3) / 1e12, 3),
            "serial_ms_per_step": round(serial_ms, 6),
            "speedup_vs_serial": round(serial_ms / ms_per_step, 4),
        }
    elif wl.kind == "decode":
        per_wave = [decode_bytes(wl, tabs, list(range(r * wsz, (r + 1) * wsz))) for r in range(R)]
        work = float(np.mean([per_wave[(warmup + i) % R] for i in range(ksteps)]))
        step_work = float(np.mean([per_wave[(warmup + i) % R] for i in range(steps)]))
        part["value"], part["unit"] = step_work / (ms_per_step * 1e-3) / 1e9, "GB/s"
        n_red = len(dur_cold.get("decode_reduce", [])) // max(ksteps, 1)
        kerns = ["decode_partial", "decode_reduce"] if n_red else ["decode_partial"]
        traffic = counter_traffic_step({"decode_partial": nl, **({"decode_reduce": n_red} if n_red else {})}, tag)
        part["roofline"] = roofline_entry(kerns, dur_cold, ksteps, work, "hbm", traffic,
                                          {"traffic_per": "step"})
        part["roofline_partial_only"] = roofline_entry(["decode_partial"], dur_cold, ksteps, work, "hbm")
        part["roofline_warm"] = roofline_entry(kerns, dur_warm, ksteps, work, "hbm")
        if nl > 1:
            by = {}
            for k in kerns:
                dd = dur_cold.get(k, [])
                per = len(dd) // max(ksteps, 1)
                if per == nl:  # one launch per layer and step, in layer order
                    by[k] = {L.name: round(float(np.mean(dd[i::nl])) * 1e3, 3) for i, L in enumerate(wl.layers)}
            extra["kernel_us_by_layer"] = by
            extra["work_by_layer"] = decode_kv_bytes_per_layer(wl, tabs, list(range(wsz)))
    else:
        work = prefill_flops(wl)
        part["value"], part["unit"] = work / (ms_per_step * 1e-3) / 1e12, "TFLOP/s"
        # With a key split the prefill's time is its two kernels together.
        pk_names = ["prefill", "prefill_reduce"] if dur_cold.get("prefill_reduce") else ["prefill"]
        traffic = counter_traffic_step({"prefill": nl}, tag) if len(pk_names) == 1 else None
        part["roofline"] = roofline_entry(pk_names, dur_cold, ksteps, work, "mfma", traffic, {"traffic_per": "step"})
        part["roofline_warm"] = roofline_entry(pk_names, dur_warm, ksteps, work, "mfma")
        if nl > 1:
            dd = dur_cold.get("prefill", [])
            extra["kernel_us_by_layer"] = {"prefill": {L.name: round(float(np.mean(dd[i::nl])) * 1e3, 3)
                                                       for i, L in enumerate(wl.layers)}}
    part["kernels"] = {k: {"launches": len(v), "avg_us": round(float(np.mean(v)) * 1e3, 3)}
                       for k, v in dur_cold.items() if v}
    part["extra"] = extra
    part["config"] = {
        "workload": WORKLOAD_TITLES[name] + (f", head_dim {args.head_dim}" if args.head_dim else ""),
        "batch": int(wsz), "num_q_heads": wl.hq, "num_kv_heads": wl.hkv, "head_dim": wl.head_dim,
        "block_size": wl.block_size, "max_seq_len": wl.max_seq_len,
        "layers": [L.name for L in wl.layers], "waves_rotated": R,
        "pool_blocks": [L.num_blocks for L in wl.layers if not L.alias_of],
        "kv_dtype": "fp8_e4m3" if fp8 else wl.dtype,
    }
    if shard_split:
        part["config"]["shard"] = {"of_gpus": args.shard, "split": shard_split}
    if mixed_step:
        part["config"]["decode_rows"] = wl.num_decode
        part["config"]["chunk_tokens"] = [int(c) for c in wl.chunk_lens[wl.num_decode:]]
    log(f"[bench] {name}: step {ms_per_step * 1e3:.1f} us, kernels {part['kernels']}")
    del dev, outs, ws, calls
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return part


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="headline",
                    choices=["headline", "qwen3", "mixed", "hybrid", "prefill", "hprefill", "mixedstep", "tiny"])
    ap.add_argument("--waves", type=int, default=None, help="independent batches rotated through")
    ap.add_argument("--kv", default="bf16", choices=["bf16", "fp8"], help="KV pool element type")
    ap.add_argument("--head-dim", type=int, default=None, help="head_dim override (e.g. 512 for the hybrid decode)")
    ap.add_argument("--partition-tokens", type=int, default=None,
                    help="decode split-K partition size (default: the workload's, else the library rule)")
    ap.add_argument("--shard", type=int, default=1,
                    help="time one GPU's share of an N-GPU run (KV heads split N ways when they divide, else rows)")
    ap.add_argument("--warm", action="store_true",
                    help="time kernels back to back only (no 1 GiB read before each attention launch)")
    ap.add_argument("--scrub", action="store_true", help="(default; kept for older command lines)")
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

    import torch  # noqa: F401

    import block_paged_kv_amd as pk

    headline = args.workload == "headline"
    first = "hybrid" if headline else args.workload
    steps = args.steps or DEFAULT_STEPS[first]
    p = run_part(pk, args, first, steps, args.warmup)
    result = {
        "metric": METRIC,
        "value": round(p["value"], 3),
        "unit": p["unit"],
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(p["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p["wl"].dtype,
        "data": "synthetic",
        "config": p["config"],
        "roofline": p["roofline"],
    }
    for k in ("roofline_partial_only", "roofline_warm"):
        if k in p:
            result[k] = p[k]
    result.update(p["extra"])
    result["kernels"] = p["kernels"]
    result["timing"] = p["timing"]
    result["kernel_timing"] = f"{p['ksteps']} eager steps, caches {p['caches']}"
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(p["wl"], args)
    del p
    if headline:
        # The metric's second half on the same line: the chunked prefill.
        q = run_part(pk, args, "prefill", args.steps or DEFAULT_STEPS["prefill"], args.warmup)
        result["prefill"] = {"value": round(q["value"], 3), "unit": q["unit"],
                             "ms_per_step": round(q["ms_per_step"], 6), "config": q["config"]}
        result["roofline_prefill"] = q["roofline"]
        result["roofline_prefill_warm"] = q["roofline_warm"]
        result["kernels_prefill"] = q["kernels"]
        if not args.no_cpu_baseline:
            log("[bench] timing the CPU oracle on a bounded prefill sample")
            result["cpu_baseline_prefill"] = cpu_baseline(q["wl"], args)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
