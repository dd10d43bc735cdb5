"""Run synthetic workloads through the library (GPU side) and the oracle (CPU side).

Two separate halves that share only ``synth``'s inputs:

* ``gpu_*`` -- allocate device pools with torch, write the cached context with
  ``paged_kv_write`` (untimed set-up), then run one step of the hot path: the
  step's KV write followed by decode (every layer) or the prefill chunk.
* ``oracle_*`` -- build float32 pools with ``oracle.kv_write`` from the
  reference allocator's slot mappings and run ``oracle.decode`` /
  ``oracle.prefill_chunk`` in float64.

Used by the tests, the smoke check and the benchmark. Nothing here is part of
the library; the library never imports this module.
"""

from __future__ import annotations

import os
import sys

import numpy as np

import synth

VERBOSE = os.environ.get("PAGEDKV_VERBOSE", "0") == "1"


def say(msg):
    if VERBOSE:
        print(msg, file=sys.stderr, flush=True)


# ====================================================================== GPU
def torch_dtype(wl):
    import torch

    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def gpu_setup(wl, tabs, fill=float("nan"), device="cuda"):
    """Device pools with the cached context written; returns per-layer dicts.

    FP8 workloads get float8_e4m3fn pools (the fill becomes its code: NaN is
    0x7F) written by the quantizing write with the layer's scales."""
    import torch

    import block_paged_kv_amd as pk

    dt = torch_dtype(wl)
    fp8 = wl.kv_dtype == "fp8"
    pool_dt = torch.float8_e4m3fn if fp8 else dt
    dev = {}
    for L in wl.layers:
        if L.alias_of:
            continue
        shape = (L.num_blocks, wl.hkv, wl.block_size, wl.head_dim)
        kp = torch.full(shape, fill, dtype=pool_dt, device=device)
        vp = torch.full(shape, fill, dtype=pool_dt, device=device)
        t = tabs[L.name]
        sk, sv = synth.setup_kv(wl, L)
        slots = np.concatenate(t["setup_slots"]) if t["setup_slots"] else np.zeros(0, np.int64)
        say(f"[gpu] setup write {wl.name}/{L.name}: {slots.shape[0]} tokens")
        if slots.shape[0]:
            ksrc = torch.from_numpy(sk).to(device=device, dtype=dt)
            vsrc = torch.from_numpy(sv).to(device=device, dtype=dt)
            sl = torch.from_numpy(slots).to(device)
            if fp8:
                pk.paged_kv_write_fp8(kp, vp, ksrc, vsrc, sl, L.k_scale, L.v_scale)
            else:
                pk.paged_kv_write(kp, vp, ksrc, vsrc, sl)
        stk, stv = synth.step_kv(wl, L)
        dev[L.name] = dict(
            k_pool=kp, v_pool=vp,
            tables=torch.from_numpy(t["tables"]).to(device),
            step_k=torch.from_numpy(stk).to(device=device, dtype=dt),
            step_v=torch.from_numpy(stv).to(device=device, dtype=dt),
            step_slots=torch.from_numpy(np.concatenate(t["step_slots"])).to(device),
        )
    for L in wl.layers:
        if L.alias_of:
            dev[L.name] = dict(dev[L.alias_of])
        dev[L.name]["q"] = torch.from_numpy(L.q).to(device=device, dtype=dt)
        dev[L.name]["window"] = L.window
        dev[L.name]["k_scale"] = L.k_scale
        dev[L.name]["v_scale"] = L.v_scale
    dev["_seq_lens"] = torch.from_numpy(wl.seq_lens.astype(np.int32)).to(device)
    if wl.kind == "prefill":
        cu = np.concatenate([[0], np.cumsum(wl.chunk_lens)]).astype(np.int32)
        dev["_cu_q"] = torch.from_numpy(cu).to(device)
    return dev


def decode_max_seq_len(wl):
    """Longest context among the rows that run as decode rows."""
    if wl.kind == "decode":
        return wl.max_seq_len
    return int(wl.seq_lens[:wl.num_decode].max()) if wl.num_decode else 0


def gpu_workspace(wl, dev, partition_tokens=None, max_seq_len=None):
    """One uint8 workspace large enough for every decode layer of the step."""
    import torch

    import block_paged_kv_amd as pk

    if wl.kind != "decode" and not wl.num_decode:
        return None
    part = wl.partition_tokens if partition_tokens is None else partition_tokens
    rows = wl.batch if wl.kind == "decode" else wl.num_decode
    msl = decode_max_seq_len(wl) if max_seq_len is None else max_seq_len
    dt = "fp8" if wl.kv_dtype == "fp8" else wl.dtype
    need = max(pk.paged_attn_decode_workspace_bytes(rows, wl.hq, wl.hkv, wl.head_dim,
                                                    wl.block_size, msl, L.window, part, dt)
               for L in wl.layers)
    return torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")


def prefill_workspace(wl):
    """Workspace of the prefill's key split for a chunk-only workload (None when
    the library would not split these shapes on this device)."""
    import torch

    import block_paged_kv_amd as pk

    need = pk.paged_attn_prefill_chunk_workspace_bytes(wl.batch, int(wl.chunk_lens.sum()),
                                                       int(wl.chunk_lens.max()), wl.hq, wl.hkv, wl.head_dim)
    return torch.empty(need, dtype=torch.uint8, device="cuda") if need else None


def gpu_step(wl, dev, outs=None, workspace=None, partition_tokens=None, max_seq_len=None,
             layers=None, prefill_split=False):
    """One pass of the hot path: the step's KV writes, then attention per layer.
    ``prefill_split``: chunk-only workloads pass the prefill a workspace (key
    split where the library's rule asks for one)."""
    import torch

    import block_paged_kv_amd as pk

    names = [L.name for L in wl.layers] if layers is None else layers
    if outs is None:
        outs = {n: torch.empty_like(dev[n]["q"]) for n in names}
    fp8 = wl.kv_dtype == "fp8"
    for L in wl.layers:
        if L.alias_of or L.name not in names:
            continue
        d = dev[L.name]
        if fp8:
            pk.paged_kv_write_fp8(d["k_pool"], d["v_pool"], d["step_k"], d["step_v"], d["step_slots"],
                                  d["k_scale"], d["v_scale"])
        else:
            pk.paged_kv_write(d["k_pool"], d["v_pool"], d["step_k"], d["step_v"], d["step_slots"])
    part = wl.partition_tokens if partition_tokens is None else partition_tokens
    msl = decode_max_seq_len(wl) if max_seq_len is None else max_seq_len
    pws = prefill_workspace(wl) if prefill_split and wl.kind == "prefill" and not wl.num_decode else None
    for n in names:
        d = dev[n]
        if wl.kind == "prefill" and wl.num_decode:
            pk.paged_attn_mixed(outs[n], d["q"], d["k_pool"], d["v_pool"], d["tables"], dev["_cu_q"],
                                dev["_seq_lens"], wl.num_decode, int(wl.chunk_lens.max()), wl.scale, msl,
                                sliding_window=d["window"], partition_tokens=part, workspace=workspace,
                                k_scale=d["k_scale"], v_scale=d["v_scale"])
        elif wl.kind == "decode":
            if fp8:
                pk.paged_attn_decode_fp8(outs[n], d["q"], d["k_pool"], d["v_pool"], d["tables"],
                                         dev["_seq_lens"], wl.scale, d["k_scale"], d["v_scale"], msl,
                                         sliding_window=d["window"], partition_tokens=part,
                                         workspace=workspace)
            else:
                pk.paged_attn_decode(outs[n], d["q"], d["k_pool"], d["v_pool"], d["tables"],
                                     dev["_seq_lens"], wl.scale, msl, sliding_window=d["window"],
                                     partition_tokens=part, workspace=workspace)
        elif fp8:
            pk.paged_attn_prefill_chunk_fp8(outs[n], d["q"], d["k_pool"], d["v_pool"], d["tables"],
                                            dev["_cu_q"], dev["_seq_lens"], int(wl.chunk_lens.max()),
                                            wl.scale, d["k_scale"], d["v_scale"],
                                            sliding_window=d["window"], workspace=pws)
        else:
            pk.paged_attn_prefill_chunk(outs[n], d["q"], d["k_pool"], d["v_pool"], d["tables"],
                                        dev["_cu_q"], dev["_seq_lens"], int(wl.chunk_lens.max()),
                                        wl.scale, sliding_window=d["window"], workspace=pws)
    return outs


# ====================================================================== oracle
def oracle_setup(wl, tabs_ref):
    """float32 pools (NaN canaries elsewhere) holding the same tokens as the GPU pools.

    FP8 workloads: the oracle quantizes the same inputs into uint8 code pools
    (canary code 0x7F, NaN); ``pools["_codes"][layer]`` keeps them for the
    bit-exact write check, and the attention pools hold their dequantized
    values (scale * E4M3 value, float64)."""
    import oracle

    pools = {}
    fp8 = wl.kv_dtype == "fp8"
    if fp8:
        pools["_codes"] = {}
    for L in wl.layers:
        if L.alias_of:
            continue
        shape = (L.num_blocks, wl.hkv, wl.block_size, wl.head_dim)
        t = tabs_ref[L.name]
        sk, sv = synth.setup_kv(wl, L)
        stk, stv = synth.step_kv(wl, L)
        slots = np.concatenate(t["setup_slots"] + t["step_slots"])
        new_k, new_v = np.concatenate([sk, stk]), np.concatenate([sv, stv])
        if fp8:
            kc = np.full(shape, 0x7F, dtype=np.uint8)
            vc = np.full(shape, 0x7F, dtype=np.uint8)
            kc, vc = oracle.kv_write(kc, vc, oracle.fp8.quantize(new_k, L.k_scale),
                                     oracle.fp8.quantize(new_v, L.v_scale), slots, wl.block_size)
            pools["_codes"][L.name] = (kc, vc)
            kp = oracle.fp8.dequantize(kc, L.k_scale)
            vp = oracle.fp8.dequantize(vc, L.v_scale)
        else:
            kp = np.full(shape, np.nan, dtype=np.float32)
            vp = np.full(shape, np.nan, dtype=np.float32)
            kp, vp = oracle.kv_write(kp, vp, new_k, new_v, slots, wl.block_size)
        pools[L.name] = (kp, vp, t["tables"])
    for L in wl.layers:
        if L.alias_of:
            pools[L.name] = pools[L.alias_of]
    return pools


def oracle_step(wl, pools, rows=None, layers=None):
    """float64 reference outputs per layer; ``rows`` limits prefill to some query rows."""
    import oracle

    out = {}
    for L in wl.layers:
        if layers is not None and L.name not in layers:
            continue
        kp, vp, tables = pools[L.name]
        if wl.kind == "decode":
            out[L.name] = oracle.decode(L.q, kp, vp, tables, wl.seq_lens, wl.scale, L.window,
                                        wl.block_size)
        else:
            cu = np.concatenate([[0], np.cumsum(wl.chunk_lens)]).astype(np.int64)
            out[L.name] = oracle.prefill_chunk(L.q, kp, vp, tables, cu, wl.seq_lens, wl.scale,
                                               L.window, wl.block_size, query_rows=rows)
    return out


# ====================================================================== compare
def compare(gpu, ref, dtype, rows=None):
    """(max_abs, rel_l2) of a GPU output against the float64 oracle."""
    g = gpu.double().cpu().numpy()
    r = np.asarray(ref, dtype=np.float64)
    if rows is not None:
        g, r = g[rows], r[rows]
    err = np.abs(g - r)
    denom = np.linalg.norm(r)
    return float(err.max()) if err.size else 0.0, float(np.linalg.norm(g - r) / denom) if denom else 0.0


TOL = {"f32": dict(max_abs=1e-5, rel_l2=None), "bf16": dict(max_abs=2e-2, rel_l2=5e-3)}


def within(dtype, max_abs, rel_l2):
    t = TOL[dtype]
    return max_abs <= t["max_abs"] and (t["rel_l2"] is None or rel_l2 <= t["rel_l2"])
