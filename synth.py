"""Seeded synthetic workloads for tests, the smoke check and the benchmark.

This module draws random inputs and drives an allocator through the request
lifecycle; it holds none of the attention arithmetic. It serves both sides of
every parity check: the HIP path and the CPU oracle receive the same arrays.

Workloads (shapes from the mlx-node pages' models; values are N(0, 1) float32,
rounded to bf16 with round-to-nearest-even for bf16 workloads):

* ``tiny``    -- fp32 decode: 1 layer, B=2, Hq=4, Hkv=2, D=64, context 40 and 75
                 tokens, the first 32 tokens (2 blocks) a shared prefix, a
                 512-block pool with a seeded physical permutation, scale 1/8.
* ``qwen3``   -- Qwen3-0.6B-shaped decode step: B=4, Hq=16, Hkv=8, D=128, bf16,
                 2048-token contexts whose first 512 tokens are a shared prefix
                 chain, a 2048 MiB pool (32768 blocks of 64 KiB), plus the write
                 of 1 new token per row.
* ``mixed``   -- continuous-batching decode: B=32, Hq=32, Hkv=8, D=128, bf16,
                 contexts uniform in [128, 8192], each row taking one of 4 shared
                 prefixes of 0..1024 tokens, 512-token split-K partitions.
* ``hybrid``  -- Gemma-style layers: B=8, Hq=8, Hkv=1, D=256, bf16, 32768-token
                 contexts: a sliding-window layer (window 512, its own 1024-block
                 pool and tables with null entries), a full-attention layer and a
                 KV-shared layer that reads the full layer's pool and tables.
* ``prefill`` -- chunked prefill: B=1, Hq=32, Hkv=8, D=128, bf16, a 2048-token
                 chunk over a 63488-token cached prefix (65536-token context,
                 4096 blocks of a 32768-block pool), chunk K/V written first.
* ``hprefill`` -- Gemma-style hybrid chunked prefill: B=4, Hq=8, Hkv=1, D=256,
                 bf16, a 2048-token chunk per row over a 6144-token cached prefix;
                 the same three layers as ``hybrid`` (sliding window 512 with its
                 own 1024-block pool and null entries for expired blocks, full
                 attention, and a KV-shared layer reading the full layer's pool
                 and tables, which writes nothing).
* ``mixedstep`` -- one continuous-batching step: 32 decode rows (contexts uniform
                 in [128, 8192], one new token each, 512-token split-K
                 partitions) and one joining request whose 2048-token chunk
                 follows a 6144-token cached prefix; Hq=32, Hkv=8, D=128, bf16,
                 a 32768-block pool. Rows with one query come first.

Random draw order per workload (``numpy.random.default_rng(seed)``): the
allocator free-list permutation, then lengths and prefix choices, then the
logical K/V of every prefix and row suffix, then Q, then the new tokens' K/V.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16
SEEDS = {"tiny": 1000, "qwen3": 1001, "mixed": 1002, "hybrid": 1003, "prefill": 1004, "hprefill": 1005,
         "mixedstep": 1006}


def round_bf16(x):
    """float32 -> nearest-even bf16 value, returned as float32 (exact bf16 values)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


@dataclass
class Layer:
    """One attention layer's inputs."""

    name: str
    num_blocks: int
    window: int = 0                      # 0 = full attention
    alias_of: str | None = None          # KV-shared layer: reads this layer's pool/tables
    free_order: np.ndarray | None = None  # int32 permutation of 1..NB-1
    k: list = field(default_factory=list)    # per row float32 [n_b, Hkv, D] (None for alias)
    v: list = field(default_factory=list)
    live_from: list = field(default_factory=list)  # per row: first position with data
    q: np.ndarray | None = None          # decode [B, Hq, D]; prefill [T, Hq, D]
    k_scale: float = 1.0                 # FP8 pools: per-layer scales (float32 values)
    v_scale: float = 1.0


@dataclass
class Workload:
    name: str
    kind: str                 # "decode" or "prefill"
    batch: int
    hq: int
    hkv: int
    head_dim: int
    dtype: str                # "f32" or "bf16"
    seq_lens: np.ndarray      # int32 [B], tokens in cache after the step's write
    tokens: list              # per row int32 token ids (length seq_lens[b])
    layers: list
    scale: float
    partition_tokens: int = 0
    chunk_lens: np.ndarray | None = None  # prefill: query tokens per row
    block_size: int = BLOCK_SIZE
    domain: int = 0
    wave_size: int = 0        # rows per benchmark step when several batches share a pool
    kv_dtype: str = ""        # "" = the pools hold ``dtype``; "fp8" = E4M3 codes with per-layer scales
    num_decode: int = 0       # prefill kind: leading rows that are decode rows (one query each)

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max()) if len(self.seq_lens) else 0

    @property
    def new_tokens(self):
        """Tokens written in the timed step, per row (decode: 1; prefill: the chunk)."""
        if self.kind == "prefill":
            return [int(c) for c in self.chunk_lens]
        return [1] * self.batch

    def layer(self, name):
        return next(L for L in self.layers if L.name == name)


def _normal(rng, shape, bf16):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return round_bf16(x) if bf16 else x


def _prefix_tokens(k, length):
    return np.arange(length, dtype=np.int64).astype(np.int32) + np.int32(1_000_000 * (k + 1))


def _suffix_tokens(b, length):
    return -(np.arange(length, dtype=np.int64).astype(np.int32) + np.int32(1_000_000 * (b + 1)))


def make(name, *, batch=None, hq=None, hkv=None, head_dim=None, context=None, prefix=None,
         num_blocks=None, seed=None, chunk=None, window=None, dtype=None, part=None,
         num_prefixes=None, sliding_blocks=None, waves=None, block_size=None, kv_dtype=None,
         k_growth=None):
    """Build workload ``name`` at its published sizes; keyword overrides shrink it for tests.

    ``block_size`` (a power of two in [8, 64], default 16) changes only the paging:
    the random draws are the same, prefix lengths round to whole blocks.
    ``kv_dtype="fp8"`` (bf16 workloads) stores the pools as FP8 E4M3 codes with a
    K and a V scale per layer: max |x| of the layer's K (V) over 448, so nothing
    saturates; the draws are the same.
    ``k_growth=g`` multiplies the key of position t by 2^min(t // g, 12) (exact in
    bf16 and float32): the largest score of a row then jumps every g positions, so an
    online softmax has to rescale accumulators that already hold data."""
    bs = BLOCK_SIZE if block_size is None else int(block_size)
    seed = SEEDS[name] if seed is None else seed
    rng = np.random.default_rng(seed)
    wl = _make(name, rng, bs, batch=batch, hq=hq, hkv=hkv, head_dim=head_dim, context=context,
               prefix=prefix, num_blocks=num_blocks, chunk=chunk, window=window, dtype=dtype,
               part=part, num_prefixes=num_prefixes, sliding_blocks=sliding_blocks, waves=waves)
    if k_growth:
        for L in wl.layers:
            if L.alias_of:
                continue
            for b, x in enumerate(L.k):
                t = L.live_from[b] + np.arange(x.shape[0])
                f = np.exp2(np.minimum(t // int(k_growth), 12)).astype(np.float32)
                L.k[b] = (x * f[:, None, None]).astype(np.float32)
    if kv_dtype:
        if kv_dtype != "fp8" or wl.dtype != "bf16":
            raise ValueError("kv_dtype='fp8' needs a bf16 workload")
        wl.kv_dtype = "fp8"
        for L in wl.layers:
            if L.alias_of:
                continue
            kmax = max(float(np.abs(x).max()) if x.size else 0.0 for x in L.k)
            vmax = max(float(np.abs(x).max()) if x.size else 0.0 for x in L.v)
            L.k_scale = float(np.float32(max(kmax, 1e-6) / 448.0))
            L.v_scale = float(np.float32(max(vmax, 1e-6) / 448.0))
        for L in wl.layers:
            if L.alias_of:
                A = wl.layer(L.alias_of)
                L.k_scale, L.v_scale = A.k_scale, A.v_scale
    return wl


def _make(name, rng, bs, *, batch=None, hq=None, hkv=None, head_dim=None, context=None, prefix=None,
          num_blocks=None, chunk=None, window=None, dtype=None, part=None, num_prefixes=None,
          sliding_blocks=None, waves=None):

    if name == "tiny":
        B, Hq, Hkv, D = batch or 2, hq or 4, hkv or 2, head_dim or 64
        NB = num_blocks or 512
        bf16 = (dtype or "f32") == "bf16"
        free = rng.permutation(np.arange(1, NB)).astype(np.int32)
        lens = np.array(context if context is not None else [40, 75][:B], dtype=np.int32)
        pre = 32 if prefix is None else prefix
        return _decode_from_prefixes(name, rng, B, Hq, Hkv, D, bf16, lens, [pre], [0] * B,
                                     [("main", NB, 0, None, free)], part or 0, bs=bs)

    if name == "qwen3":
        # ``waves`` > 1 stacks that many independent batches (each with its own
        # shared prefix chain) in the same pool; a benchmark step serves one.
        B, Hq, Hkv, D = batch or 4, hq or 16, hkv or 8, head_dim or 128
        R = waves or 1
        NB = num_blocks or 32768
        free = rng.permutation(np.arange(1, NB)).astype(np.int32)
        n = context or 2048
        lens = np.full(B * R, n, dtype=np.int32)
        pre = 512 if prefix is None else prefix
        wl = _decode_from_prefixes(name, rng, B * R, Hq, Hkv, D, (dtype or "bf16") == "bf16", lens,
                                   [pre] * R, [b // B for b in range(B * R)],
                                   [("main", NB, 0, None, free)], part or 0, bs=bs)
        wl.wave_size = B
        return wl

    if name == "mixed":
        B, Hq, Hkv, D = batch or 32, hq or 32, hkv or 8, head_dim or 128
        NB = num_blocks or 32768
        free = rng.permutation(np.arange(1, NB)).astype(np.int32)
        lo, hi = context if context is not None else (128, 8192)
        lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
        npre = num_prefixes or 4
        pmax = 1024 if prefix is None else prefix
        pre_lens = [int(bs * (x // bs)) for x in rng.integers(0, pmax + 1, size=npre)]
        choice = [int(c) for c in rng.integers(0, npre, size=B)]
        return _decode_from_prefixes(name, rng, B, Hq, Hkv, D, (dtype or "bf16") == "bf16", lens,
                                     pre_lens, choice, [("main", NB, 0, None, free)],
                                     512 if part is None else part, bs=bs)

    if name == "hybrid":
        B, Hq, Hkv, D = batch or 8, hq or 8, hkv or 1, head_dim or 256
        NB = num_blocks or 32768
        NBS = sliding_blocks or 1024
        W = 512 if window is None else window
        free_full = rng.permutation(np.arange(1, NB)).astype(np.int32)
        free_slide = rng.permutation(np.arange(1, NBS)).astype(np.int32)
        n = context or 32768
        lens = np.full(B, n, dtype=np.int32)
        layers = [("sliding", NBS, W, None, free_slide), ("full", NB, 0, None, free_full),
                  ("shared", NB, 0, "full", None)]
        return _decode_from_prefixes(name, rng, B, Hq, Hkv, D, (dtype or "bf16") == "bf16", lens,
                                     [0], [0] * B, layers, part or 0, bs=bs)

    if name == "prefill":
        B, Hq, Hkv, D = batch or 1, hq or 32, hkv or 8, head_dim or 128
        NB = num_blocks or 32768
        W = window or 0
        free = rng.permutation(np.arange(1, NB)).astype(np.int32)
        C = np.array(chunk if chunk is not None else [2048] * B, dtype=np.int32).reshape(-1)
        P = np.array(context if context is not None else [63488] * B, dtype=np.int32).reshape(-1)
        lens = (P + C).astype(np.int32)
        layer = Layer("main", NB, W, None, free)
        toks = []
        for b in range(B):
            layer.k.append(_normal(rng, (int(P[b]), Hkv, D), True))
            layer.v.append(_normal(rng, (int(P[b]), Hkv, D), True))
            layer.live_from.append(0)
            toks.append(_suffix_tokens(b, int(lens[b])))
        layer.q = _normal(rng, (int(C.sum()), Hq, D), True)
        for b in range(B):  # the chunk's own K/V: the tokens the step writes
            layer.k[b] = np.concatenate([layer.k[b], _normal(rng, (int(C[b]), Hkv, D), True)])
            layer.v[b] = np.concatenate([layer.v[b], _normal(rng, (int(C[b]), Hkv, D), True)])
        return Workload(name, "prefill", B, Hq, Hkv, D, "bf16", lens, toks, [layer],
                        1.0 / math.sqrt(D), chunk_lens=C, block_size=bs)

    if name == "mixedstep":
        ND, Hq, Hkv, D = 32 if batch is None else batch, hq or 32, hkv or 8, head_dim or 128
        NB = num_blocks or 32768
        free = rng.permutation(np.arange(1, NB)).astype(np.int32)
        lo, hi = context if context is not None else (128, 8192)
        dec = rng.integers(lo, hi + 1, size=ND).astype(np.int32)
        Cp = np.array(chunk if chunk is not None else [2048], dtype=np.int32).reshape(-1)
        Pp = np.array(prefix if prefix is not None else [6144] * len(Cp), dtype=np.int32).reshape(-1)
        C = np.concatenate([np.ones(ND, np.int32), Cp]).astype(np.int32)
        P = np.concatenate([dec - 1, Pp]).astype(np.int32)
        lens = (P + C).astype(np.int32)
        B = len(C)
        layer = Layer("main", NB, window or 0, None, free)
        toks = []
        for b in range(B):
            layer.k.append(_normal(rng, (int(P[b]), Hkv, D), True))
            layer.v.append(_normal(rng, (int(P[b]), Hkv, D), True))
            layer.live_from.append(0)
            toks.append(_suffix_tokens(b, int(lens[b])))
        layer.q = _normal(rng, (int(C.sum()), Hq, D), True)
        for b in range(B):  # the step's new tokens: one per decode row, the chunk
            layer.k[b] = np.concatenate([layer.k[b], _normal(rng, (int(C[b]), Hkv, D), True)])
            layer.v[b] = np.concatenate([layer.v[b], _normal(rng, (int(C[b]), Hkv, D), True)])
        return Workload(name, "prefill", B, Hq, Hkv, D, "bf16", lens, toks, [layer],
                        1.0 / math.sqrt(D), partition_tokens=512 if part is None else part,
                        chunk_lens=C, block_size=bs, num_decode=ND)

    if name == "hprefill":
        B, Hq, Hkv, D = batch or 4, hq or 8, hkv or 1, head_dim or 256
        NB = num_blocks or 32768
        NBS = sliding_blocks or 1024
        W = 512 if window is None else window
        free_full = rng.permutation(np.arange(1, NB)).astype(np.int32)
        free_slide = rng.permutation(np.arange(1, NBS)).astype(np.int32)
        C = np.array(chunk if chunk is not None else [2048] * B, dtype=np.int32).reshape(-1)
        P = np.array(context if context is not None else [6144] * B, dtype=np.int32).reshape(-1)
        lens = (P + C).astype(np.int32)
        layers = [Layer("sliding", NBS, W, None, free_slide), Layer("full", NB, 0, None, free_full),
                  Layer("shared", NB, 0, "full", None)]
        toks = [_suffix_tokens(b, int(lens[b])) for b in range(B)]
        for L in layers:  # cached prefix K/V per layer (a sliding layer: from its first live block)
            if L.alias_of:
                continue
            for b in range(B):
                start = (max(0, int(P[b]) - W) // bs) * bs if W and L.window else 0
                L.k.append(_normal(rng, (int(P[b]) - start, Hkv, D), True))
                L.v.append(_normal(rng, (int(P[b]) - start, Hkv, D), True))
                L.live_from.append(start)
        for L in layers:
            L.q = _normal(rng, (int(C.sum()), Hq, D), True)
        for L in layers:  # the chunk's own K/V: the tokens the step writes
            if L.alias_of:
                continue
            for b in range(B):
                L.k[b] = np.concatenate([L.k[b], _normal(rng, (int(C[b]), Hkv, D), True)])
                L.v[b] = np.concatenate([L.v[b], _normal(rng, (int(C[b]), Hkv, D), True)])
        return Workload(name, "prefill", B, Hq, Hkv, D, "bf16", lens, toks, layers,
                        1.0 / math.sqrt(D), chunk_lens=C, block_size=bs)

    raise ValueError(f"unknown workload {name}")


def _decode_from_prefixes(name, rng, B, Hq, Hkv, D, bf16, lens, pre_lens, choice, layer_specs, part,
                          bs=BLOCK_SIZE):
    layers = [Layer(nm, nb, w, alias, free) for nm, nb, w, alias, free in layer_specs]
    toks = []
    for b in range(B):
        k = choice[b]
        plen = min(pre_lens[k], int(lens[b]) - 1)  # the newest token is never a prefix token
        toks.append(np.concatenate([_prefix_tokens(k, plen), _suffix_tokens(b, int(lens[b]) - plen)]))
    # Logical K/V: per prefix, then per row suffix (positions up to n-2); each
    # layer draws its own. A sliding layer only needs the positions of its live
    # blocks, counted from the block holding n - W.
    for L in layers:
        if L.alias_of:
            continue
        pk = [(_normal(rng, (pl, Hkv, D), bf16), _normal(rng, (pl, Hkv, D), bf16)) for pl in pre_lens]
        for b in range(B):
            n = int(lens[b])
            start = 0
            if L.window:
                start = (max(0, n - L.window) // bs) * bs
            plen = min(pre_lens[choice[b]], n - 1)
            body_from = max(start, plen)
            ks = [pk[choice[b]][0][start:plen]] if start < plen else []
            vs = [pk[choice[b]][1][start:plen]] if start < plen else []
            # suffix positions [body_from, n - 1); the newest token comes later
            m = max(0, n - 1 - body_from)
            ks.append(_normal(rng, (m, Hkv, D), bf16))
            vs.append(_normal(rng, (m, Hkv, D), bf16))
            L.k.append(np.concatenate(ks) if ks else np.zeros((0, Hkv, D), np.float32))
            L.v.append(np.concatenate(vs) if vs else np.zeros((0, Hkv, D), np.float32))
            L.live_from.append(start)
    for L in layers:
        L.q = _normal(rng, (B, Hq, D), bf16)
    for L in layers:
        if L.alias_of:
            continue
        for b in range(B):  # the newest token of every row: written in the step
            L.k[b] = np.concatenate([L.k[b], _normal(rng, (1, Hkv, D), bf16)])
            L.v[b] = np.concatenate([L.v[b], _normal(rng, (1, Hkv, D), bf16)])
    return Workload(name, "decode", B, Hq, Hkv, D, "bf16" if bf16 else "f32", lens, toks, layers,
                    1.0 / math.sqrt(D), partition_tokens=part, block_size=bs)


# --------------------------------------------------------------------- tables
def build_tables(alloc_factory, wl: Workload, share=True):
    """Drive allocators through the lifecycle; return per-layer tables and write plans.

    ``alloc_factory(num_blocks, block_size, free_order)`` builds one allocator
    per pool (the library's ``Allocator`` or the oracle's ``RefAllocator``).
    ``share=False`` gives every row its own prefix domain, so equal prefixes
    get private copies instead of shared blocks.
    Returns ``{layer: dict(alloc, tables [B, MB] int32, setup_slots, step_slots)}``
    where ``setup_slots[b]`` are the slots of the positions written before the
    step (cached context) and ``step_slots[b]`` those written in the step.
    """
    out = {}
    B = wl.batch
    bs = wl.block_size
    for L in wl.layers:
        if L.alias_of:
            out[L.name] = out[L.alias_of]
            continue
        a = alloc_factory(L.num_blocks, bs, L.free_order)
        setup, step = [], []
        for b in range(B):
            n = int(wl.seq_lens[b])
            new = wl.new_tokens[b]
            toks = wl.tokens[b]
            a.add(b)
            if L.window:
                # Sliding group: grow in steps of the window, dropping expired blocks
                # as the context advances. The last drop happens before the step's
                # tokens are committed, so every query of the step keeps its keys.
                target = n - new
                written = 0
                while written < target:
                    upto = min(target, written + L.window)
                    a.reserve(b, upto)
                    a.commit_tokens(b, toks[written:upto])
                    a.drop_outside_window(b, L.window)
                    written = upto
                a.reserve(b, n)
                a.commit_tokens(b, toks[target:n])
                first = setup_first(wl, L, b)
                setup.append(np.asarray(a.slot_mapping(b, first, target - first), dtype=np.int64))
            else:
                dom = wl.domain if share else 1_000_003 * (b + 1)
                cached = a.match_prefix(b, toks[:n - 1], dom)
                a.reserve(b, n)
                a.commit_tokens(b, toks[cached:n])
                a.publish_full_blocks(b, dom)
                # Shared blocks already hold their K/V; writing them again with the
                # same values is harmless, so the setup simply writes 0..n-new.
                setup.append(np.asarray(a.slot_mapping(b, 0, n - new), dtype=np.int64))
            step.append(np.asarray(a.slot_mapping(b, n - new, new), dtype=np.int64))
        mb = max(a.num_blocks_of(b) for b in range(B))
        out[L.name] = dict(alloc=a, tables=np.asarray(a.block_tables(list(range(B)), mb), dtype=np.int32),
                           setup_slots=setup, step_slots=step)
    return out


def kv_rows(wl: Workload, layer: Layer, b, which, start, stop):
    """Rows [start, stop) of row b's logical K or V for ``layer`` (positions, not indices)."""
    arr = (layer.k if which == "k" else layer.v)[b]
    off = layer.live_from[b]
    return arr[start - off:stop - off]


def step_kv(wl: Workload, layer: Layer):
    """K/V of the tokens the step writes, concatenated over rows: ([T,Hkv,D], [T,Hkv,D])."""
    ks, vs = [], []
    for b in range(wl.batch):
        n = int(wl.seq_lens[b])
        new = wl.new_tokens[b]
        ks.append(kv_rows(wl, layer, b, "k", n - new, n))
        vs.append(kv_rows(wl, layer, b, "v", n - new, n))
    return np.concatenate(ks), np.concatenate(vs)


def setup_first(wl: Workload, layer: Layer, b):
    """First position of row b written before the step (sliding: its first live block)."""
    first = layer.live_from[b]
    if layer.window:
        target = int(wl.seq_lens[b]) - wl.new_tokens[b]
        first = max(first, (max(0, target - layer.window) // wl.block_size) * wl.block_size)
    return first


def setup_kv(wl: Workload, layer: Layer):
    """K/V of the cached positions written before the step (from each row's live start)."""
    ks, vs = [], []
    for b in range(wl.batch):
        n = int(wl.seq_lens[b])
        new = wl.new_tokens[b]
        first = setup_first(wl, layer, b)
        ks.append(kv_rows(wl, layer, b, "k", first, n - new))
        vs.append(kv_rows(wl, layer, b, "v", first, n - new))
    return np.concatenate(ks), np.concatenate(vs)


def unique_kv_bytes(wl: Workload, tables, layer_name, elem_bytes):
    """Bytes of distinct K/V token rows a decode step must read for one layer.

    Counts each (physical block, offset) the rows attend to once, K and V:
    shared prefix blocks are counted once however many rows read them.
    """
    L = wl.layer(layer_name)
    t = tables[layer_name]["tables"]
    seen = set()
    for b in range(wl.batch):
        n = int(wl.seq_lens[b])
        lo = max(0, n - L.window) if L.window else 0
        for p in range(lo, n):
            seen.add((int(t[b][p // wl.block_size]), p % wl.block_size))
    return len(seen) * wl.hkv * wl.head_dim * elem_bytes * 2
