"""Float64 reference for the paged KV write, gather, decode and prefill chunk.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``): the product path never
imports this module.

Storage convention shared with the library (a choice of layout, not of
arithmetic): a per-layer pool is ``pool[num_blocks][num_kv_heads][block_size]
[head_dim]``; K and V live in two separate pools. The mlx-node paged-cache
doc (component table, LayerKVPool row) only says each layer owns a K buffer
and a V buffer; the block-major, head-next order is our reading.

A token slot is ``physical_block * block_size + offset``; a negative slot means
"padding, write nothing".

Arrays passed in may be any real dtype (bf16-valued data is carried as float32
holding exactly the bf16 values). Every attention computation converts to
float64 first; that conversion is exact for float32 and bf16 values.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "kv_write",
    "gather_positions",
    "attend_one",
    "decode_attended_range",
    "prefill_attended_range",
    "decode",
    "prefill_chunk",
]


def kv_write(k_pool, v_pool, new_k, new_v, slot_mapping, block_size):
    """Slot-mapped KV write: return copies of the pools with new tokens stored.

    mlx-node perf doc, paged-attention knobs table (the default-on native paged
    K/V write row): each new token's K and V rows are scattered into the pool
    slot its request owns. For token t with ``slot = slot_mapping[t] >= 0``:
    ``pool[slot // BS, :, slot % BS, :] = new[t]``. Tokens with a negative slot
    are padding and write nothing; every other pool element keeps its bits.
    Block 0 is the shared null sentinel that sliding tables point at for
    expired blocks (mlx-node paged-cache doc, hybrid coordinator paragraph);
    no request owns a slot in it, so a slot there is read as padding too
    (our reading: the pages never write the sentinel).

    The copy is element for element (numpy assignment of equal dtypes), so the
    result is bit-exact. Returns ``(k_pool', v_pool')``.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    for t in range(slots.shape[0]):
        s = int(slots[t])
        if s < 0:
            continue
        blk, off = divmod(s, block_size)
        if blk == 0:
            continue
        k_out[blk, :, off, :] = new_k[t]
        v_out[blk, :, off, :] = new_v[t]
    return k_out, v_out


def gather_positions(pool, block_table_row, positions, block_size):
    """Materialise contiguous rows ``out[i] = pool[bt[p // BS], :, p % BS, :]``.

    mlx-node perf doc, paged-attention knobs table (graph decode gather row):
    a request's logical position p lives in block ``p // BS`` of its table at
    offset ``p % BS``. The null sentinel (block 0) and padding entries are never
    dereferenced for a needed position: the mlx-node paged-cache doc (hybrid
    coordinator paragraph) replaces blocks wholly outside a sliding window by a
    shared null sentinel, so a table that maps a needed position to block 0 is a
    bookkeeping error and raises.

    Returns an array of shape ``[len(positions), num_kv_heads, head_dim]`` in
    the pool's dtype (bit copies).
    """
    positions = list(positions)
    bt = np.asarray(block_table_row)
    if len(positions) == 0:
        return np.zeros((0,) + tuple(pool.shape[1:2]) + tuple(pool.shape[3:]), dtype=pool.dtype)
    rows = []
    for p in positions:
        logical_block, off = divmod(int(p), block_size)
        phys = int(bt[logical_block])
        if phys == 0:
            raise ValueError(f"position {p} maps to the null sentinel block")
        rows.append(pool[phys, :, off, :])
    return np.stack(rows, axis=0)


def attend_one(q, keys, values, scale):
    """Plain softmax attention of one query vector over a contiguous K/V set.

    ``s_t = scale * sum_d q[d] K[t, d]``; ``m = max_t s_t``;
    ``o = sum_t exp(s_t - m) V[t] / sum_t exp(s_t - m)``.

    This is the definition the paged path must reproduce (the mlx-node
    paged-cache doc's model-status table holds paged output equal to the flat
    contiguous-cache output). Subtracting the maximum does not change the value
    of the ratio. An empty set gives exact zeros (the mlx-node perf doc,
    attention-partitions paragraph: empty stripes add exact zeros).
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros(values.shape[-1], dtype=np.float64)
    s = scale * (keys @ q)
    m = s.max()
    p = np.exp(s - m)
    return (p @ values) / p.sum()


def decode_attended_range(seq_len, window):
    """Key positions a decode query attends to: ``[max(0, n - W), n)``.

    The query is the newest token, at position ``n - 1``, whose own K/V has
    already been written (the chunked-prefill workload writes new K/V first via
    the slot mapping; decode is the one-token case). With a sliding window W > 0
    the query sees the last W positions including itself (a rotating cache holds
    min(offset, window) tokens: mlx-node paged-cache doc, Gemma4 sliding
    sidecar section). ``W = 0`` means full attention.
    """
    lo = max(0, seq_len - window) if window > 0 else 0
    return lo, seq_len


def prefill_attended_range(abs_pos, window):
    """Key positions query at absolute position ``a`` attends to: ``[lo, a]``.

    Causal: keys at or before the query. With a window W > 0,
    ``lo = max(0, a - W + 1)``, the same rule as decode for a query at ``a``.
    """
    lo = max(0, abs_pos - window + 1) if window > 0 else 0
    return lo, abs_pos + 1


def decode(q, k_pool, v_pool, block_tables, seq_lens, scale, window, block_size):
    """Batched GQA decode over a block-paged cache, in float64.

    ``q[B][Hq][D]``; ``block_tables[B][MB]``; ``seq_lens[B]`` counts the row's
    tokens including the one being decoded. Query head h reads KV head
    ``h // (Hq // Hkv)`` (contiguous grouping; the mlx-node paged-cache doc,
    model-status table, gives 32 query / 2 KV head geometry without the map,
    and contiguous grouping is the plain reading). Returns ``o[B][Hq][D]``.

    Follows the mlx-node perf doc (paged-attention knobs table: generic V2
    batched paged decode serves every row of a wave; decode gather reads
    sliding groups from their first live block).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        lo, hi = decode_attended_range(n, window)
        keys = gather_positions(k_pool, block_tables[b], range(lo, hi), block_size)
        vals = gather_positions(v_pool, block_tables[b], range(lo, hi), block_size)
        for h in range(Hq):
            kvh = h // group
            out[b, h] = attend_one(q[b, h], keys[:, kvh, :], vals[:, kvh, :], scale)
    return out


def prefill_chunk(q, k_pool, v_pool, block_tables, cu_q_lens, seq_lens, scale,
                  window, block_size, query_rows=None, q_block=256):
    """Chunked-prefill attention over a cached paged prefix, in float64.

    Row b owns query rows ``cu_q_lens[b] .. cu_q_lens[b+1]-1`` of
    ``q[T][Hq][D]`` (C = their count) and has ``seq_lens[b] = P + C`` tokens in
    the cache, its chunk's own K/V already written (the mlx-node perf doc's
    paged-attention bridge for prefill over a cache hit reads K/V through the
    pages; the chunk size knob sits in the same table). Query i of the chunk is
    at absolute position ``a = P + i`` and attends to ``[lo, a]``
    (``prefill_attended_range``).

    Queries are processed in blocks of ``q_block`` consecutive rows: per query
    head, one float64 product of the block's queries with every key the block
    can see, then the keys outside each query's range get weight exactly zero
    (``exp(-inf) = 0``, the same as leaving them out), then the softmax of each
    query row. ``query_rows`` (optional) restricts the work to a subset of the
    global query rows; other rows of the result are NaN.

    Returns ``o[T][Hq][D]`` in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    T, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    group = Hq // Hkv
    out = np.full((T, Hq, D), np.nan, dtype=np.float64)
    wanted = None if query_rows is None else set(int(r) for r in query_rows)
    B = len(seq_lens)
    for b in range(B):
        r0, r1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        C = r1 - r0
        n = int(seq_lens[b])
        P = n - C
        if P < 0:
            raise ValueError("seq_lens[b] must include the chunk")
        rows = [r for r in range(r0, r1) if wanted is None or r in wanted]
        for i0 in range(0, len(rows), q_block):
            blk_rows = rows[i0:i0 + q_block]
            spans = [prefill_attended_range(P + (r - r0), window) for r in blk_rows]
            los = np.array([lo for lo, _ in spans], dtype=np.int64)
            his = np.array([hi for _, hi in spans], dtype=np.int64)
            kmin, kmax = int(los.min()), int(his.max())
            keys = gather_positions(k_pool, block_tables[b], range(kmin, kmax), block_size)
            vals = gather_positions(v_pool, block_tables[b], range(kmin, kmax), block_size)
            key_pos = np.arange(kmin, kmax)
            visible = (key_pos[None, :] >= los[:, None]) & (key_pos[None, :] < his[:, None])
            for h in range(Hq):
                kvh = h // group
                kf = keys[:, kvh, :].astype(np.float64)
                vf = vals[:, kvh, :].astype(np.float64)
                s = scale * (q[blk_rows, h, :] @ kf.T)
                s = np.where(visible, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                p = np.exp(s - m)
                out[blk_rows, h, :] = (p @ vf) / p.sum(axis=1, keepdims=True)
    return out
