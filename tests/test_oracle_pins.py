"""Pins for the attention oracle (CPU only).

Each ``pin_*`` function checks the oracle against something other than
itself: hand-worked fixtures, closed forms that are written differently from
the softmax definition, mask sets spelled out by hand, and invariants the
pages state (paged output equals the flat contiguous output; a shared prefix
block gives the same result as a private copy; placement does not matter).
``test_mutants_are_caught`` plants plausible mistakes in the oracle and checks
that at least one pin fails for each of them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers
def scatter_flat(flat_k, flat_v, table, nb, bs):
    """Build pools from contiguous per-row K/V: position p -> (table[p//bs], p%bs).

    Written independently of the oracle's gather (a plain index walk), so a
    round trip through the oracle must return the flat arrays exactly.
    """
    hkv, d = flat_k.shape[1], flat_k.shape[2]
    kp = np.full((nb, hkv, bs, d), np.nan)
    vp = np.full((nb, hkv, bs, d), np.nan)
    for p in range(flat_k.shape[0]):
        kp[table[p // bs], :, p % bs, :] = flat_k[p]
        vp[table[p // bs], :, p % bs, :] = flat_v[p]
    return kp, vp


def brute_force(q, keys, values, scale):
    """Scalar loops, no max subtraction (inputs kept small): sum e^s v / sum e^s."""
    num = [0.0] * len(values[0]) if len(values) else []
    den = 0.0
    for k, v in zip(keys, values):
        s = scale * sum(float(a) * float(b) for a, b in zip(q, k))
        e = math.exp(s)
        den += e
        for j in range(len(num)):
            num[j] += e * float(v[j])
    return [x / den for x in num] if den else [0.0] * (len(values[0]) if len(values) else 0)


# ----------------------------------------------------------------- pins
def pin_golden_hand_worked():
    with open(os.path.join(GOLDEN, "attention_hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = oracle.attend_one(np.array(c["q"]), np.array(c["K"]), np.array(c["V"]), c["scale"])
        np.testing.assert_allclose(got, c["expected"], rtol=0, atol=1e-12, err_msg=c["name"])


def pin_closed_forms_two_and_three_keys():
    """n=2: o = V0 + sigmoid(s1 - s0) (V1 - V0); n=3: o3 = (1 - w) o2 + w V2,
    w = sigmoid(s2 - log(e^s0 + e^s1)). Different expressions from the softmax."""
    rng = np.random.default_rng(7)
    for _ in range(20):
        d = 5
        q = rng.normal(size=d)
        K = rng.normal(size=(3, d))
        V = rng.normal(size=(3, d))
        scale = 0.37
        s = [scale * float(np.dot(q, K[i])) for i in range(3)]
        sig = lambda x: 1.0 / (1.0 + math.exp(-x))  # noqa: E731
        o2 = V[0] + sig(s[1] - s[0]) * (V[1] - V[0])
        np.testing.assert_allclose(oracle.attend_one(q, K[:2], V[:2], scale), o2, atol=1e-12)
        w = sig(s[2] - math.log(math.exp(s[0]) + math.exp(s[1])))
        o3 = (1 - w) * o2 + w * V[2]
        np.testing.assert_allclose(oracle.attend_one(q, K, V, scale), o3, atol=1e-12)
        np.testing.assert_array_equal(oracle.attend_one(q, K[:1], V[:1], scale), V[0])


def pin_empty_is_zero():
    out = oracle.attend_one(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 0.5)
    assert out.shape == (4,) and np.all(out == 0)


def _one_row_decode(flat_k, flat_v, q, n, window, bs=4, nb=64, seed=0, scale=0.3):
    rng = np.random.default_rng(seed)
    nblk = -(-flat_k.shape[0] // bs)
    table = list(rng.permutation(np.arange(1, nb))[:nblk])
    kp, vp = scatter_flat(flat_k, flat_v, table, nb, bs)
    bt = np.array([table + [0] * (nb - len(table))])
    return oracle.decode(q[None], kp, vp, bt, [n], scale, window, bs)[0]


def pin_mask_sets_decode():
    """q = 0 makes every visible score equal, so o = mean of V over exactly the
    attended positions. The expected sets are written out by hand."""
    rng = np.random.default_rng(3)
    hkv, d, L = 2, 3, 40
    fk = rng.normal(size=(L, hkv, d))
    fv = rng.normal(size=(L, hkv, d))
    q = np.zeros((4, d))  # 4 query heads on 2 KV heads
    cases = [
        (40, 0, list(range(0, 40))),      # full attention over 40 tokens
        (40, 16, list(range(24, 40))),    # last 16 positions, including the query's own
        (40, 1, [39]),                    # window 1: only itself
        (17, 5, [12, 13, 14, 15, 16]),    # per-row length shorter than the cache
        (7, 100, list(range(0, 7))),      # window wider than the context
    ]
    for n, w, expect in cases:
        out = _one_row_decode(fk, fv, q, n, w)
        for h in range(4):
            kvh = h // 2
            np.testing.assert_allclose(out[h], fv[expect, kvh, :].mean(axis=0), atol=1e-12,
                                       err_msg=f"n={n} w={w} h={h}")


def pin_window_limits():
    """W = 1 gives the newest V row; W >= n gives exactly the full result."""
    rng = np.random.default_rng(4)
    hkv, d, L = 1, 8, 23
    fk = rng.normal(size=(L, hkv, d))
    fv = rng.normal(size=(L, hkv, d))
    q = rng.normal(size=(2, d))
    out = _one_row_decode(fk, fv, q, L, 1)
    np.testing.assert_array_equal(out[0], fv[L - 1, 0])
    np.testing.assert_array_equal(out[1], fv[L - 1, 0])
    full = _one_row_decode(fk, fv, q, L, 0)
    for w in (L, L + 1, 1000):
        np.testing.assert_array_equal(_one_row_decode(fk, fv, q, L, w), full)


def pin_gqa_mapping():
    """Head h reads KV head h // G: make KV heads distinguishable by V alone."""
    d, L, hkv, hq = 4, 9, 3, 6
    fk = np.zeros((L, hkv, d))
    fv = np.zeros((L, hkv, d))
    for j in range(hkv):
        fv[:, j, :] = 10.0 * (j + 1)
    q = np.random.default_rng(5).normal(size=(hq, d))
    out = _one_row_decode(fk, fv, q, L, 0)
    for h in range(hq):
        np.testing.assert_allclose(out[h], 10.0 * (h // 2 + 1), atol=1e-12)


def pin_paged_equals_flat_brute_force():
    """Paged decode over a permuted pool == scalar brute force on the flat K/V."""
    rng = np.random.default_rng(11)
    hkv, hq, d, L = 2, 4, 6, 13
    fk = rng.normal(size=(L, hkv, d)) * 0.5
    fv = rng.normal(size=(L, hkv, d))
    q = rng.normal(size=(hq, d))
    for n, w in ((13, 0), (13, 5), (1, 0), (2, 0), (3, 0), (9, 4)):
        out = _one_row_decode(fk, fv, q, n, w, scale=0.41, seed=n + w)
        lo = max(0, n - w) if w else 0
        for h in range(hq):
            kvh = h // 2
            ref = brute_force(q[h], fk[lo:n, kvh], fv[lo:n, kvh], 0.41)
            np.testing.assert_allclose(out[h], ref, atol=1e-12)


def pin_shared_prefix_equals_private_copy():
    """Two rows with the same data, one sharing physical prefix blocks with a
    third row, one with private copies: outputs are bit-identical (mlx-node
    paged-cache doc: requests share refcounted blocks for a common prefix)."""
    rng = np.random.default_rng(12)
    bs, nb, hkv, d = 4, 32, 1, 5
    fk = rng.normal(size=(14, hkv, d))
    fv = rng.normal(size=(14, hkv, d))
    q = rng.normal(size=(1, 2, d))
    shared = [5, 9]              # blocks holding positions 0..7
    row_a = shared + [3, 17]     # shares blocks 5 and 9
    row_b = [20, 21, 3 + 20, 17 + 7]  # private copies of everything
    kp = np.full((nb, hkv, bs, d), np.nan)
    vp = np.full((nb, hkv, bs, d), np.nan)
    for tbl in (row_a, row_b):
        for p in range(14):
            kp[tbl[p // bs], :, p % bs] = fk[p]
            vp[tbl[p // bs], :, p % bs] = fv[p]
    bt = np.array([row_a, row_b])
    out = oracle.decode(np.concatenate([q, q]), kp, vp, bt, [14, 14], 0.5, 0, bs)
    np.testing.assert_array_equal(out[0], out[1])


def pin_placement_invariance():
    rng = np.random.default_rng(13)
    hkv, d, L = 2, 4, 21
    fk = rng.normal(size=(L, hkv, d))
    fv = rng.normal(size=(L, hkv, d))
    q = rng.normal(size=(4, d))
    a = _one_row_decode(fk, fv, q, L, 0, seed=1)
    b = _one_row_decode(fk, fv, q, L, 0, seed=2)
    np.testing.assert_array_equal(a, b)


def pin_write_then_gather_roundtrip():
    """kv_write through a slot mapping, then gather, returns the rows written,
    and leaves every other pool element bit-identical (NaN canaries)."""
    rng = np.random.default_rng(14)
    nb, hkv, bs, d = 16, 2, 4, 3
    kp = np.full((nb, hkv, bs, d), np.nan, dtype=np.float32)
    vp = np.full((nb, hkv, bs, d), np.nan, dtype=np.float32)
    table = [7, 2, 11]
    n = 10
    new_k = rng.normal(size=(n + 2, hkv, d)).astype(np.float32)
    new_v = rng.normal(size=(n + 2, hkv, d)).astype(np.float32)
    real = [table[p // bs] * bs + p % bs for p in range(n)]
    slots = real[:3] + [-7] + real[3:6] + [-1] + real[6:]      # padding tokens in the middle
    src = [0, 1, 2, 4, 5, 6, 8, 9, 10, 11]                      # token index holding position p
    k2, v2 = oracle.kv_write(kp, vp, new_k, new_v, slots, bs)
    bt = np.array(table)
    np.testing.assert_array_equal(oracle.gather_positions(k2, bt, range(n), bs), new_k[src])
    np.testing.assert_array_equal(oracle.gather_positions(v2, bt, range(n), bs), new_v[src])
    touched = np.zeros((nb, bs), dtype=bool)
    for p in range(n):
        touched[table[p // bs], p % bs] = True
    k2t, v2t = k2.transpose(0, 2, 1, 3), v2.transpose(0, 2, 1, 3)   # [nb][bs][hkv][d]
    assert np.all(np.isnan(k2t[~touched])) and np.all(np.isnan(v2t[~touched]))
    assert np.all(~np.isnan(k2t[touched])) and np.all(~np.isnan(v2t[touched]))


def pin_write_skips_the_null_block():
    """A slot inside block 0 (the shared null sentinel) writes nothing; the
    other tokens of the same call are written."""
    nb, hkv, bs, d = 4, 1, 4, 2
    kp = np.full((nb, hkv, bs, d), np.nan, dtype=np.float32)
    vp = kp.copy()
    new = np.arange(3 * hkv * d, dtype=np.float32).reshape(3, hkv, d)
    k2, v2 = oracle.kv_write(kp, vp, new, new + 100, [2, 9, 3], bs)   # slots 2, 3 lie in block 0
    assert np.all(np.isnan(k2[0])) and np.all(np.isnan(v2[0]))
    np.testing.assert_array_equal(k2[2, :, 1], new[1])
    np.testing.assert_array_equal(v2[2, :, 1], new[1] + 100)
    assert np.isnan(k2).sum() == k2.size - hkv * d


def pin_null_block_never_read():
    rng = np.random.default_rng(15)
    nb, hkv, bs, d = 8, 1, 4, 2
    kp = rng.normal(size=(nb, hkv, bs, d))
    kp[0] = np.nan
    vp = kp.copy()
    # Sliding row: blocks 0..2 dropped (null), live from position 12.
    bt = np.array([[0, 0, 0, 5, 6, 0, 0, 0]])
    out = oracle.decode(np.ones((1, 1, d)), kp, vp, bt, [20], 1.0, 7, bs)
    assert np.all(np.isfinite(out))
    with pytest.raises(ValueError):
        oracle.decode(np.ones((1, 1, d)), kp, vp, bt, [20], 1.0, 9, bs)


def _prefill_setup(P, C, window, seed, hkv=2, hq=4, d=6, bs=4):
    rng = np.random.default_rng(seed)
    L = P + C
    fk = rng.normal(size=(L, hkv, d))
    fv = rng.normal(size=(L, hkv, d))
    nb = -(-L // bs) + 5
    table = list(rng.permutation(np.arange(1, nb))[: -(-L // bs)])
    kp, vp = scatter_flat(fk, fv, table, nb, bs)
    return fk, fv, kp, vp, np.array([table]), rng.normal(size=(C, hq, d))


def pin_prefill_mask_sets():
    """q = 0: query i at position P+i averages V over [lo, P+i] exactly."""
    P, C, bs = 10, 6, 4
    for window, spans in ((0, [(0, P + i) for i in range(C)]),
                          (4, [(P + i - 3, P + i) for i in range(C)])):
        fk, fv, kp, vp, bt, _ = _prefill_setup(P, C, window, 21)
        q = np.zeros((C, 4, 6))
        out = oracle.prefill_chunk(q, kp, vp, bt, [0, C], [P + C], 0.3, window, bs)
        for i, (lo, hi) in enumerate(spans):
            for h in range(4):
                np.testing.assert_allclose(out[i, h], fv[lo:hi + 1, h // 2].mean(axis=0), atol=1e-12)


def pin_prefill_chunk_of_one_is_decode():
    P, bs = 17, 4
    for window in (0, 6):
        fk, fv, kp, vp, bt, q = _prefill_setup(P, 1, window, 22)
        pre = oracle.prefill_chunk(q, kp, vp, bt, [0, 1], [P + 1], 0.3, window, bs)
        dec = oracle.decode(q, kp, vp, bt, [P + 1], 0.3, window, bs)
        np.testing.assert_allclose(pre[0], dec[0], atol=1e-13)


def pin_prefill_split_chunk():
    """Chunk C split as C1 + C2 (the second with prefix P + C1) gives the same
    per-query results; the mlx-node paged-cache doc notes chunked prefill is
    mathematically equivalent to one pass (not bit-identical)."""
    P, C, C1, bs = 9, 11, 4, 4
    for window in (0, 5):
        fk, fv, kp, vp, bt, q = _prefill_setup(P, C, window, 23)
        whole = oracle.prefill_chunk(q, kp, vp, bt, [0, C], [P + C], 0.3, window, bs)
        first = oracle.prefill_chunk(q[:C1], kp, vp, bt, [0, C1], [P + C1], 0.3, window, bs)
        second = oracle.prefill_chunk(q[C1:], kp, vp, bt, [0, C - C1], [P + C], 0.3, window, bs)
        np.testing.assert_allclose(np.concatenate([first, second]), whole, atol=1e-13)


def pin_prefill_brute_force_two_rows():
    """Two requests in one varlen call: each query == brute force on its flat K/V."""
    rng = np.random.default_rng(24)
    bs, hkv, hq, d = 4, 1, 2, 3
    lens = [(5, 3), (0, 4)]        # (prefix P, chunk C) per row
    nb = 20
    perm = list(rng.permutation(np.arange(1, nb)))
    kp = np.full((nb, hkv, bs, d), np.nan)
    vp = np.full((nb, hkv, bs, d), np.nan)
    tables, flats = [], []
    for P, C in lens:
        L = P + C
        nblk = -(-L // bs)
        tbl = [perm.pop() for _ in range(nblk)]
        fk = rng.normal(size=(L, hkv, d))
        fv = rng.normal(size=(L, hkv, d))
        for p in range(L):
            kp[tbl[p // bs], :, p % bs] = fk[p]
            vp[tbl[p // bs], :, p % bs] = fv[p]
        tables.append(tbl + [0] * (4 - nblk))
        flats.append((fk, fv))
    q = rng.normal(size=(7, hq, d))
    out = oracle.prefill_chunk(q, kp, vp, np.array(tables), [0, 3, 7], [8, 4], 0.7, 0, bs)
    row = 0
    for b, (P, C) in enumerate(lens):
        fk, fv = flats[b]
        for i in range(C):
            for h in range(hq):
                ref = brute_force(q[row, h], fk[:P + i + 1, 0], fv[:P + i + 1, 0], 0.7)
                np.testing.assert_allclose(out[row, h], ref, atol=1e-12)
            row += 1


def pin_prefill_blocked_query_rows():
    """Query blocking and the query_rows subset: with blocks of 3 rows (and with
    the default 256-row blocks over a 300-row chunk), every computed row equals
    scalar brute force on its own flat K/V span [lo, P+i], and rows outside the
    subset are left NaN."""
    rng = np.random.default_rng(25)
    bs, hkv, hq, d = 4, 1, 2, 3
    for P, C, window, q_block, rows in ((13, 10, 0, 3, [0, 2, 3, 5, 7, 8, 9]),
                                        (13, 10, 5, 3, [1, 4, 6, 9]),
                                        (7, 300, 0, 256, [0, 1, 255, 256, 257, 299]),
                                        (7, 300, 9, 256, [3, 254, 256, 298])):
        L = P + C
        nblk = -(-L // bs)
        nb = nblk + 3
        table = list(rng.permutation(np.arange(1, nb))[:nblk])
        fk = rng.normal(size=(L, hkv, d))
        fv = rng.normal(size=(L, hkv, d))
        kp, vp = scatter_flat(fk, fv, table, nb, bs)
        q = rng.normal(size=(C, hq, d))
        out = oracle.prefill_chunk(q, kp, vp, np.array([table]), [0, C], [L], 0.6, window, bs,
                                   query_rows=rows, q_block=q_block)
        for i in range(C):
            if i not in rows:
                assert np.all(np.isnan(out[i])), f"row {i} outside the subset was computed"
                continue
            a = P + i
            lo = max(0, a - window + 1) if window else 0
            for h in range(hq):
                ref = brute_force(q[i, h], fk[lo:a + 1, 0], fv[lo:a + 1, 0], 0.6)
                np.testing.assert_allclose(out[i, h], ref, atol=1e-12, err_msg=f"row {i} head {h}")


def pin_pool_block_bytes():
    """mlx-node paged-cache doc, cold-tier writer table: a qwen3-0.6b block is
    1.84 MB. With that model's public geometry (28 layers, 8 KV heads, head_dim
    128, bf16) and block size 16, K+V across layers is 2*16*8*128*2*28 bytes;
    the same doc's capture budget equates 128 blocks with 2048 tokens at block 16."""
    per_layer = 2 * 16 * 8 * 128 * 2
    assert per_layer * 28 == 1_835_008
    assert round(per_layer * 28 / 1e6, 2) == 1.84
    assert 128 * 16 == 2048


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ----------------------------------------------------------------- mutants
def _mut_no_scale(q, keys, values, scale):
    return _orig_attend(q, keys, values, 1.0)


def _mut_no_max(q, keys, values, scale):
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros(values.shape[-1])
    p = np.exp(scale * (keys @ q))
    return (p @ values) / p.sum()


def _mut_drop_last(q, keys, values, scale):
    return _orig_attend(q, keys[:-1] if len(keys) > 1 else keys,
                        values[:-1] if len(values) > 1 else values, scale)


_orig_attend = A.attend_one
_orig_dec_range = A.decode_attended_range
_orig_pre_range = A.prefill_attended_range
_orig_gather = A.gather_positions

MUTANTS = {
    "attend: scale dropped": ("attend_one", _mut_no_scale),
    "attend: no max subtraction": ("attend_one", _mut_no_max),
    "attend: last key dropped": ("attend_one", _mut_drop_last),
    "decode window off by one": ("decode_attended_range",
                                 lambda n, w: (max(0, n - w + 1) if w > 0 else 0, n)),
    "decode excludes own token": ("decode_attended_range",
                                  lambda n, w: (_orig_dec_range(n, w)[0], max(0, n - 1))),
    "prefill window off by one": ("prefill_attended_range",
                                  lambda a, w: (max(0, a - w) if w > 0 else 0, a + 1)),
    "prefill not causal inside chunk": ("prefill_attended_range",
                                        lambda a, w: (_orig_pre_range(a, w)[0], a + 2)),
    "gather offset swapped": ("gather_positions",
                              lambda pool, bt, pos, bs: np.stack(
                                  [pool[int(bt[int(p) // bs]), :, (int(p) + 1) % bs, :] for p in pos])
                              if len(list(pos)) else _orig_gather(pool, bt, pos, bs)),
    "gather ignores table": ("gather_positions",
                             lambda pool, bt, pos, bs: np.stack(
                                 [pool[1 + int(p) // bs, :, int(p) % bs, :] for p in pos])
                             if len(list(pos)) else _orig_gather(pool, bt, pos, bs)),
}


def _mut_gqa(q, k_pool, v_pool, block_tables, seq_lens, scale, window, block_size):
    # head h reads KV head h % Hkv instead of h // G
    q = np.asarray(q, dtype=np.float64)
    Bq, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    out = np.zeros((Bq, Hq, D))
    for b in range(Bq):
        n = int(seq_lens[b])
        lo, hi = A.decode_attended_range(n, window)
        keys = A.gather_positions(k_pool, block_tables[b], range(lo, hi), block_size)
        vals = A.gather_positions(v_pool, block_tables[b], range(lo, hi), block_size)
        for h in range(Hq):
            out[b, h] = A.attend_one(q[b, h], keys[:, h % Hkv], vals[:, h % Hkv], scale)
    return out


MUTANTS["decode GQA map h % Hkv"] = ("decode", _mut_gqa)


def _mut_write_skips_last(k_pool, v_pool, new_k, new_v, slot_mapping, block_size):
    return _orig_write(k_pool, v_pool, new_k[:-1], new_v[:-1], list(slot_mapping)[:-1], block_size)


_orig_write = A.kv_write
MUTANTS["write drops the last token"] = ("kv_write", _mut_write_skips_last)


def _prefill_variant(shift_later_blocks=0, subset_index=False):
    """prefill_chunk with a blocking slip: rows of every block after the first
    shifted by ``shift_later_blocks`` positions, or each row's position taken
    from its index inside the query_rows subset instead of the chunk."""
    def f(q, k_pool, v_pool, block_tables, cu_q_lens, seq_lens, scale, window, block_size,
          query_rows=None, q_block=256):
        q = np.asarray(q, dtype=np.float64)
        T, Hq, D = q.shape
        group = Hq // k_pool.shape[1]
        out = np.full((T, Hq, D), np.nan)
        wanted = None if query_rows is None else set(int(r) for r in query_rows)
        for b in range(len(seq_lens)):
            r0, r1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
            P = int(seq_lens[b]) - (r1 - r0)
            rows = [r for r in range(r0, r1) if wanted is None or r in wanted]
            for i0 in range(0, len(rows), q_block):
                blk = rows[i0:i0 + q_block]
                pos = [(i0 + j if subset_index else r - r0) + (shift_later_blocks if i0 else 0)
                       for j, r in enumerate(blk)]
                for r, i in zip(blk, pos):
                    lo, hi = A.prefill_attended_range(P + i, window)
                    hi = min(hi, int(seq_lens[b]))
                    keys = A.gather_positions(k_pool, block_tables[b], range(lo, hi), block_size)
                    vals = A.gather_positions(v_pool, block_tables[b], range(lo, hi), block_size)
                    for h in range(Hq):
                        out[r, h] = A.attend_one(q[r, h], keys[:, h // group], vals[:, h // group], scale)
        return out
    return f


MUTANTS["prefill later query blocks shifted by one row"] = ("prefill_chunk", _prefill_variant(shift_later_blocks=-1))
MUTANTS["prefill query_rows position from the subset index"] = ("prefill_chunk", _prefill_variant(subset_index=True))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    monkeypatch.setattr(oracle, attr, fn, raising=False)
    failures = 0
    for pin in PINS:
        try:
            pin()
        except (Exception, pytest.fail.Exception):
            failures += 1
    assert failures > 0, f"no pin catches the mutant '{name}'"
