"""Request lifecycle on the GPU: prefix reuse, grow-on-demand pools and LRU
eviction (paged-cache doc: component table, pool-sizing section: grow before
evicting).

The C++ allocator drives the device pools; the oracle allocator replays every
call and must return the same tables, slots and refcounts. After each phase
the decode kernels run over the device pools and are checked against plain
attention over each request's logical K/V (no tables), from the oracle.
Requests that share a token prefix share its K/V (same tokens at the same
positions give the same K/V in any model), so a reused block must hold
exactly the values the request would have written itself.
"""

import numpy as np
import pytest

import runner
import synth
from oracle import RefAllocator
from oracle.attention import attend_one
from test_gpu_parity import announce, pk  # noqa: F401 (pk: fixture)

BS, HKV, HQ, D, DOM = 16, 2, 4, 128, 7


@pytest.mark.gpu
def test_request_lifecycle_prefix_reuse_grow_and_eviction(pk):
    import torch

    announce("lifecycle: prefix reuse, grow, eviction")
    rng = np.random.default_rng(1007)
    scale = 1.0 / np.sqrt(D)
    dev = torch.device("cuda")

    def kv(n):
        k = synth.round_bf16(rng.standard_normal((n, HKV, D), dtype=np.float32))
        v = synth.round_bf16(rng.standard_normal((n, HKV, D), dtype=np.float32))
        return k, v

    order = [int(x) for x in rng.permutation(np.arange(1, 8))]
    cpp = pk.Allocator(8, BS, order)
    ref = RefAllocator(8, BS, order)
    pools = {n: torch.zeros((8, HKV, BS, D), dtype=torch.bfloat16, device=dev) for n in "kv"}
    logical = {}  # seq -> (k, v) over its positions

    def both(fn, *args):
        a = getattr(cpp, fn)(*args)
        b = getattr(ref, fn)(*args)
        assert a == b, (fn, args, a, b)
        return a

    def both_fail(fn, *args):
        for alloc in (cpp, ref):
            with pytest.raises(Exception) as e:
                getattr(alloc, fn)(*args)
            assert e.value.code == pk.PAGED_ERR_NO_BLOCKS

    def write(seq, start, k, v):
        slots = cpp.slot_mapping(seq, start, len(k))
        assert list(slots) == list(ref.slot_mapping(seq, start, len(k)))
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)  # noqa: E731
        pk.paged_kv_write(pools["k"], pools["v"], t(k), t(v), torch.from_numpy(slots).to(dev))

    def check(seqs):
        mb = max(cpp.num_blocks_of(s) for s in seqs)
        tab = cpp.block_tables(seqs, mb)
        assert [list(r) for r in tab] == [list(r) for r in ref.block_tables(seqs, mb)]
        n = [cpp.num_tokens(s) for s in seqs]
        assert n == [ref.num_tokens(s) for s in seqs]
        for b in range(1, cpp.nb):
            assert cpp.refcount(b) == ref.refcount(b)
        q = synth.round_bf16(rng.standard_normal((len(seqs), HQ, D), dtype=np.float32))
        msl = max(n)
        need = pk.paged_attn_decode_workspace_bytes(len(seqs), HQ, HKV, D, BS, msl, 0, 0, "bf16")
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        out = torch.empty((len(seqs), HQ, D), dtype=torch.bfloat16, device=dev)
        pk.paged_attn_decode(out, torch.from_numpy(q).to(dev).to(torch.bfloat16), pools["k"], pools["v"],
                             torch.from_numpy(tab).to(dev), torch.tensor(n, dtype=torch.int32, device=dev),
                             scale, msl, workspace=ws)
        torch.cuda.synchronize()
        exp = np.zeros((len(seqs), HQ, D))
        for i, s in enumerate(seqs):
            k, v = logical[s]
            for h in range(HQ):
                g = h // (HQ // HKV)
                exp[i, h] = attend_one(q[i, h], k[:n[i], g], v[:n[i], g], scale)
        max_abs, rel = runner.compare(out, exp, "bf16")
        assert runner.within("bf16", max_abs, rel), (seqs, max_abs, rel)

    # A: 100 tokens (6 full blocks published, a partial seventh), the pool's 7 usable blocks
    tok_a = list(range(1000, 1100))
    ka, va = kv(100)
    both("add", 1)
    assert both("match_prefix", 1, tok_a, DOM) == 0
    both("reserve", 1, 100)
    write(1, 0, ka, va)
    both("commit_tokens", 1, tok_a)
    both("publish_full_blocks", 1, DOM)
    logical[1] = (ka, va)
    check([1])

    # B: A's first 48 tokens, then 12 of its own; the prefix is found, the new
    # block does not fit: with a maximum of 16 blocks the reservation asks for
    # growth to min(16, max(2 * 8, 8 + 1)) = 16 blocks, the pools grow, and the
    # one retry reserves
    tok_b = tok_a[:48] + list(range(2000, 2012))
    kb_own, vb_own = kv(12)
    both("add", 2)
    assert both("match_prefix", 2, tok_b, DOM) == 48
    both_fail("reserve", 2, 60)
    both_fail("reserve_or_grow", 2, 60)          # a fixed pool (maximum = size) cannot grow
    both("set_max_blocks", 16)
    grow_to = both("reserve_or_grow", 2, 60)
    assert grow_to == 16 and cpp.num_free() == (0, 0)
    for name in "kv":
        bigger = torch.zeros((grow_to, HKV, BS, D), dtype=torch.bfloat16, device=dev)
        bigger[:8] = pools[name]
        pools[name] = bigger
    order2 = [int(x) for x in rng.permutation(np.arange(8, grow_to))]
    both("grow", grow_to, order2)
    both("reserve", 2, 60)
    write(2, 48, kb_own, vb_own)
    both("commit_tokens", 2, tok_b[48:])
    logical[2] = (np.concatenate([ka[:48], kb_own]), np.concatenate([va[:48], vb_own]))
    check([1, 2])

    # A leaves: its three blocks that B shares stay, the other published ones
    # become evictable (the release walks A's table from its last entry), the
    # partial one is freed
    both("release", 1)
    free, evictable = cpp.num_free()
    assert (free, evictable) == ref.num_free() and evictable == 3

    # C: unrelated tokens, two blocks more than the free list holds, so the
    # two least recently released of A's blocks are evicted
    n_c = (free + 2) * BS - 5
    tok_c = list(range(3000, 3000 + n_c))
    kc, vc = kv(n_c)
    both("add", 3)
    assert both("match_prefix", 3, tok_c, DOM) == 0
    both("reserve", 3, n_c)
    write(3, 0, kc, vc)
    both("commit_tokens", 3, tok_c)
    both("publish_full_blocks", 3, DOM)
    logical[3] = (kc, vc)
    assert cpp.num_free() == ref.num_free() == (0, 1)
    check([2, 3])

    # C leaves too: its full blocks become evictable, its partial one free
    both("release", 3)
    assert cpp.num_free() == ref.num_free() == (1, free + 2)

    # D: A's first 96 tokens and 4 more; A's fourth block survived the
    # eviction, its fifth and sixth did not, so 64 tokens are found and the
    # rest are written again (the same K/V, as the tokens are the same) into
    # the free block and two of C's
    tok_d = tok_a[:96] + list(range(4000, 4004))
    kd_own, vd_own = kv(4)
    both("add", 4)
    assert both("match_prefix", 4, tok_d, DOM) == 64
    both("reserve", 4, 100)
    kd = np.concatenate([ka[:96], kd_own])
    vd = np.concatenate([va[:96], vd_own])
    write(4, 64, kd[64:], vd[64:])
    both("commit_tokens", 4, tok_d[64:])
    logical[4] = (kd, vd)
    check([2, 4])


@pytest.mark.gpu
@pytest.mark.parametrize("kv,window", [("bf16", 0), ("fp8", 0), ("bf16", 48)])
def test_continuous_batching_steps(pk, kv, window):
    # Two requests served over five steps with paged_attn_mixed: X's 150-token
    # prompt in chunks of 64, 64 and 22 while Y (a 40-token prompt, one chunk)
    # decodes beside it; then both decode. Each step reserves and writes its
    # new tokens' K/V (allocator slots, paged_kv_write) before attention, and
    # every query of the step is checked against attention over the request's
    # logical K/V up to its own position. Over FP8 pools the logical K/V are
    # the values the codes stand for (the oracle's quantizer, then scale x
    # code). With a sliding window every request drops its blocks that fell
    # out of the window before a step commits new tokens (null table entries
    # the kernels must skip).
    import torch

    from oracle import fp8 as ofp8

    announce(f"continuous batching over five steps ({kv}, window {window})")
    fp8 = kv == "fp8"
    ks, vs = (np.float32(4.0 / 448), np.float32(3.5 / 448)) if fp8 else (1.0, 1.0)
    rng = np.random.default_rng(1008)
    scale = 1.0 / np.sqrt(D)
    dev = torch.device("cuda")
    order = [int(x) for x in rng.permutation(np.arange(1, 40))]
    cpp = pk.Allocator(40, BS, order)
    ref = RefAllocator(40, BS, order)
    pdt = torch.float8_e4m3fn if fp8 else torch.bfloat16
    pools = {n: torch.zeros((40, HKV, BS, D), dtype=pdt, device=dev) for n in "kv"}
    k_log = {1: np.zeros((0, HKV, D)), 2: np.zeros((0, HKV, D))}
    v_log = {1: k_log[1].copy(), 2: k_log[2].copy()}
    for s in (1, 2):
        cpp.add(s)
        ref.add(s)
    # (request, new tokens) per step, decode rows first
    steps = [[(2, 40), (1, 64)], [(2, 1), (1, 64)], [(2, 1), (1, 22)], [(2, 1), (1, 1)], [(1, 1), (2, 1)]]
    next_tok = {1: 10_000, 2: 20_000}
    for i, rows in enumerate(steps):
        nd = sum(1 for s, c in rows if c == 1 and cpp.num_tokens(s) > 0)
        starts, qs = [], []
        for s, c in rows:
            start = cpp.num_tokens(s)
            assert start == ref.num_tokens(s)
            if window:
                for alloc in (cpp, ref):
                    alloc.drop_outside_window(s, window)
            for alloc in (cpp, ref):
                alloc.reserve(s, start + c)
            k_new = synth.round_bf16(rng.standard_normal((c, HKV, D), dtype=np.float32))
            v_new = synth.round_bf16(rng.standard_normal((c, HKV, D), dtype=np.float32))
            slots = cpp.slot_mapping(s, start, c)
            assert list(slots) == list(ref.slot_mapping(s, start, c))
            t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)  # noqa: E731
            if fp8:
                pk.paged_kv_write_fp8(pools["k"], pools["v"], t(k_new), t(v_new), torch.from_numpy(slots).to(dev),
                                      float(ks), float(vs))
                k_new = ofp8.dequantize(ofp8.quantize(k_new, ks), ks)
                v_new = ofp8.dequantize(ofp8.quantize(v_new, vs), vs)
            else:
                pk.paged_kv_write(pools["k"], pools["v"], t(k_new), t(v_new), torch.from_numpy(slots).to(dev))
            toks = list(range(next_tok[s], next_tok[s] + c))
            next_tok[s] += c
            for alloc in (cpp, ref):
                alloc.commit_tokens(s, toks)
            k_log[s] = np.concatenate([k_log[s], k_new])
            v_log[s] = np.concatenate([v_log[s], v_new])
            starts.append(start)
            qs.append(synth.round_bf16(rng.standard_normal((c, HQ, D), dtype=np.float32)))
        seqs = [s for s, _ in rows]
        counts = [c for _, c in rows]
        lens = [cpp.num_tokens(s) for s in seqs]
        mb = max(cpp.num_blocks_of(s) for s in seqs)
        tab = cpp.block_tables(seqs, mb)
        assert [list(r) for r in tab] == [list(r) for r in ref.block_tables(seqs, mb)]
        q = np.concatenate(qs)
        cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        msl = max(lens)
        need = pk.paged_attn_decode_workspace_bytes(max(nd, 1), HQ, HKV, D, BS, msl, window, 0, kv)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        out = torch.empty((int(cu[-1]), HQ, D), dtype=torch.bfloat16, device=dev)
        pk.paged_attn_mixed(out, torch.from_numpy(q).to(dev).to(torch.bfloat16), pools["k"], pools["v"],
                            torch.from_numpy(tab).to(dev), torch.from_numpy(cu).to(dev),
                            torch.tensor(lens, dtype=torch.int32, device=dev), nd,
                            max(c for _, c in rows), scale, msl, sliding_window=window, workspace=ws,
                            k_scale=float(ks), v_scale=float(vs))
        torch.cuda.synchronize()
        exp = np.zeros((int(cu[-1]), HQ, D))
        for r, (s, c) in enumerate(rows):
            for j in range(c):
                a = starts[r] + j  # absolute position of this query
                lo = max(0, a - window + 1) if window else 0
                for h in range(HQ):
                    g = h // (HQ // HKV)
                    exp[cu[r] + j, h] = attend_one(q[cu[r] + j, h], k_log[s][lo:a + 1, g], v_log[s][lo:a + 1, g],
                                                   scale)
        max_abs, rel = runner.compare(out, exp, "bf16")
        assert runner.within("bf16", max_abs, rel), (i, max_abs, rel)
        if window and i >= 1:
            # the chunked request's first block expired and is a null entry
            assert tab[seqs.index(1)][0] == 0
