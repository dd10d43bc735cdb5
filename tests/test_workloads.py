"""CPU checks of the synthetic workloads' paging (no GPU).

The hybrid chunked-prefill workload pages three layers through two pools: a
sliding layer whose expired blocks are null entries in its tables, a full
layer, and a KV-shared layer that reads the full layer's pool and tables.
The oracle run through those tables must equal plain windowed attention over
the workload's logical (flat) K/V, computed here without any table.
"""

import numpy as np

import runner
import synth
from oracle import RefAllocator


def flat_attention(q, k, v, lo, hi, scale):
    """softmax(scale * q.k) v over key positions [lo, hi] of flat k/v, float64."""
    kk = k[lo:hi + 1].astype(np.float64)
    vv = v[lo:hi + 1].astype(np.float64)
    s = scale * (kk @ q.astype(np.float64))
    w = np.exp(s - s.max())
    return (w[:, None] * vv).sum(0) / w.sum()


def test_hybrid_prefill_paging_matches_flat_attention():
    wl = synth.make("hprefill", batch=3, context=[200, 0, 77], chunk=[40, 25, 1], window=24,
                    num_blocks=80, sliding_blocks=40, hq=4)
    tabs = synth.build_tables(RefAllocator, wl)
    # the sliding layer's expired blocks really are null entries
    st = tabs["sliding"]["tables"]
    assert (st[0][:(200 - 24) // wl.block_size] == 0).all()
    pools = runner.oracle_setup(wl, tabs)
    out = runner.oracle_step(wl, pools)
    G = wl.hq // wl.hkv
    cu = np.concatenate([[0], np.cumsum(wl.chunk_lens)])
    for L in wl.layers:
        src = wl.layer(L.alias_of) if L.alias_of else L
        for b in range(wl.batch):
            C = int(wl.chunk_lens[b])
            P = int(wl.seq_lens[b]) - C
            off = src.live_from[b]
            for i in range(C):
                a = P + i
                lo = max(0, a - L.window + 1) if L.window else 0
                t = int(cu[b]) + i
                for h in range(wl.hq):
                    kvh = h // G
                    exp = flat_attention(L.q[t, h], src.k[b][:, kvh], src.v[b][:, kvh], lo - off, a - off,
                                         wl.scale)
                    np.testing.assert_allclose(out[L.name][t, h], exp, rtol=0, atol=1e-12,
                                               err_msg=f"{L.name} row {b} query {i} head {h}")


def test_hybrid_prefill_shapes():
    wl = synth.make("hprefill")
    assert (wl.batch, wl.hq, wl.hkv, wl.head_dim) == (4, 8, 1, 256)
    assert wl.chunk_lens.tolist() == [2048] * 4 and wl.seq_lens.tolist() == [8192] * 4
    assert [L.name for L in wl.layers] == ["sliding", "full", "shared"]
    assert wl.layer("sliding").window == 512 and wl.layer("shared").alias_of == "full"


def test_growing_keys_are_exact_powers_of_two_of_the_plain_draws():
    # k_growth scales the key at position t by 2^min(t // g, 12) and changes nothing else
    for name, kw in [("prefill", dict(batch=2, context=[300, 64], chunk=[150, 100], num_blocks=64)),
                     ("mixed", dict(batch=3, context=(20, 400), prefix=100, num_blocks=100)),
                     ("hprefill", dict(batch=2, context=[300, 700], chunk=[100, 37], window=64,
                                       num_blocks=200, sliding_blocks=64))]:
        a = synth.make(name, **kw)
        g = synth.make(name, k_growth=32, **kw)
        for La, Lg in zip(a.layers, g.layers):
            if La.alias_of:
                assert Lg.alias_of == La.alias_of
                continue
            np.testing.assert_array_equal(La.q, Lg.q)
            for xa, xg, va, vg, lf in zip(La.k, Lg.k, La.v, Lg.v, La.live_from):
                np.testing.assert_array_equal(va, vg)
                f = np.exp2(np.minimum((lf + np.arange(len(xa))) // 32, 12)).astype(np.float32)
                np.testing.assert_array_equal(xg, xa * f[:, None, None])
    # the largest score of a long row does grow past the kernels' rescale threshold (2^8)
    wl = synth.make("prefill", batch=1, context=[300], chunk=[100], num_blocks=64, k_growth=32)
    k = wl.layers[0].k[0][:, 0].astype(np.float64)
    q = wl.layers[0].q[-1, 0].astype(np.float64)
    s = wl.scale * (k @ q) / np.log(2.0)
    running = np.maximum.accumulate(s)
    assert np.count_nonzero(np.diff(running) > 8.0) >= 2
