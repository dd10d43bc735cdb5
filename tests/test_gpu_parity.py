"""GPU parity: the HIP path against the float64 oracle, through the C ABI.

Bit-exact for the KV write, the gather and the block tables; attention within
max-abs 1e-5 (fp32) or max-abs 2e-2 and relative L2 5e-3 (bf16). Every case
prints its name before touching the GPU.
"""

import sys

import numpy as np
import pytest

import runner
import synth
import oracle
from oracle import RefAllocator

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pk():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_paged_kv_amd

    return block_paged_kv_amd


def announce(msg):
    print(f"\n[case] {msg}", file=sys.stderr, flush=True)


def tables_both(pk, wl, share=True):
    tc = synth.build_tables(pk.Allocator, wl, share=share)
    tr = synth.build_tables(RefAllocator, wl, share=share)
    for name in tc:
        np.testing.assert_array_equal(tc[name]["tables"], tr[name]["tables"])
        for x, y in zip(tc[name]["step_slots"], tr[name]["step_slots"]):
            np.testing.assert_array_equal(x, y)
    return tc, tr


def pool_bits(t):
    """Device pool -> float32 bit patterns (bf16 upcasts exactly)."""
    import torch

    return t.float().cpu().numpy().view(np.uint32) if t.dtype != torch.float32 else \
        t.cpu().numpy().view(np.uint32)


def check_attention(wl, outs, ref, rows=None, label=""):
    for name, o in outs.items():
        max_abs, rel = runner.compare(o, ref[name], wl.dtype, rows)
        assert np.all(np.isfinite(o.float().cpu().numpy()[rows] if rows is not None else o.float().cpu().numpy()))
        assert runner.within(wl.dtype, max_abs, rel), f"{label}/{name}: max_abs={max_abs:.3g} rel_l2={rel:.3g}"


def run_case(pk, wl, rows=None, label="", **step_kw):
    announce(f"{label} {wl.name} B={wl.batch} Hq={wl.hq} Hkv={wl.hkv} D={wl.head_dim} {wl.dtype} "
             f"lens={wl.seq_lens[:8].tolist()}")
    tc, tr = tables_both(pk, wl)
    dev = runner.gpu_setup(wl, tc)
    ws = runner.gpu_workspace(wl, dev, step_kw.get("partition_tokens"), step_kw.get("max_seq_len"))
    outs = runner.gpu_step(wl, dev, workspace=ws, **step_kw)
    import torch

    torch.cuda.synchronize()
    pools = runner.oracle_setup(wl, tr)
    ref = runner.oracle_step(wl, pools, rows=rows)
    check_attention(wl, outs, ref, rows, label)
    return wl, tc, dev, outs, pools


# --------------------------------------------------------------- write/gather
@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("qwen3", dict(context=300, prefix=64, num_blocks=200)),
    ("hybrid", dict(batch=3, context=700, window=64, sliding_blocks=40, num_blocks=200)),
    ("prefill", dict(batch=3, context=[70, 33, 0], chunk=[40, 9, 17], num_blocks=64)),
    ("mixed", dict(batch=5, context=(20, 300), prefix=100, num_blocks=200, head_dim=256, hq=4, hkv=2)),
    ("mixed", dict(batch=5, context=(20, 300), prefix=100, num_blocks=300, block_size=8)),
    ("hybrid", dict(batch=2, context=500, window=100, hq=8, hkv=1, head_dim=256, sliding_blocks=30,
                    num_blocks=100, block_size=64)),
    ("hprefill", dict(batch=2, context=[300, 700], chunk=[100, 37], window=64, num_blocks=200,
                      sliding_blocks=64)),
    ("hybrid", dict(batch=2, context=300, window=64, head_dim=512, sliding_blocks=40, num_blocks=100)),
])
def test_write_is_bit_exact(pk, name, kw):
    import torch

    wl = synth.make(name, **kw)
    announce(f"write {name}")
    tc, tr = tables_both(pk, wl)
    dev = runner.gpu_setup(wl, tc)
    runner.gpu_step(wl, dev, workspace=runner.gpu_workspace(wl, dev))
    torch.cuda.synchronize()
    pools = runner.oracle_setup(wl, tr)
    for L in wl.layers:
        if L.alias_of:
            continue
        kp, vp, _ = pools[L.name]
        np.testing.assert_array_equal(pool_bits(dev[L.name]["k_pool"]), kp.view(np.uint32))
        np.testing.assert_array_equal(pool_bits(dev[L.name]["v_pool"]), vp.view(np.uint32))


def test_write_skips_padding_and_out_of_range_slots(pk):
    import torch

    announce("write padding")
    kp = torch.full((4, 2, 16, 64), float("nan"), device="cuda")
    vp = torch.full_like(kp, float("nan"))
    new = torch.arange(5 * 2 * 64, dtype=torch.float32, device="cuda").reshape(5, 2, 64)
    slots = torch.tensor([17, -1, 4 * 16, 63, -5], dtype=torch.int64, device="cuda")
    pk.paged_kv_write(kp, vp, new, -new, slots)
    k = kp.cpu()
    assert torch.equal(k[1, :, 1], new[0].cpu()) and torch.equal(k[3, :, 15], new[3].cpu())
    assert int(torch.isnan(k).sum()) == (4 * 16 - 2) * 2 * 64
    assert torch.equal(vp.cpu()[1, :, 1], -new[0].cpu())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_write_leaves_the_null_block_alone(pk, dtype):
    """Slots inside block 0 (the shared null sentinel) write nothing: whole
    pools bit-exact against the oracle's write, NaN canaries everywhere else."""
    import torch

    announce(f"write null block {dtype}")
    rng = np.random.default_rng(5)
    nb, hkv, bs, d, T = 6, 2, 16, 128, 7
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    kp = torch.full((nb, hkv, bs, d), float("nan"), dtype=dt, device="cuda")
    vp = torch.full_like(kp, float("nan"))
    x = torch.from_numpy(rng.standard_normal((T, hkv, d)).astype(np.float32)).to(dt).cuda()
    slots = [0, 17, 15, 5 * 16 + 3, 8, -1, 2 * 16]   # 0, 15 and 8 lie in block 0
    pk.paged_kv_write(kp, vp, x, -x, torch.tensor(slots, dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    ek, ev = oracle.kv_write(kp.float().cpu().numpy() * np.nan, vp.float().cpu().numpy() * np.nan,
                             x.float().cpu().numpy(), -x.float().cpu().numpy(), slots, bs)
    got_k, got_v = kp.float().cpu().numpy(), vp.float().cpu().numpy()
    assert np.all(np.isnan(got_k[0])) and np.all(np.isnan(got_v[0]))
    np.testing.assert_array_equal(got_k, ek)
    np.testing.assert_array_equal(got_v, ev)


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("mixed", dict(batch=6, context=(20, 300), prefix=100, num_blocks=300)),
    ("hybrid", dict(batch=3, context=700, window=64, sliding_blocks=40, num_blocks=200)),
    ("hybrid", dict(batch=2, context=500, window=100, hq=4, hkv=2, head_dim=128, sliding_blocks=60,
                    num_blocks=200, block_size=8)),
    ("mixed", dict(batch=5, context=(1, 400), prefix=100, num_blocks=200, block_size=32)),
])
def test_gather_returns_flat_kv(pk, name, kw):
    import torch

    wl = synth.make(name, **kw)
    announce(f"gather {name}")
    tc, _ = tables_both(pk, wl)
    dev = runner.gpu_setup(wl, tc)
    runner.gpu_step(wl, dev, workspace=runner.gpu_workspace(wl, dev))
    for L in wl.layers:
        if L.alias_of:
            continue
        spans, offs = [], [0]
        for b in range(wl.batch):
            n = int(wl.seq_lens[b])
            lo = max(0, n - L.window) if L.window else 0
            spans.append((lo, n))
            offs.append(offs[-1] + n - lo)
        total = offs[-1]
        ok = torch.empty((total, wl.hkv, wl.head_dim), dtype=dev[L.name]["k_pool"].dtype, device="cuda")
        ov = torch.empty_like(ok)
        pk.paged_kv_gather(ok, ov, dev[L.name]["k_pool"], dev[L.name]["v_pool"], dev[L.name]["tables"],
                           dev["_seq_lens"], torch.tensor(offs[:-1], dtype=torch.int64, device="cuda"),
                           wl.max_seq_len, sliding_window=L.window)
        exp_k = np.concatenate([synth.kv_rows(wl, L, b, "k", lo, n) for b, (lo, n) in enumerate(spans)])
        exp_v = np.concatenate([synth.kv_rows(wl, L, b, "v", lo, n) for b, (lo, n) in enumerate(spans)])
        np.testing.assert_array_equal(pool_bits(ok), exp_k.view(np.uint32))
        np.testing.assert_array_equal(pool_bits(ov), exp_v.view(np.uint32))


# --------------------------------------------------------------- decode parity
DECODE_SMALL = [
    ("tiny", {}, {}),
    ("tiny", dict(dtype="bf16"), {}),
    ("tiny", {}, dict(partition_tokens=16)),
    ("qwen3", dict(context=300, prefix=64, num_blocks=200), {}),
    ("qwen3", dict(context=300, prefix=64, num_blocks=200), dict(partition_tokens=64)),
    ("mixed", dict(batch=7, context=(1, 700), prefix=200, num_blocks=400), dict(partition_tokens=128)),
    ("mixed", dict(batch=5, hq=16, hkv=1, context=(100, 600), prefix=64, num_blocks=300), {}),
    ("mixed", dict(batch=5, hq=6, hkv=1, context=(100, 600), prefix=64, num_blocks=300), dict(partition_tokens=64)),
    ("mixed", dict(batch=5, hq=6, hkv=2, head_dim=64, context=(1, 300), prefix=32, num_blocks=200), {}),
    ("mixed", dict(batch=4, hq=8, hkv=8, head_dim=256, context=(30, 400), prefix=48, num_blocks=200), dict(partition_tokens=32)),
    ("mixed", dict(batch=4, hq=8, hkv=2, head_dim=128, dtype="f32", context=(30, 400), prefix=48, num_blocks=200), {}),
    ("mixed", dict(batch=4, hq=4, hkv=2, head_dim=256, dtype="f32", context=(30, 200), prefix=48, num_blocks=100), dict(partition_tokens=48)),
    ("hybrid", dict(batch=3, context=700, window=64, sliding_blocks=40, num_blocks=200), {}),
    ("hybrid", dict(batch=3, context=700, window=1, sliding_blocks=40, num_blocks=200), {}),
    ("hybrid", dict(batch=2, context=300, window=100, hq=4, hkv=2, head_dim=128, sliding_blocks=40, num_blocks=100), dict(partition_tokens=32)),
]


# Block sizes other than 16: two blocks per 16-token stage (8) and stages inside
# a block (32, 64), with partitions and windows that start mid-block.
DECODE_BLOCK_SIZES = [
    ("mixed", dict(batch=5, context=(1, 400), prefix=100, num_blocks=400, block_size=8), dict(partition_tokens=64)),
    ("mixed", dict(batch=5, context=(1, 400), prefix=100, num_blocks=400, block_size=8), {}),
    ("mixed", dict(batch=5, context=(1, 400), prefix=100, num_blocks=200, block_size=32), {}),
    ("mixed", dict(batch=5, context=(1, 700), prefix=130, num_blocks=100, block_size=64), dict(partition_tokens=128)),
    ("mixed", dict(batch=4, hq=6, hkv=2, head_dim=64, context=(1, 300), prefix=40, num_blocks=200, block_size=32), {}),
    ("mixed", dict(batch=3, hq=4, hkv=2, head_dim=64, dtype="f32", context=(30, 300), prefix=40, num_blocks=200,
                   block_size=8), {}),
    ("mixed", dict(batch=3, hq=4, hkv=2, head_dim=128, dtype="f32", context=(30, 300), prefix=40, num_blocks=100,
                   block_size=64), dict(partition_tokens=64)),
    ("hybrid", dict(batch=2, context=500, window=100, hq=4, hkv=2, head_dim=128, sliding_blocks=60, num_blocks=200,
                    block_size=8), {}),
    ("hybrid", dict(batch=2, context=500, window=100, hq=8, hkv=1, head_dim=256, sliding_blocks=30, num_blocks=100,
                    block_size=64), {}),
    ("hybrid", dict(batch=2, context=500, window=37, hq=4, hkv=2, head_dim=128, sliding_blocks=30, num_blocks=100,
                    block_size=32), dict(partition_tokens=32)),
]


@pytest.mark.parametrize("name,kw,step", DECODE_BLOCK_SIZES,
                         ids=[f"{n}-bs{kw['block_size']}-{i}" for i, (n, kw, _) in enumerate(DECODE_BLOCK_SIZES)])
def test_decode_block_sizes(pk, name, kw, step):
    run_case(pk, synth.make(name, **kw), label="decode-block-size", **step)


@pytest.mark.parametrize("name,kw,step", DECODE_SMALL,
                         ids=[f"{n}-{i}" for i, (n, _, _) in enumerate(DECODE_SMALL)])
def test_decode_small(pk, name, kw, step):
    run_case(pk, synth.make(name, **kw), label="decode-small", **step)


@pytest.mark.parametrize("name", ["tiny", "qwen3", "mixed", "hybrid"])
def test_decode_full_size(pk, name):
    run_case(pk, synth.make(name), label="decode-full")


# head_dim 512 (one ring slot per wave, LDS reads in halves): windows, block
# sizes, explicit partitions, group sizes, 1-token rows.
DECODE_D512 = [
    ("hybrid", dict(batch=3, context=700, window=64, head_dim=512, sliding_blocks=40, num_blocks=200), {}),
    ("hybrid", dict(batch=2, context=500, window=100, hq=4, hkv=2, head_dim=512, sliding_blocks=60,
                    num_blocks=200, block_size=8), {}),
    ("hybrid", dict(batch=2, context=500, window=37, hq=16, hkv=1, head_dim=512, sliding_blocks=30,
                    num_blocks=100, block_size=64), dict(partition_tokens=64)),
    ("mixed", dict(batch=5, hq=6, hkv=2, head_dim=512, context=(1, 300), prefix=32, num_blocks=200), {}),
    ("mixed", dict(batch=5, hq=3, hkv=1, head_dim=512, context=(1, 400), prefix=64, num_blocks=200,
                   block_size=32), dict(partition_tokens=32)),
]


@pytest.mark.parametrize("name,kw,step", DECODE_D512, ids=[f"{n}-{i}" for i, (n, _, _) in enumerate(DECODE_D512)])
def test_decode_head_dim_512(pk, name, kw, step):
    run_case(pk, synth.make(name, **kw), label="decode-d512", **step)


def test_decode_head_dim_512_full_size(pk):
    run_case(pk, synth.make("hybrid", head_dim=512), label="decode-d512-full")


def test_decode_edge_lengths(pk):
    # a 1-token row and a row one past a block boundary, full and sliding
    run_case(pk, synth.make("tiny", context=[1, 17], prefix=0), label="edge-1-17")
    run_case(pk, synth.make("tiny", context=[16, 33], prefix=16), label="edge-16-33",
             partition_tokens=16)


# ------------------------------------------------------------ maximum sizes
def test_decode_long_row(pk):
    # one 131072-token row (8192 blocks of one KV head, 8 query heads), the
    # library's partition rule
    run_case(pk, synth.make("qwen3", batch=1, context=131072, prefix=0, hq=8, hkv=1, num_blocks=8200),
             label="decode-128k")


# More partitions per row than one chunk of the reduce holds (64; 32 at
# head_dim 512): the wide reduce, four waves taking chunks in parallel (more
# than four chunks: a wave takes several in turn).
MANY_PARTS = [
    ("hybrid", dict(batch=1), {}),                        # one GPU's share of 8: 256 partitions
    ("hybrid", dict(batch=1, head_dim=512), {}),          # head_dim 512: 256 partitions
    ("tiny", dict(context=[1500, 2000], prefix=32), dict(partition_tokens=16)),  # float32: 125
    ("mixed", dict(batch=3, context=(3000, 5000), prefix=100, hq=4, hkv=2, num_blocks=1200),
     dict(partition_tokens=16)),                          # up to 313 partitions: five chunks
    ("hybrid", dict(batch=2, context=700, window=64, head_dim=512, sliding_blocks=40, num_blocks=200),
     dict(partition_tokens=16)),                          # 44 partitions at head_dim 512
]


@pytest.mark.parametrize("name,kw,step", MANY_PARTS, ids=[f"{n}-{i}" for i, (n, _, _) in enumerate(MANY_PARTS)])
def test_decode_many_partitions(pk, name, kw, step):
    run_case(pk, synth.make(name, **kw), label="decode-many-parts", **step)


def test_decode_partition_limit(pk):
    # 65535 partitions of 16 tokens (the grid's z limit): all but the first few
    # of every row are empty
    wl = synth.make("mixed", batch=2, context=(100, 300), prefix=32, hq=4, hkv=2, num_blocks=100)
    run_case(pk, wl, label="decode-65535-parts", partition_tokens=16, max_seq_len=65535 * 16)


def test_decode_large_batch(pk):
    run_case(pk, synth.make("mixed", batch=1024, context=(1, 64), prefix=16, hq=8, hkv=4, num_blocks=5000),
             label="decode-b1024")


def test_prefill_long_chunk_sampled_rows(pk):
    wl = synth.make("prefill", batch=1, context=[4096], chunk=[8192], num_blocks=800)
    rows = sorted(set([0, 1, 255, 256, 4095, 4096, 8190, 8191] +
                      list(np.random.default_rng(9).integers(0, 8192, size=24))))
    run_case(pk, wl, rows=rows, label="prefill-8k-chunk")


def test_decode_empty_row_gives_zeros(pk):
    import torch

    announce("decode empty row")
    wl = synth.make("tiny", context=[40, 75])
    tc, _ = tables_both(pk, wl)
    dev = runner.gpu_setup(wl, tc)
    dev["_seq_lens"][0] = 0
    for part in (0, 16):
        ws = runner.gpu_workspace(wl, dev, part)
        outs = runner.gpu_step(wl, dev, workspace=ws, partition_tokens=part)
        assert torch.all(outs["main"][0] == 0)
        assert torch.all(torch.isfinite(outs["main"][1]))


def _outputs(pk, wl, share=True, **step):
    tc = synth.build_tables(pk.Allocator, wl, share=share)
    dev = runner.gpu_setup(wl, tc)
    ws = runner.gpu_workspace(wl, dev, step.get("partition_tokens"), step.get("max_seq_len"))
    outs = runner.gpu_step(wl, dev, workspace=ws, **step)
    return {k: v.cpu() for k, v in outs.items()}


def test_decode_invariances_bit_exact(pk):
    import torch

    announce("decode invariances")
    kw = dict(batch=6, context=(50, 900), prefix=300, num_blocks=600)
    base = _outputs(pk, synth.make("mixed", **kw))["main"]
    # determinism
    assert torch.equal(base, _outputs(pk, synth.make("mixed", **kw))["main"])
    # physical placement does not matter
    wl = synth.make("mixed", **kw)
    wl.layers[0].free_order = np.random.default_rng(99).permutation(np.arange(1, 600)).astype(np.int32)
    assert torch.equal(base, _outputs(pk, wl)["main"])
    # shared prefix blocks == private copies of the same data
    assert torch.equal(base, _outputs(pk, synth.make("mixed", **kw), share=False)["main"])
    # extra (empty) partitions from a larger max_seq_len change nothing
    assert torch.equal(base, _outputs(pk, synth.make("mixed", **kw), max_seq_len=4000)["main"])
    # a row's result does not depend on the other rows of the batch
    sub = synth.make("mixed", **kw)
    sub.batch = 1
    sub.seq_lens = sub.seq_lens[:1].copy()
    sub.tokens = sub.tokens[:1]
    L = sub.layers[0]
    L.q, L.k, L.v, L.live_from = L.q[:1], L.k[:1], L.v[:1], L.live_from[:1]
    assert torch.equal(base[0], _outputs(pk, sub)["main"][0])


def _one_row(wl, r):
    """Row r of a workload without shared prefix blocks, alone."""
    import copy

    sub = copy.deepcopy(wl)
    sub.batch = 1
    sub.seq_lens = wl.seq_lens[r:r + 1].copy()
    sub.tokens = [wl.tokens[r]]
    for L, L0 in zip(sub.layers, wl.layers):
        L.q, L.k, L.v, L.live_from = L0.q[r:r + 1], L0.k[r:r + 1], L0.v[r:r + 1], L0.live_from[r:r + 1]
    return sub


# Rows with fewer partitions than the grid run their last (partial) partition
# from the grid's last partition slot (that partition's own slot stays
# empty). Lengths end inside every position of a grid of eight 64-token
# partitions, on a partition boundary, at one token and at the grid's end.
@pytest.mark.parametrize("kw", [dict(head_dim=128, hq=8, hkv=2), dict(head_dim=256, hq=8, hkv=1),
                                dict(head_dim=512, hq=4, hkv=2)], ids=["d128", "d256", "d512"])
def test_decode_last_partition_moved(pk, kw):
    import torch

    ctx = [512, 448, 449, 200, 64, 65, 1, 511, 130, 320]
    make = lambda: synth.make("tiny", batch=len(ctx), context=ctx, prefix=0, num_blocks=400,  # noqa: E731
                              dtype="bf16", **kw)
    run_case(pk, make(), label="decode-moved-last", partition_tokens=64)
    # bit for bit what each row gives alone, where its grid has no empty slot
    base = _outputs(pk, make(), partition_tokens=64)["main"]
    for r in range(len(ctx)):
        alone = _outputs(pk, _one_row(make(), r), partition_tokens=64)["main"]
        assert torch.equal(base[r], alone[0]), (r, ctx[r])


def test_decode_partition_sizes_agree(pk):
    import torch

    announce("decode partition sizes")
    kw = dict(batch=4, context=(300, 900), prefix=100, num_blocks=300, dtype="f32", hq=8, hkv=2)
    outs = [_outputs(pk, synth.make("mixed", **kw), partition_tokens=p)["main"] for p in (16, 64, 512, 1024)]
    for o in outs[1:]:
        assert float((o - outs[0]).abs().max()) <= 1e-6


# --------------------------------------------------------------- prefill parity
PREFILL_SMALL = [
    dict(batch=1, context=[0], chunk=[1], num_blocks=16),
    dict(batch=3, context=[70, 33, 0], chunk=[40, 9, 17], num_blocks=64),
    dict(batch=2, context=[300, 5], chunk=[200, 130], num_blocks=64),
    dict(batch=2, context=[100, 64], chunk=[64, 100], num_blocks=64, hq=8, hkv=8),
    dict(batch=2, context=[100, 64], chunk=[64, 100], num_blocks=64, hq=6, hkv=1),
    dict(batch=2, context=[100, 64], chunk=[64, 100], num_blocks=64, hq=16, hkv=2, head_dim=64),
    dict(batch=2, context=[100, 64], chunk=[64, 100], num_blocks=64, hq=4, hkv=1, head_dim=256),
    dict(batch=2, context=[300, 64], chunk=[150, 100], num_blocks=64, window=37),
    dict(batch=1, context=[500], chunk=[129], num_blocks=64, window=200, hq=4, hkv=4),
    dict(batch=2, context=[100, 37], chunk=[40, 20], num_blocks=64, block_size=8),
    dict(batch=2, context=[100, 37], chunk=[40, 20], num_blocks=64, block_size=32, window=45),
    dict(batch=2, context=[300, 5], chunk=[200, 130], num_blocks=64, block_size=64),
]


@pytest.mark.parametrize("kw", PREFILL_SMALL, ids=[str(i) for i in range(len(PREFILL_SMALL))])
def test_prefill_small(pk, kw):
    run_case(pk, synth.make("prefill", **kw), label="prefill-small")


@pytest.mark.timeout(600)  # the whole output against the float64 oracle on the host
def test_prefill_full_size_every_row(pk):
    # The whole 2048 x 32 x 128 output against the float64 oracle (about 2.2
    # TFLOP of host work).
    run_case(pk, synth.make("prefill"), label="prefill-full")


HPREFILL_SMALL = [
    dict(batch=2, context=[300, 700], chunk=[100, 37], window=64, num_blocks=200, sliding_blocks=64),
    dict(batch=3, context=[0, 90, 513], chunk=[130, 1, 64], window=100, num_blocks=200, sliding_blocks=64),
    dict(batch=2, context=[400, 33], chunk=[77, 200], window=48, num_blocks=300, sliding_blocks=80,
         block_size=8),
    dict(batch=2, context=[400, 33], chunk=[77, 200], window=200, num_blocks=100, sliding_blocks=40,
         block_size=32),
    dict(batch=1, context=[1000], chunk=[300], window=1, num_blocks=100, sliding_blocks=40, hq=4),
]


@pytest.mark.parametrize("kw", HPREFILL_SMALL, ids=[str(i) for i in range(len(HPREFILL_SMALL))])
def test_hybrid_prefill_small(pk, kw):
    """Gemma-style chunked prefill: sliding layer (own pool, null entries for
    expired blocks), full layer, and a KV-shared layer over the full layer's
    pool and tables; D=256, 8 query heads per KV head."""
    run_case(pk, synth.make("hprefill", **kw), label="hprefill-small")


@pytest.mark.timeout(600)  # the whole output against the float64 oracle on the host
def test_hybrid_prefill_full_size_every_row(pk):
    run_case(pk, synth.make("hprefill"), label="hprefill-full")


# head_dim 512 (full-attention layers of the Gemma-style models): 32-key K/V
# tiles, four waves of 16 query rows per workgroup.
PREFILL_D512 = [
    ("prefill", dict(batch=3, context=[70, 33, 0], chunk=[40, 9, 17], num_blocks=64, hq=4, hkv=1, head_dim=512)),
    ("prefill", dict(batch=2, context=[300, 64], chunk=[150, 100], num_blocks=64, hq=8, hkv=2, head_dim=512,
                     window=37)),
    ("prefill", dict(batch=2, context=[100, 37], chunk=[40, 20], num_blocks=64, hq=2, hkv=2, head_dim=512,
                     block_size=8)),
    ("prefill", dict(batch=2, context=[300, 5], chunk=[200, 130], num_blocks=64, hq=8, hkv=1, head_dim=512,
                     block_size=64)),
    ("prefill", dict(batch=1, context=[100], chunk=[64], num_blocks=64, hq=16, hkv=1, head_dim=512,
                     block_size=32, window=45)),
    ("hprefill", dict(batch=2, context=[300, 700], chunk=[100, 37], window=64, num_blocks=200,
                      sliding_blocks=64, head_dim=512)),
]


@pytest.mark.parametrize("name,kw", PREFILL_D512, ids=[f"{n}-{i}" for i, (n, _) in enumerate(PREFILL_D512)])
def test_prefill_head_dim_512(pk, name, kw):
    run_case(pk, synth.make(name, **kw), label="prefill-d512")


@pytest.mark.timeout(600)  # the whole output against the float64 oracle on the host
def test_hybrid_prefill_head_dim_512_full_size_every_row(pk):
    run_case(pk, synth.make("hprefill", head_dim=512), label="hprefill-d512-full")


# Keys scaled by 2^(position // 32): the running score maximum jumps by far
# more than the kernels' rescale threshold every few tiles or stages, so the
# online softmax rescales accumulators that already hold data.
K_GROWTH = [
    ("prefill", dict(batch=2, context=[300, 64], chunk=[150, 100], num_blocks=64)),
    ("prefill", dict(batch=2, context=[100, 64], chunk=[64, 100], num_blocks=64, hq=16, hkv=2, head_dim=64)),
    ("prefill", dict(batch=2, context=[300, 64], chunk=[150, 100], num_blocks=64, hq=4, hkv=1, head_dim=256)),
    ("prefill", dict(batch=2, context=[300, 64], chunk=[150, 100], num_blocks=64, hq=8, hkv=1, head_dim=512)),
    ("hprefill", dict(batch=2, context=[300, 700], chunk=[100, 37], window=64, num_blocks=200,
                      sliding_blocks=64)),
    ("qwen3", dict(context=500, prefix=64, num_blocks=200, part=128)),
    ("mixed", dict(batch=5, context=(20, 900), prefix=100, num_blocks=300, part=64)),
    ("hybrid", dict(batch=2, context=500, window=100, head_dim=512, sliding_blocks=60, num_blocks=100)),
    ("tiny", dict()),
    ("mixedstep", dict(batch=3, context=(100, 600), chunk=[77], prefix=[500], num_blocks=200, part=64)),
]


@pytest.mark.parametrize("name,kw", K_GROWTH, ids=[f"{n}-{i}" for i, (n, _) in enumerate(K_GROWTH)])
def test_growing_scores_rescale(pk, name, kw):
    run_case(pk, synth.make(name, k_growth=32, **kw), label="k-growth")


# Key split: with a workspace and fewer query tiles than CUs, every tile's key
# range is cut into parts whose partials the prefill reduce combines. All of
# these shapes split (empty parts included: a tile with fewer key tiles than
# parts), sliding windows, GQA 1..16, block sizes 8..64, head dims 64..512.
KEY_SPLIT = [("prefill", kw) for kw in PREFILL_SMALL] + [
    ("hprefill", HPREFILL_SMALL[0]), ("hprefill", HPREFILL_SMALL[2]), PREFILL_D512[0], PREFILL_D512[1],
    PREFILL_D512[5], ("prefill", dict(K_GROWTH[0][1], k_growth=32)),
    ("prefill", dict(K_GROWTH[2][1], k_growth=32)),
]


@pytest.mark.parametrize("name,kw", KEY_SPLIT, ids=[f"{n}-{i}" for i, (n, _) in enumerate(KEY_SPLIT)])
def test_prefill_key_split(pk, name, kw):
    wl = synth.make(name, **kw)
    assert runner.prefill_workspace(wl) is not None, "expected a key split for this shape"
    run_case(pk, wl, label="prefill-split", prefill_split=True)


@pytest.mark.timeout(600)  # the whole output against the float64 oracle on the host
def test_prefill_key_split_shard_shape_every_row(pk):
    # One GPU's share of the chunked prefill over 8 GPUs by KV head: 4 query
    # heads on 1 KV head, 32 query tiles, each key range cut in 8.
    wl = synth.make("prefill", hq=4, hkv=1)
    assert runner.prefill_workspace(wl) is not None
    run_case(pk, wl, label="prefill-shard8-split", prefill_split=True)


def test_prefill_workspace_bytes_rule(pk):
    import torch

    announce("prefill workspace bytes")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows_per_wg = {64: 256, 128: 256, 256: 128, 512: 64}
    for B, T, C, hq, hkv, d in [(1, 2048, 2048, 32, 8, 128), (1, 2048, 2048, 4, 1, 128),
                                (4, 8192, 2048, 8, 1, 256), (2, 100, 64, 8, 1, 512), (1, 1, 1, 4, 2, 64),
                                (3, 300, 100, 16, 2, 64)]:
        items = -(-C * (hq // hkv) // rows_per_wg[d]) * hkv * B
        S = 1
        while S < 16 and items * S < cus:
            S *= 2
        expect = 0 if S == 1 else S * T * hq * (d + 2) * 4
        assert pk.paged_attn_prefill_chunk_workspace_bytes(B, T, C, hq, hkv, d) == expect, (B, T, C, hq, hkv, d)


# One continuous-batching step: decode rows (split-K decode kernels on the
# caller's stream) and prefill chunks (prefill kernel on the side stream) in
# one call, checked against the oracle's varlen prefill over all rows.
MIXED_STEP = [
    dict(batch=5, context=(20, 900), chunk=[150, 64], prefix=[300, 0], num_blocks=200, part=128),
    dict(batch=3, context=(1, 300), chunk=[1, 200], prefix=[40, 33], num_blocks=100, part=0),
    dict(batch=4, context=(100, 600), chunk=[77], prefix=[500], num_blocks=200, window=100, part=64),
    dict(batch=6, context=(1, 400), chunk=[33, 129], prefix=[64, 17], num_blocks=300, block_size=8, part=64),
    dict(batch=2, context=(300, 700), chunk=[100], prefix=[250], num_blocks=100, block_size=64, hq=8, hkv=1,
         head_dim=256, part=128),
    dict(batch=3, context=(200, 600), chunk=[90], prefix=[150], num_blocks=200, hq=8, hkv=1, head_dim=512,
         part=128),
    dict(batch=0, chunk=[120, 5], prefix=[30, 300], num_blocks=100),
    dict(batch=4, context=(10, 200), chunk=[], prefix=[], num_blocks=100, part=32),
]


@pytest.mark.parametrize("kw", MIXED_STEP, ids=[str(i) for i in range(len(MIXED_STEP))])
def test_mixed_step_small(pk, kw):
    run_case(pk, synth.make("mixedstep", **kw), label="mixed-step")


@pytest.mark.parametrize("kw", [
    dict(batch=5, context=(20, 900), chunk=[150, 64], prefix=[300, 0], num_blocks=200, part=128),
    dict(batch=3, context=(200, 600), chunk=[90, 33], prefix=[150, 70], num_blocks=200, hq=8, hkv=1,
         head_dim=512, part=128),
], ids=["d128", "d512"])
def test_mixed_step_fp8(pk, kw):
    run_case(pk, synth.make("mixedstep", kv_dtype="fp8", **kw), label="mixed-step-fp8")


@pytest.mark.timeout(600)  # the whole output against the float64 oracle on the host
def test_mixed_step_full_size_every_row(pk):
    run_case(pk, synth.make("mixedstep"), label="mixed-step-full")


def test_prefill_chunk_of_one_matches_decode(pk):
    import torch

    announce("prefill C=1 vs decode")
    wl = synth.make("prefill", batch=2, context=[77, 300], chunk=[1, 1], num_blocks=64)
    tc, _ = tables_both(pk, wl)
    dev = runner.gpu_setup(wl, tc)
    pre = runner.gpu_step(wl, dev)["main"]
    out = torch.empty_like(pre)
    d = dev["main"]
    pk.paged_attn_decode(out, d["q"], d["k_pool"], d["v_pool"], d["tables"], dev["_seq_lens"], wl.scale,
                         wl.max_seq_len, partition_tokens=1024)
    assert float((pre.float() - out.float()).abs().max()) <= 2e-2


# --------------------------------------------------------------- graph capture
@pytest.mark.parametrize("name,kw", [
    ("qwen3", dict(context=300, prefix=64, num_blocks=200)),
    ("prefill", dict(batch=2, context=[300, 64], chunk=[150, 100], num_blocks=64)),
    ("mixedstep", dict(batch=5, context=(20, 900), chunk=[150, 64], prefix=[300, 0], num_blocks=200,
                       part=128)),
    ("prefill", dict(batch=2, context=[300, 64], chunk=[150, 100], num_blocks=64, hq=8, hkv=1, head_dim=512)),
    ("mixedstep", dict(batch=3, context=(200, 600), chunk=[90], prefix=[150], num_blocks=200, hq=8, hkv=1,
                       head_dim=512, part=128)),
    # the prefill with its key split (a workspace; two kernels per call)
    ("prefill", dict(batch=2, context=[300, 64], chunk=[150, 100], num_blocks=64, hq=8, hkv=2, split=True)),
])
def test_step_graph_replays_match_eager(pk, name, kw):
    """The step (KV write + attention) captured in a HIP graph, with the
    library's timing events inside, replays bit-identically to eager launches,
    with eager work and synchronizations between replays."""
    import torch

    announce(f"graph replay {name} {kw}")
    kw = dict(kw)
    split = kw.pop("split", False)
    wl = synth.make(name, **kw)
    tc, _ = tables_both(pk, wl)
    dev = runner.gpu_setup(wl, tc)
    ws = runner.gpu_workspace(wl, dev)
    d = dev["main"]
    out = torch.empty_like(d["q"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    calls = [pk.paged_kv_write(d["k_pool"], d["v_pool"], d["step_k"], d["step_v"], d["step_slots"],
                               stream=s, prepare=True)]
    if wl.kind == "decode":
        calls.append(pk.paged_attn_decode(out, d["q"], d["k_pool"], d["v_pool"], d["tables"], dev["_seq_lens"],
                                          wl.scale, wl.max_seq_len, workspace=ws, stream=s, prepare=True))
    elif wl.num_decode:
        # decode rows on `s`, chunk rows on the library's side stream, joined into `s`
        calls.append(pk.paged_attn_mixed(out, d["q"], d["k_pool"], d["v_pool"], d["tables"], dev["_cu_q"],
                                         dev["_seq_lens"], wl.num_decode, int(wl.chunk_lens.max()), wl.scale,
                                         runner.decode_max_seq_len(wl), partition_tokens=wl.partition_tokens,
                                         workspace=ws, stream=s, prepare=True))
    else:
        pws = runner.prefill_workspace(wl) if split else None
        assert not split or pws is not None
        calls.append(pk.paged_attn_prefill_chunk(out, d["q"], d["k_pool"], d["v_pool"], d["tables"], dev["_cu_q"],
                                                 dev["_seq_lens"], int(wl.chunk_lens.max()), wl.scale,
                                                 workspace=pws, stream=s, prepare=True))
    with torch.cuda.stream(s):
        for c in calls:
            c()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    pk.trace_reset()
    pk.trace_enable(True)
    with torch.cuda.graph(g, stream=s):
        for c in calls:
            c()
    pk.trace_enable(False)
    for r in range(3):
        out.fill_(float("nan"))
        x = torch.randn(256, 256, device="cuda")
        (x @ x).sum().item()          # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs"
    kern = "decode_partial" if wl.kind == "decode" else "prefill"
    assert pk.trace_query(kern) == (0.0, 0)   # captured launches record no events
    pk.trace_enable(True)
    with torch.cuda.stream(s):
        for c in calls:
            c()
    torch.cuda.synchronize()
    pk.trace_enable(False)
    ms, n = pk.trace_query(kern)
    assert n == 1 and ms > 0.0 and torch.equal(out, eager)


# --------------------------------------------------------------- absent table entries
@pytest.mark.parametrize("kind", ["decode", "prefill", "mixed"])
@pytest.mark.parametrize("d,bs", [(128, 16), (256, 16), (128, 8)])
def test_absent_entries_get_no_weight(pk, kind, d, bs):
    """Table entries that are 0, past num_blocks, or columns past the table's
    width, inside the attended range: decode, prefill and the mixed step all
    treat those keys as absent (weight zero). Expected: the oracle's plain
    attention over the keys that remain."""
    import torch

    announce(f"absent entries {kind} D={d} block_size={bs}")
    rng = np.random.default_rng(31)
    hq, hkv, nb, mb = 4, 2, 40, 6
    lens = [100, 75]                        # rows longer than 6 blocks: later columns lie past the width
    chunks = {"decode": [1, 1], "prefill": [20, 10], "mixed": [1, 10]}[kind]
    perm = list(rng.permutation(np.arange(1, nb)))
    tables = np.zeros((2, mb), dtype=np.int32)
    flat_k, flat_v = [], []
    kp = np.full((nb, hkv, bs, d), np.nan, dtype=np.float32)
    vp = kp.copy()
    for b, n in enumerate(lens):
        fk = synth.round_bf16(rng.standard_normal((n, hkv, d)).astype(np.float32))
        fv = synth.round_bf16(rng.standard_normal((n, hkv, d)).astype(np.float32))
        flat_k.append(fk)
        flat_v.append(fv)
        for j in range(min(mb, -(-n // bs))):
            tables[b, j] = perm.pop()
            kp[tables[b, j], :, :min(bs, n - j * bs)] = fk[j * bs:(j + 1) * bs].transpose(1, 0, 2)
            vp[tables[b, j], :, :min(bs, n - j * bs)] = fv[j * bs:(j + 1) * bs].transpose(1, 0, 2)
    tables[0, 2] = 0            # a null entry inside row 0's range
    tables[1, 1] = nb + 5       # an out-of-range block id inside row 1's range
    absent = [set(range(2 * bs, 3 * bs)) | set(range(mb * bs, lens[0])),
              set(range(bs, 2 * bs)) | set(range(mb * bs, lens[1]))]
    kp = np.nan_to_num(kp, nan=0.0)      # never-written slots of used blocks hold zeros
    vp = np.nan_to_num(vp, nan=0.0)
    kp[0] = np.nan                       # the null block: must never be read
    vp[0] = np.nan
    T = sum(chunks)
    q = synth.round_bf16(rng.standard_normal((T, hq, d)).astype(np.float32))
    scale = 1.0 / np.sqrt(d)
    expect = np.zeros((T, hq, d))
    row = 0
    for b, n in enumerate(lens):
        for i in range(chunks[b]):
            a = n - chunks[b] + i
            keep = [p for p in range(a + 1) if p not in absent[b]]
            for h in range(hq):
                expect[row, h] = oracle.attend_one(q[row, h], flat_k[b][keep, h // (hq // hkv)],
                                                   flat_v[b][keep, h // (hq // hkv)], scale)
            row += 1
    dev = lambda x, dt=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(x)).to(dt).cuda()  # noqa: E731
    k_d, v_d, q_d = dev(kp), dev(vp), dev(q)
    t_d = dev(tables, torch.int32)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    cu = torch.tensor(np.concatenate([[0], np.cumsum(chunks)]), dtype=torch.int32, device="cuda")
    out = torch.full_like(q_d, float("nan"))
    part = 32
    ws_bytes = pk.paged_attn_decode_workspace_bytes(2, hq, hkv, d, bs, 128, 0, part, "bf16")
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    if kind == "decode":
        pk.paged_attn_decode(out, q_d, k_d, v_d, t_d, sl, scale, 128, partition_tokens=part, workspace=ws)
    elif kind == "prefill":
        pk.paged_attn_prefill_chunk(out, q_d, k_d, v_d, t_d, cu, sl, max(chunks), scale)
    else:
        pk.paged_attn_mixed(out, q_d, k_d, v_d, t_d, cu, sl, 1, max(chunks), scale, 128, partition_tokens=part,
                            workspace=ws)
    torch.cuda.synchronize()
    max_abs, rel = runner.compare(out, expect, "bf16")
    assert np.all(np.isfinite(out.float().cpu().numpy()))
    assert runner.within("bf16", max_abs, rel), f"max_abs={max_abs:.3g} rel_l2={rel:.3g}"
