"""GPU parity of the FP8 (E4M3) KV cache, through the C ABI.

The quantizing write is bit-exact against the oracle's quantizer (per-layer
scale, float32 division, nearest E4M3 value with ties to even, saturation);
the gather copies codes bit for bit; decode and prefill over FP8 pools match
the float64 oracle run on the dequantized pools within the bf16 tolerances
(max-abs 2e-2, relative L2 5e-3): the kernels read exactly those values.
"""

import numpy as np
import pytest

import oracle
import runner
import synth
from oracle import fp8 as ofp8
from test_gpu_parity import announce, pk, run_case, tables_both  # noqa: F401 (pk: fixture)

pytestmark = pytest.mark.gpu


def codes(t):
    import torch

    return t.view(torch.uint8).cpu().numpy()


@pytest.mark.parametrize("name,kw", [
    ("qwen3", dict(context=300, prefix=64, num_blocks=200)),
    ("hybrid", dict(batch=3, context=700, window=64, sliding_blocks=40, num_blocks=200)),
    ("prefill", dict(batch=3, context=[70, 33, 0], chunk=[40, 9, 17], num_blocks=64)),
    ("mixed", dict(batch=5, context=(20, 300), prefix=100, num_blocks=300, head_dim=64, hq=4, hkv=2,
                   block_size=8)),
    ("mixed", dict(batch=4, context=(20, 300), prefix=100, num_blocks=100, head_dim=256, hq=4, hkv=2,
                   block_size=32)),
])
def test_fp8_write_is_bit_exact(pk, name, kw):
    import torch

    wl = synth.make(name, kv_dtype="fp8", **kw)
    announce(f"fp8 write {name} D={wl.head_dim} bs={wl.block_size}")
    tc, tr = tables_both(pk, wl)
    dev = runner.gpu_setup(wl, tc)
    runner.gpu_step(wl, dev, workspace=runner.gpu_workspace(wl, dev))
    torch.cuda.synchronize()
    pools = runner.oracle_setup(wl, tr)
    for L in wl.layers:
        if L.alias_of:
            continue
        kc, vc = pools["_codes"][L.name]
        np.testing.assert_array_equal(codes(dev[L.name]["k_pool"]), kc)
        np.testing.assert_array_equal(codes(dev[L.name]["v_pool"]), vc)


@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_fp8_quantizer_rounding_and_saturation(pk, src):
    """Magnitudes over 7 decades, exact ties of the E4M3 grid, values past the
    saturation point, both signs; bf16 and float32 sources."""
    import torch

    announce(f"fp8 quantizer {src}")
    rng = np.random.default_rng(11)
    T, H, D, NB, BS = 48, 2, 128, 5, 16
    x = rng.standard_normal((T, H, D)) * 10.0 ** rng.uniform(-5, 3, size=(T, H, D))
    ties = np.array([1.0625, 1.1875, 432.0, 464.0, 500.0, 1e4, 2.0 ** -10, 1.5 * 2.0 ** -9,
                     0.5 * 2.0 ** -9, 3 * 2.0 ** -10], dtype=np.float64)
    x[0, 0, :ties.size] = ties
    x[0, 1, :ties.size] = -ties
    dt = torch.bfloat16 if src == "bf16" else torch.float32
    xt = torch.from_numpy(x.astype(np.float32)).to(dtype=dt, device="cuda")
    xs = xt.float().cpu().numpy()  # the exact source values (bf16-rounded for bf16)
    slots = torch.arange(T, dtype=torch.int64, device="cuda") + BS + 3  # block 1 onwards
    for k_scale, v_scale in ((1.0, 1.0), (0.0123, 7.5)):
        kp = torch.full((NB, H, BS, D), float("nan"), dtype=torch.float8_e4m3fn, device="cuda")
        vp = torch.full_like(kp, float("nan"))
        pk.paged_kv_write_fp8(kp, vp, xt, -xt, slots, k_scale, v_scale)
        torch.cuda.synchronize()
        ek = np.full((NB, H, BS, D), 0x7F, dtype=np.uint8)
        ev = np.full((NB, H, BS, D), 0x7F, dtype=np.uint8)
        ek, ev = oracle.kv_write(ek, ev, ofp8.quantize(xs, k_scale), ofp8.quantize(-xs, v_scale),
                                 slots.cpu().numpy(), BS)
        np.testing.assert_array_equal(codes(kp), ek)
        np.testing.assert_array_equal(codes(vp), ev)


def test_fp8_gather_copies_codes(pk):
    import torch

    wl = synth.make("hybrid", batch=3, context=700, window=64, sliding_blocks=40, num_blocks=200,
                    kv_dtype="fp8")
    announce("fp8 gather")
    tc, tr = tables_both(pk, wl)
    dev = runner.gpu_setup(wl, tc)
    runner.gpu_step(wl, dev, workspace=runner.gpu_workspace(wl, dev))
    pools = runner.oracle_setup(wl, tr)
    for L in wl.layers:
        if L.alias_of:
            continue
        spans, offs = [], [0]
        for b in range(wl.batch):
            n = int(wl.seq_lens[b])
            lo = max(0, n - L.window) if L.window else 0
            spans.append((lo, n))
            offs.append(offs[-1] + n - lo)
        ok = torch.empty((offs[-1], wl.hkv, wl.head_dim), dtype=torch.float8_e4m3fn, device="cuda")
        ov = torch.empty_like(ok)
        pk.paged_kv_gather(ok, ov, dev[L.name]["k_pool"], dev[L.name]["v_pool"], dev[L.name]["tables"],
                           dev["_seq_lens"], torch.tensor(offs[:-1], dtype=torch.int64, device="cuda"),
                           wl.max_seq_len, sliding_window=L.window)
        kc, vc = pools["_codes"][L.name]
        tab = tr[L.name]["tables"]
        ek = np.concatenate([oracle.gather_positions(kc, tab[b], range(lo, n), wl.block_size)
                             for b, (lo, n) in enumerate(spans)])
        ev = np.concatenate([oracle.gather_positions(vc, tab[b], range(lo, n), wl.block_size)
                             for b, (lo, n) in enumerate(spans)])
        np.testing.assert_array_equal(codes(ok), ek)
        np.testing.assert_array_equal(codes(ov), ev)


FP8_DECODE = [
    ("qwen3", dict(context=300, prefix=64, num_blocks=200), {}),
    ("qwen3", dict(context=300, prefix=64, num_blocks=200), dict(partition_tokens=64)),
    ("mixed", dict(batch=7, context=(1, 700), prefix=200, num_blocks=400), dict(partition_tokens=128)),
    ("mixed", dict(batch=5, hq=16, hkv=1, context=(100, 600), prefix=64, num_blocks=300), {}),
    ("mixed", dict(batch=5, hq=6, hkv=2, head_dim=64, context=(1, 300), prefix=32, num_blocks=200), {}),
    ("mixed", dict(batch=4, hq=8, hkv=8, head_dim=256, context=(30, 400), prefix=48, num_blocks=200),
     dict(partition_tokens=32)),
    ("mixed", dict(batch=5, context=(1, 400), prefix=100, num_blocks=400, block_size=8), {}),
    ("mixed", dict(batch=4, hq=8, hkv=2, head_dim=64, context=(1, 400), prefix=100, num_blocks=400,
                   block_size=8), {}),
    ("mixed", dict(batch=5, context=(1, 700), prefix=130, num_blocks=100, block_size=64),
     dict(partition_tokens=128)),
    ("hybrid", dict(batch=3, context=700, window=64, sliding_blocks=40, num_blocks=200), {}),
    ("hybrid", dict(batch=2, context=500, window=37, hq=4, hkv=2, head_dim=128, sliding_blocks=30,
                    num_blocks=100, block_size=32), dict(partition_tokens=32)),
    ("hybrid", dict(batch=3, context=700, window=64, head_dim=512, sliding_blocks=40, num_blocks=200), {}),
    ("mixed", dict(batch=5, hq=6, hkv=2, head_dim=512, context=(1, 300), prefix=32, num_blocks=200,
                   block_size=8), dict(partition_tokens=32)),
]


@pytest.mark.parametrize("name,kw,step", FP8_DECODE,
                         ids=[f"{n}-{i}" for i, (n, _, _) in enumerate(FP8_DECODE)])
def test_fp8_decode_small(pk, name, kw, step):
    run_case(pk, synth.make(name, kv_dtype="fp8", **kw), label="fp8-decode", **step)


def test_fp8_decode_one_row_many_partitions(pk):
    # one row of the hybrid workload: 256 partitions, the wide reduce
    run_case(pk, synth.make("hybrid", batch=1, kv_dtype="fp8"), label="fp8-decode-many-parts")


@pytest.mark.parametrize("name", ["qwen3", "mixed", "hybrid"])
def test_fp8_decode_full_size(pk, name):
    run_case(pk, synth.make(name, kv_dtype="fp8"), label="fp8-decode-full")


@pytest.mark.parametrize("kw", [
    dict(batch=3, context=[70, 33, 0], chunk=[40, 9, 17], num_blocks=64),
    dict(batch=2, context=[300, 64], chunk=[150, 100], num_blocks=64, window=37),
    dict(batch=2, context=[100, 64], chunk=[64, 100], num_blocks=64, hq=16, hkv=2, head_dim=64),
    dict(batch=2, context=[100, 64], chunk=[64, 100], num_blocks=64, hq=4, hkv=1, head_dim=256),
    dict(batch=2, context=[100, 37], chunk=[40, 20], num_blocks=64, block_size=8),
    dict(batch=2, context=[300, 64], chunk=[150, 100], num_blocks=64, hq=8, hkv=1, head_dim=512, window=37),
    dict(batch=2, context=[100, 37], chunk=[40, 20], num_blocks=64, hq=4, hkv=2, head_dim=512, block_size=8),
], ids=[str(i) for i in range(7)])
def test_fp8_prefill_small(pk, kw):
    run_case(pk, synth.make("prefill", kv_dtype="fp8", **kw), label="fp8-prefill")


@pytest.mark.parametrize("kw", [
    dict(batch=3, context=[70, 33, 0], chunk=[40, 9, 17], num_blocks=64),
    dict(batch=2, context=[300, 64], chunk=[150, 100], num_blocks=64, hq=8, hkv=1, head_dim=512, window=37),
], ids=["d128", "d512"])
def test_fp8_prefill_key_split(pk, kw):
    wl = synth.make("prefill", kv_dtype="fp8", **kw)
    assert runner.prefill_workspace(wl) is not None
    run_case(pk, wl, label="fp8-prefill-split", prefill_split=True)


@pytest.mark.timeout(600)  # the whole output against the float64 oracle on the host
def test_fp8_prefill_full_size_every_row(pk):
    run_case(pk, synth.make("prefill", kv_dtype="fp8"), label="fp8-prefill-full")


def test_plain_entry_points_reject_fp8_pools(pk):
    import torch

    announce("fp8 pools on the plain entry points")
    kp = torch.zeros((4, 2, 16, 128), dtype=torch.float8_e4m3fn, device="cuda")
    q = torch.zeros((1, 2, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    bt = torch.ones((1, 4), dtype=torch.int32, device="cuda")
    sl = torch.tensor([5], dtype=torch.int32, device="cuda")
    L = pk.lib
    rc = L.paged_attn_decode(out.data_ptr(), q.data_ptr(), kp.data_ptr(), kp.data_ptr(), bt.data_ptr(), 4,
                             sl.data_ptr(), 1, 2, 2, 128, 16, 4, 0.1, 0, 64, 64, None, 0,
                             pk.PAGED_FP8_E4M3, None)
    assert rc == pk.PAGED_ERR_DTYPE
    with pytest.raises(pk.PagedError):
        pk.paged_attn_decode_fp8(out, q, kp, kp, bt, sl, 0.1, 0.0, 1.0, 64)  # k_scale must be > 0


@pytest.mark.parametrize("name,kw", [
    ("prefill", dict(batch=2, context=[300, 64], chunk=[150, 100], num_blocks=64)),
    ("prefill", dict(batch=2, context=[300, 64], chunk=[150, 100], num_blocks=64, hq=8, hkv=1, head_dim=512)),
    ("mixed", dict(batch=5, context=(20, 900), prefix=100, num_blocks=300, part=64)),
    ("hybrid", dict(batch=2, context=500, window=100, head_dim=256, sliding_blocks=60, num_blocks=100)),
], ids=["prefill", "prefill-d512", "mixed", "hybrid"])
def test_fp8_growing_scores_rescale(pk, name, kw):
    # keys scaled by 2^(position // 32): the online softmax over FP8 codes
    # rescales accumulators that already hold data
    run_case(pk, synth.make(name, kv_dtype="fp8", k_growth=32, **kw), label="fp8-k-growth")
