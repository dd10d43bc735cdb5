"""The decode entry point that allocates nothing (``paged_attn_decode_noalloc``)
against ``paged_attn_decode`` with a caller workspace, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input, each compared
bit for bit with the workspace entry point (same kernels, same partitions)
and within the bf16 / fp32 tolerance of the float64 oracle. The library's
per-GPU scratch keeps the first call's partials when the second runs; the
second must not depend on them.
"""

import numpy as np
import pytest

import runner
import synth
from oracle import RefAllocator

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pk():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_paged_kv_amd

    return block_paged_kv_amd


def _one(pk, wl, label):
    import torch

    print(f"[no_alloc] {label}: {wl.name} B={wl.batch} D={wl.head_dim} {wl.dtype} "
          f"lens={wl.seq_lens[:6].tolist()}", flush=True)
    tc = synth.build_tables(pk.Allocator, wl)
    tr = synth.build_tables(RefAllocator, wl)
    dev = runner.gpu_setup(wl, tc)
    runner.gpu_step(wl, dev, workspace=runner.gpu_workspace(wl, dev))  # writes + reference outputs
    msl = runner.decode_max_seq_len(wl)
    pools = runner.oracle_setup(wl, tr)
    ref = runner.oracle_step(wl, pools)
    for L in wl.layers:
        d = dev[L.name]
        ws = runner.gpu_workspace(wl, dev)
        want = torch.full_like(d["q"], float("nan"))
        got = torch.full_like(d["q"], float("nan"))
        pk.paged_attn_decode(want, d["q"], d["k_pool"], d["v_pool"], d["tables"], dev["_seq_lens"], wl.scale,
                             msl, sliding_window=d["window"], partition_tokens=wl.partition_tokens, workspace=ws)
        pk.paged_attn_decode_noalloc(got, d["q"], d["k_pool"], d["v_pool"], d["tables"], dev["_seq_lens"],
                                     wl.scale, msl, sliding_window=d["window"],
                                     partition_tokens=wl.partition_tokens)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                           want.view(torch.int16) if want.dtype == torch.bfloat16 else want.view(torch.int32)), \
            f"{label}/{L.name}: differs from paged_attn_decode"
        max_abs, rel = runner.compare(got, ref[L.name], wl.dtype)
        assert runner.within(wl.dtype, max_abs, rel), f"{label}/{L.name}: max_abs={max_abs:.3g} rel_l2={rel:.3g}"


def test_noalloc_matches_workspace_decode_twice(pk):
    # Large first (partials across many partitions), then a smaller call.
    _one(pk, synth.make("mixed", batch=12, context=(300, 4000), prefix=256, num_blocks=4000), "first")
    _one(pk, synth.make("hybrid", batch=2, context=900, window=64, sliding_blocks=40, num_blocks=200), "second")


def test_noalloc_fp32_and_direct(pk):
    _one(pk, synth.make("tiny"), "fp32 tiny")
    _one(pk, synth.make("tiny", context=[5, 9]), "fp32 one partition")


def test_noalloc_rejects_what_does_not_fit(pk):
    import torch

    # 64 rows x 64 heads x 1024 partitions x 130 floats > 16 MiB: refused before any launch.
    need = pk.paged_attn_decode_workspace_bytes(64, 64, 8, 128, 16, 1024 * 16, 0, 16, "bf16")
    assert need > 16 << 20
    q = torch.zeros((64, 64, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    kp = torch.zeros((4, 8, 16, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((64, 1024), dtype=torch.int32, device="cuda")
    sl = torch.ones(64, dtype=torch.int32, device="cuda")
    with pytest.raises(pk.PagedError) as e:
        pk.paged_attn_decode_noalloc(out, q, kp, kp, bt, sl, 0.1, 1024 * 16, partition_tokens=16)
    assert e.value.code == pk.PAGED_ERR_CAPACITY
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
