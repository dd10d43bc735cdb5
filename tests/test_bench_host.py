"""CPU checks of bench.py's host-side bookkeeping (no GPU): one GPU's share
of an N-GPU run, the kernel identity that guards recorded counters, and the
roofline arithmetic."""

import pytest

import bench


@pytest.mark.parametrize("name,n,kw,split", [
    ("prefill", 8, {"hq": 4, "hkv": 1}, "kv_heads"),
    ("prefill", 2, {"hq": 16, "hkv": 4}, "kv_heads"),
    ("mixed", 8, {"hq": 4, "hkv": 1}, "kv_heads"),
    ("qwen3", 4, {"hq": 4, "hkv": 2}, "kv_heads"),
    ("hybrid", 8, {"batch": 1}, "rows"),       # one KV head: split the rows
    ("hprefill", 4, {"batch": 1}, "rows"),
    ("mixedstep", 8, {"hq": 4, "hkv": 1}, "kv_heads"),
])
def test_shard_overrides(name, n, kw, split):
    assert bench.shard_overrides(name, n) == (kw, split)


def test_shard_of_one_gpu_is_the_workload():
    assert bench.shard_overrides("hybrid", 1) == ({}, None)


def test_shard_that_divides_nothing_exits():
    # tiny: 2 KV heads and 2 rows do not split 4 ways
    with pytest.raises(SystemExit):
        bench.shard_overrides("tiny", 4)


def test_kernel_identity_ignores_comments_and_layout():
    a = "int x = 1;  // one\n\n    return x;\n"
    b = "// header\nint x = 1;\n  return x; // done\n"
    assert bench.code_lines(a) == bench.code_lines(b) == "int x = 1;\nreturn x;"
    assert bench.code_lines("int x = 2;") != bench.code_lines(a)


def test_roofline_entry_arithmetic():
    # two kernels, 3 steps: 6 ms of launches in all -> 2 ms per step
    dur = {"decode_partial": [1.0, 1.0, 1.0], "decode_reduce": [1.0, 1.0, 1.0]}
    e = bench.roofline_entry(["decode_partial", "decode_reduce"], dur, 3, 8e9, "hbm")
    assert e["kernel_us_per_step"] == pytest.approx(2000.0)
    assert e["achieved"] == pytest.approx(4000.0)          # 8 GB per 2 ms
    assert e["frac"] == pytest.approx(0.5)
    m = bench.roofline_entry(["prefill"], {"prefill": [2.0]}, 1, 2.5e12, "mfma")
    assert m["unit"] == "TFLOP/s" and m["achieved"] == pytest.approx(1250.0) and m["frac"] == pytest.approx(0.5)
