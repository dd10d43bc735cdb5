"""The library's C++ allocator against the oracle's RefAllocator (CPU only).

Both implement the written policy independently; every observable outcome
must agree exactly: return values, error codes, block tables, slot mappings,
refcounts and free/evictable counts.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

import block_paged_kv_amd as pk
import synth
from oracle import RefAllocator

from test_ref_allocator import GROW_SCRIPTS, apply, check_invariants, random_script, run_script

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_golden_script_cpp():
    run_script(pk.Allocator, None)


@pytest.mark.parametrize("idx", range(len(GROW_SCRIPTS)), ids=[s["name"] for s in GROW_SCRIPTS])
def test_golden_grow_script_cpp(idx):
    run_script(pk.Allocator, None, GROW_SCRIPTS[idx])


def _snapshot(a, nb, ids):
    tables = [list(r) for r in a.block_tables(ids, 64)] if ids else []
    return (a.num_free(), [a.refcount(b) for b in range(nb)], [[int(x) for x in r] for r in tables])


@pytest.mark.parametrize("seed", range(8))
def test_random_scripts_match(seed):
    nb = 40
    order, ops = random_script(seed, nb=nb)
    ref = RefAllocator(nb, 4, order)
    cpp = pk.Allocator(nb, 4, order)
    log_r, log_c = [], []
    for i, op in enumerate(ops):
        apply(ref, op, log_r)
        apply(cpp, op, log_c)
        assert log_c == log_r, f"op {i}: {op}"
        ids = sorted(ref.seqs)
        assert _snapshot(cpp, nb, ids) == _snapshot(ref, nb, ids), f"op {i}: {op}"
        check_invariants(ref)
        for sid in ids:
            n = ref.num_tokens(sid)
            if n and all(b != 0 for b in ref.seqs[sid].blocks):
                assert list(cpp.slot_mapping(sid, 0, n)) == ref.slot_mapping(sid, 0, n)


def test_grow_matches():
    ref = RefAllocator(6, 4, [5, 4, 3, 2, 1])
    cpp = pk.Allocator(6, 4, [5, 4, 3, 2, 1])
    for a in (ref, cpp):
        a.add(1)
        a.reserve(1, 20)
        with pytest.raises(Exception) as e:
            a.reserve(1, 24)
        assert e.value.code == pk.PAGED_ERR_NO_BLOCKS
        a.grow(9, [8, 6, 7])
        a.reserve(1, 32)
    assert [list(r) for r in cpp.block_tables([1], 8)] == ref.block_tables([1], 8)
    assert cpp.nb == ref.nb == 9
    with pytest.raises(pk.PagedError):
        cpp.grow(10, [3])


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("qwen3", dict(context=300, prefix=64, num_blocks=300)),
    ("mixed", dict(batch=12, context=(20, 400), prefix=200, num_blocks=600)),
    ("hybrid", dict(batch=3, context=900, window=64, sliding_blocks=40, num_blocks=300)),
    ("prefill", dict(batch=3, context=[70, 33, 0], chunk=[40, 9, 17], num_blocks=64)),
])
def test_workload_tables_match(name, kw):
    wl = synth.make(name, **kw)
    tc = synth.build_tables(pk.Allocator, wl)
    tr = synth.build_tables(RefAllocator, wl)
    for L in tc:
        np.testing.assert_array_equal(tc[L]["tables"], tr[L]["tables"])
        for x, y in zip(tc[L]["setup_slots"] + tc[L]["step_slots"], tr[L]["setup_slots"] + tr[L]["step_slots"]):
            np.testing.assert_array_equal(x, y)
        # block 0 never handed out to a live position; pads are 0
        t = tc[L]["tables"]
        for b in range(wl.batch):
            n = int(wl.seq_lens[b])
            lo = synth.BLOCK_SIZE * (max(0, n - wl.layer(L).window) // synth.BLOCK_SIZE) if wl.layer(L).window else 0
            live = t[b][lo // 16: -(-n // 16)]
            assert np.all(live > 0)


def test_shared_prefix_refcounts_full_size_qwen3_tables():
    wl = synth.make("qwen3", num_blocks=32768)
    t = synth.build_tables(pk.Allocator, wl)["main"]
    tab = t["tables"]
    # 512-token shared chain = 32 blocks, identical in all four rows
    assert all(np.array_equal(tab[0][:32], tab[b][:32]) for b in range(4))
    assert all(t["alloc"].refcount(int(x)) == 4 for x in tab[0][:32])
    assert len(set(tab[:, 32:].ravel().tolist())) == 4 * (128 - 32)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_allocator_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "alloc_sanitize"
    src = [os.path.join(ROOT, "tests", "alloc_sanitize.cpp"),
           os.path.join(ROOT, "block_paged_kv_amd", "csrc", "allocator.cpp"),
           os.path.join(ROOT, "block_paged_kv_amd", "csrc", "status.cpp")]
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "block_paged_kv_amd", "csrc"),
           *src, "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "OK" in r.stdout
