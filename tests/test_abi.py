"""CPU-only checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments on the host before touching a device."""

import ctypes
import os
import re

import pytest

import block_paged_kv_amd as pk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(paged_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 25
    lib = ctypes.CDLL(pk.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding declares a signature for each of them
    assert set(names) <= set(pk._SIGNATURES), set(names) - set(pk._SIGNATURES)


def test_abi_version_matches_header():
    m = re.search(r"#define PAGEDKV_ABI_VERSION (\d+)", open(HEADER).read())
    assert pk.abi_version() == int(m.group(1))


def test_write_argument_errors():
    L = pk.lib
    # unknown dtype
    assert L.paged_kv_write(None, None, None, None, None, 1, 8, 16, 1, 128, 7, None) == pk.PAGED_ERR_DTYPE
    assert b"dtype" in pk.lib.paged_last_error()
    # head_dim, block size, nulls
    assert L.paged_kv_write(None, None, None, None, None, 1, 8, 16, 1, 100, 1, None) == pk.PAGED_ERR_INVALID_ARG
    assert L.paged_kv_write(None, None, None, None, None, 1, 8, 12, 1, 128, 1, None) == pk.PAGED_ERR_INVALID_ARG
    assert L.paged_kv_write(None, None, None, None, None, 1, 8, 16, 1, 128, 1, None) == pk.PAGED_ERR_INVALID_ARG
    # nothing to do is a success without any device call
    assert L.paged_kv_write(None, None, None, None, None, 0, 8, 16, 1, 128, 1, None) == pk.PAGED_OK
    # misaligned pointers are rejected
    assert L.paged_kv_write(16, 16, 16, 17, 8, 1, 8, 16, 1, 128, 1, None) == pk.PAGED_ERR_INVALID_ARG


def test_decode_argument_errors():
    L = pk.lib
    args = dict(out=None, q=None, k=None, v=None, bt=None, mb=4, sl=None, B=2, hq=6, hkv=4, d=128,
                bs=16, nb=8, scale=0.1, w=0, part=64, msl=64, ws=None, wsb=0, dt=1, s=None)

    def call(**kw):
        a = dict(args, **kw)
        return L.paged_attn_decode(a["out"], a["q"], a["k"], a["v"], a["bt"], a["mb"], a["sl"], a["B"],
                                   a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["scale"], a["w"],
                                   a["part"], a["msl"], a["ws"], a["wsb"], a["dt"], a["s"])

    assert call() == pk.PAGED_ERR_INVALID_ARG              # 6 q heads on 4 kv heads
    assert call(hq=8, part=24) == pk.PAGED_ERR_INVALID_ARG  # partition not a multiple of 16
    assert call(hq=8, dt=3) == pk.PAGED_ERR_DTYPE
    assert call(hq=8, scale=float("inf")) == pk.PAGED_ERR_INVALID_ARG
    assert call(hq=8, B=0) == pk.PAGED_OK                   # empty batch: nothing enqueued
    assert call(hq=8) == pk.PAGED_ERR_INVALID_ARG           # NULL pointers


def test_prefill_argument_errors():
    L = pk.lib
    rc = L.paged_attn_prefill_chunk(None, None, None, None, None, 4, None, None, 1, 8, 8, 8, 8, 128,
                                    16, 8, 0.1, 0, None, 0, pk.PAGED_F32, None)
    assert rc == pk.PAGED_ERR_DTYPE
    rc = L.paged_attn_prefill_chunk(None, None, None, None, None, 4, None, None, 1, 8, 8, 8, 3, 128,
                                    16, 8, 0.1, 0, None, 0, pk.PAGED_BF16, None)
    assert rc == pk.PAGED_ERR_INVALID_ARG
    rc = L.paged_attn_prefill_chunk(None, None, None, None, None, 4, None, None, 1, 0, 8, 8, 8, 128,
                                    16, 8, 0.1, 0, None, 0, pk.PAGED_BF16, None)
    assert rc == pk.PAGED_OK
    # negative or non-finite scale
    for bad in (-0.1, float("nan")):
        rc = L.paged_attn_prefill_chunk(None, None, None, None, None, 4, None, None, 1, 8, 8, 8, 8, 128,
                                        16, 8, bad, 0, None, 0, pk.PAGED_BF16, None)
        assert rc == pk.PAGED_ERR_INVALID_ARG


@pytest.mark.parametrize("B,hq,hkv,d,msl,w,part,dt", [
    (4, 16, 8, 128, 2048, 0, 128, "bf16"), (32, 32, 8, 128, 8192, 0, 512, "bf16"),
    (8, 8, 1, 256, 32768, 512, 64, "bf16"), (2, 4, 2, 64, 75, 0, 16, "f32"),
    (3, 6, 3, 64, 100, 0, 128, "bf16"), (2, 4, 2, 64, 75, 0, 48, "f32"),
    (8, 8, 1, 512, 32768, 0, 512, "bf16"), (8, 8, 1, 512, 32768, 512, 64, "fp8")])
def test_workspace_bytes(B, hq, hkv, d, msl, w, part, dt):
    span = min(msl, w + 15) if w else msl
    parts = -(-span // part)
    expect = 0 if parts == 1 else B * hq * parts * (d + 2) * 4
    assert pk.paged_attn_decode_workspace_bytes(B, hq, hkv, d, 16, msl, w, part, dt) == expect


def test_partition_must_fit_the_kernel():
    # bf16 partitions are whole 16-token stages; fp32 ones whole blocks
    with pytest.raises(pk.PagedError):
        pk.paged_attn_decode_workspace_bytes(2, 4, 2, 64, 8, 100, 0, 24, "bf16")
    assert pk.paged_attn_decode_workspace_bytes(2, 4, 2, 64, 8, 100, 0, 24, "f32") > 0
    with pytest.raises(pk.PagedError) as e:
        pk.paged_attn_decode_workspace_bytes(2, 4, 2, 64, 16, 100, 0, 64, "f16")
    assert e.value.code == pk.PAGED_ERR_DTYPE


def test_head_dim_512_limits():
    # head_dim 512 over bf16 and FP8 pools, not float32; no head_dim outside {64, 128, 256, 512}
    assert pk.paged_attn_decode_workspace_bytes(2, 4, 2, 512, 16, 100, 0, 32, "bf16") > 0
    with pytest.raises(pk.PagedError) as e:
        pk.paged_attn_decode_workspace_bytes(2, 4, 2, 512, 16, 100, 0, 32, "f32")
    assert e.value.code == pk.PAGED_ERR_INVALID_ARG
    for d in (96, 384, 1024):
        rc = pk.lib.paged_attn_prefill_chunk(None, None, None, None, None, 4, None, None, 1, 8, 8, 8, 8, d,
                                             16, 8, 0.1, 0, None, 0, pk.PAGED_BF16, None)
        assert rc == pk.PAGED_ERR_INVALID_ARG
        assert b"head_dim" in pk.lib.paged_last_error()
    assert pk.lib.paged_kv_write(None, None, None, None, None, 1, 8, 16, 1, 1024, 1, None) == \
        pk.PAGED_ERR_INVALID_ARG


def test_partition_count_limit():
    # at most 65535 partitions (the grid's z dimension): rejected before any device call
    L = pk.lib
    rc = L.paged_attn_decode(None, None, None, None, None, 4, None, 2, 4, 2, 128, 16, 8, 0.1, 0, 16,
                             65536 * 16, None, 0, pk.PAGED_BF16, None)
    assert rc == pk.PAGED_ERR_INVALID_ARG
    assert b"65535" in L.paged_last_error()
    assert pk.paged_attn_decode_workspace_bytes(2, 4, 2, 128, 16, 65535 * 16, 0, 16, "bf16") == \
        2 * 4 * 65535 * (128 + 2) * 4


def test_span_limit():
    # an attended span above 2^30 tokens is rejected (positions stay in 32 bits)
    assert pk.paged_attn_decode_workspace_bytes(1, 8, 1, 128, 16, 1 << 30, 0, 65536, "bf16") > 0
    with pytest.raises(pk.PagedError, match="2\\^30"):
        pk.paged_attn_decode_workspace_bytes(1, 8, 1, 128, 16, (1 << 30) + 1, 0, 65536, "bf16")
    # a window bounds the span whatever max_seq_len is
    assert pk.paged_attn_decode_workspace_bytes(1, 8, 1, 128, 16, 2**31 - 1, 512, 64, "bf16") > 0


def test_mixed_step_argument_errors():
    L = pk.lib

    def call(B=3, nd=2, T=10, d=128, dt=pk.PAGED_BF16, ks=1.0, vs=1.0, part=64, ws=None, wsb=0, ptr=None,
             msl=64, scale=0.1):
        return L.paged_attn_mixed(ptr, ptr, ptr, ptr, ptr, 4, ptr, ptr, B, nd, T, 8, 8, 8, d, 16, 8, scale, ks, vs,
                                  0, part, msl, ws, wsb, dt, None)

    assert call(dt=pk.PAGED_F32) == pk.PAGED_ERR_DTYPE
    assert call(nd=4) == pk.PAGED_ERR_INVALID_ARG           # more decode rows than rows
    assert call(T=1) == pk.PAGED_ERR_INVALID_ARG            # fewer queries than decode rows
    assert call(ks=2.0) == pk.PAGED_ERR_INVALID_ARG         # scales belong to FP8 pools
    assert call(B=0, nd=0, T=0) == pk.PAGED_OK              # nothing to do
    assert call() == pk.PAGED_ERR_INVALID_ARG               # NULL pointers
    # everything below is rejected before any device call
    assert call(d=384, ptr=16) == pk.PAGED_ERR_INVALID_ARG  # no kernel for head_dim 384
    assert call(ptr=16, part=32) == pk.PAGED_ERR_INVALID_ARG  # two partitions: a workspace is needed
    assert b"workspace" in pk.lib.paged_last_error()
    assert call(ptr=16, part=32, ws=16, wsb=64) == pk.PAGED_ERR_CAPACITY  # too small a workspace
    assert b"workspace" in pk.lib.paged_last_error()
    assert call(ptr=16, part=32, ws=8, wsb=1 << 20) == pk.PAGED_ERR_INVALID_ARG  # misaligned workspace
    # the decode rows' limits are checked before the chunk rows are enqueued
    assert call(ptr=16, part=16, msl=65536 * 16, ws=16, wsb=1 << 40) == pk.PAGED_ERR_INVALID_ARG
    assert b"65535" in pk.lib.paged_last_error()
    assert call(ptr=16, scale=0.0) == pk.PAGED_ERR_INVALID_ARG  # scale must be positive


def test_scale_must_be_positive():
    L = pk.lib
    for scale in (0.0, -0.5, float("nan"), float("inf")):
        rc = L.paged_attn_decode(16, 16, 16, 16, 16, 4, 16, 2, 4, 2, 128, 16, 8, scale, 0, 64, 64, None, 0,
                                 pk.PAGED_BF16, None)
        assert rc == pk.PAGED_ERR_INVALID_ARG and b"scale" in L.paged_last_error()
        rc = L.paged_attn_prefill_chunk(16, 16, 16, 16, 16, 4, 16, 16, 1, 8, 8, 4, 2, 128, 16, 8, scale, 0,
                                        None, 0, pk.PAGED_BF16, None)
        assert rc == pk.PAGED_ERR_INVALID_ARG and b"scale" in L.paged_last_error()


def test_prefill_workspace_checks():
    L = pk.lib
    # argument errors come before the device query; the rule itself needs a device
    with pytest.raises(pk.PagedError) as e:
        pk.paged_attn_prefill_chunk_workspace_bytes(1, 8, 8, 8, 8, 96)
    assert e.value.code == pk.PAGED_ERR_INVALID_ARG
    with pytest.raises(pk.PagedError) as e:
        pk.paged_attn_prefill_chunk_workspace_bytes(1, 8, 8, 6, 4, 128)
    assert e.value.code == pk.PAGED_ERR_INVALID_ARG
    assert pk.paged_attn_prefill_chunk_workspace_bytes(0, 0, 0, 8, 8, 128) == 0
    with pytest.raises(pk.PagedError) as e:
        pk.paged_attn_prefill_chunk_workspace_bytes(1, 2048, 2048, 4, 1, 128)
    assert e.value.code == pk.PAGED_ERR_HIP
    assert L.paged_attn_prefill_chunk_workspace_bytes(1, 8, 8, 8, 8, 128, None) == pk.PAGED_ERR_INVALID_ARG
    # a misaligned workspace is refused before anything is enqueued
    rc = L.paged_attn_prefill_chunk(16, 16, 16, 16, 16, 4, 16, 16, 1, 8, 8, 4, 2, 128, 16, 8, 0.1, 0,
                                    8, 1 << 20, pk.PAGED_BF16, None)
    assert rc == pk.PAGED_ERR_INVALID_ARG and b"workspace" in L.paged_last_error()
    rc = L.paged_attn_prefill_chunk_fp8(16, 16, 16, 16, 16, 4, 16, 16, 1, 8, 8, 4, 2, 128, 16, 8, 0.1, 1.0,
                                        1.0, 0, 24, 1 << 20, None)
    assert rc == pk.PAGED_ERR_INVALID_ARG and b"workspace" in L.paged_last_error()


def test_library_rule_needs_a_device_here():
    # No GPU in this container: the rule's device query fails cleanly.
    with pytest.raises(pk.PagedError) as e:
        pk.paged_attn_decode_partition_tokens(4, 16, 8, 128, 16, 2048, 0)
    assert e.value.code == pk.PAGED_ERR_HIP
    with pytest.raises(pk.PagedError) as e:
        pk.paged_attn_decode_workspace_bytes(4, 16, 8, 128, 16, 2048, 0, 0, "f32")
    assert e.value.code == pk.PAGED_ERR_HIP


def test_trace_api_without_launches():
    pk.trace_reset()
    assert pk.trace_query("decode_partial") == (0.0, 0)
    with pytest.raises(KeyError):
        pk.trace_query("nope")
    assert pk.lib.paged_trace_query(9, None, None) == pk.PAGED_ERR_INVALID_ARG


def test_header_is_plain_c_and_links(tmp_path):
    # A C99 program using only the header and the library (no Python, no
    # torch): the host allocator through the ABI, from create to destroy.
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text(r'''
#include <stdio.h>
#include "pagedkv.h"
int main(void) {
  paged_alloc* a = NULL;
  int32_t table[4] = {0}, needed = 0, nb = 0;
  int64_t seq = 7, slots[20];
  if (paged_alloc_create(8, 16, NULL, &a) != PAGED_OK) return 1;
  if (paged_seq_add(a, seq) != PAGED_OK) return 2;
  if (paged_seq_reserve(a, seq, 20) != PAGED_OK) return 3;
  if (paged_alloc_block_tables(a, &seq, 1, 4, table, &needed) != PAGED_OK) return 4;
  if (paged_alloc_slot_mapping(a, seq, 0, 20, slots) != PAGED_OK) return 5;
  if (paged_seq_reserve(a, seq, 16 * 8) != PAGED_ERR_NO_BLOCKS) return 6;
  paged_alloc_num_blocks(a, &nb);
  printf("%d %d %d %d %lld %lld\n", paged_abi_version(), nb, table[0], table[1],
         (long long)slots[0], (long long)slots[19]);
  return paged_alloc_destroy(a) == PAGED_OK ? 0 : 7;
}
''')
    exe = tmp_path / "abi"
    lib_dir = os.path.dirname(pk.LIB_PATH)
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-L", lib_dir, "-lpagedkv", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)], check=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, (run.returncode, run.stderr)
    ver, nb, b0, b1, s0, s19 = (int(x) for x in run.stdout.split())
    assert ver == pk.abi_version() and nb == 8
    # blocks 1..7 in ascending order without a free-list permutation; slots follow the table
    assert (b0, b1) == (1, 2) and s0 == b0 * 16 and s19 == b1 * 16 + 3
