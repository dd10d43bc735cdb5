"""Pins for the reference allocator (CPU only).

The hand-worked script in ``tests/golden/allocator_script.json`` was derived
from the written policy by hand; random scripts check the invariants the
policy implies: every non-null block is free, evictable or referenced
(exactly once in that sense), refcounts equal the number of live tables
holding a block, block 0 is never handed out and rows that matched a prefix
share identical leading entries.
"""

import json
import os

import numpy as np
import pytest

from oracle import RefAllocator, AllocError

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def run_script(make, steps, script=None):
    """Run a golden script (default: allocator_script.json) on an allocator
    built by ``make(nb, bs, order)``.

    The allocator must offer the RefAllocator method names; failures must
    raise an exception with a ``.code`` attribute.
    """
    g = script if script is not None else load_golden("allocator_script.json")
    a = make(g["num_blocks"], g["block_size"], g["free_order"])
    for i, st in enumerate(g["steps"][:steps] if steps else g["steps"]):
        op, where = st["op"], f"step {i}: {st}"
        if op == "add":
            a.add(st["seq"])
        elif op == "match":
            assert a.match_prefix(st["seq"], st["tokens"], st["domain"]) == st["expect_cached"], where
        elif op == "reserve":
            a.reserve(st["seq"], st["tokens"])
        elif op == "reserve_fail":
            before = (a.num_free(), [list(map(int, r)) for r in a.block_tables([st["seq"]], 64)])
            with pytest.raises(Exception) as ei:
                a.reserve(st["seq"], st["tokens"])
            assert ei.value.code == st["code"], where
            assert (a.num_free(), [list(map(int, r)) for r in a.block_tables([st["seq"]], 64)]) == before, where
        elif op == "commit":
            a.commit_tokens(st["seq"], st["tokens"])
        elif op == "publish":
            a.publish_full_blocks(st["seq"], st["domain"])
        elif op == "tables":
            assert [list(r) for r in a.block_tables(st["seqs"], st["max_blocks"])] == st["expect"], where
        elif op == "tables_fail":
            with pytest.raises(Exception) as ei:
                a.block_tables(st["seqs"], st["max_blocks"])
            assert ei.value.code == st["code"], where
        elif op == "num_free":
            assert list(a.num_free()) == st["expect"], where
        elif op == "refcount":
            assert a.refcount(st["block"]) == st["expect"], where
        elif op == "slots":
            assert list(a.slot_mapping(st["seq"], st["start"], st["n"])) == st["expect"], where
        elif op == "slots_fail":
            with pytest.raises(Exception) as ei:
                a.slot_mapping(st["seq"], st["start"], st["n"])
            assert ei.value.code == st["code"], where
        elif op == "release":
            a.release(st["seq"])
        elif op == "drop":
            a.drop_outside_window(st["seq"], st["window"])
        elif op == "grow":
            a.grow(st["blocks"], st["order"])
        elif op == "set_max":
            a.set_max_blocks(st["blocks"])
        elif op == "set_max_fail":
            with pytest.raises(Exception) as ei:
                a.set_max_blocks(st["blocks"])
            assert ei.value.code == st["code"], where
        elif op == "reserve_or_grow":
            assert a.reserve_or_grow(st["seq"], st["tokens"]) == st["expect_grow"], where
        elif op == "reserve_or_grow_fail":
            before = (a.num_free(), [list(map(int, r)) for r in a.block_tables([st["seq"]], 64)])
            with pytest.raises(Exception) as ei:
                a.reserve_or_grow(st["seq"], st["tokens"])
            assert ei.value.code == st["code"], where
            assert (a.num_free(), [list(map(int, r)) for r in a.block_tables([st["seq"]], 64)]) == before, where
        else:
            raise AssertionError(f"unknown op {op}")
    return a


def test_golden_script():
    run_script(RefAllocator, None)


GROW_SCRIPTS = load_golden("allocator_grow_script.json")["scripts"]


@pytest.mark.parametrize("idx", range(len(GROW_SCRIPTS)), ids=[s["name"] for s in GROW_SCRIPTS])
def test_golden_grow_script(idx):
    a = run_script(RefAllocator, None, GROW_SCRIPTS[idx])
    check_invariants(a)


def _grow_ignoring_order(self, new_num_blocks, new_order=None):
    return _orig_grow(self, new_num_blocks, None)


def _grow_prepending(self, new_num_blocks, new_order=None):
    old = list(self.free)
    _orig_grow(self, new_num_blocks, new_order)
    added = list(self.free)[len(old):]
    self.free.clear()
    self.free.extend(added + old)


def _reserve_or_grow_doubling_only(self, seq_id, total_tokens):
    r = _orig_rog(self, seq_id, total_tokens)
    return min(self.max_nb, 2 * self.nb) if r else r


def _reserve_or_grow_on_free_only(self, seq_id, total_tokens):
    """Grows whenever the free list alone is short (before any eviction)."""
    s = self._seq(seq_id)
    needed = -(-int(total_tokens) // self.bs) - len(s.blocks)
    if needed > len(self.free) and self.nb < self.max_nb:
        return min(self.max_nb, max(2 * self.nb, self.nb + needed))
    return _orig_rog(self, seq_id, total_tokens)


_orig_grow = RefAllocator.grow
_orig_rog = RefAllocator.reserve_or_grow
GROW_MUTANTS = {
    "grow ignores the given order": ("grow", _grow_ignoring_order),
    "grow puts new blocks at the free head": ("grow", _grow_prepending),
    "grow-on-demand only doubles": ("reserve_or_grow", _reserve_or_grow_doubling_only),
    "grow-on-demand when the free list alone is short": ("reserve_or_grow", _reserve_or_grow_on_free_only),
}


@pytest.mark.parametrize("name", sorted(GROW_MUTANTS))
def test_grow_mutants_are_caught(name, monkeypatch):
    attr, fn = GROW_MUTANTS[name]
    monkeypatch.setattr(RefAllocator, attr, fn)
    failures = 0
    for sc in GROW_SCRIPTS:
        try:
            run_script(RefAllocator, None, sc)
        except (Exception, pytest.fail.Exception):
            failures += 1
    assert failures > 0, f"no grow script catches the mutant '{name}'"


def check_invariants(a: RefAllocator):
    nb = a.nb
    holders = [0] * nb
    for s in a.seqs.values():
        for b in s.blocks:
            if b:
                holders[b] += 1
    assert holders[0] == 0
    for b in range(1, nb):
        assert a.ref[b] == holders[b], f"block {b}"
    free, lru = set(a.free), set(a.lru)
    used = {b for b in range(1, nb) if a.ref[b] > 0}
    assert 0 not in free | lru | used
    assert not (free & lru) and not (free & used) and not (lru & used)
    assert len(free) + len(lru) + len(used) == nb - 1
    assert len(free) == len(a.free) and len(lru) == len(a.lru)
    for b in lru:
        assert a.chain_id[b] != 0 and a.table[a.key_of[b]] == b
    for key, b in a.table.items():
        assert a.key_of[b] == key and a.chain_id[b] != 0


def random_script(seed, nb=40, bs=4, n_ops=400):
    """Random lifecycle calls over a small vocabulary so prefixes collide often."""
    rng = np.random.default_rng(seed)
    order = list(rng.permutation(np.arange(1, nb)))
    ops = []
    live = []
    next_id = 0
    prompts = [list(rng.integers(0, 3, size=int(rng.integers(1, 20)))) for _ in range(6)]
    for _ in range(n_ops):
        r = rng.random()
        if r < 0.3 or not live:
            sid = next_id
            next_id += 1
            toks = list(prompts[int(rng.integers(0, len(prompts)))])
            toks += list(rng.integers(0, 3, size=int(rng.integers(0, 9))))
            ops.append(("start", sid, toks, int(rng.integers(0, 2))))
            live.append(sid)
        elif r < 0.55:
            sid = live[int(rng.integers(0, len(live)))]
            ops.append(("extend", sid, list(rng.integers(0, 3, size=int(rng.integers(1, 6))))))
        elif r < 0.65:
            sid = live[int(rng.integers(0, len(live)))]
            ops.append(("drop", sid, int(rng.integers(1, 12))))
        elif r < 0.75 and len(live) > 0:
            src = live[int(rng.integers(0, len(live)))]
            ops.append(("fork", next_id, src, int(rng.integers(0, 4))))
            live.append(next_id)
            next_id += 1
        else:
            sid = live.pop(int(rng.integers(0, len(live))))
            ops.append(("release", sid))
    return order, ops


def apply(a, op, log):
    """Apply one scripted op; record every observable outcome in ``log``."""
    def attempt(fn, *args):
        try:
            r = fn(*args)
            log.append(("ok", r if not isinstance(r, list) else list(r)))
            return True
        except Exception as e:  # noqa: BLE001
            log.append(("err", e.code))
            return False

    kind = op[0]
    if kind == "start":
        _, sid, toks, dom = op
        attempt(a.add, sid)
        attempt(a.match_prefix, sid, toks[:-1], dom)
        if attempt(a.reserve, sid, len(toks)):
            cached = a.num_tokens(sid)
            attempt(a.commit_tokens, sid, toks[cached:])
            attempt(a.publish_full_blocks, sid, dom)
    elif kind == "extend":
        _, sid, toks = op
        n = a.num_tokens(sid)
        if attempt(a.reserve, sid, n + len(toks)):
            attempt(a.commit_tokens, sid, toks)
            attempt(a.publish_full_blocks, sid, 0)
    elif kind == "drop":
        attempt(a.drop_outside_window, op[1], op[2])
    elif kind == "fork":
        _, dst, src, nblk = op
        attempt(a.add, dst)
        attempt(a.share_prefix, dst, src, min(nblk, a.num_tokens(src) // a.bs))
    elif kind == "release":
        attempt(a.release, op[1])
    log.append(("free", a.num_free()))


@pytest.mark.parametrize("seed", range(6))
def test_random_scripts_keep_invariants(seed):
    order, ops = random_script(seed)
    a = RefAllocator(40, 4, order)
    log = []
    for op in ops:
        apply(a, op, log)
        check_invariants(a)
    assert any(x == ("err", -3) for x in log), "script never exhausted the pool"


def test_prefix_rows_share_leading_entries():
    a = RefAllocator(64, 4, None)
    prompt = list(range(10))
    for sid in range(3):
        a.add(sid)
        a.match_prefix(sid, prompt + [100 + sid], 0)
        a.reserve(sid, 11 + sid)
        cached = a.num_tokens(sid)
        a.commit_tokens(sid, (prompt + [100 + sid] + [7] * sid)[cached:])
        a.publish_full_blocks(sid, 0)
    t = a.block_tables([0, 1, 2], 8)
    assert t[0][:2] == t[1][:2] == t[2][:2]
    assert len({t[0][2], t[1][2], t[2][2]}) == 3
    assert a.refcount(t[0][0]) == 3


def test_invalid_arguments():
    with pytest.raises(AllocError) as e:
        RefAllocator(8, 4, [1, 2, 3])
    assert e.value.code == -1
    a = RefAllocator(8, 4)
    with pytest.raises(AllocError) as e:
        a.release(5)
    assert e.value.code == -5
    a.add(1)
    with pytest.raises(AllocError) as e:
        a.add(1)
    assert e.value.code == -5
    with pytest.raises(AllocError) as e:
        a.refcount(8)
    assert e.value.code == -1
