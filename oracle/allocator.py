"""Reference host block allocator (pure Python).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``). The C++ allocator in the
library implements the same written policy independently; the tests compare
the two call by call, bit for bit (block tables, slot mappings, refcounts,
free/evictable counts, error codes).

What the pages fix (mlx-node paged-cache doc, component table): a
BlockAllocator owns the logical lifecycle -- per-block refcounts, LRU eviction
and a prefix table for cross-request reuse -- and the per-request lifecycle is
reset -> find cached prefix -> allocate suffix blocks -> record tokens ->
register full blocks for reuse -> release. Only whole blocks are shared. A
block's identity is inherited through its parent chain (Gemma4 sliding sidecar
section). A caller-chosen cache salt selects a domain used for both lookup and
publication (cache-salt section). Sliding groups keep their absolute table
width and turn blocks wholly outside the window into a shared null sentinel
(hybrid coordinator paragraph).

The written policy (our reading where the pages leave details open):

* Block 0 is the null sentinel: never handed out, never refcounted.
* Free list: a FIFO of block ids, initially ``free_order`` (the caller draws
  it; default ascending 1..NB-1). Allocation pops the head; a released
  unpublished block is appended at the tail.
* Publishing gives a block a fresh chain id (a counter from 1 that is never
  reused) and enters it in the prefix table under the key
  ``(domain, parent chain id or 0 for the first block, the block's BS token
  ids)``. Keys are exact; no hash collisions are possible.
* A published block whose refcount drops to 0 joins the tail of the evictable
  (LRU) queue; it stays matchable. Matching it takes it out of the queue.
* Allocation takes the free list first, then evicts the LRU head (its key and
  chain id are dropped). All-or-nothing: if free + evictable < needed, nothing
  changes and the call fails.
* Release walks the row's table from the last entry to the first (deepest
  first, so chain tails reach the LRU queue before their parents), skipping
  null entries.
* Grow-on-demand (pool-sizing section): the pool has a maximum block count,
  by default its size at creation (a fixed pool). A reservation that needs
  more blocks than free + evictable hold asks for growth first, to
  ``min(max, max(2 * current, current + needed))`` blocks, where ``needed`` is
  the number of new blocks the reservation takes; the caller grows its pools
  and retries the reservation once, which then allocates (free blocks first,
  then LRU eviction) or fails. A pool already at its maximum fails at once.
"""

from __future__ import annotations

from collections import OrderedDict, deque

OK = 0
ERR_INVALID_ARG = -1
ERR_NO_BLOCKS = -3
ERR_CAPACITY = -4
ERR_STATE = -5


class AllocError(Exception):
    """Raised with the library's status code in ``.code``."""

    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class _Seq:
    __slots__ = ("blocks", "tokens")

    def __init__(self):
        self.blocks = []   # physical ids in logical order; 0 = dropped (null)
        self.tokens = []   # committed token ids, one per cached position


class RefAllocator:
    """Block allocator for one pool (one cache group)."""

    def __init__(self, num_blocks, block_size, free_order=None):
        if num_blocks < 2 or block_size < 1:
            raise AllocError(ERR_INVALID_ARG, "num_blocks >= 2 and block_size >= 1 required")
        self.nb = int(num_blocks)
        self.bs = int(block_size)
        if free_order is None:
            order = list(range(1, self.nb))
        else:
            order = [int(x) for x in free_order]
            if sorted(order) != list(range(1, self.nb)):
                raise AllocError(ERR_INVALID_ARG, "free_order must be a permutation of 1..NB-1")
        self.free = deque(order)
        self.lru = OrderedDict()          # evictable published blocks, oldest first
        self.ref = [0] * self.nb
        self.chain_id = [0] * self.nb     # 0 = unpublished
        self.key_of = [None] * self.nb
        self.table = {}                   # key -> block
        self.next_chain_id = 1
        self.seqs = {}
        self.max_nb = self.nb             # grow-on-demand ceiling; a fixed pool by default

    # -- helpers ---------------------------------------------------------
    def _seq(self, seq_id):
        s = self.seqs.get(int(seq_id))
        if s is None:
            raise AllocError(ERR_STATE, f"unknown sequence {seq_id}")
        return s

    def _take_new(self):
        if self.free:
            b = self.free.popleft()
        else:
            b, _ = self.lru.popitem(last=False)
            del self.table[self.key_of[b]]
            self.key_of[b] = None
            self.chain_id[b] = 0
        self.ref[b] = 1
        return b

    def _unref(self, b):
        self.ref[b] -= 1
        if self.ref[b] < 0:
            raise AllocError(ERR_STATE, f"refcount underflow on block {b}")
        if self.ref[b] == 0:
            if self.chain_id[b]:
                self.lru[b] = None
            else:
                self.free.append(b)

    # -- lifecycle -------------------------------------------------------
    def grow(self, new_num_blocks, new_order=None):
        """Append blocks nb..new_nb-1 to the free tail (the mlx-node paged-cache
        doc's pool-sizing section grows the pool before evicting)."""
        new_num_blocks = int(new_num_blocks)
        if new_num_blocks < self.nb:
            raise AllocError(ERR_INVALID_ARG, "cannot shrink")
        added = list(range(self.nb, new_num_blocks)) if new_order is None else [int(x) for x in new_order]
        if sorted(added) != list(range(self.nb, new_num_blocks)):
            raise AllocError(ERR_INVALID_ARG, "new_order must be a permutation of the new ids")
        grow_by = new_num_blocks - self.nb
        self.ref += [0] * grow_by
        self.chain_id += [0] * grow_by
        self.key_of += [None] * grow_by
        self.free.extend(added)
        self.nb = new_num_blocks
        self.max_nb = max(self.max_nb, self.nb)

    def set_max_blocks(self, max_blocks):
        """Ceiling of grow-on-demand (the pool-sizing section's maximum pool
        size); at least the current block count."""
        if int(max_blocks) < self.nb:
            raise AllocError(ERR_INVALID_ARG, "max_blocks below the current pool size")
        self.max_nb = int(max_blocks)

    def reserve_or_grow(self, seq_id, total_tokens):
        """allocate_suffix_blocks with grow-on-demand (mlx-node paged-cache doc,
        pool-sizing section: a reservation that outruns free + evictable
        blocks grows the pool before evicting, to min(max, max(2 x current,
        current + needed)) blocks; one grow, then one retry).

        Returns 0 when the reservation was made here. Otherwise nothing has
        changed and the return value is the block count the pool must grow to;
        the caller grows its pools, calls ``grow`` and retries with
        ``reserve``. A pool at its maximum raises ERR_NO_BLOCKS."""
        s = self._seq(seq_id)
        if total_tokens < 0:
            raise AllocError(ERR_INVALID_ARG, "negative token count")
        needed = -(-int(total_tokens) // self.bs) - len(s.blocks)
        if needed <= 0 or len(self.free) + len(self.lru) >= needed:
            self.reserve(seq_id, total_tokens)
            return 0
        if self.nb >= self.max_nb:
            raise AllocError(ERR_NO_BLOCKS, f"need {needed} blocks and the pool is at its maximum")
        return min(self.max_nb, max(2 * self.nb, self.nb + needed))

    def add(self, seq_id):
        if int(seq_id) in self.seqs:
            raise AllocError(ERR_STATE, f"sequence {seq_id} exists")
        self.seqs[int(seq_id)] = _Seq()

    def match_prefix(self, seq_id, tokens, domain):
        """Share the longest published chain of full blocks that prefixes ``tokens``.

        Only for a sequence that holds no blocks yet. Returns the number of
        cached tokens (a multiple of the block size).
        """
        s = self._seq(seq_id)
        if s.blocks:
            raise AllocError(ERR_STATE, "match_prefix needs an empty sequence")
        parent = 0
        tokens = [int(t) for t in tokens]
        for i in range(len(tokens) // self.bs):
            blk_tokens = tuple(tokens[i * self.bs:(i + 1) * self.bs])
            b = self.table.get((int(domain), parent, blk_tokens))
            if b is None:
                break
            if self.ref[b] == 0:
                del self.lru[b]
            self.ref[b] += 1
            s.blocks.append(b)
            s.tokens.extend(blk_tokens)
            parent = self.chain_id[b]
        return len(s.blocks) * self.bs

    def share_prefix(self, dst_id, src_id, num_blocks):
        """Make ``dst`` (empty) reference the first ``num_blocks`` full blocks of ``src``."""
        d = self._seq(dst_id)
        s = self._seq(src_id)
        if d.blocks:
            raise AllocError(ERR_STATE, "share_prefix needs an empty destination")
        if num_blocks < 0 or num_blocks > len(s.blocks) or num_blocks * self.bs > len(s.tokens):
            raise AllocError(ERR_STATE, "source does not hold that many full blocks")
        if any(b == 0 for b in s.blocks[:num_blocks]):
            raise AllocError(ERR_STATE, "cannot share a dropped block")
        for b in s.blocks[:num_blocks]:
            self.ref[b] += 1
            d.blocks.append(b)
        d.tokens = list(s.tokens[:num_blocks * self.bs])

    def reserve(self, seq_id, total_tokens):
        """Grow the table to ``ceil(total_tokens / BS)`` entries (all or nothing)."""
        s = self._seq(seq_id)
        if total_tokens < 0:
            raise AllocError(ERR_INVALID_ARG, "negative token count")
        need = -(-int(total_tokens) // self.bs) - len(s.blocks)
        if need <= 0:
            return
        if len(self.free) + len(self.lru) < need:
            raise AllocError(ERR_NO_BLOCKS, f"need {need} blocks")
        for _ in range(need):
            s.blocks.append(self._take_new())

    def commit_tokens(self, seq_id, tokens):
        """Record the token ids of the next positions (they must be reserved)."""
        s = self._seq(seq_id)
        tokens = [int(t) for t in tokens]
        if len(s.tokens) + len(tokens) > len(s.blocks) * self.bs:
            raise AllocError(ERR_CAPACITY, "commit beyond reserved blocks")
        s.tokens.extend(tokens)

    def publish_full_blocks(self, seq_id, domain):
        """Enter every full, unpublished block in the prefix table (stops at a null entry)."""
        s = self._seq(seq_id)
        parent = 0
        for i in range(len(s.tokens) // self.bs):
            b = s.blocks[i]
            if b == 0:
                break
            if self.chain_id[b]:
                parent = self.chain_id[b]
                continue
            key = (int(domain), parent, tuple(s.tokens[i * self.bs:(i + 1) * self.bs]))
            other = self.table.get(key)
            if other is not None:
                # Same content already published by another block: keep ours
                # private and continue the chain through the published one.
                parent = self.chain_id[other]
                continue
            self.chain_id[b] = self.next_chain_id
            self.next_chain_id += 1
            self.key_of[b] = key
            self.table[key] = b
            parent = self.chain_id[b]

    def drop_outside_window(self, seq_id, window):
        """Null every block wholly before position ``committed - window``."""
        s = self._seq(seq_id)
        if window <= 0:
            raise AllocError(ERR_INVALID_ARG, "window must be positive")
        first_needed = len(s.tokens) - int(window)
        for i, b in enumerate(s.blocks):
            if b != 0 and (i + 1) * self.bs <= first_needed:
                self._unref(b)
                s.blocks[i] = 0

    def release(self, seq_id):
        s = self._seq(seq_id)
        for b in reversed(s.blocks):
            if b != 0:
                self._unref(b)
        del self.seqs[int(seq_id)]

    # -- queries ---------------------------------------------------------
    def block_tables(self, seq_ids, max_blocks):
        need = max((len(self._seq(i).blocks) for i in seq_ids), default=0)
        if need > max_blocks:
            raise AllocError(ERR_CAPACITY, f"needs {need} columns")
        out = []
        for i in seq_ids:
            row = list(self._seq(i).blocks)
            out.append(row + [0] * (max_blocks - len(row)))
        return out

    def slot_mapping(self, seq_id, start_pos, n):
        s = self._seq(seq_id)
        out = []
        for p in range(int(start_pos), int(start_pos) + int(n)):
            i, off = divmod(p, self.bs)
            if p < 0 or i >= len(s.blocks):
                raise AllocError(ERR_CAPACITY, f"position {p} is not reserved")
            b = s.blocks[i]
            if b == 0:
                raise AllocError(ERR_STATE, f"position {p} lies in a dropped block")
            out.append(b * self.bs + off)
        return out

    def refcount(self, block_id):
        if not 0 <= block_id < self.nb:
            raise AllocError(ERR_INVALID_ARG, "block id out of range")
        return self.ref[block_id]

    def num_free(self):
        return len(self.free), len(self.lru)

    def num_tokens(self, seq_id):
        return len(self._seq(seq_id).tokens)

    def num_blocks_of(self, seq_id):
        return len(self._seq(seq_id).blocks)
