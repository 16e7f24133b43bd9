"""Block manager and block movement — oracle side, TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module; the library never does, and this module imports
nothing from it.

What it follows:

* page "vLLM推理引擎深度解析" §三 (``PagedAttentionManager``): physical blocks
  carry a share count; a request of n tokens takes ceil(n / block_size) blocks
  from the head of the free list and is refused when fewer are free; appending
  a token fills the request's last block and takes a new block from the head
  of the free list once that block is full; freeing a request lowers the count
  of each of its blocks and a block whose count reaches zero goes back to the
  tail of the free list; sharing a prefix raises the counts of the blocks that
  hold it.
* page "vLLM 原理与源码阅读" (PagedAttention 显存管理 → Block 管理器): requests
  that share a prompt prefix share its physical blocks, and a shared block is
  copied only when one of them has to write into it (copy-on-write).
* page "vLLM推理引擎深度实战" §5.3 (推理优化配置): a CPU swap space beside the
  GPU pool, i.e. whole blocks move between a device pool and a host pool.
* page "vLLM 原理与源码阅读" (Prefix Caching → 自动检测与复用): the prompt content
  is hashed into cache keys; a new request looks up the longest cached prefix;
  only the uncached suffix needs its KV computed; the hit blocks are shared
  through the block share counts.

Reading taken where the pages leave a step open or contradict themselves:
the §三 ``share_prefix`` listing can hand out a partly filled block and then
append into it, which would overwrite the other request's tokens. Here a
request whose last block is shared and not full gets a fresh block on its next
append: the manager reports the (source, destination) pair that the device
must copy before the token is written, and the shared block's count drops by
one. A full shared block needs no copy: the next token starts a new block.

Prefix caching, readings: the cache works on whole blocks. The key of full
block i of a prompt stands for the whole prefix tokens[0 : 16(i+1)] (here the
tuple of those tokens itself, so keys never collide); partly filled blocks
are never cached. A request's full prompt blocks enter the cache when the
caller publishes them (after their KV is written); an entry that exists
already keeps its block. A cached block whose count drops to zero stays
cached while it waits in the free list; taking it from the free list for
another use evicts its entry, and a cache hit on it takes it out of the
free list. A hit never covers more blocks than the prompt has full blocks.

Functions:

* ``BlockManager``: allocate / append / fork / share_prefix / free / slots, with
  the invariants checked by ``check_invariants``; prefix caching through
  ``allocate_cached`` (longest cached prefix, shared) and ``publish`` (a
  request's full prompt blocks enter the cache).
* ``copy_blocks``: for each (src, dst) pair, K and V of block dst become those
  of block src (the device copy that copy-on-write asks for); pairs with an
  index outside the pool are skipped.
* ``swap_blocks``: for each (src, dst) pair, block dst of the destination pool
  becomes block src of the source pool (device <-> host moves).

Pinned in ``tests/test_block_manager_oracle.py`` by the worked cases below the
pages' rules fix, by a contents check (every live request reads back exactly
its own tokens through its table, so a skipped copy-on-write is caught), by
invariants under random operation sequences, and by mutation tests.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK_SIZE = 16


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE,
                 free_order: Optional[Sequence[int]] = None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = range(self.num_blocks) if free_order is None else free_order
        self.free: List[int] = [int(b) for b in order]
        self.ref: List[int] = [0] * self.num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.cache: Dict[tuple, int] = {}          # whole-prefix key -> block
        self.key_of: Dict[int, tuple] = {}         # block -> its cache key

    # -- taking and returning blocks (head of the free list out, tail in) --
    def _take(self) -> int:
        if not self.free:
            raise MemoryError("no free block")
        b = self.free.pop(0)
        self.ref[b] = 1
        if b in self.key_of:                       # reused for other tokens: leaves the cache
            del self.cache[self.key_of.pop(b)]
        return b

    def _drop(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    # -- requests --
    def allocate(self, seq: int, num_tokens: int) -> List[int]:
        """A new request of num_tokens tokens: ceil(n / block_size) blocks, all or nothing."""
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        need = -(-int(num_tokens) // self.block_size)
        if need > len(self.free):
            raise MemoryError(f"need {need} blocks, {len(self.free)} free")
        self.tables[seq] = [self._take() for _ in range(need)]
        self.lens[seq] = int(num_tokens)
        return list(self.tables[seq])

    def append(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """One new token: returns its slot and the copy-on-write pair (src, dst) or None."""
        table, pos = self.tables[seq], self.lens[seq]
        cow = None
        if pos % self.block_size == 0:           # no block yet, or the last one is full
            table.append(self._take())
        elif self.ref[table[-1]] > 1:            # shared and not full: copy before writing
            old = table[-1]
            new = self._take()
            self._drop(old)
            table[-1] = new
            cow = (old, new)
        self.lens[seq] = pos + 1
        return table[pos // self.block_size] * self.block_size + pos % self.block_size, cow

    def fork(self, parent: int, child: int) -> None:
        """The child shares every block of the parent (one more count each)."""
        self.share_prefix(parent, child, self.lens[parent])

    def share_prefix(self, src: int, child: int, num_tokens: int) -> None:
        """The child's first num_tokens tokens are the source's: it shares the blocks holding them."""
        if child in self.tables:
            raise KeyError(f"sequence {child} exists")
        if not 0 <= num_tokens <= self.lens[src]:
            raise ValueError("prefix longer than the source")
        k = -(-int(num_tokens) // self.block_size)
        shared = self.tables[src][:k]
        for b in shared:
            self.ref[b] += 1
        self.tables[child] = list(shared)
        self.lens[child] = int(num_tokens)

    # -- prefix caching --
    def prefix_keys(self, tokens: Sequence[int]) -> List[tuple]:
        """Key of every full block of a prompt: the whole prefix up to the block's end."""
        bs = self.block_size
        return [tuple(int(t) for t in tokens[:bs * (i + 1)]) for i in range(len(tokens) // bs)]

    def allocate_cached(self, seq: int, tokens: Sequence[int]) -> int:
        """A new request for a prompt: the longest run of cached full blocks from its start
        is shared, fresh blocks cover the rest, all or nothing. Returns the number of leading
        tokens whose KV is already in the cache (a multiple of block_size)."""
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        hit = []
        for key in self.prefix_keys(tokens):
            if key not in self.cache:
                break
            hit.append(self.cache[key])
        need = -(-len(tokens) // self.block_size) - len(hit)
        idle = sum(1 for b in hit if self.ref[b] == 0)
        if need > len(self.free) - idle:
            raise MemoryError(f"need {need} blocks, {len(self.free) - idle} free")
        for b in hit:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
        self.tables[seq] = hit + [self._take() for _ in range(need)]
        self.lens[seq] = len(tokens)
        return len(hit) * self.block_size

    def publish(self, seq: int, tokens: Sequence[int]) -> int:
        """Enter the request's full blocks covering ``tokens`` (its first tokens, KV written)
        into the cache; returns how many entries were added."""
        n = min(len(tokens), self.lens[seq])
        added = 0
        for i, key in enumerate(self.prefix_keys(tokens[:n])):
            b = self.tables[seq][i]
            if key in self.cache or b in self.key_of:
                continue
            self.cache[key] = b
            self.key_of[b] = key
            added += 1
        return added

    def free_seq(self, seq: int) -> None:
        for b in self.tables.pop(seq):
            self._drop(b)
        del self.lens[seq]

    def slots(self, seq: int, pos0: int, count: int) -> List[int]:
        t = self.tables[seq]
        return [t[p // self.block_size] * self.block_size + p % self.block_size
                for p in range(pos0, pos0 + count)]

    def check_invariants(self) -> None:
        """Counts equal the number of tables holding a block; free list = blocks counted zero."""
        held = np.zeros(self.num_blocks, dtype=np.int64)
        for seq, t in self.tables.items():
            assert len(t) == -(-self.lens[seq] // self.block_size), f"table length of {seq}"
            for b in t:
                held[b] += 1
        assert list(held) == self.ref, "share counts"
        assert sorted(self.free) == [b for b in range(self.num_blocks) if self.ref[b] == 0], "free list"
        assert len(set(self.free)) == len(self.free), "free list duplicates"
        assert all(self.key_of[b] == k for k, b in self.cache.items()), "cache maps"
        assert len(self.key_of) == len(self.cache), "cache maps"


def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray, pairs) -> Tuple[np.ndarray, np.ndarray]:
    """K and V of block dst become those of block src, pair by pair; out-of-pool pairs skipped."""
    k, v = k_pool.copy(), v_pool.copy()
    n = k.shape[0]
    for s, d in pairs:
        if 0 <= s < n and 0 <= d < n:
            k[d] = k[s]
            v[d] = v[s]
    return k, v


def swap_blocks(dst_pool: np.ndarray, src_pool: np.ndarray, pairs) -> np.ndarray:
    """Block dst of the destination pool becomes block src of the source pool, pair by pair."""
    out = dst_pool.copy()
    for s, d in pairs:
        out[d] = src_pool[s]
    return out
