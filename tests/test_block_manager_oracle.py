"""Pins of the block-manager oracle (CPU only).

The oracle follows page "vLLM推理引擎深度解析" §三 (share counts, head-of-free-list
allocation, fill-then-new-block append, free to the tail), the copy-on-write of
shared blocks on page "vLLM 原理与源码阅读" (Block 管理器), and the device <-> host
block moves behind the swap space of page "vLLM推理引擎深度实战" §5.3. The pins
below do not re-run its code: worked cases whose numbers follow from those rules
by hand, a contents check that simulates the tokens each request writes (so a
request that ever reads another request's write is caught), invariants under
random operation sequences, and mutation tests that plant mistakes.
"""
import numpy as np
import pytest

from oracle import block_manager as OBM


def test_worked_case_from_the_rules():
    bm = OBM.BlockManager(16)
    assert bm.allocate(1, 50) == [0, 1, 2, 3]          # ceil(50/16) = 4 blocks from the head
    assert bm.allocate(2, 30) == [4, 5]
    assert bm.append(1) == (3 * 16 + 2, None)          # position 50: block 3, offset 2
    assert bm.allocate(3, 48) == [6, 7, 8]
    assert bm.append(3) == (9 * 16, None)              # 48 tokens fill 3 blocks: new block 9
    bm.share_prefix(1, 4, 50)                          # blocks holding positions 0..49
    assert bm.tables[4] == [0, 1, 2, 3] and bm.ref[:4] == [2, 2, 2, 2]
    # position 50 of request 4 lies in shared block 3, which request 1 has already
    # written past: copy it to the head of the free list (10), then write there
    assert bm.append(4) == (10 * 16 + 2, (3, 10))
    assert bm.tables[4] == [0, 1, 2, 10] and bm.ref[3] == 1 and bm.ref[10] == 1
    bm.free_seq(1)
    assert bm.ref[:4] == [1, 1, 1, 0]
    assert bm.free == [11, 12, 13, 14, 15, 3]          # freed blocks go to the tail
    assert bm.slots(4, 47, 4) == [2 * 16 + 15, 10 * 16, 10 * 16 + 1, 10 * 16 + 2]
    bm.check_invariants()


def test_full_shared_block_needs_no_copy():
    bm = OBM.BlockManager(8)
    bm.allocate(1, 32)
    bm.fork(1, 2)
    assert bm.append(2) == (2 * 16, None)              # 32 tokens: both shared blocks are full
    assert bm.tables[2] == [0, 1, 2] and bm.tables[1] == [0, 1]
    bm.check_invariants()


def test_refusal_changes_nothing():
    bm = OBM.BlockManager(4)
    bm.allocate(1, 40)                                 # 3 blocks
    before = (list(bm.free), list(bm.ref), {k: list(v) for k, v in bm.tables.items()})
    with pytest.raises(MemoryError):
        bm.allocate(2, 33)                             # needs 3, 1 free
    assert (bm.free, bm.ref, bm.tables) == (before[0], before[1], before[2])
    bm.append(1)                                       # 41 tokens fit in block 2
    bm.allocate(3, 16)                                 # takes the last block
    with pytest.raises(MemoryError):
        for _ in range(8):
            bm.append(1)                               # position 48 needs a fourth block
    bm.check_invariants()


class Contents:
    """Simulated pool contents: slot -> (request, position) of the token written there."""

    def __init__(self, bm):
        self.bm = bm
        self.pool = {}
        self.expect = {}                               # request -> list of (owner, position)

    def allocate(self, seq, n):
        self.bm.allocate(seq, n)
        for p, s in enumerate(self.bm.slots(seq, 0, n)):
            self.pool[s] = (seq, p)
        self.expect[seq] = [(seq, p) for p in range(n)]

    def append(self, seq):
        slot, cow = self.bm.append(seq)
        if cow is not None:                            # the device copy, then the write
            src, dst = cow
            for o in range(self.bm.block_size):
                if src * self.bm.block_size + o in self.pool:
                    self.pool[dst * self.bm.block_size + o] = self.pool[src * self.bm.block_size + o]
        p = len(self.expect[seq])
        self.pool[slot] = (seq, p)
        self.expect[seq].append((seq, p))

    def share(self, src, child, n):
        self.bm.share_prefix(src, child, n)
        self.expect[child] = list(self.expect[src][:n])

    def free(self, seq):
        self.bm.free_seq(seq)
        del self.expect[seq]

    def check(self):
        for seq, want in self.expect.items():
            got = [self.pool.get(s) for s in self.bm.slots(seq, 0, len(want))]
            assert got == want, f"request {seq} reads {got[:4]}... instead of its own tokens"


def random_ops(seed, num_blocks=64, steps=400):
    """A seeded mix of allocate / append / fork / share_prefix / free on one manager."""
    rng = np.random.default_rng(seed)
    c = Contents(OBM.BlockManager(num_blocks, free_order=rng.permutation(num_blocks)))
    nxt = 0
    for _ in range(steps):
        live = list(c.expect)
        op = rng.integers(0, 10)
        try:
            if op < 2 or not live:
                c.allocate(nxt, int(rng.integers(0, 70)))
                nxt += 1
            elif op < 6:
                c.append(live[int(rng.integers(0, len(live)))])
            elif op < 8:
                src = live[int(rng.integers(0, len(live)))]
                c.share(src, nxt, int(rng.integers(0, len(c.expect[src]) + 1)))
                nxt += 1
            else:
                c.free(live[int(rng.integers(0, len(live)))])
        except MemoryError:
            pass
        c.bm.check_invariants()
        c.check()
    return c


@pytest.mark.parametrize("seed", range(12))
def test_random_operation_sequences_keep_contents_and_invariants(seed):
    c = random_ops(seed)
    assert c.expect, "the sequence should leave live requests"


def test_copy_and_swap_blocks_by_block_identity():
    k = np.arange(8)[:, None, None].repeat(16, 1).repeat(3, 2).astype(np.float32)
    v = -k
    k2, v2 = OBM.copy_blocks(k, v, [(1, 5), (2, 6), (7, 9), (-1, 0)])  # the last two leave the pool
    assert [int(b[0, 0]) for b in k2] == [0, 1, 2, 3, 4, 1, 2, 7]
    assert [int(b[0, 0]) for b in v2] == [0, -1, -2, -3, -4, -1, -2, -7]
    host = np.zeros((4, 16, 3), np.float32)
    h2 = OBM.swap_blocks(host, k, [(6, 0), (3, 2)])
    assert [int(b[0, 0]) for b in h2] == [6, 0, 3, 0]


# -- mutation tests: plant a mistake in the oracle, some pin must catch it --

def test_mutation_no_copy_on_write_is_caught(monkeypatch):
    def append(self, seq):
        table, pos = self.tables[seq], self.lens[seq]
        if pos % self.block_size == 0:
            table.append(self._take())
        self.lens[seq] = pos + 1
        return table[pos // self.block_size] * self.block_size + pos % self.block_size, None
    monkeypatch.setattr(OBM.BlockManager, "append", append)
    with pytest.raises(AssertionError):
        for seed in range(12):
            random_ops(seed)


def test_mutation_lifo_free_list_is_caught(monkeypatch):
    def _take(self):
        if not self.free:
            raise MemoryError
        b = self.free.pop()
        self.ref[b] = 1
        return b
    monkeypatch.setattr(OBM.BlockManager, "_take", _take)
    with pytest.raises(AssertionError):
        test_worked_case_from_the_rules()


def test_mutation_prefix_rounds_down_is_caught(monkeypatch):
    orig = OBM.BlockManager.share_prefix

    def share_prefix(self, src, child, n):
        orig(self, src, child, n - n % self.block_size)
        self.lens[child] = n
    monkeypatch.setattr(OBM.BlockManager, "share_prefix", share_prefix)
    with pytest.raises((AssertionError, IndexError)):
        for seed in range(12):
            random_ops(seed)


# -- prefix caching (page "vLLM 原理与源码阅读", Prefix Caching: hash the prompt, find the
# -- longest cached prefix, compute only the suffix, share the hit blocks) --

def test_prefix_cache_worked_case():
    bm = OBM.BlockManager(8)
    a = list(range(100, 140))                          # 40 tokens: 2 full blocks + 8
    assert bm.allocate_cached(1, a) == 0               # empty cache: nothing cached
    assert bm.tables[1] == [0, 1, 2]
    assert bm.publish(1, a) == 2                       # the two full blocks enter the cache
    b = a[:35] + [7] * 15                              # shares 35 tokens = 2 full blocks
    assert bm.allocate_cached(2, b) == 32
    assert bm.tables[2] == [0, 1, 3, 4] and bm.ref[:5] == [2, 2, 1, 1, 1]
    c = [5] + a[1:32]                                  # first block differs, second equal
    assert bm.allocate_cached(3, c) == 0               # keys stand for whole prefixes
    assert bm.tables[3] == [5, 6]
    bm.free_seq(1)
    bm.free_seq(2)
    # freed blocks go to the tail in table order: request 1 frees 2, request 2 frees 0 1 3 4
    assert bm.ref[:2] == [0, 0] and bm.free == [7, 2, 0, 1, 3, 4]
    # blocks 0 and 1 wait in the free list, still cached: a new request hits them
    assert bm.allocate_cached(4, a[:33]) == 32
    assert bm.tables[4] == [0, 1, 7] and bm.free == [2, 3, 4]
    bm.free_seq(4)                                     # free list: 2 3 4 0 1 7 (0, 1 cached)
    assert bm.free == [2, 3, 4, 0, 1, 7] and len(bm.cache) == 2
    assert bm.allocate_cached(5, list(range(80))) == 0 # takes 2 3 4 0 1: both leave the cache
    assert bm.free == [7] and bm.cache == {}
    assert bm.allocate_cached(6, a[:16]) == 0          # nothing cached any more
    bm.check_invariants()


def test_prefix_cache_refusal_counts_idle_hits():
    bm = OBM.BlockManager(3)
    a = list(range(32))
    bm.allocate_cached(1, a)
    bm.publish(1, a)
    bm.free_seq(1)                                     # blocks 0, 1 cached and idle; 2 free
    # 48 tokens: 2 hits (idle, leave the free list) + 1 fresh = all 3 blocks
    assert bm.allocate_cached(2, a + [9] * 16) == 32
    bm.free_seq(2)
    before = (list(bm.free), list(bm.ref), dict(bm.cache))
    with pytest.raises(MemoryError):                   # 2 idle hits + 2 fresh > 3 blocks
        bm.allocate_cached(3, a + [9] * 17)
    assert (bm.free, bm.ref, bm.cache) == before
    bm.check_invariants()


class PrefixContents:
    """Simulated pool: every slot records the whole token prefix whose last token it holds
    (K/V of a token depend on all tokens before it). Every live request must read, at each
    position p, exactly its own tokens[0 : p+1]."""

    def __init__(self, bm):
        self.bm, self.pool, self.toks = bm, {}, {}

    def _write(self, seq, positions):
        t = self.toks[seq]
        for p, s in zip(positions, self.bm.slots(seq, positions[0], len(positions))):
            self.pool[s] = tuple(t[:p + 1])

    def allocate(self, seq, tokens):
        cached = self.bm.allocate_cached(seq, tokens)
        self.toks[seq] = list(tokens)
        if cached < len(tokens):                       # compute the suffix only
            self._write(seq, list(range(cached, len(tokens))))
        return cached

    def publish(self, seq):
        self.bm.publish(seq, self.toks[seq])

    def append(self, seq, token):
        slot, cow = self.bm.append(seq)
        bs = self.bm.block_size
        if cow is not None:
            src, dst = cow
            for o in range(bs):
                if src * bs + o in self.pool:
                    self.pool[dst * bs + o] = self.pool[src * bs + o]
        self.toks[seq].append(token)
        self.pool[slot] = tuple(self.toks[seq])

    def fork(self, src, child):
        self.bm.fork(src, child)
        self.toks[child] = list(self.toks[src])

    def free(self, seq):
        self.bm.free_seq(seq)
        del self.toks[seq]

    def check(self):
        for seq, t in self.toks.items():
            got = [self.pool.get(s) for s in self.bm.slots(seq, 0, len(t))]
            want = [tuple(t[:p + 1]) for p in range(len(t))]
            assert got == want, f"request {seq} reads another prefix's KV"


def prefix_ops(seed, num_blocks=48, steps=300):
    rng = np.random.default_rng(seed)
    c = PrefixContents(OBM.BlockManager(num_blocks, free_order=rng.permutation(num_blocks)))
    # three system prompts; the second starts like the first, the third ends like the first
    sp0 = [int(x) for x in rng.integers(0, 50, 40)]
    systems = [sp0, sp0[:16] + [int(x) for x in rng.integers(0, 50, 24)], [999] * 16 + sp0[16:]]
    nxt, hits = 0, 0
    for _ in range(steps):
        live = list(c.toks)
        op = int(rng.integers(0, 10))
        try:
            if op < 3 or not live:
                sp = systems[int(rng.integers(0, 3))]
                prompt = sp[:int(rng.integers(0, len(sp) + 1))] + [int(x) for x in rng.integers(0, 50, int(rng.integers(0, 30)))]
                hits += c.allocate(nxt, prompt) > 0
                if rng.random() < 0.8:
                    c.publish(nxt)
                nxt += 1
            elif op < 6:
                c.append(live[int(rng.integers(0, len(live)))], int(rng.integers(0, 50)))
            elif op < 7:
                c.fork(live[int(rng.integers(0, len(live)))], nxt)
                nxt += 1
            else:
                c.free(live[int(rng.integers(0, len(live)))])
        except MemoryError:
            pass
        c.bm.check_invariants()
        c.check()
    return c, hits


@pytest.mark.parametrize("seed", range(10))
def test_prefix_cache_random_sequences_read_their_own_prefixes(seed):
    c, hits = prefix_ops(seed)
    assert hits > 0, "the sequence should exercise cache hits"


def test_mutation_unchained_block_keys_are_caught(monkeypatch):
    def prefix_keys(self, tokens):                     # a block's own tokens only
        bs = self.block_size
        return [(i, tuple(tokens[bs * i:bs * (i + 1)])) for i in range(len(tokens) // bs)]
    monkeypatch.setattr(OBM.BlockManager, "prefix_keys", prefix_keys)
    with pytest.raises(AssertionError):
        for seed in range(10):
            prefix_ops(seed)


def test_mutation_no_eviction_on_reuse_is_caught(monkeypatch):
    def _take(self):
        if not self.free:
            raise MemoryError
        b = self.free.pop(0)
        self.ref[b] = 1
        return b                                       # keeps a stale cache entry
    monkeypatch.setattr(OBM.BlockManager, "_take", _take)
    with pytest.raises(AssertionError):
        for seed in range(10):
            prefix_ops(seed)
