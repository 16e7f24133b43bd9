"""Seeded synthetic inputs for the paged KV-cache attention path.

Both sides of every parity check consume what this module builds: the HIP
library (through its Python binding) and the CPU oracle. It holds none of the
attention arithmetic. It only

* draws context lengths and N(0, 1) values from ``numpy.random.default_rng``
  sub-streams of one seed, rounded to the storage dtype (round to nearest even);
* plays the block manager: hands out 16-token physical blocks from a seeded
  shuffled free list, builds per-sequence block tables, shares whole prefix
  blocks with a reference count, and places every prior token's K/V in the slot
  its table names;
* records where each new token must go (``slot_mapping``), following the append
  rule of the page "vLLM推理引擎深度解析" §三 (``PagedAttentionManager.append_token``:
  a token goes into the last block while it has room, otherwise into a freshly
  taken block);
* NaN-poisons every slot that holds no live token (free blocks, the tails of
  last blocks, and the new tokens' own slots until they are scattered), since
  recycled blocks carry stale data (same page, ``free_request``; page
  "vLLM推理引擎深度实战" §1.2, ``free_sequence``).

Block geometry: the page "vLLM 原理与源码阅读" (PagedAttention 显存管理 → Block
管理器) gives 16 tokens per block as the default; the page "vLLM推理引擎深度实战"
§1.2 sets ``BLOCK_SIZE = 16``. One logical block maps to one physical block
(page "vLLM推理引擎深度解析" §三). Each physical block stores its tokens
token-major, ``[16][num_kv_heads][head_dim]``, as the ``(block_size, n_heads,
head_dim)`` per-block K and V planes of ``PagedAttention.forward`` (same page,
§五); K and V live in two separate pools.

Storage dtypes: ``f32`` -> ``numpy.float32``, ``f16`` -> ``numpy.float16``,
``bf16`` -> ``numpy.uint16`` bit patterns (numpy has no bfloat16).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

BLOCK_SIZE = 16
DTYPES = ("f32", "f16", "bf16")
_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
# Element size in bytes for each storage dtype.
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
# dtype codes of the C ABI (include/pa.h, pa_dtype_t)
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


# ----------------------------------------------------------------------------
# value generation and storage
# ----------------------------------------------------------------------------
def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype, round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        u = x.view(np.uint32)
        # finite inputs only (N(0,1) draws): add 0x7FFF plus the lsb of the kept half
        bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        return ((u + bias) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(dtype)


def poison_value(dtype: str):
    """A quiet NaN in the storage dtype."""
    if dtype == "f32":
        return np.float32(np.nan)
    if dtype == "f16":
        return np.float16(np.nan)
    if dtype == "bf16":
        return np.uint16(0x7FC0)
    raise ValueError(dtype)


def normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0, 1) drawn in float32, then rounded to ``dtype``."""
    return round_to(rng.standard_normal(shape, dtype=np.float32), dtype)


def is_nan_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Elementwise NaN test on storage arrays (bf16 bit patterns included)."""
    if dtype == "bf16":
        return ((a & 0x7F80) == 0x7F80) & ((a & 0x007F) != 0)
    return np.isnan(a)


# ----------------------------------------------------------------------------
# block manager (harness role)
# ----------------------------------------------------------------------------
class BlockAllocator:
    """Physical block pool with a seeded shuffled free list and reference counts.

    Taking blocks pops the head of the free list; running out raises
    ``MemoryError``, the convention of the page "vLLM推理引擎深度实战" §1.2
    (``allocate_sequence``). Shared blocks carry ``ref_count > 1``, as
    ``share_prefix`` on the page "vLLM推理引擎深度解析" §三 counts them.
    """

    def __init__(self, num_blocks: int, rng: np.random.Generator):
        self.num_blocks = int(num_blocks)
        self.free: List[int] = [int(i) for i in rng.permutation(self.num_blocks)]
        self.ref_count = np.zeros(self.num_blocks, dtype=np.int32)

    def take(self, n: int) -> List[int]:
        if n > len(self.free):
            raise MemoryError(f"need {n} blocks, {len(self.free)} free")
        ids, self.free = self.free[:n], self.free[n:]
        for i in ids:
            self.ref_count[i] = 1
        return ids

    def share(self, ids: List[int]) -> List[int]:
        for i in ids:
            self.ref_count[i] += 1
        return list(ids)

    def release(self, ids: List[int]) -> None:
        for i in ids:
            self.ref_count[i] -= 1
            if self.ref_count[i] == 0:
                self.free.append(int(i))


def slot_of(table_row, pos: int, block_size: int = BLOCK_SIZE) -> int:
    """Flat slot of logical position ``pos``: physical block * block_size + offset."""
    return int(table_row[pos // block_size]) * block_size + pos % block_size


def slots_of(table_row: np.ndarray, positions: np.ndarray, block_size: int = BLOCK_SIZE) -> np.ndarray:
    positions = np.asarray(positions, dtype=np.int64)
    return (np.asarray(table_row, dtype=np.int64)[positions // block_size] * block_size
            + positions % block_size)


def _pool_arrays(num_blocks, num_kv_heads, head_dim, dtype):
    shape = (num_blocks, BLOCK_SIZE, num_kv_heads, head_dim)
    k = np.empty(shape, dtype=_STORAGE[dtype])
    v = np.empty(shape, dtype=_STORAGE[dtype])
    k.fill(poison_value(dtype))
    v.fill(poison_value(dtype))
    return k, v


def _place(pool: np.ndarray, slots: np.ndarray, rows: np.ndarray) -> None:
    """Write token rows into their slots (harness placement of prior context)."""
    flat = pool.reshape(-1, pool.shape[2], pool.shape[3])
    flat[slots] = rows


# ----------------------------------------------------------------------------
# decode cases
# ----------------------------------------------------------------------------
@dataclass
class DecodeCase:
    name: str
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    context_lens: np.ndarray          # int32 [B], tokens in cache after the scatter
    block_tables: np.ndarray          # int32 [B, max_blocks], padding -1
    num_blocks: int
    k_pool: np.ndarray                # [num_blocks, 16, H_kv, D] storage dtype (new slots NaN)
    v_pool: np.ndarray
    query: np.ndarray                 # [B, H_q, D]
    k_new: np.ndarray                 # [B, H_kv, D]
    v_new: np.ndarray
    slot_mapping: np.ndarray          # int32 [B]
    ref_count: np.ndarray             # int32 [num_blocks]
    shared_blocks: List[int] = field(default_factory=list)
    sharers: List[int] = field(default_factory=list)
    dense_k: Optional[List[np.ndarray]] = None   # per sequence [L_b, H_kv, D], built before paging
    dense_v: Optional[List[np.ndarray]] = None

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def block_stride(self) -> int:
        """Elements between consecutive physical blocks of one pool."""
        return BLOCK_SIZE * self.num_kv_heads * self.head_dim

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0


def make_decode(name: str, dtype: str, context_lens, num_q_heads: int, num_kv_heads: int,
                head_dim: int, seed: int, num_blocks: Optional[int] = None,
                pool_factor: float = 1.1, prefix_tokens: int = 0, sharers=None,
                keep_dense: bool = False, table_pad: int = 0) -> DecodeCase:
    """One decode step: every sequence has ``L_b - 1`` prior tokens cached and one new token.

    ``context_lens`` counts tokens in cache after the new token's scatter, so the new
    token sits at position ``L_b - 1``. ``sharers`` (sequence indices) share the first
    ``prefix_tokens // 16`` blocks, which must be whole blocks strictly below every
    sharer's new position, so no write ever lands in a shared block.
    """
    lens = np.asarray(context_lens, dtype=np.int64)
    B = len(lens)
    ss = np.random.SeedSequence(seed)
    s_perm, s_q, s_kv, s_new = (np.random.default_rng(s) for s in ss.spawn(4))
    sharers = sorted(int(i) for i in (sharers or []))
    if prefix_tokens % BLOCK_SIZE:
        raise ValueError("shared prefix must be whole blocks")
    n_prefix_blocks = prefix_tokens // BLOCK_SIZE
    for b in sharers:
        if lens[b] <= prefix_tokens:
            raise ValueError("a sharer's new token would land in a shared block")

    need_per_seq = [ceil_div(int(L), BLOCK_SIZE) for L in lens]
    own = [n - (n_prefix_blocks if b in sharers else 0) for b, n in enumerate(need_per_seq)]
    need = sum(own) + (n_prefix_blocks if sharers else 0)
    if num_blocks is None:
        num_blocks = max(1, math.ceil(pool_factor * need))
    alloc = BlockAllocator(num_blocks, s_perm)

    shared = alloc.take(n_prefix_blocks) if sharers and n_prefix_blocks else []
    tables = []
    for b in range(B):
        if b in sharers:
            row = list(shared) + alloc.take(own[b])
        else:
            row = alloc.take(own[b])
        tables.append(row)
    if shared:
        # the first taker already holds one reference per block
        for _ in range(len(sharers) - 1):
            alloc.share(shared)

    max_blocks = max(need_per_seq + [1]) + table_pad
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    for b, row in enumerate(tables):
        bt[b, : len(row)] = row

    k_pool, v_pool = _pool_arrays(num_blocks, num_kv_heads, head_dim, dtype)
    q = normal(s_q, (B, num_q_heads, head_dim), dtype)
    k_new = normal(s_new, (B, num_kv_heads, head_dim), dtype)
    v_new = normal(s_new, (B, num_kv_heads, head_dim), dtype)

    prefix_k = prefix_v = None
    if sharers and prefix_tokens:
        prefix_k = normal(s_kv, (prefix_tokens, num_kv_heads, head_dim), dtype)
        prefix_v = normal(s_kv, (prefix_tokens, num_kv_heads, head_dim), dtype)
        pos = np.arange(prefix_tokens)
        _place(k_pool, slots_of(bt[sharers[0]], pos), prefix_k)
        _place(v_pool, slots_of(bt[sharers[0]], pos), prefix_v)

    dense_k = [] if keep_dense else None
    dense_v = [] if keep_dense else None
    slot_mapping = np.empty(B, dtype=np.int32)
    for b in range(B):
        L = int(lens[b])
        start = prefix_tokens if b in sharers else 0
        n_own_prior = max(L - 1 - start, 0)
        kk = normal(s_kv, (n_own_prior, num_kv_heads, head_dim), dtype)
        vv = normal(s_kv, (n_own_prior, num_kv_heads, head_dim), dtype)
        if n_own_prior:
            pos = np.arange(start, L - 1)
            _place(k_pool, slots_of(bt[b], pos), kk)
            _place(v_pool, slots_of(bt[b], pos), vv)
        slot_mapping[b] = slot_of(bt[b], L - 1) if L >= 1 else -1
        if keep_dense:
            parts_k = ([prefix_k] if start else []) + [kk, k_new[b:b + 1]]
            parts_v = ([prefix_v] if start else []) + [vv, v_new[b:b + 1]]
            dense_k.append(np.concatenate(parts_k, axis=0)[:L])
            dense_v.append(np.concatenate(parts_v, axis=0)[:L])

    return DecodeCase(name=name, dtype=dtype, num_seqs=B, num_q_heads=num_q_heads,
                      num_kv_heads=num_kv_heads, head_dim=head_dim,
                      scale=float(np.float32(1.0 / math.sqrt(head_dim))),
                      context_lens=lens.astype(np.int32), block_tables=bt,
                      num_blocks=num_blocks, k_pool=k_pool, v_pool=v_pool, query=q,
                      k_new=k_new, v_new=v_new, slot_mapping=slot_mapping,
                      ref_count=alloc.ref_count.copy(), shared_blocks=list(shared),
                      sharers=sharers, dense_k=dense_k, dense_v=dense_v)


# ----------------------------------------------------------------------------
# FP8 (e4m3) cache contents for a decode case
# ----------------------------------------------------------------------------
E4M3_NAN_CODES = (0x7F, 0xFF)     # S.1111.111 in the OCP E4M3 format


@dataclass
class Fp8Pools:
    k_pool: np.ndarray                # uint8 codes [num_blocks, 16, H_kv, D]
    v_pool: np.ndarray
    k_scale: np.ndarray               # float32 [H_kv]
    v_scale: np.ndarray


def fp8_pools(case: DecodeCase, seed: int = 0) -> Fp8Pools:
    """Cache contents of ``case`` as e4m3 codes: every live slot holds codes drawn
    uniformly from the 254 non-NaN codes (magnitudes spread over the whole format,
    subnormals included); every slot the 16-bit pools poison (free blocks, tails,
    the new tokens' slots) holds a NaN code. Per-kv-head scales are drawn from
    [1/448, 1/112], so stored values reach +-1 to +-4."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 8]))
    finite = np.array([c for c in range(256) if c not in E4M3_NAN_CODES], dtype=np.uint8)
    out = []
    for pool in (case.k_pool, case.v_pool):
        codes = finite[rng.integers(0, len(finite), size=pool.shape, dtype=np.uint8)]
        codes[is_nan_storage(pool, case.dtype)] = E4M3_NAN_CODES[0]
        out.append(codes)
    ks = rng.uniform(1 / 448, 1 / 112, case.num_kv_heads).astype(np.float32)
    vs = rng.uniform(1 / 448, 1 / 112, case.num_kv_heads).astype(np.float32)
    return Fp8Pools(out[0], out[1], ks, vs)


# ----------------------------------------------------------------------------
# prefill cases
# ----------------------------------------------------------------------------
@dataclass
class PrefillCase:
    name: str
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    prior_lens: np.ndarray            # int32 [B], tokens already cached before the chunk
    q_lens: np.ndarray                # int32 [B], new tokens in this chunk
    seq_lens: np.ndarray              # int32 [B] = prior + q_len, keys including the chunk
    cu_q_lens: np.ndarray             # int32 [B+1]
    block_tables: np.ndarray
    num_blocks: int
    k_pool: np.ndarray
    v_pool: np.ndarray
    query: np.ndarray                 # [T, H_q, D], T = sum(q_lens)
    k_new: np.ndarray                 # [T, H_kv, D]
    v_new: np.ndarray
    slot_mapping: np.ndarray          # int32 [T]
    dense_k: Optional[List[np.ndarray]] = None
    dense_v: Optional[List[np.ndarray]] = None

    @property
    def num_q_tokens(self) -> int:
        return int(self.cu_q_lens[-1])

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def block_stride(self) -> int:
        return BLOCK_SIZE * self.num_kv_heads * self.head_dim

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def make_prefill(name: str, dtype: str, prior_lens, q_lens, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, seed: int, pool_factor: float = 1.1,
                 keep_dense: bool = False) -> PrefillCase:
    """A chunk of ``q_lens[b]`` new tokens appended after ``prior_lens[b]`` cached ones."""
    prior = np.asarray(prior_lens, dtype=np.int64)
    ql = np.asarray(q_lens, dtype=np.int64)
    B = len(prior)
    total = prior + ql
    ss = np.random.SeedSequence(seed)
    s_perm, s_q, s_kv, s_new = (np.random.default_rng(s) for s in ss.spawn(4))
    need_per_seq = [ceil_div(int(t), BLOCK_SIZE) for t in total]
    num_blocks = max(1, math.ceil(pool_factor * sum(need_per_seq)))
    alloc = BlockAllocator(num_blocks, s_perm)
    tables = [alloc.take(n) for n in need_per_seq]
    bt = np.full((B, max(need_per_seq + [1])), -1, dtype=np.int32)
    for b, row in enumerate(tables):
        bt[b, : len(row)] = row
    k_pool, v_pool = _pool_arrays(num_blocks, num_kv_heads, head_dim, dtype)
    T = int(ql.sum())
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ql)
    q = normal(s_q, (T, num_q_heads, head_dim), dtype)
    k_new = normal(s_new, (T, num_kv_heads, head_dim), dtype)
    v_new = normal(s_new, (T, num_kv_heads, head_dim), dtype)
    slot_mapping = np.empty(T, dtype=np.int32)
    dense_k = [] if keep_dense else None
    dense_v = [] if keep_dense else None
    for b in range(B):
        P = int(prior[b])
        kk = normal(s_kv, (P, num_kv_heads, head_dim), dtype)
        vv = normal(s_kv, (P, num_kv_heads, head_dim), dtype)
        if P:
            _place(k_pool, slots_of(bt[b], np.arange(P)), kk)
            _place(v_pool, slots_of(bt[b], np.arange(P)), vv)
        slot_mapping[cu[b]:cu[b + 1]] = slots_of(bt[b], np.arange(P, P + int(ql[b])))
        if keep_dense:
            dense_k.append(np.concatenate([kk, k_new[cu[b]:cu[b + 1]]], axis=0))
            dense_v.append(np.concatenate([vv, v_new[cu[b]:cu[b + 1]]], axis=0))
    return PrefillCase(name=name, dtype=dtype, num_seqs=B, num_q_heads=num_q_heads,
                       num_kv_heads=num_kv_heads, head_dim=head_dim,
                       scale=float(np.float32(1.0 / math.sqrt(head_dim))),
                       prior_lens=prior.astype(np.int32), q_lens=ql.astype(np.int32),
                       seq_lens=total.astype(np.int32), cu_q_lens=cu, block_tables=bt,
                       num_blocks=num_blocks, k_pool=k_pool, v_pool=v_pool, query=q,
                       k_new=k_new, v_new=v_new, slot_mapping=slot_mapping,
                       dense_k=dense_k, dense_v=dense_v)


# ----------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------
def _log_uniform_lens(rng, n, lo, hi):
    # integers with log-uniform density on [lo, hi], both ends reachable
    return np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi + 1), size=n))).astype(np.int64).clip(lo, hi)


def tiny_fp32(seed: int = 1, keep_dense: bool = True) -> DecodeCase:
    """4 sequences, lengths {5, 16, 17, 40}, 4 heads (MHA), head_dim 64, fp32, 32-block pool."""
    return make_decode("tiny_fp32_mha_d64", "f32", [5, 16, 17, 40], 4, 4, 64, seed,
                       num_blocks=32, keep_dense=keep_dense)


def llama2_7b_fp16(seed: int = 2, keep_dense: bool = False) -> DecodeCase:
    """Batch 64, 32 q = 32 kv heads, head_dim 128, fp16, lengths uniform on [128, 2048]."""
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(5)[4])
    lens = rng.integers(128, 2048, size=64, endpoint=True)
    return make_decode("llama2_7b_fp16_b64", "f16", lens, 32, 32, 128, seed, keep_dense=keep_dense)


def llama3_8b_gqa_bf16(seed: int = 3, keep_dense: bool = False) -> DecodeCase:
    """Batch 256, 32 q / 8 kv heads, head_dim 128, bf16, log-uniform lengths on [64, 4096];
    the 128 longest sequences share one 512-token system-prompt prefix (32 whole blocks)."""
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(5)[4])
    lens = _log_uniform_lens(rng, 256, 64, 4096)
    order = np.argsort(-lens, kind="stable")
    sharers = [int(i) for i in order[:128]]
    lens[sharers] = np.maximum(lens[sharers], 513)
    return make_decode("llama3_8b_gqa_bf16_b256", "bf16", lens, 32, 8, 128, seed,
                       prefix_tokens=512, sharers=sharers, keep_dense=keep_dense)


def long_context_bf16(seed: int = 4, keep_dense: bool = False) -> DecodeCase:
    """Batch 8, 64 q / 8 kv heads, head_dim 128, bf16, lengths uniform on [32768, 131072]."""
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(5)[4])
    lens = rng.integers(32768, 131072, size=8, endpoint=True)
    return make_decode("long_ctx_splitkv_bf16_b8", "bf16", lens, 64, 8, 128, seed, keep_dense=keep_dense)


def chunked_prefill_bf16(seed: int = 5, keep_dense: bool = False) -> PrefillCase:
    """16 sequences, 2048 cached tokens plus a 512-token chunk, 32 q / 8 kv heads, head_dim 128."""
    return make_prefill("chunked_prefill_bf16_16x2048p512", "bf16", [2048] * 16, [512] * 16,
                        32, 8, 128, seed, keep_dense=keep_dense)


NAMED = {
    "tiny": tiny_fp32,
    "llama2_7b_fp16": llama2_7b_fp16,
    "llama3_8b_gqa_bf16": llama3_8b_gqa_bf16,
    "long_context_bf16": long_context_bf16,
    "chunked_prefill_bf16": chunked_prefill_bf16,
}


# ----------------------------------------------------------------------------
# host-side validator of index preconditions
# ----------------------------------------------------------------------------
def validate_indices(num_blocks: int, block_tables: np.ndarray, lens: np.ndarray,
                     slot_mapping: Optional[np.ndarray] = None) -> None:
    """Raise ``ValueError`` unless tables cover ceil(L/16) in-range ids and live slots are unique."""
    lens = np.asarray(lens)
    if (lens < 0).any():
        raise ValueError("negative length")
    for b, L in enumerate(lens):
        n = ceil_div(int(L), BLOCK_SIZE)
        if n > block_tables.shape[1]:
            raise ValueError(f"table of sequence {b} too short")
        row = block_tables[b, :n]
        if ((row < 0) | (row >= num_blocks)).any():
            raise ValueError(f"table of sequence {b} names a block out of range")
    if slot_mapping is not None:
        live = slot_mapping[slot_mapping >= 0]
        if (live >= num_blocks * BLOCK_SIZE).any():
            raise ValueError("slot out of range")
        if len(np.unique(live)) != len(live):
            raise ValueError("duplicate slot")
