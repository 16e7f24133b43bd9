"""Plain fp64 NumPy oracle of paged attention — TEST INFRASTRUCTURE ONLY.

See the package docstring for what may import this module. Nothing here is
blocked, fused or reordered beyond what the definitions state.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK_SIZE = 16


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of storage values to float64 (bf16 arrives as uint16 bit patterns)."""
    if dtype == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype in ("f16", "f32"):
        return np.asarray(a).astype(np.float64)
    raise ValueError(dtype)


def _scale64(scale: float) -> float:
    # the library receives the scale as a float32 argument
    return float(np.float32(scale))


def kv_head_of(q_head: int, num_q_heads: int, num_kv_heads: int) -> int:
    """Grouped-query mapping: query heads form contiguous groups of size H_q / H_kv.

    The pages only show multi-head attention (one K/V head per query head, page
    "vLLM推理引擎深度解析" §五); with H_q == H_kv this is the identity.
    """
    return q_head // (num_q_heads // num_kv_heads)


# ----------------------------------------------------------------------------
# cache write
# ----------------------------------------------------------------------------
def scatter(k_pool: np.ndarray, v_pool: np.ndarray, key: np.ndarray, value: np.ndarray,
            slot_mapping: np.ndarray, block_size: int = BLOCK_SIZE):
    """Return copies of the pools with token t's K/V rows written at slot ``slot_mapping[t]``.

    A slot names physical block ``slot // block_size`` and offset ``slot % block_size``
    (one slot per token of a block; page "vLLM推理引擎深度解析" §三). Negative slots are
    skipped. Values are copied bit for bit in the storage dtype; later tokens win on a
    repeated slot.
    """
    out_k = k_pool.copy()
    out_v = v_pool.copy()
    for t, s in enumerate(np.asarray(slot_mapping)):
        s = int(s)
        if s < 0:
            continue
        out_k[s // block_size, s % block_size] = key[t]
        out_v[s // block_size, s % block_size] = value[t]
    return out_k, out_v


# ----------------------------------------------------------------------------
# gather through the block table
# ----------------------------------------------------------------------------
def gather(pool: np.ndarray, table_row: np.ndarray, length: int, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Logical rows ``0 .. length-1`` of one sequence: ``[length, H_kv, D]`` in storage dtype.

    Logical block ``i`` of the sequence is physical block ``table_row[i]``; token ``j`` is row
    ``j % block_size`` of logical block ``j // block_size``, and ``ceil(length / block_size)``
    table entries are read (page "vLLM推理引擎深度解析" §五, ``PagedAttention.forward``).
    """
    n_blocks = math.ceil(length / block_size)
    rows = []
    for i in range(n_blocks):
        block = pool[int(table_row[i])]                # [block_size, H_kv, D]
        take = min(block_size, length - i * block_size)
        rows.append(block[:take])
    if not rows:
        return pool[:0, 0]
    return np.concatenate(rows, axis=0)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one query vector over rows of K/V, in float64.

    ``scores = scale * K q``; ``weights = softmax(scores)``; ``out = weights @ V``
    (page "vLLM推理引擎深度解析" §五: einsum of q with the keys, divide by sqrt(head_dim),
    softmax over the cached positions, weighted sum of the values). The max is subtracted
    before exponentiating, which leaves the softmax unchanged.
    """
    s = scale * (K @ q)
    m = s.max()
    p = np.exp(s - m)
    return (p @ V) / p.sum()


def paged_decode(query, k_pool, v_pool, block_tables, context_lens, scale, num_kv_heads,
                 dtype, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Decode attention: each sequence's one query per head over its ``L_b`` cached tokens.

    ``context_lens[b]`` counts the tokens in cache after this step's new token was
    written, so the new token (position ``L_b - 1``) attends to itself and all earlier
    ones. No mask is needed: every cached position precedes the query. ``L_b = 0``
    yields zeros. Returns float64 ``[B, H_q, D]``.
    """
    B, Hq, D = query.shape
    sc = _scale64(scale)
    q64 = to_f64(query, dtype)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        K = to_f64(gather(k_pool, block_tables[b], L, block_size), dtype)   # [L, H_kv, D]
        V = to_f64(gather(v_pool, block_tables[b], L, block_size), dtype)
        for h in range(Hq):
            g = kv_head_of(h, Hq, num_kv_heads)
            out[b, h] = attend(q64[b, h], K[:, g], V[:, g], sc)
    return out


def append_slot(table_row: np.ndarray, length: int, block_size: int = BLOCK_SIZE) -> int:
    """Slot of the newest token of a sequence holding ``length`` tokens: position
    ``length - 1`` sits in row ``(length-1) % block_size`` of the physical block that
    table entry ``(length-1) // block_size`` names (the append of page
    "vLLM推理引擎深度解析" §三: the last block while it has room, else a fresh block the
    manager has put at the end of the table). ``length == 0``: no token, -1."""
    if length <= 0:
        return -1
    pos = length - 1
    return int(table_row[pos // block_size]) * block_size + pos % block_size


def paged_decode_step(query, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale, num_kv_heads,
                      dtype, block_size: int = BLOCK_SIZE):
    """One decode step: each sequence's new K/V row is written at its newest position
    (``append_slot``), then every sequence attends over its ``L_b`` cached tokens.
    Returns ``(out, k_pool', v_pool')``."""
    slots = np.array([append_slot(block_tables[b], int(context_lens[b]), block_size)
                      for b in range(len(context_lens))], dtype=np.int64)
    kp, vp = scatter(k_pool, v_pool, k_new, v_new, slots, block_size)
    out = paged_decode(query, kp, vp, block_tables, context_lens, scale, num_kv_heads, dtype, block_size)
    return out, kp, vp


# ----------------------------------------------------------------------------
# split-KV: partition partials and their log-sum-exp merge
# ----------------------------------------------------------------------------
def decode_partials(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, partition: int):
    """For each token range ``[partition*p, partition*(p+1))``: (max score, sum of
    exp(score - max), normalised partial output)."""
    s_all = scale * (K @ q)
    parts = []
    for start in range(0, len(s_all), partition):
        s = s_all[start:start + partition]
        m = s.max()
        p = np.exp(s - m)
        ell = p.sum()
        parts.append((m, ell, (p @ V[start:start + partition]) / ell))
    return parts


def lse_merge(parts) -> np.ndarray:
    """Combine partials: weights ``ell_p * exp(m_p - M)`` with ``M = max_p m_p``."""
    M = max(m for m, _, _ in parts)
    w = np.array([ell * math.exp(m - M) for m, ell, _ in parts])
    o = np.array([op for _, _, op in parts])
    return (w @ o) / w.sum()


def paged_decode_splitkv(query, k_pool, v_pool, block_tables, context_lens, scale, num_kv_heads,
                         dtype, partition: int, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Split-KV decode: per-partition partials merged by log-sum-exp. Equals ``paged_decode``
    in exact arithmetic; kept to pin the decomposition itself."""
    B, Hq, D = query.shape
    sc = _scale64(scale)
    q64 = to_f64(query, dtype)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        K = to_f64(gather(k_pool, block_tables[b], L, block_size), dtype)
        V = to_f64(gather(v_pool, block_tables[b], L, block_size), dtype)
        for h in range(Hq):
            g = kv_head_of(h, Hq, num_kv_heads)
            out[b, h] = lse_merge(decode_partials(q64[b, h], K[:, g], V[:, g], sc, partition))
    return out


# ----------------------------------------------------------------------------
# chunked prefill
# ----------------------------------------------------------------------------
def visible_keys(num_keys: int, q_len: int, causal: bool) -> np.ndarray:
    """Boolean ``[q_len, num_keys]``: query ``i`` sits at absolute position
    ``num_keys - q_len + i`` and, when causal, sees keys up to and including it."""
    if not causal:
        return np.ones((q_len, num_keys), dtype=bool)
    pos = num_keys - q_len + np.arange(q_len)
    return np.arange(num_keys)[None, :] <= pos[:, None]


def paged_prefill(query, k_pool, v_pool, block_tables, seq_lens, cu_q_lens, scale, num_kv_heads,
                  dtype, causal: bool = True, block_size: int = BLOCK_SIZE,
                  seqs=None, heads=None) -> np.ndarray:
    """Attention of each chunk query over its sequence's cached keys (chunk included).

    Sequence ``b`` owns query rows ``cu_q_lens[b] .. cu_q_lens[b+1]-1``; it has
    ``seq_lens[b]`` keys in cache after the chunk was written. Query ``i`` of the chunk
    sits at absolute position ``P_i = seq_lens[b] - q_len + i``; with ``causal`` it sees
    keys ``0 .. P_i`` (itself included), otherwise all ``seq_lens[b]`` keys.
    ``seqs``/``heads`` restrict the work to a sample; other rows stay zero.
    Returns float64 ``[T, H_q, D]``.
    """
    T, Hq, D = query.shape
    sc = _scale64(scale)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    seqs = range(len(seq_lens)) if seqs is None else seqs
    heads = range(Hq) if heads is None else heads
    for b in seqs:
        q0, q1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        qlen, L = q1 - q0, int(seq_lens[b])
        if qlen == 0 or L == 0:
            continue
        K = to_f64(gather(k_pool, block_tables[b], L, block_size), dtype)
        V = to_f64(gather(v_pool, block_tables[b], L, block_size), dtype)
        Q = to_f64(query[q0:q1], dtype)                                    # [qlen, H_q, D]
        visible = visible_keys(L, qlen, causal)                            # [qlen, L]
        for h in heads:
            g = kv_head_of(h, Hq, num_kv_heads)
            S = sc * (Q[:, h] @ K[:, g].T)                                 # [qlen, L]
            S = np.where(visible, S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            P = np.exp(S - m)
            out[q0:q1, h] = (P @ V[:, g]) / P.sum(axis=1, keepdims=True)
    return out
