"""Pins of the CPU oracle against things other than itself (CPU only).

Each pin is a function returning an error figure, so the mutation tests at the
end can plant a mistake in the oracle and show that some pin catches it.

Pins used:
* torch's float64 ``scaled_dot_product_attention`` (a library routine) on the
  contiguous per-sequence K/V the generator built before paging them;
* a 40-digit ``decimal`` brute force on tiny inputs;
* closed forms (one key, zero query, constant values, one dominant key);
* invariants: relabelling physical blocks, shared prefix blocks versus private
  copies, NaN in slots that hold no live token;
* the flat-slot view of the pool for the scatter (a NumPy fancy-index write);
* golden slot positions worked by hand from the pages' append rule.
"""
import decimal
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.paged_attention as OPA
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "slot_positions.json")


# ----------------------------------------------------------------------------
# pin functions
# ----------------------------------------------------------------------------
def _sdpa(q, K, V, scale, mask=None):
    """torch fp64 SDPA on [H_q, Lq, D] x [H_kv, L, D] with grouped heads."""
    return F.scaled_dot_product_attention(q, K, V, attn_mask=mask, scale=scale, enable_gqa=True)


def pin_decode_vs_sdpa(case: W.DecodeCase) -> float:
    out = oracle.paged_decode(case.query, *_scattered(case), case.block_tables, case.context_lens,
                              case.scale, case.num_kv_heads, case.dtype)
    err = 0.0
    for b in range(case.num_seqs):
        L = int(case.context_lens[b])
        q = torch.from_numpy(oracle.to_f64(case.query[b], case.dtype))[:, None, :]       # [Hq,1,D]
        K = torch.from_numpy(oracle.to_f64(case.dense_k[b], case.dtype)).permute(1, 0, 2)  # [Hkv,L,D]
        V = torch.from_numpy(oracle.to_f64(case.dense_v[b], case.dtype)).permute(1, 0, 2)
        ref = _sdpa(q, K, V, float(np.float32(case.scale)))[:, 0, :].numpy()
        if L == 0:
            ref = np.zeros_like(ref)
        err = max(err, _maxerr(out[b], ref))
    return err


def pin_prefill_vs_sdpa(case: W.PrefillCase, causal=True) -> float:
    kp, vp = oracle.scatter(case.k_pool, case.v_pool, case.k_new, case.v_new, case.slot_mapping)
    out = oracle.paged_prefill(case.query, kp, vp, case.block_tables, case.seq_lens, case.cu_q_lens,
                               case.scale, case.num_kv_heads, case.dtype, causal=causal)
    err = 0.0
    for b in range(case.num_seqs):
        q0, q1 = int(case.cu_q_lens[b]), int(case.cu_q_lens[b + 1])
        qlen, L = q1 - q0, int(case.seq_lens[b])
        if qlen == 0:
            continue
        q = torch.from_numpy(oracle.to_f64(case.query[q0:q1], case.dtype)).permute(1, 0, 2)
        K = torch.from_numpy(oracle.to_f64(case.dense_k[b], case.dtype)).permute(1, 0, 2)
        V = torch.from_numpy(oracle.to_f64(case.dense_v[b], case.dtype)).permute(1, 0, 2)
        # bottom-right aligned causal mask built from torch ops, independent of the oracle's
        mask = torch.ones(qlen, L, dtype=torch.bool)
        if causal:
            mask = torch.tril(mask, diagonal=L - qlen)
        ref = _sdpa(q, K, V, float(np.float32(case.scale)), mask).permute(1, 0, 2).numpy()
        err = max(err, _maxerr(out[q0:q1], ref))
    return err


def _maxerr(a, b) -> float:
    """Max abs difference; a NaN anywhere counts as an infinite error."""
    d = np.abs(np.asarray(a) - np.asarray(b))
    return float("inf") if not np.isfinite(d).all() else float(d.max(initial=0.0))


def _scattered(case):
    return oracle.scatter(case.k_pool, case.v_pool, case.k_new, case.v_new, case.slot_mapping)


def _decimal_attention(q, K, V, scale, digits=40):
    ctx = decimal.Context(prec=digits)
    D = decimal.Decimal
    sc = D(float(scale))
    s = [ctx.multiply(sc, sum((D(float(a)) * D(float(b)) for a, b in zip(q, k)), D(0))) for k in K]
    m = max(s)
    p = [ctx.exp(x - m) for x in s]
    tot = sum(p, D(0))
    return np.array([float(sum((pi * D(float(v[d])) for pi, v in zip(p, V)), D(0)) / tot)
                     for d in range(len(V[0]))])


def _small_decode(dtype, G=2, Hkv=2, D=16, lens=(1, 15, 16, 17, 33, 64), seed=11, **kw):
    return W.make_decode("pin", dtype, list(lens), G * Hkv, Hkv, D, seed, keep_dense=True, **kw)


# ----------------------------------------------------------------------------
# scatter and slots
# ----------------------------------------------------------------------------
def test_golden_slot_positions():
    g = json.load(open(GOLDEN))
    bs = g["block_size"]
    for c in g["new_token_position"]["cases"]:
        n = c["cached_before"]
        row = np.arange(1000, 1000 + n // bs + 1)            # any distinct physical ids
        slot = W.slot_of(row, n)
        assert (slot // bs - 1000, slot % bs) == (c["logical_block"], c["offset"])
        assert (n % bs == 0) == c["fresh_block"]
    for tokens, blocks in g["blocks_needed"]["cases"]:
        assert W.ceil_div(tokens, bs) == blocks
        assert math.ceil(tokens / bs) == blocks
    kb = g["kv_bytes_per_token"]
    assert 2 * kb["layers"] * kb["kv_heads"] * kb["head_dim"] * kb["elem_bytes"] == kb["all_layers"]
    assert kb["all_layers"] // kb["layers"] == kb["one_layer"]


def test_tiny_case_slots_follow_append_rule():
    c = W.tiny_fp32()
    got = [(int(np.where(c.block_tables[b] == s // 16)[0][0]), int(s % 16))
           for b, s in enumerate(c.slot_mapping)]
    assert got == [(0, 4), (0, 15), (1, 0), (2, 7)]


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_scatter_matches_flat_slot_write(dtype):
    rng = np.random.default_rng(0)
    nb, H, D = 9, 3, 8
    kp = W.normal(rng, (nb, 16, H, D), dtype)
    vp = W.normal(rng, (nb, 16, H, D), dtype)
    slots = rng.choice(nb * 16, size=20, replace=False).astype(np.int32)
    slots[[3, 7]] = -1
    key = W.normal(rng, (20, H, D), dtype)
    val = W.normal(rng, (20, H, D), dtype)
    ok, ov = oracle.scatter(kp, vp, key, val, slots)
    live = slots >= 0
    rk = kp.copy().reshape(nb * 16, H, D)
    rv = vp.copy().reshape(nb * 16, H, D)
    rk[slots[live]] = key[live]
    rv[slots[live]] = val[live]
    assert ok.tobytes() == rk.reshape(kp.shape).tobytes()
    assert ov.tobytes() == rv.reshape(vp.shape).tobytes()
    # untouched slots keep their bits, inputs are not modified
    untouched = np.setdiff1d(np.arange(nb * 16), slots[live])
    assert ok.reshape(nb * 16, H, D)[untouched].tobytes() == kp.reshape(nb * 16, H, D)[untouched].tobytes()


def test_append_slot_matches_golden_positions():
    g = json.load(open(GOLDEN))
    bs = g["block_size"]
    for c in g["new_token_position"]["cases"]:
        n = c["cached_before"]                                 # the new token makes it n + 1
        row = np.arange(1000, 1000 + n // bs + 1)
        slot = oracle.append_slot(row, n + 1)
        assert (slot // bs - 1000, slot % bs) == (c["logical_block"], c["offset"])
    assert oracle.append_slot(np.array([5]), 0) == -1


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_step_equals_scatter_then_decode(dtype):
    """The step writes each new token where the harness's append rule put it (the slots are
    derived independently, from the case's own slot_mapping) and then decodes."""
    c = _small_decode(dtype, lens=(0, 1, 15, 16, 17, 33, 64))
    out, kp, vp = oracle.paged_decode_step(c.query, c.k_new, c.v_new, c.k_pool, c.v_pool, c.block_tables,
                                           c.context_lens, c.scale, c.num_kv_heads, dtype)
    rk, rv = oracle.scatter(c.k_pool, c.v_pool, c.k_new, c.v_new, c.slot_mapping)
    assert kp.tobytes() == rk.tobytes() and vp.tobytes() == rv.tobytes()
    ref = oracle.paged_decode(c.query, rk, rv, c.block_tables, c.context_lens, c.scale, c.num_kv_heads, dtype)
    assert np.array_equal(out, ref)
    assert np.all(out[0] == 0)                                 # empty sequence: zeros, nothing written


def test_mutation_append_slot_off_by_one_is_caught(monkeypatch):
    def bad(table_row, length, block_size=16):
        return -1 if length <= 0 else int(table_row[length // block_size]) * block_size + length % block_size
    monkeypatch.setattr(OPA, "append_slot", bad)
    with pytest.raises((AssertionError, IndexError)):
        test_decode_step_equals_scatter_then_decode("f32")


def test_scatter_then_gather_returns_new_token():
    c = _small_decode("bf16")
    kp, vp = _scattered(c)
    for b in range(c.num_seqs):
        L = int(c.context_lens[b])
        assert oracle.gather(kp, c.block_tables[b], L)[L - 1].tobytes() == c.k_new[b].tobytes()
        assert oracle.gather(vp, c.block_tables[b], L)[L - 1].tobytes() == c.v_new[b].tobytes()
        assert oracle.gather(kp, c.block_tables[b], L).tobytes() == c.dense_k[b].tobytes()


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,G,Hkv,D", [("f32", 1, 4, 64), ("f16", 1, 3, 32), ("bf16", 4, 2, 16),
                                          ("bf16", 8, 1, 8), ("f16", 2, 2, 128)])
def test_decode_matches_sdpa(dtype, G, Hkv, D):
    c = _small_decode(dtype, G=G, Hkv=Hkv, D=D)
    assert pin_decode_vs_sdpa(c) < 1e-12


def test_tiny_config_matches_sdpa():
    assert pin_decode_vs_sdpa(W.tiny_fp32()) < 1e-12


def test_decode_matches_decimal_bruteforce():
    rng = np.random.default_rng(5)
    for L in (1, 2, 5):
        q = rng.standard_normal(3)
        K = rng.standard_normal((L, 3)) * 2
        V = rng.standard_normal((L, 3))
        got = oracle.attend(q, K, V, 0.7)
        ref = _decimal_attention(q, K, V, 0.7)      # same binary64 scale on both sides
        assert np.abs(got - ref).max() < 1e-14


def test_closed_forms():
    rng = np.random.default_rng(6)
    q = rng.standard_normal(8)
    K = rng.standard_normal((33, 8))
    V = rng.standard_normal((33, 8))
    # a single key returns its value exactly
    assert np.array_equal(oracle.attend(q, K[:1], V[:1], 0.3), V[0])
    # a zero query weights every value equally
    assert np.abs(oracle.attend(np.zeros(8), K, V, 0.3) - V.mean(axis=0)).max() < 1e-15
    # constant values come back unchanged
    C = np.tile(rng.standard_normal(8), (33, 1))
    assert np.abs(oracle.attend(q, K, C, 0.3) - C[0]).max() < 1e-15
    # one key whose score dominates by > 50 returns its value
    K2 = K.copy()
    K2[17] = q / np.linalg.norm(q) * 400.0
    assert np.abs(oracle.attend(q, K2, V, 1.0) - V[17]).max() < 1e-15
    # scores shifted by a constant leave the result unchanged (softmax shift invariance)
    out1 = oracle.attend(q, K, V, 0.5)
    qs = np.concatenate([q, [1.0]])
    Ks = np.concatenate([K, np.full((33, 1), 7.0)], axis=1)
    assert np.abs(oracle.attend(qs, Ks, V, 0.5) - out1).max() < 1e-13


def test_zero_length_sequence_gives_zeros():
    c = _small_decode("f32", lens=(3, 20))
    lens = c.context_lens.copy()
    lens[0] = 0
    out = oracle.paged_decode(c.query, *_scattered(c), c.block_tables, lens, c.scale,
                              c.num_kv_heads, c.dtype)
    assert not out[0].any() and out[1].any()


def _relabel(case, seed):
    """Move every physical block to a new id; tables follow."""
    perm = np.random.default_rng(seed).permutation(case.num_blocks)
    kp, vp = _scattered(case)
    nk, nv = np.empty_like(kp), np.empty_like(vp)
    nk[perm] = kp
    nv[perm] = vp
    bt = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1)
    return nk, nv, bt


def test_block_relabelling_is_bitwise_invariant():
    c = _small_decode("bf16", G=4, Hkv=2, D=32, lens=(7, 16, 40, 100))
    base = oracle.paged_decode(c.query, *_scattered(c), c.block_tables, c.context_lens, c.scale,
                               c.num_kv_heads, c.dtype)
    for seed in range(3):
        nk, nv, bt = _relabel(c, seed)
        out = oracle.paged_decode(c.query, nk, nv, bt, c.context_lens, c.scale, c.num_kv_heads, c.dtype)
        assert out.tobytes() == base.tobytes()


def _unshare(case):
    """Give every sharer private copies of the shared prefix blocks."""
    kp, vp = _scattered(case)
    n_sh = len(case.shared_blocks)
    extra = n_sh * len(case.sharers)
    nk = np.concatenate([kp, np.empty((extra,) + kp.shape[1:], kp.dtype)])
    nv = np.concatenate([vp, np.empty((extra,) + vp.shape[1:], vp.dtype)])
    bt = case.block_tables.copy()
    nxt = case.num_blocks
    for b in case.sharers:
        for i, blk in enumerate(case.shared_blocks):
            nk[nxt], nv[nxt] = kp[blk], vp[blk]
            assert bt[b, i] == blk
            bt[b, i] = nxt
            nxt += 1
    return nk, nv, bt


def test_shared_prefix_equals_private_copies():
    c = _small_decode("bf16", G=4, Hkv=2, D=32, lens=(40, 70, 33, 90, 20), prefix_tokens=32,
                      sharers=[0, 1, 3])
    assert c.ref_count[c.shared_blocks].tolist() == [3, 3]
    shared = oracle.paged_decode(c.query, *_scattered(c), c.block_tables, c.context_lens, c.scale,
                                 c.num_kv_heads, c.dtype)
    nk, nv, bt = _unshare(c)
    private = oracle.paged_decode(c.query, nk, nv, bt, c.context_lens, c.scale, c.num_kv_heads, c.dtype)
    assert shared.tobytes() == private.tobytes()
    assert pin_decode_vs_sdpa(c) < 1e-12


def test_poisoned_slots_never_reach_the_output():
    c = _small_decode("f16", lens=(3, 17, 31))
    kp, vp = _scattered(c)
    assert W.is_nan_storage(kp, c.dtype).any()      # free blocks and tails are poisoned
    out = oracle.paged_decode(c.query, kp, vp, c.block_tables, c.context_lens, c.scale,
                              c.num_kv_heads, c.dtype)
    assert np.isfinite(out).all()


# ----------------------------------------------------------------------------
# split-KV
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("partition", [16, 48, 512, 4096])
def test_lse_merge_reaches_direct_result(partition):
    rng = np.random.default_rng(partition)
    for L in (1, 17, 600, 1500):
        q = rng.standard_normal(64)
        K = rng.standard_normal((L, 64)) * 1.5
        V = rng.standard_normal((L, 64))
        parts = oracle.decode_partials(q, K, V, 0.125, partition)
        assert len(parts) == math.ceil(L / partition)
        assert np.abs(oracle.lse_merge(parts) - oracle.attend(q, K, V, 0.125)).max() < 1e-14


def test_splitkv_oracle_equals_decode_oracle():
    c = _small_decode("bf16", G=8, Hkv=1, D=32, lens=(1, 16, 100, 513))
    kp, vp = _scattered(c)
    a = oracle.paged_decode(c.query, kp, vp, c.block_tables, c.context_lens, c.scale, 1, c.dtype)
    for part in (16, 64, 512):
        s = oracle.paged_decode_splitkv(c.query, kp, vp, c.block_tables, c.context_lens, c.scale, 1,
                                        c.dtype, part)
        assert np.abs(a - s).max() < 1e-14


# ----------------------------------------------------------------------------
# prefill
# ----------------------------------------------------------------------------
def _small_prefill(dtype="bf16", prior=(0, 5, 32, 47), qlens=(9, 16, 1, 37), G=4, Hkv=2, D=16, seed=3):
    return W.make_prefill("pin", dtype, list(prior), list(qlens), G * Hkv, Hkv, D, seed, keep_dense=True)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_matches_sdpa(causal):
    assert pin_prefill_vs_sdpa(_small_prefill(), causal) < 1e-12


def test_prefill_causality():
    c = _small_prefill(prior=(20,), qlens=(30,), G=2, Hkv=2)
    kp, vp = oracle.scatter(c.k_pool, c.v_pool, c.k_new, c.v_new, c.slot_mapping)
    base = oracle.paged_prefill(c.query, kp, vp, c.block_tables, c.seq_lens, c.cu_q_lens, c.scale,
                                c.num_kv_heads, c.dtype)
    cut = 33                         # perturb keys at positions >= 33
    kq, vq = kp.copy(), vp.copy()
    for j in range(cut, int(c.seq_lens[0])):
        blk, off = c.block_tables[0, j // 16], j % 16
        kq[blk, off] = W.normal(np.random.default_rng(j), kq.shape[2:], c.dtype)
        vq[blk, off] = W.normal(np.random.default_rng(j + 999), vq.shape[2:], c.dtype)
    pert = oracle.paged_prefill(c.query, kq, vq, c.block_tables, c.seq_lens, c.cu_q_lens, c.scale,
                                c.num_kv_heads, c.dtype)
    first_affected = cut - int(c.prior_lens[0])          # query i sits at position prior + i
    assert pert[:first_affected].tobytes() == base[:first_affected].tobytes()
    assert not np.array_equal(pert[first_affected:], base[first_affected:])


def test_prefill_last_query_equals_decode():
    c = _small_prefill(prior=(40, 3), qlens=(24, 13), G=4, Hkv=2, D=32)
    kp, vp = oracle.scatter(c.k_pool, c.v_pool, c.k_new, c.v_new, c.slot_mapping)
    pre = oracle.paged_prefill(c.query, kp, vp, c.block_tables, c.seq_lens, c.cu_q_lens, c.scale,
                               c.num_kv_heads, c.dtype)
    last = c.cu_q_lens[1:] - 1
    dec = oracle.paged_decode(c.query[last], kp, vp, c.block_tables, c.seq_lens, c.scale,
                              c.num_kv_heads, c.dtype)
    assert np.abs(pre[last] - dec).max() < 1e-14


# ----------------------------------------------------------------------------
# mutation tests: plant a mistake in the oracle, some pin must catch it
# ----------------------------------------------------------------------------
def test_mutation_wrong_gqa_mapping_is_caught(monkeypatch):
    c = _small_decode("f32", G=4, Hkv=2, D=16)
    monkeypatch.setattr(OPA, "kv_head_of", lambda h, hq, hkv: h % hkv)
    assert pin_decode_vs_sdpa(c) > 1e-3


def test_mutation_missing_scale_is_caught(monkeypatch):
    c = _small_decode("f32")
    monkeypatch.setattr(OPA, "_scale64", lambda s: 1.0)
    assert pin_decode_vs_sdpa(c) > 1e-3


def test_mutation_gather_token_order_is_caught(monkeypatch):
    # decode attention cannot see key order, causal prefill can
    c = _small_prefill()
    real = OPA.gather
    monkeypatch.setattr(OPA, "gather", lambda pool, row, length, block_size=16:
                        np.roll(real(pool, row, length, block_size), 1, axis=0))
    assert not pin_prefill_vs_sdpa(c) < 1e-3


def test_mutation_gather_wrong_block_is_caught(monkeypatch):
    c = _small_decode("f32", lens=(20, 40, 64))
    real = OPA.gather

    def wrong(pool, row, length, block_size=16):
        return real(pool, np.roll(np.asarray(row)[:W.ceil_div(length, 16)], 1), length, block_size)
    monkeypatch.setattr(OPA, "gather", wrong)
    assert not pin_decode_vs_sdpa(c) < 1e-3


def test_mutation_gather_reading_whole_last_block_is_caught(monkeypatch):
    c = _small_decode("f32", lens=(20, 40))
    real = OPA.gather
    monkeypatch.setattr(OPA, "gather", lambda pool, row, length, block_size=16:
                        real(pool, row, W.ceil_div(length, 16) * 16, block_size))
    assert not pin_decode_vs_sdpa(c) < 1e-3      # NaN tails or extra keys


def test_mutation_causal_off_by_one_is_caught(monkeypatch):
    c = _small_prefill()
    real = OPA.visible_keys
    monkeypatch.setattr(OPA, "visible_keys", lambda L, q, causal: np.roll(real(L, q, causal), -1, axis=1))
    assert not pin_prefill_vs_sdpa(c) < 1e-3


def test_mutation_unmasked_prefill_is_caught(monkeypatch):
    c = _small_prefill()
    monkeypatch.setattr(OPA, "visible_keys", lambda L, q, causal: np.ones((q, L), bool))
    assert pin_prefill_vs_sdpa(c) > 1e-3


def test_mutation_merge_without_rescale_is_caught(monkeypatch):
    rng = np.random.default_rng(9)
    q, K, V = rng.standard_normal(32), rng.standard_normal((300, 32)) * 2, rng.standard_normal((300, 32))
    direct = oracle.attend(q, K, V, 0.2)

    def bad_merge(parts):
        w = np.array([ell for _, ell, _ in parts])
        return (w @ np.array([o for _, _, o in parts])) / w.sum()
    monkeypatch.setattr(OPA, "lse_merge", bad_merge)
    assert np.abs(OPA.lse_merge(OPA.decode_partials(q, K, V, 0.2, 64)) - direct).max() > 1e-3


def test_mutation_scatter_offset_is_caught(monkeypatch):
    c = _small_decode("f32", lens=(5, 17))
    real = OPA.scatter

    def bad(kp, vp, key, val, slots, block_size=16):
        return real(kp, vp, key, val, np.where(slots >= 0, slots + 1, slots), block_size)
    monkeypatch.setattr(OPA, "scatter", bad)
    kp, vp = OPA.scatter(c.k_pool, c.v_pool, c.k_new, c.v_new, c.slot_mapping)
    L = int(c.context_lens[0])
    assert OPA.gather(kp, c.block_tables[0], L)[L - 1].tobytes() != c.k_new[0].tobytes()
