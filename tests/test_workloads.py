"""Host-side harness checks (CPU only): block manager, tables, slots, poisoning, validator."""
import numpy as np
import pytest

import workloads as W


def test_allocator_exhaustion_raises_memory_error():
    a = W.BlockAllocator(5, np.random.default_rng(0))
    a.take(3)
    with pytest.raises(MemoryError):
        a.take(3)
    assert len(a.free) == 2


def test_allocator_refcounts_and_release():
    a = W.BlockAllocator(6, np.random.default_rng(1))
    ids = a.take(2)
    a.share(ids)
    assert a.ref_count[ids].tolist() == [2, 2]
    a.release(ids)
    assert a.ref_count[ids].tolist() == [1, 1] and len(a.free) == 4
    a.release(ids)
    assert len(a.free) == 6


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 3.140625], dtype=np.float32)
    bits = W.round_to(x, "bf16")
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    # 1+2^-8 is a tie between 1 and 1+2^-7 -> even (1.0); 1+3*2^-8 ties up to 1+2^-6
    assert back.tolist() == [1.0, 1.0, 1.0 + 2**-6, 1.0, -2.5, 3.140625]


def test_tiny_config_shape():
    c = W.tiny_fp32()
    assert c.context_lens.tolist() == [5, 16, 17, 40]
    assert c.num_blocks == 32 and c.head_dim == 64 and c.num_q_heads == c.num_kv_heads == 4
    used = c.block_tables[c.block_tables >= 0]
    assert len(used) == 1 + 1 + 2 + 3 and len(np.unique(used)) == len(used)
    W.validate_indices(c.num_blocks, c.block_tables, c.context_lens, c.slot_mapping)


def test_new_slots_and_free_blocks_are_poisoned():
    c = W.make_decode("t", "bf16", [3, 16, 33], 4, 2, 16, seed=2, keep_dense=True)
    flat = c.k_pool.reshape(-1, 2, 16)
    assert W.is_nan_storage(flat[c.slot_mapping], "bf16").all()
    used = set(c.block_tables[c.block_tables >= 0].tolist())
    free = [i for i in range(c.num_blocks) if i not in used]
    assert free and W.is_nan_storage(c.k_pool[free], "bf16").all()
    # prior tokens are live values
    for b in range(c.num_seqs):
        L = int(c.context_lens[b])
        for p in range(L - 1):
            s = W.slot_of(c.block_tables[b], p)
            assert not W.is_nan_storage(flat[s], "bf16").any()


def test_shared_prefix_structure():
    c = W.make_decode("t", "f16", [40, 70, 33, 90, 20], 4, 2, 16, seed=3, prefix_tokens=32,
                      sharers=[0, 1, 3], keep_dense=True)
    assert len(c.shared_blocks) == 2
    for b in c.sharers:
        assert c.block_tables[b, :2].tolist() == c.shared_blocks
    assert c.ref_count[c.shared_blocks].tolist() == [3, 3]
    # no sharer writes its new token into a shared block
    assert not set((c.slot_mapping // 16).tolist()) & set(c.shared_blocks)
    with pytest.raises(ValueError):
        W.make_decode("t", "f16", [40, 30], 4, 2, 16, seed=3, prefix_tokens=32, sharers=[0, 1])


def test_validator_rejects_bad_indices():
    c = W.make_decode("t", "f32", [3, 20], 2, 2, 8, seed=4)
    W.validate_indices(c.num_blocks, c.block_tables, c.context_lens, c.slot_mapping)
    with pytest.raises(ValueError):
        W.validate_indices(c.num_blocks, c.block_tables, c.context_lens + 16, c.slot_mapping)
    bad = c.block_tables.copy()
    bad[1, 0] = c.num_blocks
    with pytest.raises(ValueError):
        W.validate_indices(c.num_blocks, bad, c.context_lens)
    with pytest.raises(ValueError):
        W.validate_indices(c.num_blocks, c.block_tables, c.context_lens,
                           np.array([c.slot_mapping[0]] * 2, dtype=np.int32))


def test_prefill_case_layout():
    c = W.make_prefill("t", "bf16", [0, 5, 32], [9, 16, 1], 4, 2, 16, seed=5, keep_dense=True)
    assert c.cu_q_lens.tolist() == [0, 9, 25, 26]
    assert c.seq_lens.tolist() == [9, 21, 33]
    # the chunk's slots follow the table at positions prior .. prior+q_len-1
    for b in range(3):
        for i in range(int(c.q_lens[b])):
            s = c.slot_mapping[c.cu_q_lens[b] + i]
            assert s == W.slot_of(c.block_tables[b], int(c.prior_lens[b]) + i)
    W.validate_indices(c.num_blocks, c.block_tables, c.seq_lens, c.slot_mapping)


def test_named_configs_are_seeded():
    a, b = W.tiny_fp32(), W.tiny_fp32()
    assert a.k_pool.tobytes() == b.k_pool.tobytes() and a.query.tobytes() == b.query.tobytes()
    assert not np.array_equal(a.query, W.tiny_fp32(seed=7).query)
