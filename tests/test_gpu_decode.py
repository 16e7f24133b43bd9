"""GPU parity of reshape_and_cache + pa_decode against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_463_amd as P
import workloads as W
from gpu_cases import DeviceDecode, assert_close, assert_scatter_exact, oracle_decode, out_f64, say, dev, i32

pytestmark = pytest.mark.gpu


def _run_and_check(case, split=0, seqs=None, what=None):
    what = what or f"{case.name} {case.dtype} G={case.group} D={case.head_dim} split={split}"
    say(f"case: {what}")
    d = DeviceDecode(case)
    d.scatter()
    out = d.decode(split=split)
    torch.cuda.synchronize()
    kp, vp = assert_scatter_exact(case, d.kp, d.vp)
    ref = oracle_decode(case, kp, vp, seqs)
    got = out_f64(out) if seqs is None else out_f64(out)[np.asarray(seqs)]
    assert_close(got, ref, case.dtype, what)
    return d, out


def test_tiny_fp32_config():
    _run_and_check(W.tiny_fp32())


LENS = [1, 2, 15, 16, 17, 31, 33, 64, 100, 257, 513]


@pytest.mark.parametrize("dtype", W.DTYPES)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_shapes(dtype, D, G):
    hkv = 2 if G < 8 else 1
    case = W.make_decode("shapes", dtype, LENS, G * hkv, hkv, D, seed=100 + G + D, table_pad=3)
    _run_and_check(case)


def test_zero_length_rows_are_zero():
    case = W.make_decode("zero", "bf16", [5, 40, 1], 8, 2, 128, seed=7)
    d = DeviceDecode(case)
    d.scatter()
    lens0 = case.context_lens.copy()
    lens0[1] = 0
    d.lens = i32(lens0)
    out = out_f64(d.decode())
    assert not out[1].any()
    kp, vp = oracle.scatter(case.k_pool, case.v_pool, case.k_new, case.v_new, case.slot_mapping)
    ref = oracle.paged_decode(case.query, kp, vp, case.block_tables, lens0, case.scale, 2, "bf16")
    assert_close(out, ref, "bf16", "zero-length row")


@pytest.mark.parametrize("lens", [[17] * 300, [5, 300, 16, 300] * 75, list(range(1, 601)), [0, 3, 0, 1] * 40,
                                  [(7 * i) % 61 + 1 for i in range(1100)]],
                         ids=["equal-lengths", "tied-pairs", "600-distinct", "zeros-and-ones",
                              "1100-grid-order"])
def test_many_sequences_each_written_once(lens):
    """Grid rows take sequences longest first through a bucketed ranking on the device; every
    sequence must be computed exactly once (the output starts NaN-filled). Batches above 1024
    sequences keep grid order."""
    case = W.make_decode("order", "bf16", lens, 8, 2, 64, seed=31)
    _run_and_check(case)


def test_llama2_7b_fp16_full_size():
    _run_and_check(W.llama2_7b_fp16())


def test_llama3_8b_gqa_bf16_full_size():
    _run_and_check(W.llama3_8b_gqa_bf16())


def test_block_relabelling_is_bit_identical():
    case = W.make_decode("relabel", "bf16", [7, 16, 40, 300, 1000], 32, 8, 128, seed=21)
    d = DeviceDecode(case)
    d.scatter()
    base = d.decode().clone()
    perm = np.random.default_rng(3).permutation(case.num_blocks)
    inv = torch.from_numpy(np.argsort(perm)).cuda()
    kp2, vp2 = d.kp[inv].contiguous(), d.vp[inv].contiguous()      # new id perm[i] holds old block i
    bt2 = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1)
    out2 = torch.empty_like(base)
    P.decode(out2, d.q, kp2, vp2, i32(bt2), d.lens, case.scale)
    torch.cuda.synchronize()
    assert torch.equal(base.view(torch.int16), out2.view(torch.int16))


def test_shared_prefix_equals_private_copies_bitwise():
    case = W.make_decode("shared", "bf16", [600, 700, 40, 900, 520, 70], 32, 8, 128, seed=22,
                         prefix_tokens=512, sharers=[0, 1, 3, 4])
    d = DeviceDecode(case)
    d.scatter()
    shared = d.decode().clone()
    # private copies of the 32 shared blocks for every sharer
    n_sh = len(case.shared_blocks)
    extra = n_sh * len(case.sharers)
    kp2 = torch.cat([d.kp, torch.empty((extra,) + tuple(d.kp.shape[1:]), dtype=d.kp.dtype, device="cuda")])
    vp2 = torch.cat([d.vp, torch.empty_like(kp2[-extra:])])
    bt2 = case.block_tables.copy()
    nxt = case.num_blocks
    for b in case.sharers:
        for i, blk in enumerate(case.shared_blocks):
            kp2[nxt], vp2[nxt] = d.kp[blk], d.vp[blk]
            bt2[b, i] = nxt
            nxt += 1
    out2 = torch.empty_like(shared)
    P.decode(out2, d.q, kp2, vp2, i32(bt2), d.lens, case.scale)
    torch.cuda.synchronize()
    assert torch.equal(shared.view(torch.int16), out2.view(torch.int16))


def test_rerun_is_bit_identical():
    case = W.make_decode("determinism", "f16", [33, 2048, 700, 5], 32, 32, 128, seed=23)
    d = DeviceDecode(case)
    d.scatter()
    a = d.decode().clone()
    b = d.decode(out=torch.empty_like(a))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_interleaved_block_layout():
    """Per-block (2, 16, H, D) tensors as in the pages: K plane then V plane of each block."""
    case = W.make_decode("interleaved", "f16", [3, 16, 17, 90], 8, 4, 64, seed=24)
    big = torch.empty((case.num_blocks, 2) + case.k_pool.shape[1:], dtype=torch.float16, device="cuda")
    big[:, 0] = dev(case.k_pool, "f16")
    big[:, 1] = dev(case.v_pool, "f16")
    kp, vp = big[:, 0], big[:, 1]
    q, kn, vn = dev(case.query, "f16"), dev(case.k_new, "f16"), dev(case.v_new, "f16")
    P.reshape_and_cache(kn, vn, kp, vp, i32(case.slot_mapping))
    out = torch.empty_like(q)
    P.decode(out, q, kp, vp, i32(case.block_tables), i32(case.context_lens), case.scale)
    torch.cuda.synchronize()
    rk, rv = oracle.scatter(case.k_pool, case.v_pool, case.k_new, case.v_new, case.slot_mapping)
    ref = oracle.paged_decode(case.query, rk, rv, case.block_tables, case.context_lens, case.scale, 4, "f16")
    assert_close(out_f64(out), ref, "f16", "interleaved layout")


def test_out_of_range_table_entries_do_not_fault():
    """An out-of-range block id is read as block 0 and masked: no fault, finite output."""
    case = W.make_decode("badtable", "bf16", [40, 40], 8, 2, 128, seed=25)
    d = DeviceDecode(case)
    d.scatter()
    bt = case.block_tables.copy()
    bt[1, 1] = case.num_blocks + 1000
    out = torch.empty_like(d.q)
    P.decode(out, d.q, d.kp, d.vp, i32(bt), d.lens, case.scale)
    torch.cuda.synchronize()
    kp, vp = oracle.scatter(case.k_pool, case.v_pool, case.k_new, case.v_new, case.slot_mapping)
    ref = oracle_decode(case, kp, vp, [0])
    assert_close(out_f64(out)[[0]], ref, "bf16", "untouched sequence")
    assert torch.isfinite(out.float()).all()
